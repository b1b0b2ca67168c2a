// Embedding backward: dwte[v] += sum of dx0 rows whose token is v, and
// dwpe[p] += sum of dx0 rows at position p (the scatter-add that inverts the
// gather x0 = wte[tok] + wpe[pos]; Feste page, "Model Architecture" for the
// forward, "Manual Backpropagation" for the chain rule).
//
// Deterministic and atomic-free in floating point: a stable counting sort of
// the keys (integer atomics for the counts, whose result is order-free; each
// row's slot is the count of equal keys before it) lists every key's rows in
// ascending index order. Rows are then summed in that order in chunks of
// kSegRows rows (so a hot token, id 0 under a Zipf law carries ~14% of the
// rows, is spread over many blocks), and a key's chunk sums are added in
// chunk order.
#include "kernels.h"

namespace lm {

long embed_bwd_max_chunks(int M, int nkeys) {
  long distinct = M < nkeys ? M : nkeys;
  return (long)M / kSegRows + distinct + 1;
}

__device__ __forceinline__ int clamp_key(int k, int nkeys) { return k < 0 ? 0 : (k >= nkeys ? nkeys - 1 : k); }

__global__ void csr_count_kernel(const int32_t* __restrict__ keys, int M, int nkeys, int32_t* __restrict__ counts) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < M) atomicAdd(&counts[clamp_key(keys[i], nkeys)], 1);
}

// Exclusive scans of counts (-> offsets) and of ceil(count / kSegRows)
// (-> chunk_base), each with nkeys + 1 entries. One block of 1024 threads;
// every thread scans a contiguous slice serially (its loads issued in
// batches of 8), then the slice totals are scanned in LDS.
__global__ void __launch_bounds__(1024) csr_scan_kernel(const int32_t* __restrict__ counts, int nkeys,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ chunk_base) {
  __shared__ int s_a[1024], s_b[1024];
  const int n = nkeys + 1;
  const int per = (n + 1023) / 1024;
  const int t = threadIdx.x, lo = t * per, hi = min(n, lo + per);
  auto cnt = [&](int v) { return v < hi && v < nkeys ? counts[v] : 0; };
  int sa = 0, sb = 0;
  for (int v = lo; v < hi; v += 8) {
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = cnt(v + u);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sa += c[u];
      sb += (c[u] + kSegRows - 1) / kSegRows;
    }
  }
  s_a[t] = sa;
  s_b[t] = sb;
  __syncthreads();
  // Hillis-Steele inclusive scan of the 1024 slice totals
  for (int o = 1; o < 1024; o <<= 1) {
    int a = t >= o ? s_a[t - o] : 0, b = t >= o ? s_b[t - o] : 0;
    __syncthreads();
    s_a[t] += a;
    s_b[t] += b;
    __syncthreads();
  }
  int ra = s_a[t] - sa, rb = s_b[t] - sb;
  for (int v = lo; v < hi; v += 8) {
    int c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = cnt(v + u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (v + u < hi) {
        offsets[v + u] = ra;
        chunk_base[v + u] = rb;
        ra += c[u];
        rb += (c[u] + kSegRows - 1) / kSegRows;
      }
  }
}

// rank[i] += #{j < i in row block jb : key_j == key_i} for the rows i of row
// block b (blocks of 256 rows; grid (b, jb), jb <= b). Integer sums, so the
// result does not depend on the order of the atomic additions.
__global__ void __launch_bounds__(256) csr_rank_kernel(const int32_t* __restrict__ keys, int M, int nkeys,
                                                       int32_t* __restrict__ rank) {
  const int b = blockIdx.x, jb = blockIdx.y;
  if (jb > b) return;
  __shared__ int s_k[256];
  const int j = jb * 256 + threadIdx.x;
  s_k[threadIdx.x] = j < M ? clamp_key(keys[j], nkeys) : -2;
  __syncthreads();
  const int i = b * 256 + threadIdx.x;
  if (i >= M) return;
  const int my = clamp_key(keys[i], nkeys);
  const int lim = jb == b ? (int)threadIdx.x : 256;
  int cnt = 0;
#pragma unroll 8
  for (int q = 0; q < lim; ++q) cnt += (s_k[q] == my);
  if (cnt) atomicAdd(&rank[i], cnt);
}

// perm[offsets[key_i] + rank_i] = i.
__global__ void __launch_bounds__(256) csr_place_kernel(const int32_t* __restrict__ keys, int M, int nkeys,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ rank,
                                                        int32_t* __restrict__ perm) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < M) perm[offsets[clamp_key(keys[i], nkeys)] + rank[i]] = i;
}

__device__ __forceinline__ int find_key(const int32_t* __restrict__ chunk_base, int nkeys, int w) {
  // largest v in [0, nkeys) with chunk_base[v] <= w
  int lo = 0, hi = nkeys - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (chunk_base[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One block per chunk (grid-stride): sum its rows in sorted order. A key with
// a single chunk is added to dst directly; otherwise the chunk sum goes to
// partial[w].
__global__ void __launch_bounds__(256) segsum_chunks_kernel(const float* __restrict__ dx, int C, int nkeys,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ perm,
                                                            float* __restrict__ partial, float* __restrict__ dst) {
  const int total = chunk_base[nkeys];
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int v = find_key(chunk_base, nkeys, w);
    const int j = w - chunk_base[v];
    const int s0 = offsets[v] + j * kSegRows;
    const int s1 = min(offsets[v + 1], s0 + kSegRows);
    const bool single = (chunk_base[v + 1] - chunk_base[v]) == 1;
    for (int c = threadIdx.x; c < C; c += 256) {
      float acc = 0.f;
      for (int s = s0; s < s1; ++s) acc += dx[(long)perm[s] * C + c];
      if (single) dst[(long)v * C + c] += acc;
      else partial[(long)w * C + c] = acc;
    }
  }
}

__global__ void __launch_bounds__(256) segsum_keys_kernel(int C, int nkeys, const int32_t* __restrict__ chunk_base,
                                                          const float* __restrict__ partial,
                                                          float* __restrict__ dst) {
  for (int v = blockIdx.x; v < nkeys; v += gridDim.x) {
    const int b0 = chunk_base[v], b1 = chunk_base[v + 1];
    if (b1 - b0 <= 1) continue;
    for (int c = threadIdx.x; c < C; c += 256) {
      float acc = 0.f;
      for (int w = b0; w < b1; ++w) acc += partial[(long)w * C + c];
      dst[(long)v * C + c] += acc;
    }
  }
}

void launch_csr(const int32_t* keys, int M, int nkeys, EmbedBwdWs ws, hipStream_t s) {
  launch_fill_u32(reinterpret_cast<uint32_t*>(ws.counts), 0u, nkeys + 1, s);
  if (M > 0) hipLaunchKernelGGL(csr_count_kernel, dim3((M + 255) / 256), dim3(256), 0, s, keys, M, nkeys, ws.counts);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, ws.counts, nkeys, ws.offsets, ws.chunk_base);
  if (M > 0) {
    const int nb = (M + 255) / 256;
    launch_fill_u32(reinterpret_cast<uint32_t*>(ws.rank), 0u, M, s);
    hipLaunchKernelGGL(csr_rank_kernel, dim3(nb, nb), dim3(256), 0, s, keys, M, nkeys, ws.rank);
    hipLaunchKernelGGL(csr_place_kernel, dim3(nb), dim3(256), 0, s, keys, M, nkeys, ws.offsets, ws.rank, ws.perm);
  }
}

void launch_segment_sum(const float* dx, const int32_t* keys, int M, int C, int nkeys, EmbedBwdWs ws, float* dst,
                        bool accumulate, hipStream_t s) {
  (void)keys;
  if (!accumulate) launch_fill_u32(reinterpret_cast<uint32_t*>(dst), 0u, (long)nkeys * C, s);
  long maxc = embed_bwd_max_chunks(M, nkeys);
  unsigned g1 = (unsigned)(maxc < 4096 ? maxc : 4096);
  hipLaunchKernelGGL(segsum_chunks_kernel, dim3(g1), dim3(256), 0, s, dx, C, nkeys, ws.offsets, ws.chunk_base,
                     ws.perm, ws.partial, dst);
  unsigned g2 = (unsigned)(nkeys < 1024 ? nkeys : 1024);
  hipLaunchKernelGGL(segsum_keys_kernel, dim3(g2), dim3(256), 0, s, C, nkeys, ws.chunk_base, ws.partial, dst);
}

}  // namespace lm
