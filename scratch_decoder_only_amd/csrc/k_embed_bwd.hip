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

// counts[v] = #rows with key v. Each block of 256 rows first counts its equal
// keys in LDS and only the first row of each key adds the block's count: a
// Zipf-hot key (token id 0 holds ~14% of the rows) then takes one atomic
// addition per block instead of one per row, which serialised on its
// counter. Integer sums: the result does not depend on their order. hist
// (nullable, zeroed [blocks][nkeys]): the same first row also records the
// block's count of its key.
__global__ void __launch_bounds__(256) csr_count_kernel(const int32_t* __restrict__ keys, int M, int nkeys,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ hist) {
  __shared__ int s_k[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int my = i < M ? clamp_key(keys[i], nkeys) : -1;
  s_k[threadIdx.x] = my;
  __syncthreads();
  if (my < 0) return;
  int cnt = 0;
  bool first = true;
#pragma unroll 8
  for (int q = 0; q < 256; ++q) {
    const bool eq = s_k[q] == my;
    cnt += eq;
    first = first && !(eq && q < (int)threadIdx.x);
  }
  if (first) {
    atomicAdd(&counts[my], cnt);
    if (hist) hist[(long)blockIdx.x * nkeys + my] = cnt;
  }
}

// Linear-time rank (many row blocks): hist[b][v] becomes the number of rows
// of key v in blocks before b (an exclusive scan over the blocks, one thread
// per key, consecutive keys on consecutive threads).
// (the counts of 16 blocks are loaded before any is overwritten: a load
// after each store of the same array left a memory latency per block)
__global__ void __launch_bounds__(256) csr_block_prefix_kernel(int32_t* __restrict__ hist, int nb, int nkeys) {
  const int v = blockIdx.x * 256 + threadIdx.x;
  if (v >= nkeys) return;
  constexpr int G = 16;
  int run = 0;
  for (int b0 = 0; b0 < nb; b0 += G) {
    int c[G];
#pragma unroll
    for (int i = 0; i < G; ++i) c[i] = b0 + i < nb ? hist[(long)(b0 + i) * nkeys + v] : 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      if (b0 + i < nb) hist[(long)(b0 + i) * nkeys + v] = run;
      run += c[i];
    }
  }
}

// perm[offsets[key_i] + (rows of key_i in earlier blocks) + (rows of key_i
// before i in its block)] = i, the last term counted in LDS.
__global__ void __launch_bounds__(256) csr_place_blocks_kernel(const int32_t* __restrict__ keys, int M, int nkeys,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ hist,
                                                               int32_t* __restrict__ perm) {
  __shared__ int s_k[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int my = i < M ? clamp_key(keys[i], nkeys) : -1;
  s_k[threadIdx.x] = my;
  __syncthreads();
  if (my < 0) return;
  int before = 0;
  for (int q = 0; q < (int)threadIdx.x; ++q) before += (s_k[q] == my);
  perm[offsets[my] + hist[(long)blockIdx.x * nkeys + my] + before] = i;
}

// Exclusive scans of counts (-> offsets) and of ceil(count / kSegRows)
// (-> chunk_base), each with nkeys + 1 entries, by one block of 512 threads
// in rounds of 4096 keys, the loads of RB rounds issued at once (8
// consecutive keys per thread per round, held in registers), so the memory
// latency is paid once per RB rounds rather than once per round: per round a
// wavefront scan; then the first wavefront turns the wavefront totals of the
// batch into exclusive prefixes in LDS (carrying the running totals between
// batches), and each thread writes its keys.
template <int RB>
__global__ void __launch_bounds__(512) csr_scan_pre_kernel(const int32_t* __restrict__ counts, int nkeys,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ chunk_base) {
  constexpr int NW = 8, KPT = 8, RK = 512 * KPT;
  __shared__ int s_a[RB][NW], s_b[RB][NW];
  const int n = nkeys + 1;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int carry_a = 0, carry_b = 0;  // (wavefront 0)
  for (int base = 0; base < n; base += RB * RK) {
    int c[RB][KPT];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int i0 = base + r * RK + t * KPT;
      if (i0 + KPT <= nkeys) {  // two 16-byte loads (the arrays are 16-byte aligned)
        const int4 lo = *reinterpret_cast<const int4*>(counts + i0), hi = *reinterpret_cast<const int4*>(counts + i0 + 4);
        c[r][0] = lo.x; c[r][1] = lo.y; c[r][2] = lo.z; c[r][3] = lo.w;
        c[r][4] = hi.x; c[r][5] = hi.y; c[r][6] = hi.z; c[r][7] = hi.w;
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u) c[r][u] = i0 + u < nkeys ? counts[i0 + u] : 0;
      }
    }
    int ea[RB], eb[RB];  // exclusive prefix of the thread's keys within its wavefront
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      int a = 0, b = 0;
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        a += c[r][u];
        b += (c[r][u] + kSegRows - 1) / kSegRows;
      }
      int xa = a, xb = b;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int ya = __shfl_up(xa, o, 64), yb = __shfl_up(xb, o, 64);
        if (lane >= o) {
          xa += ya;
          xb += yb;
        }
      }
      ea[r] = xa - a;
      eb[r] = xb - b;
      if (lane == 63) {
        s_a[r][w] = xa;
        s_b[r][w] = xb;
      }
    }
    __syncthreads();
    if (w == 0) {
      // the RB x NW wavefront totals of the batch, one per lane in key order,
      // scanned across the wavefront
      static_assert(RB * NW <= 64, "one wavefront holds the batch's totals");
      const int r = lane / NW, q = lane % NW;
      const bool in = lane < RB * NW;
      const int va = in ? s_a[r][q] : 0, vb = in ? s_b[r][q] : 0;
      int xa = va, xb = vb;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int ya = __shfl_up(xa, o, 64), yb = __shfl_up(xb, o, 64);
        if (lane >= o) {
          xa += ya;
          xb += yb;
        }
      }
      if (in) {
        s_a[r][q] = carry_a + xa - va;
        s_b[r][q] = carry_b + xb - vb;
      }
      carry_a += __shfl(xa, 63, 64);
      carry_b += __shfl(xb, 63, 64);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      int ra = s_a[r][w] + ea[r], rb = s_b[r][w] + eb[r];
      int oa[KPT], ob[KPT];
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        oa[u] = ra;
        ob[u] = rb;
        ra += c[r][u];
        rb += (c[r][u] + kSegRows - 1) / kSegRows;
      }
      const int i0 = base + r * RK + t * KPT;
      if (i0 + KPT <= n) {
        *reinterpret_cast<int4*>(offsets + i0) = make_int4(oa[0], oa[1], oa[2], oa[3]);
        *reinterpret_cast<int4*>(offsets + i0 + 4) = make_int4(oa[4], oa[5], oa[6], oa[7]);
        *reinterpret_cast<int4*>(chunk_base + i0) = make_int4(ob[0], ob[1], ob[2], ob[3]);
        *reinterpret_cast<int4*>(chunk_base + i0 + 4) = make_int4(ob[4], ob[5], ob[6], ob[7]);
      } else {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
          if (i0 + u < n) {
            offsets[i0 + u] = oa[u];
            chunk_base[i0 + u] = ob[u];
          }
      }
    }
    __syncthreads();  // the prefixes are read before the next batch overwrites them
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
// partial[w]. The chunk's row ids are staged in LDS; with C a multiple of 4
// each thread sums 4 columns and keeps 8 rows' loads in flight (the additions
// stay in row order).
__global__ void __launch_bounds__(256) segsum_chunks_kernel(const float* __restrict__ dx, int C, int nkeys,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ perm,
                                                            float* __restrict__ partial, float* __restrict__ dst) {
  __shared__ int s_rows[kSegRows];
  const int total = chunk_base[nkeys];
  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    const int v = find_key(chunk_base, nkeys, w);
    const int j = w - chunk_base[v];
    const int s0 = offsets[v] + j * kSegRows;
    const int s1 = min(offsets[v + 1], s0 + kSegRows);
    const int nr = s1 - s0;
    const bool single = (chunk_base[v + 1] - chunk_base[v]) == 1;
    __syncthreads();  // the previous chunk's rows are no longer read
    if ((int)threadIdx.x < nr) s_rows[threadIdx.x] = perm[s0 + threadIdx.x];
    __syncthreads();
    if ((C & 3) == 0) {
      for (int c4 = threadIdx.x; c4 < (C >> 2); c4 += 256) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        int r = 0;
        for (; r + 8 <= nr; r += 8) {
          f32x4_t x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const f32x4_t*>(dx + (long)s_rows[r + u] * C + 4 * c4);
#pragma unroll
          for (int u = 0; u < 8; ++u) acc += x[u];
        }
        for (; r < nr; ++r) acc += *reinterpret_cast<const f32x4_t*>(dx + (long)s_rows[r] * C + 4 * c4);
        float* o = single ? dst + (long)v * C + 4 * c4 : partial + (long)w * C + 4 * c4;
        if (single) *reinterpret_cast<f32x4_t*>(o) += acc;
        else *reinterpret_cast<f32x4_t*>(o) = acc;
      }
    } else {
      for (int c = threadIdx.x; c < C; c += 256) {
        float acc = 0.f;
        for (int r = 0; r < nr; ++r) acc += dx[(long)s_rows[r] * C + c];
        if (single) dst[(long)v * C + c] += acc;
        else partial[(long)w * C + c] = acc;
      }
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
      // chunk sums added in chunk order, the loads of 8 chunks issued
      // together (a Zipf-hot key has tens of chunks, all in this block)
      float acc = 0.f;
      int w = b0;
      for (; w + 8 <= b1; w += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = partial[(long)(w + u) * C + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += x[u];
      }
      for (; w < b1; ++w) acc += partial[(long)w * C + c];
      dst[(long)v * C + c] += acc;
    }
  }
}

// Position gradient of rows without packed documents: the position of row
// b T + t is t, so dst[t] = sum over b of dx[b T + t] (t < T; rows T..S-1 of
// dst are zero). The sum is taken as the sorted path takes it, so the result
// is bit-identical to it: the B rows of a position in ascending order in
// chunks of kSegRows rows, each chunk summed from zero, the chunk sums added
// from zero in order, and the total added onto the zeroed destination.
__global__ void __launch_bounds__(256) pos_colsum_kernel(const float* __restrict__ dx, int B, int T, int C, int S,
                                                         float* __restrict__ dst) {
  const int nq = C >> 2;
  const long q = (long)blockIdx.x * 256 + threadIdx.x;
  if (q >= (long)S * nq) return;
  const int t = (int)(q / nq), c = (int)(q - (long)t * nq) * 4;
  f32x4_t out = {0.f, 0.f, 0.f, 0.f};
  if (t < T) {
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    f32x4_t tot = zero;
    for (int b0 = 0; b0 < B; b0 += kSegRows) {
      const int b1 = min(B, b0 + kSegRows);
      f32x4_t acc = zero;
      for (int b = b0; b < b1; ++b) acc += *reinterpret_cast<const f32x4_t*>(dx + ((long)b * T + t) * C + c);
      if (B <= kSegRows) tot = acc;  // one chunk: added onto the zeroed row as it is
      else tot += acc;
    }
    out = zero + tot;
  }
  *reinterpret_cast<f32x4_t*>(dst + (long)t * C + c) = out;
}

void launch_pos_colsum(const float* dx, int B, int T, int C, int S, float* dst, hipStream_t s) {
  const long n = (long)S * (C >> 2);
  if (n <= 0) return;
  hipLaunchKernelGGL(pos_colsum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dx, B, T, C, S, dst);
}

// The rank of a row among the rows of its key: pairwise within and across
// blocks of 256 rows (O(M^2) comparisons, the fewest launches: at 8192 rows
// 7 us), or from per-block key counts scanned over the blocks (O(M + blocks
// x keys), 2 launches more) from 128 blocks on, where the scratch for the
// [blocks][nkeys] table (at most 2^24 ints) is there. Measured per step (both
// sorts of a packed step): at 32768 rows the per-block counts 5 us faster
// each, at 16384 rows 6 us slower each; beyond, the pairwise count grows as
// the square of the rows.
constexpr int kCsrLinearMinBlocks = 128;
constexpr long kCsrHistMax = 1L << 24;
static bool csr_linear(int M, int nkeys, long cap) {
  const long nb = ((long)M + 255) / 256;
  return nb >= kCsrLinearMinBlocks && nb * nkeys <= kCsrHistMax && nb * nkeys <= cap;
}
long csr_rank_ints(int M, int nkeys) {
  // the largest table of any row count up to M that takes the linear rank
  long need = M;
  for (long nb = ((long)M + 255) / 256; nb >= kCsrLinearMinBlocks; --nb)
    if (nb * nkeys <= kCsrHistMax) {
      need = std::max(need, nb * nkeys);
      break;
    }
  return need;
}

void launch_csr(const int32_t* keys, int M, int nkeys, EmbedBwdWs ws, hipStream_t s) {
  launch_fill_u32(reinterpret_cast<uint32_t*>(ws.counts), 0u, nkeys + 1, s);
  const int nb = (M + 255) / 256;
  const bool lin = M > 0 && csr_linear(M, nkeys, ws.rank_cap > 0 ? ws.rank_cap : M);
  if (lin) launch_fill_u32(reinterpret_cast<uint32_t*>(ws.rank), 0u, (long)nb * nkeys, s);
  if (M > 0)
    hipLaunchKernelGGL(csr_count_kernel, dim3(nb), dim3(256), 0, s, keys, M, nkeys, ws.counts,
                       lin ? ws.rank : nullptr);
  if (nkeys + 1 <= 4096)
    hipLaunchKernelGGL(csr_scan_pre_kernel<1>, dim3(1), dim3(512), 0, s, ws.counts, nkeys, ws.offsets, ws.chunk_base);
  else
    hipLaunchKernelGGL(csr_scan_pre_kernel<8>, dim3(1), dim3(512), 0, s, ws.counts, nkeys, ws.offsets, ws.chunk_base);
  if (lin) {
    hipLaunchKernelGGL(csr_block_prefix_kernel, dim3((nkeys + 255) / 256), dim3(256), 0, s, ws.rank, nb, nkeys);
    hipLaunchKernelGGL(csr_place_blocks_kernel, dim3(nb), dim3(256), 0, s, keys, M, nkeys, ws.offsets, ws.rank,
                       ws.perm);
  } else if (M > 0) {
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
