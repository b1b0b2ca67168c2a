// Device helpers shared by the gfx950 kernels of the training step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lm {

typedef uint16_t bf16;  // storage of a bfloat16 value (upper half of an fp32)
typedef _Float16 f16;   // IEEE binary16

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16 with round-to-nearest-even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16, b);
}

// Activation storage type helpers: float (fp32 path) or bf16 (bf16 path).
template <typename T> struct Act;
template <> struct Act<float> {
  static __device__ __forceinline__ float ld(const float* p, long i) { return p[i]; }
  static __device__ __forceinline__ void st(float* p, long i, float v) { p[i] = v; }
};
template <> struct Act<bf16> {
  static __device__ __forceinline__ float ld(const bf16* p, long i) { return bf2f(p[i]); }
  static __device__ __forceinline__ void st(bf16* p, long i, float v) { p[i] = f2bf(v); }
};
template <> struct Act<f16> {
  static __device__ __forceinline__ float ld(const f16* p, long i) { return (float)p[i]; }
  static __device__ __forceinline__ void st(f16* p, long i, float v) { p[i] = (f16)v; }
};

// The two 16-bit operand types (bf16, f16) as raw bits: conversions of one
// value and of a packed pair (low half first), round to nearest even; fp16
// overflows to +-inf.
template <typename E> struct H16;
template <> struct H16<bf16> {
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  static __device__ __forceinline__ uint32_t bits(float f) { return f2bf(f); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, v2));
  }
};
template <> struct H16<f16> {
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
  static __device__ __forceinline__ uint32_t bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
  static __device__ __forceinline__ uint32_t pack(float a, float b) {
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, v2));
  }
};

// 32x32x16 matrix-core product with fp32 accumulation, operands as 8 raw
// 16-bit values per lane of the type E.
template <typename E>
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c);
template <>
__device__ __forceinline__ f32x16_t mfma32<bf16>(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16_t mfma32<f16>(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Wavefront reductions in registers (no LDS round trip): DPP moves within
// each row of 16 lanes (partners l ^ 1, l ^ 2, then the mirrored lane in the
// other quad and in the other half-row) leave every lane with its row's
// result; two row broadcasts combine rows 0 + 1 into row 1 and (0 + 1) +
// (2 + 3) into row 3, whose lane 63 is read back as a scalar, so all 64
// lanes get the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// src from the DPP pattern in the rows of ROW_MASK, `old` in the others
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                                               CTRL, ROW_MASK, 0xf, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op, float identity) {
  v = op(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]: lane l ^ 1
  v = op(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]: lane l ^ 2
  v = op(v, dpp_mov<0x141>(v));  // row_half_mirror: the other quad of 8 lanes
  v = op(v, dpp_mov<0x140>(v));  // row_mirror: the other half of 16 lanes
  v = op(v, dpp_rows<0x142, 0xa>(identity, v));  // row_bcast:15 into rows 1, 3
  v = op(v, dpp_rows<0x143, 0xc>(identity, v));  // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
struct AddOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, AddOp(), 0.f); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp(), -INFINITY); }
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// GELU, tanh form: 0.5 u (1 + tanh(y)), y = sqrt(2/pi) (u + 0.044715 u^3),
// evaluated as g = u s with s = 0.5 (1 + tanh(y)) = 1 / (1 + exp(-2y)) (the
// same function; it saturates to 0 or 1 without overflow trouble), and its
// derivative 0.5 (1 + t) + 0.5 u (1 - t^2) c (1 + 3 a u^2), t = tanh(y), which
// in terms of s is s + u s (1 - s) 2c (1 + 3 a u^2) = s + g (1 - s) (2c + 6ac
// u^2). One exp2 of -2y log2(e) = u (k0 + k1 u^2) and the hardware reciprocal
// (about 1 ulp, no IEEE division sequence) give s; with the constants folded
// both results take 11 vector instructions. The MLP-in forward stores both
// (the activation for the MLP-out GEMM, the derivative for the backward), so
// the backward's GELU' epilogue is a product.
__device__ __forceinline__ void gelu_and_grad(float u, float& g, float& d) {
  constexpr float c = 0.7978845608028654f, a = 0.044715f, l2e = 1.4426950408889634f;
  constexpr float k0 = -2.0f * c * l2e, k1 = -2.0f * c * a * l2e;
  const float u2 = u * u;
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u * __builtin_fmaf(k1, u2, k0)));
  g = u * s;
  d = __builtin_fmaf(g * (1.0f - s), __builtin_fmaf(6.0f * a * c, u2, 2.0f * c), s);
}

// Wait until at most n vector-memory operations of this wavefront are
// outstanding (loads, stores and direct-to-LDS loads count alike, in order).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: LDS data from direct loads is
// made visible by each wavefront's own vmcnt wait before it; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// f(integral_constant<int, i>) for i = 0 .. N-1 (compile-time indices).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr unsigned kOutOfRange = 0x80000000u;  // a byte offset past every buffer's range
typedef __attribute__((address_space(3))) void lds_void_t;

}  // namespace lm
