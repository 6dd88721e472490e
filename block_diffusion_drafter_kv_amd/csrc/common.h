// Shared device helpers for the DFlash drafter kernels (gfx950 / CDNA4).
//
// Element types.  An fp32 drafter computes in fp32 throughout (weights,
// activations, KV cache; v_mfma_f32_16x16x4_f32).  A bf16 drafter (weights and
// target hidden states given in bf16) multiplies fp16 operands with fp32
// accumulation (v_mfma_f32_16x16x32_f16, the bf16 rate on CDNA4): its weight
// matrices are converted once, exactly, to fp16 scaled by a power of two; its
// activations, block q/k/v, attention weights and KV cache are fp16 (three more
// significand bits than bf16 at the same size); the residual stream stays fp32.
// Only the fc product, whose two operands both arrive in bf16, runs on
// v_mfma_f32_16x16x32_bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16_t;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

static constexpr int WAVE = 64;
static constexpr int EPI_ROWS = 64;  // rows staged per GEMM epilogue pass

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) { return (f16_t)x; }

// Storage type of the weights read elementwise (norm gains, embedding) by a
// kernel whose operand type is C: the caller's bf16 for an fp16-operand drafter.
template <typename C> struct WeightOf { typedef C type; };
template <> struct WeightOf<f16_t> { typedef bf16_t type; };

// ---- MFMA fragments: one lane holds 8 consecutive k-values of one row ----
// For a 16x16 output tile with k = 32 per step, lane l supplies row (l % 16) of
// the A operand and column (l % 16) of the B operand, with k-values
// 8*(l/16) .. 8*(l/16)+7; its 4 results are rows 4*(l/16)+i, column l % 16.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  typedef bf16x8 type;
  __device__ __forceinline__ static void mma(f32x4& c, const bf16x8& a, const bf16x8& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<f16_t> {
  typedef f16x8 type;
  __device__ __forceinline__ static void mma(f32x4& c, const f16x8& a, const f16x8& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<float> {
  typedef f32x8 type;
  // eight k=4 steps; step j pairs k-value j of every lane group (same mapping on A and B)
  __device__ __forceinline__ static void mma(f32x4& c, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  }
};

// 16-byte vector of T
template <typename T> struct Vec16;
template <> struct Vec16<bf16_t> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<f16_t> { typedef f16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

// ---- wave reductions ----
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// sum over a group of `width` lanes (width power of two, groups aligned)
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ----
struct U4 { uint32_t x, y, z, w; };
__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    U4 n;
    n.x = hi1 ^ c.y ^ k0;
    n.y = lo1;
    n.z = hi0 ^ c.w ^ k1;
    n.w = lo0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}
// u in [0,1) with 24 random bits; counter (position, slot, step, purpose), key = seed
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t slot, uint64_t step,
                                                uint32_t position, uint32_t purpose) {
  U4 c{position, slot, (uint32_t)step, purpose};
  U4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (float)(o.x >> 8) * (1.0f / 16777216.0f);
}

enum : uint32_t { PURPOSE_DRAFT = 0, PURPOSE_ACCEPT = 1, PURPOSE_RESAMPLE = 2, PURPOSE_NOISE = 3, PURPOSE_TREE_WALK = 4 };

// device error word bits
enum : int32_t { ERR_CAPACITY = 1, ERR_BAD_SLOT = 2, ERR_ROWS = 4, ERR_BAD_TOKEN = 8, ERR_PAGE = 16,
                 ERR_NONFINITE = 32 };

__device__ __forceinline__ void raise_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Store conversion of an activation or cache value.  16-bit: a value beyond fp16's
// largest finite magnitude (or NaN) sets `bad` and is stored saturated (NaN stays
// NaN), so later kernels see finite values while the caller is told.  fp32: as is.
template <typename T>
__device__ __forceinline__ T store_cvt(float x, bool& bad) {
  if constexpr (sizeof(T) == 2) {
    if (!(fabsf(x) <= 65504.f)) {
      bad = true;
      if (x == x) x = x > 0.f ? 65504.f : -65504.f;
    }
  }
  return from_f32<T>(x);
}

// After an epilogue pass: one lane of each wave that met an out-of-range value reports it
// (every lane of the wave must reach this call).
__device__ __forceinline__ void report_nonfinite(int32_t* err, bool bad, int tid) {
  if (__any(bad) && (tid & 63) == 0) raise_error(err, ERR_NONFINITE);
}

}  // namespace dfl
