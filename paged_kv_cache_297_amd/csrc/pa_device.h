// Device helpers for the gfx950 paged-attention kernels: element types and
// conversions, 16-byte loads, dot products and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_params.h"

namespace pa {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One byte of OCP FP8 E4M3FN storage.
struct fp8e4m3 {
  uint8_t bits;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// 16-byte loads.  KV tiles are streamed once, so they bypass reuse-oriented
// caching with the nontemporal hint.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T load_stream(const void *p) {
#if PA_NONTEMPORAL
  return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
#else
  return *reinterpret_cast<const T *>(p);
#endif
}
__device__ __forceinline__ u32x4 load16_stream(const void *p) { return load_stream<u32x4>(p); }
__device__ __forceinline__ u32x2 load8_stream(const void *p) { return load_stream<u32x2>(p); }
__device__ __forceinline__ unsigned load4_stream(const void *p) { return load_stream<unsigned>(p); }
__device__ __forceinline__ u32x4 load16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// Read-only tables (block tables) are read through the constant address
// space: a wave-uniform index then compiles to a scalar load, which waits on
// its own counter instead of behind the KV tile loads in flight.
typedef const int32_t __attribute__((address_space(4))) *const_i32_ptr;
__device__ __forceinline__ const_i32_ptr as_const_table(const int32_t *p) {
  return (const_i32_ptr)(uintptr_t)p;
}

// ---------------------------------------------------------------------------
// Packed dot products with fp32 accumulation.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dot2(float acc, unsigned a, unsigned b, __bf16) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ float dot2(float acc, unsigned a, unsigned b, _Float16) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                false);
}

// fp8 E4M3FN pair (bytes 0,1 or 2,3 of a word) -> packed 16-bit pair, exact.
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to(unsigned w, __bf16) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to(unsigned w, _Float16) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// fp32 pair -> packed 16-bit pair (round to nearest even).
__device__ __forceinline__ unsigned pack2(float a, float b, __bf16) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}
__device__ __forceinline__ unsigned pack2(float a, float b, _Float16) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Whether token t lies in [lo, lo + span) (span >= 1).  Without a sliding
// window (WIN false) lo is at or before the first token a workgroup loads,
// so only the upper bound is tested: one compare against a per-block scalar
// instead of a subtraction and a compare per element.
template <bool WIN>
__device__ __forceinline__ bool in_span(int t, int lo, int span) {
  if constexpr (WIN) return (unsigned)(t - lo) < (unsigned)span;
  else return t < lo + span;
}

// Keep-mask of a 32-bit word holding two 16-bit elements of tokens t, t + 1:
// the half of a token outside [lo, lo + span) is cleared.  Straight-line
// selects, so the window and tail masks can be applied on every step without
// a divergent branch.
template <bool WIN>
__device__ __forceinline__ unsigned keep_pair_mask(int t, int lo, int span) {
  return (in_span<WIN>(t, lo, span) ? 0x0000FFFFu : 0u) |
         (in_span<WIN>(t + 1, lo, span) ? 0xFFFF0000u : 0u);
}

// A key's logit in log2 units, before the ALiBi term, from its dot product
// with the query: scale * k_scale * q.K, or under a soft cap c (CAP)
// c * tanh(scale * k_scale * q.K / c).  The 16-bit kernels take
// tanh(y) = 1 - 2 / (exp(2y) + 1) from the hardware exp2 and reciprocal (an
// exp that overflows to +inf gives 1, one that underflows to 0 gives -1): it
// cancels near y = 0, a few ulps of 1 absolute, far below 16-bit tolerances.
// ACCURATE (fp32 queries) takes tanh(y) = expm1(2y) / (expm1(2y) + 2), which
// keeps a relative error of a few ulps at every y; 2y is clamped at 20,
// where tanh is 1 in fp32 (a NaN passes the clamp).
// The cap is a compile-time choice: a run-time branch here, even a uniform
// one, splits the tile loop and costs the loads their overlap.
template <bool CAP, bool ACCURATE = false, typename P>
__device__ __forceinline__ float scaled_logit(const P &p, float dot) {
  if constexpr (CAP && ACCURATE) {
    float y2 = dot * p.cap_in_nat;
    y2 = y2 > 20.0f ? 20.0f : y2;
    const float em = expm1f(y2);
    return p.cap_out * (em / (em + 2.0f));
  } else if constexpr (CAP) {
    const float e = fast_exp2(dot * p.cap_in);
    return fmaf(-2.0f * p.cap_out, __builtin_amdgcn_rcpf(e + 1.0f), p.cap_out);
  } else {
    return dot * p.scale_log2;
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
  return (float)v;
}
template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  return (T)v;
}

// ---------------------------------------------------------------------------
// Cross-lane operations (wave64).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return bits_f(__builtin_amdgcn_mov_dpp((int)f_bits(v), CTRL, 0xF, 0xF, false));
}

// All lanes of each 16-lane row get the row's max / sum.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp<0x128>(v));  // row_ror:8
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x124>(v);
  v += dpp<0x128>(v);
  return v;
}

// v_permlane16_swap swaps the odd rows of its first operand with the even
// rows of its second; v_permlane32_swap swaps the upper half of the first
// with the lower half of the second.  Called as swap(lo, hi) and summed, a
// lane whose bit (16 or 32) is clear ends with lo(self) + lo(partner) and a
// lane whose bit is set ends with hi(self) + hi(partner): one instruction per
// pair performs a "transpose-reduce" step.
template <int M>
__device__ __forceinline__ void swap_pair(float lo, float hi, float &a, float &b) {
  static_assert(M == 16 || M == 32, "permlane swap distance");
  if constexpr (M == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(f_bits(lo), f_bits(hi), false, false);
    a = bits_f(r[0]);
    b = bits_f(r[1]);
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(f_bits(lo), f_bits(hi), false, false);
    a = bits_f(r[0]);
    b = bits_f(r[1]);
  }
}
template <int M>
__device__ __forceinline__ float xor_sum(float v) {
  float a, b;
  swap_pair<M>(v, v, a, b);
  return a + b;
}
template <int M>
__device__ __forceinline__ float xor_max(float v) {
  float a, b;
  swap_pair<M>(v, v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float readlane(float v, int lane) {
  return bits_f(__builtin_amdgcn_readlane(f_bits(v), lane));
}

// Orders LDS traffic of one wave (no workgroup barrier needed: the data is
// produced and consumed by the same wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Per-sequence path choice (host mirror: pa_should_use_v2).  seq_len is the
// length the rule sees: the window-clipped min(L, W + 1) under a window.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool seq_uses_v2(const Params &p, int seq_len) {
  if (p.mode == kModeV1) return false;
  if (p.mode == kModeV2 || p.auto_all_v2) return true;
  const int parts = (seq_len + kPartitionSize - 1) / kPartitionSize;
  return (long long)p.num_kv_heads * parts > (long long)p.auto_tile_limit;
}

}  // namespace pa
