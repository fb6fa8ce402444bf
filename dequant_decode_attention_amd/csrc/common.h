// Shared device/host helpers of the dqattn library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dqattn.h"

namespace dqa {

constexpr int kGroup = 32;       // quantization group length ([P1 para 1])
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxRecent = 128;  // residual-buffer bound ([P1 para 8])

// Launch geometry target: enough workgroups to give every one of the 256
// compute units several resident workgroups.  Fixed (not queried) so that
// workspace sizes depend on the shape only.
constexpr int kTargetWorkgroups = 1024;

// Device pointers handed to the library must be 16-byte aligned (the
// kernels move 16-byte pieces); DQA_ERR_ALIGN otherwise.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define DQA_CHECK_LAUNCH()                               \
  do {                                                   \
    if (hipPeekAtLastError() != hipSuccess) return DQA_ERR_HIP; \
  } while (0)

__device__ __forceinline__ float h2f(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, bits));
}

__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Arithmetic stays in C rather than inline asm: gfx950 needs independent
// instructions between some dependent pairs (a transcendental result and
// the next VALU instruction that reads it, a VALU result and a matrix
// instruction or a lane permute that reads it), and the compiler inserts
// them only around instructions it generates itself.
//
// Half H of a word of two fp16 values, widened to fp32 (exact).  An FMA
// with one or two such operands compiles to one mixed-precision FMA.
typedef _Float16 fp16x2 __attribute__((ext_vector_type(2)));
template <int H>
__device__ __forceinline__ float half_of(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(fp16x2, w)[H]);
}
// A constant the optimizer does not see through (held in a scalar
// register), so that fma(h, +-1, x) stays one mixed-precision FMA instead
// of becoming a widening conversion and an addition.
__device__ __forceinline__ float opaque_const(float c) {
  asm("" : "+s"(c));
  return c;
}

// Butterfly exchange inside a quad / half-row with DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror (lane i <-> 7-i in 8)
constexpr int kDppRowMirror = 0x140;    // row_mirror (lane i <-> 15-i in 16)

// Sum over N adjacent lanes (N in {1, 2, 4, 8, 16}); every lane of the
// aligned N-lane block receives the block sum.
template <int N>
__device__ __forceinline__ float sum_adjacent(float v) {
  if constexpr (N >= 2) v += dpp<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppRowMirror>(v);
  return v;
}

// Max over N adjacent lanes (as sum_adjacent).
template <int N>
__device__ __forceinline__ float max_adjacent(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppRowMirror>(v));
  return v;
}

// Combine lane L with lane L ^ 32 (rows32) or L ^ 16 through the VALU
// row-swap permutes; every lane gets the result.  The two values returned by
// the permute are copied into scalars before they are reinterpreted (a bit
// cast of an element of the returned vector reads element 0).
template <bool MAX>
__device__ __forceinline__ float swap_rows(float v, bool rows32) {
  const unsigned x = __builtin_bit_cast(unsigned, v);
  unsigned r0, r1;
  if (rows32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  const float f0 = __builtin_bit_cast(float, r0), f1 = __builtin_bit_cast(float, r1);
  return MAX ? fmaxf(f0, f1) : f0 + f1;
}

// Sum / max over all 64 lanes, and sum over each 32-lane half; every lane
// gets the result.  Call with the whole wave active.
__device__ __forceinline__ float wave_sum(float v) {
  return swap_rows<false>(swap_rows<false>(sum_adjacent<16>(v), true), false);
}
__device__ __forceinline__ float wave_max(float v) {
  return swap_rows<true>(swap_rows<true>(max_adjacent<16>(v), true), false);
}
__device__ __forceinline__ float half_sum(float v) { return swap_rows<false>(sum_adjacent<16>(v), false); }

// Wave-wide reduction over lanes with stride S (S a power of two): every
// lane ends with the reduction over its residue class lane % S.
template <int S>
__device__ __forceinline__ float max_strided(float v) {
#pragma unroll
  for (int m = S; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
template <int S>
__device__ __forceinline__ float sum_strided(float v) {
#pragma unroll
  for (int m = S; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Merge weight of a partial softmax state with running max m (log2 domain)
// into a combined max M; empty partials carry m = -inf.
__device__ __forceinline__ float merge_weight(float m, float M) {
  return (m == -INFINITY) ? 0.0f : exp2f(m - M);
}

}  // namespace dqa
