// Shared pieces of the uniform-layout decode kernels: the kernel argument
// block and the device helpers both decode kernels use.
#pragma once

#include <cmath>

#include "common.h"

namespace dqa {

// The split of one (batch, KV head)'s tiles over its waves, computed on the
// host.  The n_q quantized tiles (one work unit each) and n_r <= 4 fp16
// recent tiles (W units each: their set-up costs more) lie on a line of
// total = n_q + W n_r units: recent tile r takes the W units from rstart[r]
// (centred in the r-th of n_r equal segments), the quantized tiles fill the
// other units in order.  Wave gw of the (batch, KV head) takes the units
// [gw per_wave + min(gw, extra), ...) -- per_wave of them, one more when
// gw < extra: the quantized tiles among them (a contiguous run) and the
// recent tiles that start among them.
struct TileSplit {
  int per_wave, extra, n_r, W;
  int rstart[4];
};

struct KiviArgs {
  const uint16_t* q;
  const uint32_t* k_codes;
  const uint16_t* k_scale;
  const uint16_t* k_zero;
  const uint32_t* v_codes;
  const uint16_t* v_scale;
  const uint16_t* v_zero;
  const uint16_t* k_recent;
  const uint16_t* v_recent;
  float* out;
  float* partials;
  uint32_t* counters;   // merge counters, one per (batch, KV head)
  int Hq, Hkv, T_q, R;
  int qtile_stride;     // 32-token tiles of quantized-buffer capacity per (batch, KV head)
  int R_cap;            // recent-buffer rows per (batch, KV head)
  int n_qtiles;         // T_q / 32
  int n_rtiles;         // ceil(R / 32)
  int total_splits;     // splits (partial-state slots) per (batch, KV head)
  TileSplit split;      // tiles -> waves
  float q_scale;        // sm_scale * log2(e): logits in the log2 domain
  float rope_theta;
  const uint32_t* rope_table;   // the cache's built in-tile trig table, or null
  double omega[64];     // RoPE frequencies theta^(-2i/d), i < d/2 (host fp64)
};

// RoPE frequencies omega_i = theta^(-2i/d), i < d/2, in fp64 on the host
// (zero past d/2); the same values reach every kernel that rotates.
inline void rope_omega(float theta, int d, double* omega) {
  for (int i = 0; i < 64; ++i)
    omega[i] = (theta > 0.0f && i < d / 2) ? std::pow(static_cast<double>(theta), -2.0 * i / d) : 0.0;
}
struct RopeOmega {
  double omega[64];
  float theta;
};

// The feature-product decode kernel (2- and 4-bit codes with RoPE; see
// decode_feat.hip): its resident workgroup target and its launch.
int feat_decode_workgroups();
int feat_recent_weight();
int feat_waves_per_wg();
int launch_feat_decode(const KiviArgs& a, int d, int G, int bits, dim3 grid, hipStream_t s);
// The in-tile trig table of a cache (kivi_rope_table): its size in uint32
// words for head dim d, and its build kernel (bits 2 or 4, d 64 or 128).
size_t feat_rope_table_words(int d);
int launch_rope_table(float theta, int d, int bits, uint32_t* table, hipStream_t s);

namespace {


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Host side of TileSplit for n_q quantized and n_r recent tiles, recent
// weight W, over nw waves (total units below 2^31).
inline TileSplit make_tile_split(int n_q, int n_r, int W, long long nw) {
  TileSplit t{};
  const long long total = n_q + static_cast<long long>(W) * n_r;
  t.per_wave = static_cast<int>(total / nw);
  t.extra = static_cast<int>(total % nw);
  t.n_r = n_r;
  t.W = W;
  for (int r = 0; r < n_r && r < 4; ++r) {
    const long long lo = r * total / n_r, hi = (r + 1) * total / n_r;
    t.rstart[r] = static_cast<int>(lo + (hi - lo - W) / 2);
  }
  return t;
}

// The tiles of wave gw under a TileSplit: its quantized run [qb, qb + nq)
// and its r_mine recent tiles from r_first.
struct WaveTiles {
  int qb, nq, r_first, r_mine;
};
__device__ __forceinline__ WaveTiles wave_tiles(const TileSplit& t, int gw) {
  const int u0 = gw * t.per_wave + min(gw, t.extra);
  const int u1 = u0 + t.per_wave + (gw < t.extra ? 1 : 0);
  int before0 = 0, before1 = 0;   // recent units below u0 and below u1
  WaveTiles w{0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (r < t.n_r) {
      const int start = t.rstart[r];
      before0 += min(max(u0 - start, 0), t.W);
      before1 += min(max(u1 - start, 0), t.W);
      if (start >= u0 && start < u1) {
        if (w.r_mine == 0) w.r_first = r;
        ++w.r_mine;
      }
    }
  }
  w.qb = u0 - before0;
  w.nq = (u1 - before1) - w.qb;
  return w;
}

// Accurate unit complex number e^{i * pos * omega}: the angle is formed and
// reduced modulo 2*pi in fp64, then sin/cos are taken in fp32 on [-pi, pi].
__device__ __forceinline__ void rope_unit(double pos, double omega, float& c, float& s) {
  const double kTwoPiHi = 6.283185307179586;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double ang = pos * omega;
  const double k = rint(ang * 0.15915494309189535);
  double r = fma(-k, kTwoPiHi, ang);
  r = fma(-k, kTwoPiLo, r);
  sincosf(static_cast<float>(r), &s, &c);
}

// Orders LDS traffic of the lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// NB consecutive bytes (4, 8, 16 or 32; NB-aligned, at most 16-aligned) as
// 32-bit words.
template <int NB>
struct Words {
  uint32_t w[NB / 4];
};
template <int NB>
__device__ __forceinline__ Words<NB> load_words(const void* p) {
  Words<NB> r;
  if constexpr (NB == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NB == 8) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r.w[0] = u.x;
    r.w[1] = u.y;
  } else {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i] = u.x;
      r.w[4 * i + 1] = u.y;
      r.w[4 * i + 2] = u.z;
      r.w[4 * i + 3] = u.w;
    }
  }
  return r;
}

// A kernel-argument pointer as a wave-uniform value.  A lane-dependent
// choice between two argument pointers would otherwise be folded into a
// per-lane vector load of the pointer from the argument segment, issued
// again on every use.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  // rebuilt as a global-memory pointer, so loads through it stay global loads
  using GT = const __attribute__((address_space(1))) T;
  GT* g = reinterpret_cast<GT*>((static_cast<uint64_t>(hi) << 32) | lo);
  return (const T*)g;
}

// A value the compiler must treat as unknown (keeps a VGPR constant out of
// the scalar constant bus, and keeps shifted words from being folded back
// into bit-field extracts).  The asm statement is empty: no instruction.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Key codes as fp16 subnormals.  A code c placed in the low bits of an fp16
// bit pattern whose exponent field is zero is the value c * 2^-24; a code
// left at bit offset 2p (2-bit) or 4p (4-bit) inside its 16-bit half is
// c * 2^(bits * p) * 2^-24, still subnormal while it stays below bit 10.  One
// mask of the packed word therefore yields two such values (one per half),
// and the mixed-precision FMA widens them exactly and multiplies by the fp32
// scale pre-multiplied by 2^(24 - bits * p): code * scale + zero with one
// rounding, the same result as an fp32 FMA on the integer code.
//
// Position p of K-step element e (channel c0 + e) inside its half.
template <int BITS>
__device__ __forceinline__ constexpr int key_code_pos(int e) {
  return BITS == 2 ? (e <= 4 ? e : e - 5) : (BITS == 4 ? (e & 1) : 0);
}
// The lane's masked key-code registers (key_code_reg / key_code_half give
// the register and half of K-step element e).  2-bit: one word = 16
// channels (two K-steps); register e holds channel e in the low half (even
// K-step) and channel e + 8 in the high half (odd K-step).  4-bit: one word
// = one K-step; register e & 3 holds channel e in half e >> 2.  8-bit: two
// words = one K-step; word i gives registers 2i (channels 4i, 4i + 2) and
// 2i + 1 (channels 4i + 1, 4i + 3).
template <int BITS>
__device__ __forceinline__ void key_code_regs(const uint32_t* w, int ks, uint32_t* m) {
  if constexpr (BITS == 2) {
    const uint32_t x = w[ks >> 1], x1 = opaque(x >> 10);
#pragma unroll
    for (int e = 0; e < 5; ++e) m[e] = x & (0x00030003u << (2 * e));
#pragma unroll
    for (int e = 5; e < 8; ++e) m[e] = x1 & (0x00030003u << (2 * (e - 5)));
  } else if constexpr (BITS == 4) {
    const uint32_t x = w[ks], x1 = opaque(x >> 8);
    m[0] = x & 0x000F000Fu;    // channels 0, 4
    m[1] = x & 0x00F000F0u;    // channels 1, 5
    m[2] = x1 & 0x000F000Fu;   // channels 2, 6
    m[3] = x1 & 0x00F000F0u;   // channels 3, 7
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t x = w[2 * ks + i];
      m[2 * i] = x & 0x00FF00FFu;                 // channels 4i, 4i + 2
      m[2 * i + 1] = opaque(x >> 8) & 0x00FF00FFu; // channels 4i + 1, 4i + 3
    }
  }
}
// register and half of K-step element e (ks: the K-step, for 2-bit)
template <int BITS>
__device__ __forceinline__ constexpr int key_code_reg(int e) {
  return BITS == 2 ? e : (BITS == 4 ? (e & 3) : (2 * (e >> 2) + (e & 1)));
}
template <int BITS>
__device__ __forceinline__ constexpr int key_code_half(int e, int ks) {
  return BITS == 2 ? (ks & 1) : (BITS == 4 ? (e >> 2) : ((e >> 1) & 1));
}

// code (fp16 half A of m) * s + zero (fp16 half Z of z), one rounding
template <int A, int Z>
__device__ __forceinline__ float mix_dequant(uint32_t m, float s, uint32_t z) {
  return __builtin_fmaf(half_of<A>(m), s, half_of<Z>(z));
}

// Value chunk (8 tokens of one channel) -> fp16 operand holding the codes as
// fp16 subnormals, each code at the top of the 10-bit mantissa field: bits
// 8-9 (2-bit: code * 2^-16), 6-9 (4-bit: code * 2^-18) or 2-9 (8-bit: code *
// 2^-22).  The matrix cores multiply subnormal inputs exactly, but they sum
// the products of subnormal operands as if each had the smallest normal
// exponent, so a code in the low mantissa bits would lose up to 10 bits of
// its product (measured on MI355X: sums of 32 such products off by up to
// 1.5e-4 relative, biased toward zero; with the codes at the top, within a
// few fp32 ulps).  The accumulator runs in the code * 2^-kCodeShift domain and
// is rescaled once.  Element 2i holds token i, element 2i+1 token i+4 (the
// same order is used for the probabilities).
template <int BITS>
constexpr int kCodeShift = BITS == 2 ? 16 : (BITS == 4 ? 18 : 22);
template <int BITS>
constexpr float kCodeScale = static_cast<float>(1u << kCodeShift<BITS>);

template <int BITS>
__device__ __forceinline__ half8 value_codes8(uint64_t chunk, uint32_t mask) {
  uint32_t r[4];
  if constexpr (BITS == 2) {
    // tokens 0..3 at bits 0..7, tokens 4..7 at bits 16..23; token i (and
    // i + 4) shifted to bits 8..9 (24..25)
    const uint32_t v = static_cast<uint32_t>(chunk);
    const uint32_t u = v | (v << 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (u << (8 - 2 * i)) & mask;
  } else if constexpr (BITS == 4) {
    // token i at bits 4i..4i+3 and token i + 4 at 16 + 4i; moved to bits 6..9
    const uint32_t w = static_cast<uint32_t>(chunk);
    r[0] = (w << 6) & mask;
    r[1] = (w << 2) & mask;
    r[2] = (w >> 2) & mask;
    r[3] = (w >> 6) & mask;
  } else {
    const uint32_t lo = static_cast<uint32_t>(chunk), hi = static_cast<uint32_t>(chunk >> 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_amdgcn_perm(hi, lo, static_cast<uint32_t>(i | (0x0C << 8) | ((4 + i) << 16) | (0x0C << 24))) << 2;
  }
  half8 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(half2v, r[i]);
    out[2 * i] = h[0];
    out[2 * i + 1] = h[1];
  }
  return out;
}
// token offset (inside the lane's 8-token run) of operand element e
__device__ __forceinline__ constexpr int vtok(int e) { return (e >> 1) + 4 * (e & 1); }

// Token (0..31) of key-operand row m in half s of a tile: rows 4g..4g+3 of
// the two halves cover tokens 8g..8g+7, so that output row 4g + r of half s
// is token 8g + 4s + r.
__device__ __forceinline__ constexpr int row_token(int s, int m) { return 8 * (m >> 2) + 4 * s + (m & 3); }

// x - (fp32) of the low / high fp16 half of h, exact (the fp16 value is
// widened exactly and one fp32 rounding applies, none here since hi is x
// rounded toward zero): one mixed-precision FMA each.
__device__ __forceinline__ float minus_half_lo(uint32_t h, float x) {
  return __builtin_fmaf(half_of<0>(h), opaque_const(-1.0f), x);
}
__device__ __forceinline__ float minus_half_hi(uint32_t h, float x) {
  return __builtin_fmaf(half_of<1>(h), opaque_const(-1.0f), x);
}

// Split 8 fp32 values into fp16 hi + lo (hi rounded toward zero; lo the
// exact fp32 remainder rounded toward zero).
__device__ __forceinline__ void split8(const float* x, half8& hi, half8& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[2 * p], x[2 * p + 1]));
    const half2v hv = __builtin_bit_cast(half2v, h);
    const half2v l = __builtin_bit_cast(
        half2v, __builtin_amdgcn_cvt_pkrtz(minus_half_lo(h, x[2 * p]), minus_half_hi(h, x[2 * p + 1])));
    hi[2 * p] = hv[0];
    hi[2 * p + 1] = hv[1];
    lo[2 * p] = l[0];
    lo[2 * p + 1] = l[1];
  }
}

// Reductions over the 4 lanes L, L^16, L^32, L^48 (the four 16-lane rows),
// with the row-swap permutes of the VALU; every lane gets the result.  Each
// permute swaps rows between two copies of v.  The two results are copied
// into scalars before they are reinterpreted: a bit cast applied directly
// to an element of the returned vector reads element 0.
template <bool MAX>
__device__ __forceinline__ float combine2(float v, bool rows32) {
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
__device__ __forceinline__ float max_rows(float v) { return combine2<true>(combine2<true>(v, true), false); }
__device__ __forceinline__ float sum_rows(float v) { return combine2<false>(combine2<false>(v, true), false); }

// First float of row j (token j of a tile) of the in-tile rotation table,
// whose rows are ERF floats apart.
template <int ERF>
__device__ __forceinline__ constexpr int erow(int j) { return j * ERF + 16 * ((j >> 3) & 3); }

}  // namespace
}  // namespace dqa
