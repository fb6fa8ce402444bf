// Split-K decode attention over the uniform (KIVI) 2- and 4-bit cache with
// RoPE: the key logits as one matrix product of per-token "features" and
// per-tile factors, with no rotation or dequantization of keys on the VALU.
//
// [P1 para 7]: keys are quantized before RoPE and rotated after
// dequantization.  [P1 para 4, 5]: one key scale/zero per (channel, 32-token
// block), one value scale/zero per (token, 32-channel group).  [P1 para 2]:
// the whole cache is read at every decode step, so the codes are read once
// and expanded in registers.
//
// For channel pair i (channels a = 2i, b = 2i + 1) of the token at position
// t0 + j of a 32-token tile that starts at t0, with codes c, the tile's
// scales s and zeros z, and the query rotated back to t0 (q' = R(t0)^T q):
//   q . R(t0 + j) khat = q' . R(j) khat
//     = c_a cos(j w_i) (s_a q'_a) + c_a sin(j w_i) (s_a q'_b)
//     + c_b cos(j w_i) (s_b q'_b) + c_b sin(j w_i) (-s_b q'_a)
//     + cos(j w_i) (z_a q'_a + z_b q'_b) + sin(j w_i) (z_a q'_b - z_b q'_a).
// Every term is a per-token factor (code times a trigonometric value of the
// token's in-tile offset, or the trigonometric value alone) times a per-tile
// factor of one query head.  So the logits of a tile are one matrix product:
//   A (rows = tokens) = [code * trig | trig] features,
//   B (columns = query heads) = the per-tile factors.
// A trig value is held as a head with few significant bits (9 for 2-bit
// codes, 7 for 4-bit) plus the exact tail, so code * head is exact in fp16
// and code * tail errs by < 2^-20 of the feature; the per-tile factors are
// formed in fp32 and split into fp16 hi + lo, which occupy separate B
// columns (hi of head h in column h, lo in column G + h).  Two products per
// K-step (A head, A tail) and one cross-lane add per logit give the logit to
// about 2^-20 relative.  The trig values of a lane's two tokens and sixteen
// pairs stay in registers for the whole kernel; per key element the VALU does
// a share of the code extraction and two packed fp16 multiplies.
//
// Scale bookkeeping: a key code is extracted to bit 4 of its fp16 half (the
// subnormal code * 2^-20) and the trig head/tail registers hold
// trig * 2^15, so a feature is code * trig * 2^-5 (normal fp16 for all but
// tiny trig values, whose errors are then tiny in absolute terms).  The code
// factors of B carry 2^5; the zero-point features (trig * 2^15 alone) are
// accumulated first, against B = z q' * 2^5, and that partial sum is scaled
// by 2^-20 before the code features add to it.
//
// Values: as in the other decode kernel (A = value codes as fp16 subnormals,
// B = p * scale), with the codes extracted near the top of the mantissa:
// the matrix cores sum products of subnormal inputs as if their exponent were
// the smallest normal one, so a code in the low mantissa bits would lose
// precision.  Codes at two positions (2-bit: 6 and 8, 4-bit: 4 and 6); the
// lower position's tokens carry a factor 4 in their value scales.
//
// Recent fp16 tokens (at most 4 tiles per (batch, KV head), spread over
// different waves): keys rotated in fp32 from the trig table, split into
// fp16 hi + lo, against the query rotated to the tile start.
#include <type_traits>

#include "decode_common.h"
#include "merge.h"

namespace dqa {
namespace {

constexpr int kFWaves = 8;          // waves per workgroup (one workgroup per compute unit)
constexpr int kFWavesPerSimd = 2;   // resident waves per SIMD (register budget 256)
// work units of an fp16 recent tile in the split of tiles over waves (its
// query rotation and fp32 key rotation cost about two more quantized tiles)
constexpr int kRecentWeight = 3;

// ---------------------------------------------------------------- helpers

// Packed fp16 products with one code half broadcast: (c * t.x, c * t.y) for
// c the low (HALF = 0) or high (HALF = 1) half of `code` (one packed
// multiply with the broadcast in its operand selection).
template <int HALF>
__device__ __forceinline__ uint32_t pk_mul_bcast(uint32_t code, uint32_t t) {
  const half2v c = __builtin_bit_cast(half2v, code);
  const half2v b = {c[HALF], c[HALF]};
  return __builtin_bit_cast(uint32_t, b * __builtin_bit_cast(half2v, t));
}

// Mixed-precision products with an fp16 operand taken from half H of a
// word (one mixed-precision FMA, no conversion): h * x (NEG: h * -x) and
// h * x + c, in fp32.  The zero addend keeps the FMA form (h * x + 0 is
// h * x except for the sign of a zero product).
template <int H, bool NEG = false>
__device__ __forceinline__ float mix_mul(uint32_t h2, float x) {
  return __builtin_fmaf(half_of<H>(h2), NEG ? -x : x, 0.0f);
}
template <int H>
__device__ __forceinline__ float mix_fma(uint32_t h2, float x, float c) {
  return __builtin_fmaf(half_of<H>(h2), x, c);
}

// fp32 x with all but its top `bits` significant bits cleared (toward zero).
__device__ __forceinline__ float trunc_sig(float x, int bits) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return __builtin_bit_cast(float, u & ~((1u << (24 - bits)) - 1u));
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  half2v h;
  h[0] = static_cast<_Float16>(lo);
  h[1] = static_cast<_Float16>(hi);
  return __builtin_bit_cast(uint32_t, h);
}

// fp32 x -> fp16 hi (toward zero) + lo (the exact remainder, toward zero),
// for two values: returns (hi pair, lo pair).  Subnormal remainders are kept.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(minus_half_lo(hi, x0), minus_half_hi(hi, x1)));
}

// Key code register e of a packed word (channels e and e + 16/BITS of the
// word's 32/BITS channels, one per fp16 half), each code moved to bit 4 of
// its half: the fp16 subnormal code * 2^-20.
template <int BITS>
__device__ __forceinline__ uint32_t key_code_at4(uint32_t w, int e) {
  constexpr uint32_t kMask = BITS == 2 ? 0x00300030u : 0x00F000F0u;
  const int sh = BITS * e - 4;
  return (sh < 0 ? (w << (-sh)) : (w >> sh)) & kMask;
}

// Value chunk (8 tokens of one channel) -> fp16 operand, element 2i = token
// i, 2i + 1 = token i + 4.  2-bit: tokens with i even at bits 6..7 of their
// half, odd at 8..9; 4-bit: i = 0, 1 at bits 4..7, i = 2, 3 at bits 6..9.
// The value codes' product domain is code * 2^-kVShift; tokens at the lower
// position carry a factor 4 in their scale (feat_vscale_factor).
template <int BITS>
constexpr int kVShift = BITS == 2 ? 16 : 18;
template <int BITS>
__device__ __forceinline__ bool feat_vlow(int t) {
  return BITS == 2 ? ((t & 1) == 0) : ((t & 3) < 2);
}
template <int BITS>
__device__ __forceinline__ half8 feat_value_codes8(uint32_t chunk) {
  uint32_t r[4];
  if constexpr (BITS == 2) {
    const uint32_t v = chunk & 0xFFFFu;
    const uint32_t u = v | (v << 8);          // tokens 0..3 at bits 0..7, 4..7 at 16..23
    const uint32_t u6 = u << 6, u2 = u << 2;
    r[0] = u6 & 0x00C000C0u;                  // token 0 (bit 0 -> 6)
    r[1] = u6 & 0x03000300u;                  // token 1 (bit 2 -> 8)
    r[2] = u2 & 0x00C000C0u;                  // token 2 (bit 4 -> 6)
    r[3] = u2 & 0x03000300u;                  // token 3 (bit 6 -> 8)
  } else {
    const uint32_t w = chunk;                 // token i at bits 4i, i + 4 at 16 + 4i
    r[0] = (w << 4) & 0x00F000F0u;            // token 0 -> bits 4..7
    r[1] = w & 0x00F000F0u;                   // token 1 at bits 4..7
    r[2] = (w >> 2) & 0x03C003C0u;            // token 2 -> bits 6..9
    r[3] = (w >> 6) & 0x03C003C0u;            // token 3 -> bits 6..9
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

// Operand order of a lane group's trig registers.  Quad q (4 consecutive
// registers, one MFMA A operand) holds the pairs zero-point K-step q reads:
// those of code K-steps 2q and 2q + 1, each (pa, pb) with pa the pair of the
// code word's low half and pb = pa + HPW the matching pair of its high half.
// pair_at: position -> pair (relative to the lane group); pos_of: inverse.
template <int EPW>
__host__ __device__ constexpr int pair_at(int pos) {
  constexpr int HPW = EPW / 2;
  const int k = 2 * (pos / 4) + ((pos % 4) >> 1);
  return (k / HPW) * EPW + k % HPW + (pos & 1) * HPW;
}
template <int EPW>
__host__ __device__ constexpr int pos_of(int pair) {
  constexpr int HPW = EPW / 2;
  const int k = (pair / EPW) * HPW + pair % HPW;
  return 4 * (k / 2) + 2 * (k % 2) + (pair % EPW) / HPW;
}

template <int EPW, int PPG>
constexpr bool operand_order_is_permutation() {
  for (int p = 0; p < PPG; ++p)
    if (pair_at<EPW>(p) < 0 || pair_at<EPW>(p) >= PPG || pos_of<EPW>(pair_at<EPW>(p)) != p) return false;
  return true;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------- in-tile trig table
// For the token at offset j = 0..31 of a tile and RoPE pair i: e^{i j w_i}
// as a head with kTrigHeadBits significant bits plus the tail, both times
// kTrigScale, packed as fp16 (cos, sin) words at the pair's position in the
// operand order of its lane group; and e^{i 32 w_i}, the step from one tile
// start to the next.  e^{i j w} for j = 4a + b is the product of two of 11
// accurately rounded unit numbers (angle 4a w, a = 1..8, and b w, b = 1..3).
// The decode kernel builds the table in LDS at its start, or copies it from a
// table built once per cache by kivi_rope_table (same arithmetic, same bits).
template <int BITS>
constexpr int kTrigHeadBits = BITS == 2 ? 9 : 7;
constexpr float kTrigScale = 32768.0f;   // 2^15
constexpr uint32_t kRopeTableMagic = 0x52545442u;   // header word 0 of a built table
// Layout of a built table (uint32 words): header [magic, bits, d, theta bits],
// then head words [32][NP], tail words [32][NP] (NP = d / 2 pairs, at their
// operand-order positions), then the steps as float (cos, sin) [NP].
constexpr int kRopeTableHeader = 4;
inline size_t rope_table_words(int d) { return kRopeTableHeader + 2 * 32 * (d / 2) + 2 * (d / 2); }

// Builds the table with the NT threads of a workgroup (tid = thread index).
// base: LDS scratch of 11 * NP float2.  put(j, ps, head, tail) stores token
// j's words at operand position ps, put_step(i, e^{i 32 w_i}).  Ends with
// every base read done (a barrier inside, none at the end).
template <int D, int BITS, int NT, typename Put, typename PutStep>
__device__ __forceinline__ void build_trig_table(const double* omega, float2 (*base)[D / 2], int tid, Put put,
                                                 PutStep put_step) {
  constexpr int NP = D / 2, PPG = NP / 4, EPW = 16 / BITS, HB = kTrigHeadBits<BITS>;
  for (int e = tid; e < 11 * NP; e += NT) {
    const int r = e / NP, i = e % NP;
    float c, s;
    rope_unit(static_cast<double>(r < 8 ? 4 * (r + 1) : r - 7), omega[i], c, s);
    base[r][i] = float2{c, s};
  }
  __syncthreads();
  for (int e = tid; e < kGroup * NP; e += NT) {
    const int j = e / NP, i = e % NP;
    const int ja = j >> 2, jb = j & 3;
    const float2 u = ja ? base[ja - 1][i] : float2{1.0f, 0.0f};
    const float2 v = jb ? base[7 + jb][i] : float2{1.0f, 0.0f};
    const float c = fmaf(u.x, v.x, -(u.y * v.y)), s = fmaf(u.y, v.x, u.x * v.y);
    const float ch = trunc_sig(c, HB), sh = trunc_sig(s, HB);
    const int ps = (i / PPG) * PPG + pos_of<EPW>(i % PPG);
    put(j, ps, pack_f16(ch * kTrigScale, sh * kTrigScale), pack_f16((c - ch) * kTrigScale, (s - sh) * kTrigScale));
  }
  if (tid < NP) put_step(tid, base[7][tid]);
}

// kivi_rope_table's kernel: one workgroup of 256 threads.
template <int D, int BITS>
__global__ __launch_bounds__(256) void rope_table_kernel(RopeOmega w, uint32_t* __restrict__ table) {
  constexpr int NP = D / 2;
  __shared__ float2 base[11][NP];
  uint32_t* const th = table + kRopeTableHeader;
  uint32_t* const tl = th + kGroup * NP;
  float2* const st = reinterpret_cast<float2*>(tl + kGroup * NP);
  build_trig_table<D, BITS, 256>(
      w.omega, base, static_cast<int>(threadIdx.x),
      [&](int j, int ps, uint32_t h, uint32_t l) {
        th[j * NP + ps] = h;
        tl[j * NP + ps] = l;
      },
      [&](int i, float2 v) { st[i] = v; });
  if (threadIdx.x == 0) {
    table[0] = kRopeTableMagic;
    table[1] = BITS;
    table[2] = D;
    table[3] = __builtin_bit_cast(uint32_t, w.theta);
  }
}

// ----------------------------------------------------------------- kernel

template <int D, int BITS, int G>
__global__ __launch_bounds__(64 * kFWaves) __attribute__((amdgpu_waves_per_eu(kFWavesPerSimd))) void kivi_feat_kernel(
    KiviArgs a) {
  static_assert(BITS == 2 || BITS == 4, "feature kernel: 2- and 4-bit codes");
  constexpr int NP = D / 2;              // RoPE pairs
  constexpr int PPG = NP / 4;            // pairs of one lane group (16 lanes)
  constexpr int EPW = 16 / BITS;         // channels per fp16 half of a packed key word
  constexpr int HPW = EPW / 2;           // pairs per fp16 half of a word
  constexpr int NW = PPG * BITS / 16;    // key words per token of a lane group
  constexpr int KSC = PPG / 2;           // code K-steps (2 pairs per lane group each)
  constexpr int KSB = PPG / 4;           // zero-point K-steps (4 pairs per lane group each)
  constexpr int KTOT = 32 * (KSC + KSB); // B rows
  constexpr int BST = KTOT + 8;          // B column stride (halves): columns in different banks
  constexpr int NBC = 2 * G;             // B columns in use (hi, lo per head)
  constexpr int NITEM = G * 4 * KSB;     // per-tile factor items (head, lane group, K-step pair)
  constexpr int MB = D / 16;             // channel blocks of the value product
  constexpr int NVG = D / kGroup;        // value groups per token
  constexpr int NCOL = G * NVG;          // value-operand columns in use
  constexpr int KROW = D * BITS / 8;     // key bytes per token
  constexpr int LROW = NW * 4;           // key bytes per token of one lane group
  constexpr int VBLK = 4 * D * BITS;     // value bytes per 32-token block
  constexpr int VST = 24;                // row stride of the fp16 value staging area (halves)
  constexpr int KSR = D / 32;            // K-steps of a recent tile (channels)
  constexpr int TPR = NP + 4;            // packed trig row (padded: 16 rows start in different banks)
  static_assert(NCOL <= 16, "value-operand columns");
  static_assert(NITEM <= kWave, "one factor item per lane");
  static_assert(G * 4 * KSR <= kWave, "one recent-query item per lane");
  static_assert(HPW % 2 == 0 && KSC % 2 == 0, "K-step pairs share a word");
  static_assert(operand_order_is_permutation<EPW, PPG>(), "trig operand order");

  // ---- LDS.  Per wave, two slots (tiles t and t + 1) of: the B operand
  // [column][K], the key scales and zeros [scale/zero][channel], the value
  // scales and zeros [scale/zero][group][token].  During the set-up the B
  // area holds the trig bases and the packed trig table instead.
  constexpr int kBBytes = kFWaves * 2 * NBC * BST * 2;
  constexpr int kBaseBytes = 11 * NP * 8;
  constexpr int kTrigPackBytes = 2 * kGroup * TPR * 4;
  constexpr int kBigBytes = kBBytes > kBaseBytes + kTrigPackBytes ? kBBytes : kBaseBytes + kTrigPackBytes;
  __shared__ __attribute__((aligned(16))) uint8_t lds_big[kBigBytes];
  __shared__ __attribute__((aligned(16))) _Float16 lds_ksz[kFWaves][2][2][D];
  __shared__ __attribute__((aligned(16))) _Float16 lds_vsz[kFWaves][2][2][NVG][kGroup];
  __shared__ float2 lds_step[NP];        // e^{i 32 w}: one tile start to the next
  __shared__ float lds_m[kFWaves][G], lds_l[kFWaves][G];
  // per wave: the output rows (after the tiles), the recent tiles' value
  // staging, and a rotation per pair (the first quantized tile's start during
  // the set-up, a recent tile's start later)
  constexpr int kOutBytes = kFWaves * G * D * 4;
  constexpr int kVstBytes = kFWaves * kGroup * VST * 2;
  constexpr int kRotBytes = kFWaves * NP * 8;
  __shared__ __attribute__((aligned(16))) uint8_t lds_aux[kOutBytes + kVstBytes + kRotBytes];
  float2 (*const base)[NP] = reinterpret_cast<float2 (*)[NP]>(lds_big);
  uint32_t (*const lds_th)[TPR] = reinterpret_cast<uint32_t (*)[TPR]>(lds_big + kBaseBytes);
  uint32_t (*const lds_tl)[TPR] = reinterpret_cast<uint32_t (*)[TPR]>(lds_big + kBaseBytes + kTrigPackBytes / 2);
  float2 (*const lds_rot)[NP] = reinterpret_cast<float2 (*)[NP]>(lds_aux + kOutBytes + kVstBytes);
  float (*const lds_o)[G][D] = reinterpret_cast<float (*)[G][D]>(lds_aux);
  _Float16 (*const lds_vst)[kGroup * VST] = reinterpret_cast<_Float16 (*)[kGroup * VST]>(lds_aux + kOutBytes);

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * a.Hkv + kvh;
  _Float16 (*const lds_B)[NBC][BST] = reinterpret_cast<_Float16 (*)[NBC][BST]>(lds_big) + 2 * wave;

  // The wave's tiles (a recent tile weighs kRecentWeight quantized tiles):
  // its recent tiles first, then its run [qb, qb + nq) of quantized tiles.
  const WaveTiles wt = wave_tiles(a.split, split * kFWaves + wave);
  const int qb = wt.qb, nq = wt.nq, r_first = wt.r_first, r_mine = wt.r_mine;


  // ---- per-tile factor item of this lane: head ih, lane group ig, K-step
  // pair ikb (code K-steps 2 ikb, 2 ikb + 1; zero-point K-step ikb).  Its four
  // pairs (relative to the lane group): p0 = piA(2 ikb), p1 = piB(2 ikb),
  // p2 = p0 + 1, p3 = p1 + 1; channels cA..cA+3 (pairs p0, p2) and
  // cA + EPW..cA + EPW + 3 (p1, p3), cA = 2 (ig PPG + p0).
  const bool item = lane < NITEM;
  const int it = item ? lane : 0;
  const int ih = it / (4 * KSB), ig = (it / KSB) % 4, ikb = it % KSB;
  const int iks = 2 * ikb;
  const int ip0 = (iks / HPW) * EPW + iks % HPW;            // piA(2 ikb)
  const int ich = 2 * (ig * PPG + ip0);                       // first channel of chunk A
  // the item's query pairs in the order (p0, p2, p1, p3) = channels
  // (cA, cA + 2, cA + EPW, cA + EPW + 2), loaded now and rotated back to the
  // first tile after the set-up
  uint32_t qraw[4];
  {
    const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + ih) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      qraw[k] = *reinterpret_cast<const uint32_t*>(qh + ich + 2 * (k & 1) + EPW * (k >> 1));
  }

  // ---- tile inputs: key codes two tiles ahead, value codes one, scales
  // three (loads) and two (LDS staging).  The
  // first loads are issued before the set-up below, so their latency
  // overlaps it.
  const size_t qstride = static_cast<size_t>(a.qtile_stride);
  const uint16_t* const ksz_s = uniform_ptr(a.k_scale);
  const uint16_t* const ksz_z = uniform_ptr(a.k_zero);
  const uint16_t* const vsz_s = uniform_ptr(a.v_scale);
  const uint16_t* const vsz_z = uniform_ptr(a.v_zero);
  const uint8_t* const kbase = reinterpret_cast<const uint8_t*>(a.k_codes) + unit * qstride * kGroup * KROW;
  const uint8_t* const vbase = reinterpret_cast<const uint8_t*>(a.v_codes) + unit * qstride * VBLK;
  struct Codes {
    uint32_t k[2][NW];      // the lane's key words of its two tokens
    uint32_t v[MB];         // value chunks (2-bit: 16 bits used)
  };
  struct Scales {
    uint32_t ksz[D / 64];   // lanes 0..31: key scales of D / 32 channels; 32..63: zeros
    uint32_t vsz[NVG / 2];  // lanes 0..31: value scales of token lane; 32..63: zeros
  };
  auto load_keys = [&](int ti, Codes& t) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint8_t* p = kbase + (static_cast<size_t>(ti) * kGroup + row_token(s, col)) * KROW + grp * LROW;
      const Words<LROW> w = load_words<LROW>(p);
#pragma unroll
      for (int i = 0; i < NW; ++i) t.k[s][i] = w.w[i];
    }
  };
  auto load_values = [&](int ti, Codes& t) {
    const uint8_t* blk = vbase + static_cast<size_t>(ti) * VBLK;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint8_t* p = blk + (16 * mb + col) * 4 * BITS + grp * BITS;
      if constexpr (BITS == 2) t.v[mb] = *reinterpret_cast<const uint16_t*>(p);
      else t.v[mb] = *reinterpret_cast<const uint32_t*>(p);
    }
  };
  auto load_scales = [&](int ti, Scales& t) {
    const int half = lane >> 5, r = lane & 31;
    const Words<D / 16> kw = load_words<D / 16>((half ? ksz_z : ksz_s) + (unit * qstride + ti) * D + r * (D / 32));
#pragma unroll
    for (int i = 0; i < D / 64; ++i) t.ksz[i] = kw.w[i];
    const uint16_t* vsrc = (half ? vsz_z : vsz_s) + ((unit * qstride + ti) * kGroup + r) * NVG;
    const Words<2 * NVG> vw = load_words<2 * NVG>(vsrc);
#pragma unroll
    for (int i = 0; i < NVG / 2; ++i) t.vsz[i] = vw.w[i];
  };
  Codes c0, c1;
  Scales s0, s1;
  if (nq > 0) {
    load_keys(qb, c0);
    load_values(qb, c0);
    load_scales(qb, s0);
  }
  if (nq > 1) {
    load_keys(qb + 1, c1);
    load_scales(qb + 1, s1);
  }

  // ---- trig tables (build_trig_table): copied from the cache's built table
  // when its header matches (bits, d, theta), else built here; and e^{i t0 w}
  // of this wave's first quantized tile.
  if (lane < NP) {
    float c, s;
    rope_unit(static_cast<double>(qb) * kGroup, a.omega[lane], c, s);
    lds_rot[wave][lane] = float2{c, s};
  }
  {
    // the cache's built trig table (if any): header and contents requested
    // together, the header checked when they arrive (requesting them at the
    // kernel's start was measured slower: more registers live across the
    // tile loads)
    constexpr int kPieces = (2 * kGroup * NP / 4 + 64 * kFWaves - 1) / (64 * kFWaves);   // 16-byte pieces per thread
    bool copy = false;
    uint4 tv[kPieces];
    float2 step{1.0f, 0.0f};
    if (a.rope_table != nullptr) {
      const uint4 hdr = *reinterpret_cast<const uint4*>(a.rope_table);
      const uint32_t* const gt = a.rope_table + kRopeTableHeader;
#pragma unroll
      for (int k = 0; k < kPieces; ++k)
        tv[k] = reinterpret_cast<const uint4*>(gt)[min(tid + 64 * kFWaves * k, 2 * kGroup * NP / 4 - 1)];
      if (tid < NP) step = reinterpret_cast<const float2*>(gt + 2 * kGroup * NP)[tid];
      copy = hdr.x == kRopeTableMagic && hdr.y == static_cast<uint32_t>(BITS) && hdr.z == static_cast<uint32_t>(D) &&
             hdr.w == __builtin_bit_cast(uint32_t, a.rope_theta);
    }
    if (copy) {
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        const int w0 = 4 * (tid + 64 * kFWaves * k);
        if (w0 < 2 * kGroup * NP) {
          const int half = w0 / (kGroup * NP), j = (w0 % (kGroup * NP)) / NP, ps = w0 % NP;
          *reinterpret_cast<uint4*>(half ? &lds_tl[j][ps] : &lds_th[j][ps]) = tv[k];
        }
      }
      if (tid < NP) lds_step[tid] = step;
    } else {
      build_trig_table<D, BITS, 64 * kFWaves>(
          a.omega, base, tid,
          [&](int j, int ps, uint32_t h, uint32_t l) {
            lds_th[j][ps] = h;
            lds_tl[j][ps] = l;
          },
          [&](int i, float2 v) { lds_step[i] = v; });
    }
  }
  __syncthreads();

  // ---- the lane's trig registers: tokens j(s) (rows of the A operand of
  // half s), pairs grp * PPG + pair_at(pos); head (HB significant bits) and
  // tail, both times 2^15, as fp16 (cos, sin) pairs, in operand order
  u32x4 tqh[2][PPG / 4], tql[2][PPG / 4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = row_token(s, col);
#pragma unroll
    for (int q = 0; q < PPG / 4; ++q) {
      tqh[s][q] = *reinterpret_cast<const u32x4*>(&lds_th[j][grp * PPG + 4 * q]);
      tql[s][q] = *reinterpret_cast<const u32x4*>(&lds_tl[j][grp * PPG + 4 * q]);
    }
  }
  auto trig_h = [&](int s, int pair) -> uint32_t { return tqh[s][pos_of<EPW>(pair) / 4][pos_of<EPW>(pair) % 4]; };
  auto trig_l = [&](int s, int pair) -> uint32_t { return tql[s][pos_of<EPW>(pair) / 4][pos_of<EPW>(pair) % 4]; };

  float iq[4][2];
  {
    const float qs = a.q_scale * 32.0f;      // log2-domain logits, code factors carry 2^5
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = ich + 2 * (k & 1) + EPW * (k >> 1);
      const float x0 = h2f(static_cast<uint16_t>(qraw[k] & 0xFFFFu)) * qs;
      const float x1 = h2f(static_cast<uint16_t>(qraw[k] >> 16)) * qs;
      const float2 r = lds_rot[wave][c / 2];
      iq[k][0] = x0 * r.x + x1 * r.y;        // R(-t0) q
      iq[k][1] = x1 * r.x - x0 * r.y;
    }
  }
  // the set-up areas are free from here on
  __syncthreads();

  float4v acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, lsum = 0.0f, zacc = 0.0f;
  const int qh = col % G;                         // logit column -> query head
  const int vg = min(col / G, NVG - 1);           // value column -> value group
  const int bcol = col % NBC;                     // B column this lane reads

  // hi + lo logit columns: lanes col and col +- G (mod 2G) hold the same head
  auto combine_cols = [&](float x) -> float {
    if constexpr (G == 4) return x + dpp<0x124>(x);          // row_ror:4
    else if constexpr (G == 2) return x + dpp<kDppQuadXor2>(x);
    else return x + dpp<kDppQuadXor1>(x);
  };

  // online softmax over the lane's 8 logits (the column max over the 4 row
  // groups); returns the probabilities in p.  MASKED: some logits may be
  // -inf (a partial recent tile), so the running max may still be -inf.
  auto softmax_step = [&](float* lg, float* p, auto masked) {
    float tm = lg[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tm = fmaxf(tm, lg[e]);
    tm = max_rows(tm);
    const float mn = fmaxf(m, tm);
    if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {
      const float sc = merge_weight(m, mn);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= sc;
      lsum *= sc;
      zacc *= sc;
    }
    m = mn;
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (decltype(masked)::value)
        p[e] = (mn == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg[e] - mn);
      else
        p[e] = __builtin_amdgcn_exp2f(lg[e] - mn);
      ps += p[e];
    }
    lsum += ps;
  };

  // ------------------------------------------------------ fp16 recent tile
  // Keys rotated in fp32 with the trig registers (head + tail), split into
  // fp16 hi + lo, against the query rotated to the tile start.
  const uint16_t* const krb = a.k_recent + unit * a.R_cap * D;
  const uint16_t* const vrb = a.v_recent + unit * a.R_cap * D;
  auto recent_tile = [&](int rt) {
    const int r0 = rt * kGroup;
    const double t0 = static_cast<double>(a.n_qtiles + rt) * kGroup;
    _Float16* const Bw = &lds_B[0][0][0];
    // keys: the lane's 8 channels of K-step ks for its two tokens (the
    // value slabs are loaded after the key products, when these are dead)
    uint4 kin[2][KSR];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = r0 + row_token(s, col);
#pragma unroll
      for (int ks = 0; ks < KSR; ++ks) {
        kin[s][ks] = uint4{0u, 0u, 0u, 0u};
        if (r < a.R)
          kin[s][ks] = *reinterpret_cast<const uint4*>(krb + static_cast<size_t>(r) * D + 2 * PPG * grp + 8 * ks);
      }
    }
    // e^{i t0 w} once per pair, shared through LDS
    if (lane < NP) {
      float c, s;
      rope_unit(t0, a.omega[lane], c, s);
      lds_rot[wave][lane] = float2{c, s};
    }
    wave_sync();
    // B: the query rotated to t0 (no 2^5), K = the lane group's channels in
    // order: item (head, lane group, K-step) of this lane writes 8 channels
    if (lane < G * 4 * KSR) {
      const int h = lane / (4 * KSR), g = (lane / KSR) % 4, ks = lane % KSR;
      const int c0 = 2 * PPG * g + 8 * ks;
      const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c0;
      const uint4 qw = *reinterpret_cast<const uint4*>(qh);
      const uint32_t qq[4] = {qw.x, qw.y, qw.z, qw.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = h2f(static_cast<uint16_t>(qq[i] & 0xFFFFu)) * a.q_scale;
        const float x1 = h2f(static_cast<uint16_t>(qq[i] >> 16)) * a.q_scale;
        const float2 r = lds_rot[wave][c0 / 2 + i];
        split2(x0 * r.x + x1 * r.y, x1 * r.x - x0 * r.y, hi[i], lo[i]);
      }
      const int K = 32 * ks + 8 * g;
      *reinterpret_cast<uint4*>(Bw + h * BST + K) = uint4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<uint4*>(Bw + (G + h) * BST + K) = uint4{lo[0], lo[1], lo[2], lo[3]};
    }
    wave_sync();
    float4v sacc[2] = {float4v{0.0f, 0.0f, 0.0f, 0.0f}, float4v{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < KSR; ++ks) {
      const half8 bv = *reinterpret_cast<const half8*>(Bw + bcol * BST + 32 * ks + 8 * grp);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t w[4] = {kin[s][ks].x, kin[s][ks].y, kin[s][ks].z, kin[s][ks].w};
        uint32_t ah[4], al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2v th = __builtin_bit_cast(half2v, trig_h(s, 4 * ks + i));
          const half2v tl = __builtin_bit_cast(half2v, trig_l(s, 4 * ks + i));
          const float cs = (static_cast<float>(th[0]) + static_cast<float>(tl[0])) * (1.0f / kTrigScale);
          const float sn = (static_cast<float>(th[1]) + static_cast<float>(tl[1])) * (1.0f / kTrigScale);
          const float x0 = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
          const float x1 = h2f(static_cast<uint16_t>(w[i] >> 16));
          split2(x0 * cs - x1 * sn, x0 * sn + x1 * cs, ah[i], al[i]);
        }
        sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ah), bv, sacc[s], 0, 0, 0);
        sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, al), bv, sacc[s], 0, 0, 0);
      }
    }
    // value slabs: token lane / 2, 8 channels of block mb
    uint4 vin[MB];
    {
      const int r = r0 + (lane >> 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        vin[mb] = uint4{0u, 0u, 0u, 0u};
        if (r < a.R) vin[mb] = *reinterpret_cast<const uint4*>(vrb + static_cast<size_t>(r) * D + 16 * mb + 8 * (lane & 1));
      }
    }
    float lg[8], p[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[2 * r] = combine_cols(sacc[0][r]);
      lg[2 * r + 1] = combine_cols(sacc[1][r]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (r0 + 8 * grp + vtok(e) >= a.R) lg[e] = -INFINITY;
    softmax_step(lg, p, std::true_type{});
    half8 bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[e] = static_cast<_Float16>(col < NCOL ? p[e] : 0.0f);
    // values pass through LDS 16 channels at a time to form the
    // channel-major operand
    _Float16* const st = lds_vst[wave];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      *reinterpret_cast<uint4*>(&st[(lane >> 1) * VST + 8 * (lane & 1)]) = vin[mb];
      wave_sync();
      half8 av;
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = st[(8 * grp + vtok(e)) * VST + col];
      wave_sync();
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[mb], 0, 0, 0);
    }
    wave_sync();
  };

  // ------------------------------------------------------- quantized tiles
  // value-scale factor of this lane's staging token (lanes 0..31: scales)
  const uint32_t vfac = (lane < 32 && feat_vlow<BITS>(lane & 31)) ? 0x44004400u : 0x3C003C00u;  // (4, 4) or (1, 1)
  // a tile's key scales and zeros into slot sl (lanes 0..31 scales, 32..63 zeros)
  auto stage_ksz = [&](const Scales& t, int sl) {
    const int half = lane >> 5, r = lane & 31;
    if constexpr (D / 64 == 2)
      *reinterpret_cast<uint2*>(&lds_ksz[wave][sl][half][r * (D / 32)]) = uint2{t.ksz[0], t.ksz[1]};
    else
      *reinterpret_cast<uint32_t*>(&lds_ksz[wave][sl][half][r * (D / 32)]) = t.ksz[0];
  };
  // a tile's value scales (times the position factor) and zeros into slot sl
  auto stage_vsz = [&](const Scales& t, int sl) {
    const int half = lane >> 5, r = lane & 31;
#pragma unroll
    for (int i = 0; i < NVG / 2; ++i) {
      const uint32_t w = __builtin_bit_cast(
          uint32_t, __builtin_bit_cast(half2v, t.vsz[i]) * __builtin_bit_cast(half2v, vfac));
      lds_vsz[wave][sl][half][2 * i][r] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu));
      lds_vsz[wave][sl][half][2 * i + 1][r] = __builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16));
    }
  };

  // the per-tile factors of the item from the key scales and zeros in slot
  // sl -> B of slot sl (hi in column ih, lo in G + ih); then the query steps
  // to the next tile's start
  auto write_factors = [&](int sl) {
    if (!item) return;
    _Float16* const Bw = &lds_B[sl][0][0];
    // scales and zeros of channels (cA, cA+1, cA+2, cA+3) and (cA+EPW, ...)
    // as fp16 pairs: word kk of chunk c holds channels 2 kk, 2 kk + 1 (the
    // a and b channel of the chunk's pair kk)
    uint32_t sw[2][2], zw[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint2 s2 = *reinterpret_cast<const uint2*>(&lds_ksz[wave][sl][0][ich + c * EPW]);
      const uint2 z2 = *reinterpret_cast<const uint2*>(&lds_ksz[wave][sl][1][ich + c * EPW]);
      sw[c][0] = s2.x;
      sw[c][1] = s2.y;
      zw[c][0] = z2.x;
      zw[c][1] = z2.y;
    }
    // code K-steps 2 ikb (pairs p0 = chunk A channels 0,1; p1 = chunk B
    // channels 0,1) and 2 ikb + 1 (p2 = chunk A channels 2,3; p3 = B 2,3)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float f[8];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float qa = iq[2 * c + kk][0], qb_ = iq[2 * c + kk][1];
        f[4 * c + 0] = mix_mul<0>(sw[c][kk], qa);       // s_a q'_a
        f[4 * c + 1] = mix_mul<0>(sw[c][kk], qb_);      // s_a q'_b
        f[4 * c + 2] = mix_mul<1>(sw[c][kk], qb_);      // s_b q'_b
        f[4 * c + 3] = mix_mul<1, true>(sw[c][kk], qa);  // -s_b q'_a
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split2(f[2 * i], f[2 * i + 1], hi[i], lo[i]);
      const int K = 32 * (iks + kk) + 8 * ig;
      *reinterpret_cast<uint4*>(Bw + ih * BST + K) = uint4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<uint4*>(Bw + (G + ih) * BST + K) = uint4{lo[0], lo[1], lo[2], lo[3]};
    }
    // zero-point K-step ikb: pairs in the order p0, p1, p2, p3
    {
      float f[8];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = q4 & 1, kk = q4 >> 1;               // chunk, pair within chunk
        const float qa = iq[2 * c + kk][0], qb_ = iq[2 * c + kk][1];
        f[2 * q4 + 0] = mix_fma<0>(zw[c][kk], qa, mix_mul<1>(zw[c][kk], qb_));    // z_a q'_a + z_b q'_b
        f[2 * q4 + 1] = mix_fma<0>(zw[c][kk], qb_, mix_mul<1, true>(zw[c][kk], qa));   // z_a q'_b - z_b q'_a
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split2(f[2 * i], f[2 * i + 1], hi[i], lo[i]);
      const int K = 32 * (KSC + ikb) + 8 * ig;
      *reinterpret_cast<uint4*>(Bw + ih * BST + K) = uint4{hi[0], hi[1], hi[2], hi[3]};
      *reinterpret_cast<uint4*>(Bw + (G + ih) * BST + K) = uint4{lo[0], lo[1], lo[2], lo[3]};
    }
    // the query to the next tile's start: q' <- R(-32 w) q'
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 st = lds_step[(ich + 2 * (k & 1) + EPW * (k >> 1)) / 2];
      const float x0 = iq[k][0], x1 = iq[k][1];
      iq[k][0] = x0 * st.x + x1 * st.y;
      iq[k][1] = x1 * st.x - x0 * st.y;
    }
  };

  // Tile i of the run (slot sl = i & 1): its B, value scales and the next
  // tile's key scales are in LDS.  The logits of tile i run together with
  // the factors of tile i + 1 (other slot); at the end the next tile's value
  // scales and the key scales of tile i + 2 are staged.  `cur` holds tile
  // i's codes, `nxt` receives tile i + 1's; `sn1` holds the scales of tile
  // i + 1, `sn2` those of tile i + 2, and then receives tile i + 3's.  Key
  // codes run two tiles ahead: `cur`'s keys, once used, receive tile i + 2's.
  auto quantized_tile = [&](int i, int sl, Codes& cur, Codes& nxt, Scales& sn1, Scales& sn2) {
    wave_sync();
    // (past the run's end the last tile is loaded again, unused: no branch)
    load_values(qb + min(i + 1, nq - 1), nxt);
    const _Float16* const Bw = &lds_B[sl][0][0];

    // The wave runs at raised priority from its logit products through its
    // softmax: of the two waves on a SIMD, the one feeding the matrix cores
    // (and then needing their results) issues first, and the other fills the
    // gaps with its value product, staging and loads (measured: kernel 55
    // against 59 us at 2 bits, 62.7 against 64.4 us at 4 bits).
    __builtin_amdgcn_s_setprio(1);
    // logits: zero-point K-steps (their sums carry 2^20) and code K-steps in
    // separate accumulators
    float4v zs[2] = {float4v{0.0f, 0.0f, 0.0f, 0.0f}, float4v{0.0f, 0.0f, 0.0f, 0.0f}};
    float4v cs[2] = {float4v{0.0f, 0.0f, 0.0f, 0.0f}, float4v{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int kb = 0; kb < KSB; ++kb) {
      const half8 bv = *reinterpret_cast<const half8*>(Bw + bcol * BST + 32 * (KSC + kb) + 8 * grp);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        zs[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, tqh[s][kb]), bv, zs[s], 0, 0, 0);
        zs[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, tql[s][kb]), bv, zs[s], 0, 0, 0);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSC; ++ks) {
      const half8 bv = *reinterpret_cast<const half8*>(Bw + bcol * BST + 32 * ks + 8 * grp);
      const int w = ks / HPW, ip = ks % HPW;
      const int pa = w * EPW + ip, pb = pa + HPW;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint32_t ca = key_code_at4<BITS>(cur.k[s][w], 2 * ip);
        const uint32_t cb = key_code_at4<BITS>(cur.k[s][w], 2 * ip + 1);
        uint32_t ah[4], al[4];
        ah[0] = pk_mul_bcast<0>(ca, trig_h(s, pa));
        ah[1] = pk_mul_bcast<0>(cb, trig_h(s, pa));
        ah[2] = pk_mul_bcast<1>(ca, trig_h(s, pb));
        ah[3] = pk_mul_bcast<1>(cb, trig_h(s, pb));
        al[0] = pk_mul_bcast<0>(ca, trig_l(s, pa));
        al[1] = pk_mul_bcast<0>(cb, trig_l(s, pa));
        al[2] = pk_mul_bcast<1>(ca, trig_l(s, pb));
        al[3] = pk_mul_bcast<1>(cb, trig_l(s, pb));
        cs[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ah), bv, cs[s], 0, 0, 0);
        cs[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, al), bv, cs[s], 0, 0, 0);
      }
    }
    load_keys(qb + min(i + 2, nq - 1), cur);
    // the next tile's factors, independent of the products above (after the
    // run's last tile they are computed from stale scales and never read)
    write_factors(sl ^ 1);

    // element e of the lane's run is token 8 grp + vtok(e)
    float lg[8], p[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[2 * r] = combine_cols(fmaf(zs[0][r], 1.0f / 1048576.0f, cs[0][r]));
      lg[2 * r + 1] = combine_cols(fmaf(zs[1][r], 1.0f / 1048576.0f, cs[1][r]));
    }
    softmax_step(lg, p, std::false_type{});
    __builtin_amdgcn_s_setprio(0);

    // value product: column (head qh, group vg) holds p * scale
    const uint4 vs4 = *reinterpret_cast<const uint4*>(&lds_vsz[wave][sl][0][vg][8 * grp]);
    const uint4 vz4 = *reinterpret_cast<const uint4*>(&lds_vsz[wave][sl][1][vg][8 * grp]);
    const uint32_t vsw[4] = {vs4.x, vs4.y, vs4.z, vs4.w}, vzw[4] = {vz4.x, vz4.y, vz4.z, vz4.w};
    half8 bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // the staged scale of token t = vtok(e) is half t % 2 of word t / 2
      const int t = vtok(e);
      const float pv = (t & 1) ? mix_mul<1>(vsw[t >> 1], p[e]) : mix_mul<0>(vsw[t >> 1], p[e]);
      bv[e] = static_cast<_Float16>(col < NCOL ? pv : 0.0f);
      zacc = (t & 1) ? mix_fma<1>(vzw[t >> 1], p[e], zacc) : mix_fma<0>(vzw[t >> 1], p[e], zacc);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(feat_value_codes8<BITS>(cur.v[mb]), bv, acc[mb], 0, 0, 0);

    // stage the next tile's value scales and the key scales two tiles on,
    // then load the scales three tiles on into the buffer just staged from
    if (i + 1 < nq) stage_vsz(sn1, sl ^ 1);
    if (i + 2 < nq) stage_ksz(sn2, sl);
    if (i + 3 < nq) load_scales(qb + i + 3, sn1);
  };

  // the wave's recent tiles (B slot 0), then its quantized run
  for (int k = 0; k < r_mine; ++k) recent_tile(r_first + k);
  // fp16 value products are exact-scale; switch the accumulator to the
  // code-product domain (a power of two: exact)
  if (r_mine > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= 1.0f / static_cast<float>(1u << kVShift<BITS>);
  }
  if (nq > 0) {
    // tile 0: key and value scales into slot 0, tile 1's key scales into
    // slot 1; the factors of tile 0; tile 2's scales into the free buffer
    stage_ksz(s0, 0);
    stage_vsz(s0, 0);
    if (nq > 1) stage_ksz(s1, 1);
    wave_sync();
    write_factors(0);
    if (nq > 2) load_scales(qb + 2, s0);
  }
  for (int i = 0; i < nq; i += 2) {
    // tile i: codes c0, slot 0, scales of i + 1 in s1 and of i + 2 in s0
    quantized_tile(i, 0, c0, c1, s1, s0);
    // tile i + 1: codes c1, slot 1, scales of i + 2 in s0 and of i + 3 in s1
    if (i + 1 < nq) quantized_tile(i + 1, 1, c1, c0, s0, s1);
  }

  // ---- wave state -> LDS: row sums and zero-point sums over the 4 row
  // groups of each column
  lsum = sum_rows(lsum);
  zacc = sum_rows(zacc);
  if (col < NCOL) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (mb / 2 == vg)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          lds_o[wave][qh][16 * mb + 4 * grp + r] =
              fmaf(acc[mb][r], static_cast<float>(1u << kVShift<BITS>), zacc);
  }
  if (lane < G) {
    lds_m[wave][lane] = m;
    lds_l[wave][lane] = lsum;
  }
  __syncthreads();
  write_split_state<D, G, kFWaves>(a.partials, a.counters + unit, a.out, a.Hq, unit, b, kvh, split, a.total_splits,
                                   lds_m, lds_l, lds_o);
}

template <int D, int BITS>
int launch_feat_g(const KiviArgs& a, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((kivi_feat_kernel<D, BITS, 1>), grid, dim3(64 * kFWaves), 0, s, a); break;
    case 2: hipLaunchKernelGGL((kivi_feat_kernel<D, BITS, 2>), grid, dim3(64 * kFWaves), 0, s, a); break;
    case 4: hipLaunchKernelGGL((kivi_feat_kernel<D, BITS, 4>), grid, dim3(64 * kFWaves), 0, s, a); break;
    default: return DQA_ERR_UNSUPPORTED;
  }
  return DQA_OK;
}

}  // namespace

int feat_decode_workgroups() { return 256 * kFWavesPerSimd * 4 / kFWaves; }
int feat_waves_per_wg() { return kFWaves; }
int feat_recent_weight() { return kRecentWeight; }

size_t feat_rope_table_words(int d) { return rope_table_words(d); }

int launch_rope_table(float theta, int d, int bits, uint32_t* table, hipStream_t s) {
  RopeOmega w;
  rope_omega(theta, d, w.omega);
  w.theta = theta;
  if (d == 128) {
    if (bits == 2) hipLaunchKernelGGL((rope_table_kernel<128, 2>), dim3(1), dim3(256), 0, s, w, table);
    else hipLaunchKernelGGL((rope_table_kernel<128, 4>), dim3(1), dim3(256), 0, s, w, table);
  } else {
    if (bits == 2) hipLaunchKernelGGL((rope_table_kernel<64, 2>), dim3(1), dim3(256), 0, s, w, table);
    else hipLaunchKernelGGL((rope_table_kernel<64, 4>), dim3(1), dim3(256), 0, s, w, table);
  }
  return hipPeekAtLastError() == hipSuccess ? DQA_OK : DQA_ERR_HIP;
}

int launch_feat_decode(const KiviArgs& a, int d, int G, int bits, dim3 grid, hipStream_t s) {
  if (d == 128) return bits == 2 ? launch_feat_g<128, 2>(a, G, grid, s) : launch_feat_g<128, 4>(a, G, grid, s);
  return bits == 2 ? launch_feat_g<64, 2>(a, G, grid, s) : launch_feat_g<64, 4>(a, G, grid, s);
}

}  // namespace dqa
