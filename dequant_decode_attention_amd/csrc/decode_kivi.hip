// Split-K decode attention over the uniform (KIVI) low-bit cache, with the
// dequantization fused into the products.
//
// [P1 para 2]: every decode step reads the whole cache from HBM, so the step
// is bounded by memory traffic; the codes are read once and expanded in
// registers.  [P1 para 4, 5]: keys carry one scale/zero per (channel,
// 32-token block), values one per (token, 32-channel block).  [P1 para 7]:
// keys were quantized before RoPE; the rotation is applied here, after
// dequantization.  [P1 para 8]: up to 128 recent tokens are kept in fp16
// and attended after the quantized ones.  [P1 para 6]: the output is the
// softmax-weighted sum of the values.
//
// Work decomposition (one GPU, one launch): grid = (splits, KV heads,
// batch).  The tiles of a (batch, KV head) -- its 32-token quantized tiles,
// then its fp16 recent tiles (at most 4) -- are spread evenly over the
// splits' waves, each wave taking a contiguous run; a wave keeps the next
// tile's codes and scales in flight while it computes the current one.
// Both contractions run on the matrix cores (v_mfma_f32_16x16x32_f16):
//   * logits: A = 16 dequantized, rotated keys (rows = tokens), split into
//     fp16 hi + lo; B = the query, rotated back to the tile's first position
//     and pre-scaled, also split hi + lo, replicated over the 16 columns
//     (column n holds query head n % G).  Three products (hi.hi, lo.hi,
//     hi.lo) keep the logits close to fp32 accuracy.  Because
//     q . R(t0 + j) k = (R(t0)^T q) . R(j) k, the per-token rotation only
//     needs the 32 in-tile factors R(j), shared by every tile (LDS table).
//   * values: A = the value codes of 16 channels x 32 tokens (small
//     integers, exact in fp16); B column n = (head n % G, value group n / G)
//     holds p * scale of that group; the zero point enters as sum(p * zero)
//     in fp32.  Column n of the logit output holds the probabilities of
//     exactly the tokens that column n of the value operand needs, so no
//     data moves between the two products.
// The online softmax runs once per tile per column.  Each split writes its
// partial softmax state; the last split of every (batch, KV head) to finish
// merges them in split order (merge.h).
#include <mutex>

#include "decode_common.h"
#include "merge.h"

namespace dqa {
namespace {

constexpr int kWavesPerWG = 4;
// Waves per SIMD the decode kernel is compiled for, and the workgroups that
// are then resident at once on 256 compute units (one workgroup = 4 waves,
// so waves per SIMD = workgroups per unit).  The 2-bit kernel fits 3 waves
// per SIMD (168 registers); the 4- and 8-bit kernels measured faster at 2.
template <int BITS>
constexpr int kDecodeWavesPerSimd = BITS == 2 ? 3 : 2;
inline int decode_workgroups(int bits) { return 256 * (bits == 2 ? kDecodeWavesPerSimd<2> : kDecodeWavesPerSimd<4>); }
// 2- and 4-bit caches with RoPE run the feature-product kernel (decode_feat.hip)
inline bool use_feat(int bits, bool rope) { return rope && (bits == 2 || bits == 4); }

// ------------------------------------------------------------- the kernel

template <int D, int BITS, int G, bool ROPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kDecodeWavesPerSimd<BITS>))) void kivi_decode_kernel(KiviArgs a) {
  constexpr int KS = D / 32;            // K-steps of the logit product
  constexpr int CPL = D / 4;            // key channels per lane (per token)
  constexpr int MB = D / 16;            // channel blocks of the value product
  constexpr int NVG = D / kGroup;       // value groups per token
  constexpr int NCOL = G * NVG;         // value-operand columns in use
  constexpr int NPAIR = D / 2;          // RoPE pairs
  constexpr int LROW = CPL * BITS / 8;  // key bytes per lane per token
  constexpr int KROW = D * BITS / 8;    // key bytes per token
  constexpr int VBLK = 4 * D * BITS;    // value bytes per 32-token block
  // Row j of the in-tile rotation table starts at float j * ERF + 16 * ((j >> 3) & 3):
  // ERF = 4 (mod 32) and the extra offset put the rows that one read
  // instruction touches (tokens j, j + 8, j + 16, j + 24 of a lane group) in
  // different LDS banks.
  constexpr int ERF = ((2 * NPAIR + 44 + 31) / 32) * 32 + 4;
  constexpr int VST = 24;               // row stride of the fp16 value staging area (halves)
  constexpr int QS = D + 8;             // row stride of the query operand (halves): heads in different banks
  constexpr int QH = 2 * G * QS;        // halves of the per-wave query operand (hi, lo)
  constexpr int WQ = QH > kGroup * VST ? QH : kGroup * VST;
  constexpr int LPP = kWave / NPAIR;    // lanes per RoPE pair in the query rotation
  constexpr int HPL = (G + LPP - 1) / LPP;  // heads per lane in the query rotation
  constexpr int SZW = D / 64;           // 32-bit words per lane of a tile's scale block
  static_assert(NCOL <= 16, "value-operand columns");

  __shared__ __attribute__((aligned(16))) float lds_E[ROPE ? kGroup * ERF : 4];
  __shared__ __attribute__((aligned(16))) _Float16 lds_w[kWavesPerWG][WQ];
  // a tile's key scales (fp32, each times 2^(24 - BITS * p) for its code's
  // bit position p: key_code_pos) and zeros (fp16)
  __shared__ __attribute__((aligned(16))) float lds_ks[kWavesPerWG][D];
  __shared__ __attribute__((aligned(16))) _Float16 lds_kz[kWavesPerWG][D];
  __shared__ __attribute__((aligned(16))) _Float16 lds_vsz[kWavesPerWG][2][NVG][kGroup];
  __shared__ float lds_m[kWavesPerWG][G], lds_l[kWavesPerWG][G];
  __shared__ __attribute__((aligned(16))) float lds_o[kWavesPerWG][G][D];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * a.Hkv + kvh;
  // The wave's work (wave_tiles, every tile one work unit): its recent tiles
  // first, then its contiguous run [qb, qe) of quantized tiles.
  const WaveTiles wt = wave_tiles(a.split, split * kWavesPerWG + wave);
  const int qb = wt.qb, qe = wt.qb + wt.nq, r_first = wt.r_first, r_mine = wt.r_mine;

  // in-tile rotation table E[j][i] = e^{i j omega_i}, j = 0..31: thread
  // (pair i, block q) evaluates e^{i 8q omega_i} and e^{i omega_i} accurately
  // and steps through the block's 8 offsets by complex products
  const int pi = lane % NPAIR;
  float an_c = 1.0f, an_s = 0.0f, w32c = 1.0f, w32s = 0.0f;
  if constexpr (ROPE) {
    static_assert(kGroup * NPAIR / 8 <= 256, "one table block per thread");
    if (tid < kGroup * NPAIR / 8) {
      const int i = tid % NPAIR, q = tid / NPAIR;
      float bc, bs, sc, ss;
      rope_unit(static_cast<double>(8 * q), a.omega[i], bc, bs);
      rope_unit(1.0, a.omega[i], sc, ss);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lds_E[erow<ERF>(8 * q + j) + 2 * i] = bc;
        lds_E[erow<ERF>(8 * q + j) + 2 * i + 1] = bs;
        const float nc = bc * sc - bs * ss;
        const float ns = bc * ss + bs * sc;
        bc = nc;
        bs = ns;
      }
    }
    if (qb < qe) rope_unit(static_cast<double>(qb) * kGroup, a.omega[pi], an_c, an_s);
    rope_unit(static_cast<double>(kGroup), a.omega[pi], w32c, w32s);
    __syncthreads();
  }

  // query pairs this lane rotates: pair pi of heads lane / NPAIR + k * LPP
  float qv[HPL][2];
#pragma unroll
  for (int k = 0; k < HPL; ++k) {
    const int h = lane / NPAIR + k * LPP;
    qv[k][0] = qv[k][1] = 0.0f;
    if (h < G) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + 2 * pi);
      qv[k][0] = h2f(static_cast<uint16_t>(w & 0xFFFFu)) * a.q_scale;
      qv[k][1] = h2f(static_cast<uint16_t>(w >> 16)) * a.q_scale;
    }
  }
  _Float16* const wq = lds_w[wave];
  // B operand of the logit product for the current tile: the query rotated
  // back by the tile position, split hi/lo, [hi|lo][head][channel]
  auto write_query = [&](float cth, float sth) {
#pragma unroll
    for (int k = 0; k < HPL; ++k) {
      const int h = lane / NPAIR + k * LPP;
      if (h < G) {
        float r0 = qv[k][0], r1 = qv[k][1];
        if constexpr (ROPE) {
          r0 = qv[k][0] * cth + qv[k][1] * sth;
          r1 = qv[k][1] * cth - qv[k][0] * sth;
        }
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
        const half2v lo = __builtin_bit_cast(
            half2v, __builtin_amdgcn_cvt_pkrtz(minus_half_lo(hb, r0), minus_half_hi(hb, r1)));
        *reinterpret_cast<uint32_t*>(&wq[h * QS + 2 * pi]) = hb;
        *reinterpret_cast<half2v*>(&wq[(G + h) * QS + 2 * pi]) = lo;
      }
    }
  };
  if constexpr (!ROPE) {
    write_query(1.0f, 0.0f);
    wave_sync();
  }

  float4v acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, lsum = 0.0f, zacc = 0.0f;
  const int qh = col % G;                       // logit column -> query head
  const int vg = min(col / G, NVG - 1);         // value column -> value group

  // logits of one tile from a key provider: kf(s, ks, x) fills the 8
  // dequantized (unrotated) fp32 keys of half s, K-step ks
  auto tile_logits = [&](int tile_pos, auto&& kf, float* lg) {
    float4v sacc[2] = {float4v{0.0f, 0.0f, 0.0f, 0.0f}, float4v{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = CPL * grp + 8 * ks;
      const half8 bqh = *reinterpret_cast<const half8*>(&wq[qh * QS + c0]);
      const half8 bql = *reinterpret_cast<const half8*>(&wq[(G + qh) * QS + c0]);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];
        kf(s, ks, x);
        if constexpr (ROPE) {
          const int j = row_token(s, col);
          const float4 e01 = *reinterpret_cast<const float4*>(&lds_E[erow<ERF>(j) + c0]);
          const float4 e23 = *reinterpret_cast<const float4*>(&lds_E[erow<ERF>(j) + c0 + 4]);
          const float ec[4] = {e01.x, e01.z, e23.x, e23.z};
          const float es[4] = {e01.y, e01.w, e23.y, e23.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float x0 = x[2 * p], x1 = x[2 * p + 1];
            x[2 * p] = x0 * ec[p] - x1 * es[p];
            x[2 * p + 1] = x0 * es[p] + x1 * ec[p];
          }
        }
        half8 kh, kl;
        split8(x, kh, kl);
        sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, bqh, sacc[s], 0, 0, 0);
        sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, bqh, sacc[s], 0, 0, 0);
        sacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, bql, sacc[s], 0, 0, 0);
      }
    }
    // element e of the lane's run is token 8 grp + vtok(e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lg[2 * r] = sacc[0][r];
      lg[2 * r + 1] = sacc[1][r];
    }
    (void)tile_pos;
  };

  // online softmax over the lane's 8 logits (column max across the 4 row
  // groups); returns the probabilities in p
  auto softmax_step = [&](float* lg, float* p) {
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
      p[e] = (mn == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(lg[e] - mn);
      ps += p[e];
    }
    lsum += ps;
  };

  // ---------------------------------------------------------- quantized tile
  // key-scale staging: lane r < 32 converts the scales of channels
  // CPS * r .. CPS * r + CPS - 1, each times 2^(24 - BITS * p) for the bit
  // position p of its code inside the masked register
  constexpr int CPS = D / 32;
  float sfac[CPS];
#pragma unroll
  for (int i = 0; i < CPS; ++i)
    sfac[i] = __builtin_ldexpf(1.0f, 24 - BITS * key_code_pos<BITS>(((lane & 31) * CPS + i) & 7));
  const size_t qstride = static_cast<size_t>(a.qtile_stride);      // tiles per (batch, KV head)
  const uint16_t* const ksz_s = uniform_ptr(a.k_scale);
  const uint16_t* const ksz_z = uniform_ptr(a.k_zero);
  const uint16_t* const vsz_s = uniform_ptr(a.v_scale);
  const uint16_t* const vsz_z = uniform_ptr(a.v_zero);
  const uint8_t* const kbase = reinterpret_cast<const uint8_t*>(a.k_codes) + unit * qstride * kGroup * KROW;
  const uint8_t* const vbase = reinterpret_cast<const uint8_t*>(a.v_codes) + unit * qstride * VBLK;
  constexpr int VW = BITS == 8 ? 2 : 1;   // 32-bit words per value chunk
  // two codes per register, one in each fp16 half, at the top of the
  // subnormal mantissa (value_codes8)
  const uint32_t vmask = opaque(BITS == 2 ? 0x03000300u : 0x03C003C0u);
  // a tile's raw inputs, loaded one tile ahead into registers that are not
  // touched until the tile is processed
  struct TileIn {
    Words<LROW> k[2];
    uint32_t v[MB][VW];
    uint32_t ksz[SZW], vsz[SZW];
  };
  auto load_tile = [&](int ti, TileIn& t) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      t.k[s] = load_words<LROW>(kbase + (static_cast<size_t>(ti) * kGroup + row_token(s, col)) * KROW + grp * LROW);
    const uint8_t* blk = vbase + static_cast<size_t>(ti) * VBLK;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint8_t* p = blk + (16 * mb + col) * 4 * BITS + grp * BITS;
      if constexpr (BITS == 2) {
        t.v[mb][0] = *reinterpret_cast<const uint16_t*>(p);
      } else if constexpr (BITS == 4) {
        t.v[mb][0] = *reinterpret_cast<const uint32_t*>(p);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        t.v[mb][0] = u.x;
        t.v[mb][VW - 1] = u.y;
      }
    }
    // scale blocks: lanes 0..31 read scales, 32..63 zeros
    const int half = lane >> 5, r = lane & 31;
    const uint16_t* ksrc = (half ? ksz_z : ksz_s) + (unit * qstride + ti) * D + r * (D / 32);
    const uint16_t* vsrc = (half ? vsz_z : vsz_s) + ((unit * qstride + ti) * kGroup + r) * NVG;
    const Words<4 * SZW> kw = load_words<4 * SZW>(ksrc);
    const Words<4 * SZW> vw = load_words<4 * SZW>(vsrc);
#pragma unroll
    for (int i = 0; i < SZW; ++i) {
      t.ksz[i] = kw.w[i];
      t.vsz[i] = vw.w[i];
    }
  };
  auto quantized_tile = [&](int ti, const TileIn& cur, TileIn& nxt, bool prefetch) {
    {
      const int half = lane >> 5, r = lane & 31;
      if (half == 0) {
        float sv[CPS];
#pragma unroll
        for (int i = 0; i < CPS; ++i)
          sv[i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(cur.ksz[i >> 1] >> ((i & 1) * 16)))) *
                  sfac[i];
        if constexpr (CPS == 4) {
          *reinterpret_cast<float4*>(&lds_ks[wave][r * CPS]) = float4{sv[0], sv[1], sv[2], sv[3]};
        } else {
          *reinterpret_cast<float2*>(&lds_ks[wave][r * CPS]) = float2{sv[0], sv[1]};
        }
      } else {
        if constexpr (SZW == 2) {
          *reinterpret_cast<uint2*>(&lds_kz[wave][r * CPS]) = uint2{cur.ksz[0], cur.ksz[1]};
        } else {
          *reinterpret_cast<uint32_t*>(&lds_kz[wave][r * CPS]) = cur.ksz[0];
        }
      }
#pragma unroll
      for (int g = 0; g < NVG; ++g)
        lds_vsz[wave][half][g][r] =
            __builtin_bit_cast(_Float16, static_cast<uint16_t>(cur.vsz[g >> 1] >> ((g & 1) * 16)));
    }
    if (prefetch) load_tile(ti + 1, nxt);
    if constexpr (ROPE) {
      write_query(an_c, an_s);
      const float nc = an_c * w32c - an_s * w32s;
      const float ns = an_c * w32s + an_s * w32c;
      an_c = nc;
      an_s = ns;
    }
    wave_sync();

    float lg[8], p[8];
    uint32_t km[2][8];   // masked key-code registers of the current word(s), per half
    tile_logits(ti * kGroup,
                [&](int s, int ks, float* x) {
                  if (BITS != 2 || (ks & 1) == 0) key_code_regs<BITS>(cur.k[s].w, ks, km[s]);
                  const int c0 = CPL * grp + 8 * ks;
                  const float4 s0 = *reinterpret_cast<const float4*>(&lds_ks[wave][c0]);
                  const float4 s1 = *reinterpret_cast<const float4*>(&lds_ks[wave][c0 + 4]);
                  const uint4 zq = *reinterpret_cast<const uint4*>(&lds_kz[wave][c0]);
                  const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                  const uint32_t zw[4] = {zq.x, zq.y, zq.z, zq.w};
#pragma unroll
                  for (int e = 0; e < 8; ++e) {
                    const uint32_t mr = km[s][key_code_reg<BITS>(e)];
                    if (key_code_half<BITS>(e, ks) == 0)
                      x[e] = (e & 1) ? mix_dequant<0, 1>(mr, sc[e], zw[e >> 1]) : mix_dequant<0, 0>(mr, sc[e], zw[e >> 1]);
                    else
                      x[e] = (e & 1) ? mix_dequant<1, 1>(mr, sc[e], zw[e >> 1]) : mix_dequant<1, 0>(mr, sc[e], zw[e >> 1]);
                  }
                },
                lg);
    softmax_step(lg, p);

    // value product: column (head qh, group vg) holds p * scale
    const half8 vs = *reinterpret_cast<const half8*>(&lds_vsz[wave][0][vg][8 * grp]);
    const half8 vz = *reinterpret_cast<const half8*>(&lds_vsz[wave][1][vg][8 * grp]);
    half8 bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = vtok(e);
      bv[e] = static_cast<_Float16>(col < NCOL ? p[e] * static_cast<float>(vs[t]) : 0.0f);
      zacc = fmaf(p[e], static_cast<float>(vz[t]), zacc);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint64_t ch = VW == 2 ? (static_cast<uint64_t>(cur.v[mb][VW - 1]) << 32) | cur.v[mb][0] : cur.v[mb][0];
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(value_codes8<BITS>(ch, vmask), bv, acc[mb], 0, 0, 0);
    }
    wave_sync();
  };

  // ------------------------------------------------------ fp16 recent tile
  const uint16_t* const krb = a.k_recent + unit * a.R_cap * D;
  const uint16_t* const vrb = a.v_recent + unit * a.R_cap * D;
  auto recent_tile = [&](int rt) {
    const int r0 = rt * kGroup;
    // every load of the tile is issued before any is used: keys (the lane's
    // 8 channels of K-step ks for its two tokens) and value slabs (token
    // lane/2, 8 channels of 16-channel block mb)
    uint4 kin[2][KS], vin[MB];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int r = r0 + row_token(s2, col);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kin[s2][ks] = uint4{0u, 0u, 0u, 0u};
        if (r < a.R) kin[s2][ks] = *reinterpret_cast<const uint4*>(krb + static_cast<size_t>(r) * D + CPL * grp + 8 * ks);
      }
    }
    {
      const int r = r0 + (lane >> 1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        vin[mb] = uint4{0u, 0u, 0u, 0u};
        if (r < a.R) vin[mb] = *reinterpret_cast<const uint4*>(vrb + static_cast<size_t>(r) * D + 16 * mb + 8 * (lane & 1));
      }
    }
    float rc = 1.0f, rs = 0.0f;
    if constexpr (ROPE) rope_unit(static_cast<double>(a.n_qtiles + rt) * kGroup, a.omega[pi], rc, rs);
    write_query(rc, rs);    // the value staging below reuses the query area
    wave_sync();
    float lg[8], p[8];
    tile_logits((a.n_qtiles + rt) * kGroup,
                [&](int s2, int ks, float* x) {
                  const uint32_t w[4] = {kin[s2][ks].x, kin[s2][ks].y, kin[s2][ks].z, kin[s2][ks].w};
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    x[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
                    x[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
                  }
                },
                lg);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (r0 + 8 * grp + vtok(e) >= a.R) lg[e] = -INFINITY;
    softmax_step(lg, p);
    half8 bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[e] = static_cast<_Float16>(col < NCOL ? p[e] : 0.0f);
    wave_sync();
    // values pass through LDS 16 channels at a time to form the
    // channel-major operand
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      *reinterpret_cast<uint4*>(&wq[(lane >> 1) * VST + 8 * (lane & 1)]) = vin[mb];
      wave_sync();
      half8 av;
#pragma unroll
      for (int e = 0; e < 8; ++e) av[e] = wq[(8 * grp + vtok(e)) * VST + col];
      wave_sync();
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[mb], 0, 0, 0);
    }
  };

  // the wave's recent tiles, then its quantized run; two register buffers
  // alternate so that the loads of tile i+1 stay in flight during tile i
  TileIn buf0, buf1;
  if (qb < qe) load_tile(qb, buf0);
  for (int k = 0; k < r_mine; ++k) recent_tile(r_first + k);
  // fp16 value products are exact-scale; switch the accumulator to the
  // code-product domain (a power of two: exact)
  if (r_mine > 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= 1.0f / kCodeScale<BITS>;
  }
  if constexpr (!ROPE) {
    if (r_mine > 0) {
      write_query(1.0f, 0.0f);   // restore the query area used for staging
      wave_sync();
    }
  }
  for (int ti = qb; ti < qe; ti += 2) {
    quantized_tile(ti, buf0, buf1, ti + 1 < qe);
    if (ti + 1 < qe) quantized_tile(ti + 1, buf1, buf0, ti + 2 < qe);
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
        for (int r = 0; r < 4; ++r) lds_o[wave][qh][16 * mb + 4 * grp + r] = fmaf(acc[mb][r], kCodeScale<BITS>, zacc);
  }
  if (lane < G) {
    lds_m[wave][lane] = m;
    lds_l[wave][lane] = lsum;
  }
  __syncthreads();
  write_split_state<D, G, kWavesPerWG>(a.partials, a.counters + unit, a.out, a.Hq, unit, b, kvh, split,
                                       a.total_splits, lds_m, lds_l, lds_o);
}

// ---------------------------------------------------------------- host side

struct Plan {
  int G, n_qtiles, n_rtiles, total;
  size_t units, ws_bytes;
};

int make_plan(const dqa_kivi_cache* c, Plan* p) {
  if (!c) return DQA_ERR_NULL;
  if (c->B < 0 || c->Hq <= 0 || c->Hkv <= 0 || c->T_q < 0 || c->R < 0) return DQA_ERR_SHAPE;
  if (c->d != 64 && c->d != 128) return DQA_ERR_SHAPE;
  if (c->bits != 2 && c->bits != 4 && c->bits != 8) return DQA_ERR_BITS;
  if (c->Hq % c->Hkv != 0) return DQA_ERR_SHAPE;
  if (c->T_q % kGroup != 0 || c->R > kMaxRecent) return DQA_ERR_SHAPE;
  if (c->T_cap < 0 || c->T_cap % kGroup != 0 || (c->T_cap > 0 && c->T_cap < c->T_q)) return DQA_ERR_SHAPE;
  if (c->R_cap < 0 || (c->R_cap > 0 && c->R_cap < c->R)) return DQA_ERR_SHAPE;
  if (c->B > 65535 || c->Hkv > 65535) return DQA_ERR_SHAPE;
  p->G = c->Hq / c->Hkv;
  if (p->G != 1 && p->G != 2 && p->G != 4) return DQA_ERR_UNSUPPORTED;
  p->units = static_cast<size_t>(c->B) * c->Hkv;
  p->n_qtiles = c->T_q / kGroup;
  p->n_rtiles = (c->R + kGroup - 1) / kGroup;
  // One resident round of workgroups (as many per compute unit as the
  // kernel has waves per SIMD), at least one tile per wave when the cache is
  // long enough; an empty cache still gets one split (zero output).
  const long long n_tiles = p->n_qtiles + p->n_rtiles;
  const int wg = use_feat(c->bits, c->rope_theta > 0.0f) ? feat_decode_workgroups() : decode_workgroups(c->bits);
  long long want = (wg + static_cast<long long>(p->units) - 1) /
                   static_cast<long long>(p->units > 0 ? p->units : 1);
  long long cap = (n_tiles + kWavesPerWG - 1) / kWavesPerWG;
  if (want > cap) want = cap;
  if (want > kMaxSplitsMerge - 1) want = kMaxSplitsMerge - 1;
  if (want < 1) want = 1;
  p->total = static_cast<int>(want);
  p->ws_bytes = partial_state_bytes(p->units, p->total, p->G, c->d);
  return DQA_OK;
}

template <int D, int BITS, int G>
void launch_g(const KiviArgs& a, bool rope, dim3 grid, hipStream_t s) {
  if (rope)
    hipLaunchKernelGGL((kivi_decode_kernel<D, BITS, G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kivi_decode_kernel<D, BITS, G, false>), grid, dim3(256), 0, s, a);
}

template <int D, int BITS>
void launch_bits(const KiviArgs& a, int G, bool rope, dim3 grid, hipStream_t s) {
  if (G == 1) launch_g<D, BITS, 1>(a, rope, grid, s);
  else if (G == 2) launch_g<D, BITS, 2>(a, rope, grid, s);
  else launch_g<D, BITS, 4>(a, rope, grid, s);
}

template <int D>
void launch_decode(const KiviArgs& a, int G, int bits, bool rope, dim3 grid, hipStream_t s) {
  if (bits == 2) launch_bits<D, 2>(a, G, rope, grid, s);
  else if (bits == 4) launch_bits<D, 4>(a, G, rope, grid, s);
  else launch_bits<D, 8>(a, G, rope, grid, s);
}


}  // namespace
}  // namespace dqa

// Partial-state memory of decode_attention_qkv_noalloc: one array per GPU
// the library runs on, held until the process ends.  Host code never uses
// the array's name as an address: the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device.
constexpr size_t kNoAllocScratchBytes = size_t{2} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (nullptr if it cannot be had).  The
// first call on a device looks the symbol up with that device current.
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

using namespace dqa;

extern "C" size_t kivi_rope_table_words(int d) {
  return (d == 64 || d == 128) ? feat_rope_table_words(d) : 0;
}

extern "C" int kivi_rope_table(float rope_theta, int d, int bits, uint32_t* table, void* stream) {
  if (!table) return DQA_ERR_NULL;
  if (!(rope_theta > 0.0f) || (d != 64 && d != 128)) return DQA_ERR_SHAPE;
  if (bits != 2 && bits != 4) return DQA_ERR_BITS;
  if (!aligned16(table)) return DQA_ERR_ALIGN;
  return launch_rope_table(rope_theta, d, bits, table, static_cast<hipStream_t>(stream));
}

extern "C" size_t decode_attention_workspace_bytes(const dqa_kivi_cache* cache) {
  Plan p;
  if (make_plan(cache, &p) != DQA_OK) return 0;
  return p.ws_bytes;
}

namespace {

// Validation shared by the decode entry points; fills the plan.
int check_decode(const uint16_t* q, const dqa_kivi_cache* c, const void* ws, size_t ws_bytes,
                 const float* out, Plan* p) {
  int st = make_plan(c, p);
  if (st != DQA_OK) return st;
  if (p->units == 0) return DQA_OK;
  if (!q || !out) return DQA_ERR_NULL;
  if (c->T_q > 0 && (!c->k_codes || !c->k_scale || !c->k_zero || !c->v_codes ||
                     !c->v_scale || !c->v_zero))
    return DQA_ERR_NULL;
  if (c->R > 0 && (!c->k_recent || !c->v_recent)) return DQA_ERR_NULL;
  if (!ws) return DQA_ERR_WORKSPACE;
  if (ws_bytes < p->ws_bytes) return DQA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(ws) || !aligned16(out)) return DQA_ERR_ALIGN;
  if (c->T_q > 0 && (!aligned16(c->k_codes) || !aligned16(c->k_scale) || !aligned16(c->k_zero) ||
                     !aligned16(c->v_codes) || !aligned16(c->v_scale) || !aligned16(c->v_zero)))
    return DQA_ERR_ALIGN;
  if (c->R > 0 && (!aligned16(c->k_recent) || !aligned16(c->v_recent))) return DQA_ERR_ALIGN;
  if (c->rope_table && !aligned16(c->rope_table)) return DQA_ERR_ALIGN;
  return DQA_OK;
}

}  // namespace

extern "C" int decode_attention_qkv_partial(const uint16_t* q, const dqa_kivi_cache* c,
                                            float sm_scale, void* ws, size_t ws_bytes,
                                            float* out, void* stream) {
  Plan p;
  const int st = check_decode(q, c, ws, ws_bytes, out, &p);
  if (st != DQA_OK || p.units == 0) return st;
  KiviArgs a;
  a.q = q;
  a.k_codes = c->k_codes;
  a.k_scale = c->k_scale;
  a.k_zero = c->k_zero;
  a.v_codes = c->v_codes;
  a.v_scale = c->v_scale;
  a.v_zero = c->v_zero;
  a.k_recent = c->k_recent;
  a.v_recent = c->v_recent;
  a.out = out;
  a.partials = merge_partials(ws, p.units);
  a.counters = merge_counters(ws);
  a.Hq = c->Hq;
  a.Hkv = c->Hkv;
  a.T_q = c->T_q;
  a.R = c->R;
  a.qtile_stride = (c->T_cap > 0 ? c->T_cap : c->T_q) / kGroup;
  a.R_cap = c->R_cap > 0 ? c->R_cap : c->R;
  a.n_qtiles = p.n_qtiles;
  a.n_rtiles = p.n_rtiles;
  a.total_splits = p.total;
  a.split = make_tile_split(p.n_qtiles, p.n_rtiles, use_feat(c->bits, c->rope_theta > 0.0f) ? feat_recent_weight() : 1,
                            static_cast<long long>(p.total) * (use_feat(c->bits, c->rope_theta > 0.0f) ? feat_waves_per_wg() : kWavesPerWG));
  a.q_scale = sm_scale * 1.4426950408889634f;
  const bool rope = c->rope_theta > 0.0f;
  rope_omega(c->rope_theta, c->d, a.omega);
  a.rope_theta = c->rope_theta;
  a.rope_table = rope ? c->rope_table : nullptr;
  const dim3 grid(p.total, c->Hkv, c->B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (use_feat(c->bits, rope)) {
    const int st2 = launch_feat_decode(a, c->d, p.G, c->bits, grid, s);
    if (st2 != DQA_OK) return st2;
  } else if (c->d == 128) {
    launch_decode<128>(a, p.G, c->bits, rope, grid, s);
  } else {
    launch_decode<64>(a, p.G, c->bits, rope, grid, s);
  }
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

extern "C" int decode_attention_qkv_merge(const dqa_kivi_cache* c, const void* ws, size_t ws_bytes,
                                          float* out, void* stream) {
  Plan p;
  int st = make_plan(c, &p);
  if (st != DQA_OK || p.units == 0) return st;
  if (!out) return DQA_ERR_NULL;
  if (!ws) return DQA_ERR_WORKSPACE;
  if (ws_bytes < p.ws_bytes) return DQA_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(out)) return DQA_ERR_ALIGN;
  (void)stream;   // the split kernel merges the splits itself
  return DQA_OK;
}

extern "C" int decode_attention_qkv(const uint16_t* q, const dqa_kivi_cache* c,
                                    float sm_scale, void* ws, size_t ws_bytes,
                                    float* out, void* stream) {
  const int st = decode_attention_qkv_partial(q, c, sm_scale, ws, ws_bytes, out, stream);
  if (st != DQA_OK) return st;
  return decode_attention_qkv_merge(c, ws, ws_bytes, out, stream);
}

extern "C" size_t decode_attention_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int decode_attention_qkv_noalloc(const uint16_t* q, const dqa_kivi_cache* c, float sm_scale,
                                            float* out, void* stream) {
  Plan p;
  const int st = make_plan(c, &p);
  if (st != DQA_OK) return st;
  if (p.ws_bytes > kNoAllocScratchBytes) return DQA_ERR_WORKSPACE;
  if (p.units == 0) return DQA_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DQA_ERR_HIP;
  void* ws = scratch_address(dev);
  if (!ws) return DQA_ERR_HIP;
  return decode_attention_qkv(q, c, sm_scale, ws, kNoAllocScratchBytes, out, stream);
}
