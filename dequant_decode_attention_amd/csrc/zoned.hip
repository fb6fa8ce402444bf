// Mixed-bitwidth zoned cache: host plan, device packer and decode reader.
//
// [P3 sec 2.2, bit-allocation pipeline]: value widths per token and key
// widths per channel come from {0, 2, 4, 8, 16}; width 0 evicts.
// [P3 sec 2.2, TriZone packed decoding]: zone A holds the packed key rows and
// the kept value rows at 2/4/8 bits grouped by width; zone B the fp16 value
// rows of 16-bit tokens; zone C fp16 keys and values of the newest tokens;
// the attention kernel reads the three zones with dequantization fused into
// the products.
//
// Layout (bytes, little endian; one region per (batch, KV head) unit,
// batch-major, each starting at a multiple of 256):
//   zone A = groups of segment 2, then 4, 8, 16.  Kept tokens of a segment
//   are taken in token order, 32 slots per group, the last group padded with
//   masked (all-zero) slots.  A group holds, each block 16-byte aligned:
//     key codes [32][W_K] uint32, key scale [n_kq] fp16, key zero [n_kq] fp16,
//     and for widths 2/4/8: value codes [32][d*w/32] uint32, value scale
//     [32][d/32] fp16, value zero [32][d/32] fp16.
//   A key row is one block per key class (2, 4, 8: codes LSB first in
//   ceil(m_w*w/32) words; 16: raw fp16, two per word); channels inside a
//   class keep their order.  Key groups = (32-slot group, quantized channel)
//   over the valid slots; value groups = (token, 32 channels).
//   zone B = [P_16][d] fp16 value rows of segment 16; zone C = keys [C][d],
//   then values [C][d], fp16.
#include "common.h"
#include "merge.h"

namespace dqa {
namespace {

constexpr int kSegW[4] = {2, 4, 8, 16};
constexpr int32_t kPlanMagic = 0x5A4F4E45;  // "ZONE"
constexpr int kHeaderWords = 16;
constexpr int kUnitWords = 40;

// Header word indices.
enum { H_MAGIC, H_VERSION, H_B, H_HKV, H_TOLD, H_C, H_D, H_UNITS, H_BLOB_LO, H_BLOB_HI,
       H_MAX_GROUPS, H_UNIT_OFF, H_PERM_OFF, H_TOK_OFF };
// Unit record word indices.
enum { U_N = 0,        // [4] kept tokens per segment
       U_M = 4,        // [4] channels per key class
       U_GROUPS = 8,   // [4] groups per segment
       U_KWORDS = 12,  // [4] key-row words per class
       U_WK = 16, U_NKQ = 17, U_KCODES_B = 18, U_KSZ_B = 19,
       U_SEG_OFF = 20, // [4] byte offset of each segment (relative to unit base)
       U_GRP_B = 24,   // [4] bytes per group of each segment
       U_ZB = 28, U_ZC = 29, U_BASE_LO = 30, U_BASE_HI = 31, U_SIZE = 32,
       U_TOTAL_GROUPS = 33, U_TOK_PREFIX = 34 /* [4] token-map start per segment */ };

__host__ __device__ inline size_t pad(size_t n, size_t a) { return (n + a - 1) / a * a; }

size_t plan_words(int B, int Hkv, int T_old, int d) {
  if (B < 0 || Hkv < 0 || T_old < 0 || (d != 64 && d != 128)) return 0;
  return kHeaderWords + static_cast<size_t>(B) * Hkv * (kUnitWords + d + T_old);
}

int check_plan(const int32_t* p) {
  if (!p) return DQA_ERR_NULL;
  if (p[H_MAGIC] != kPlanMagic || p[H_VERSION] != 1) return DQA_ERR_PLAN;
  if (p[H_D] != 64 && p[H_D] != 128) return DQA_ERR_PLAN;
  if (p[H_B] < 0 || p[H_HKV] < 0 || p[H_C] < 0 || p[H_C] > 256) return DQA_ERR_PLAN;
  if (static_cast<int64_t>(p[H_B]) * p[H_HKV] != p[H_UNITS]) return DQA_ERR_PLAN;
  return DQA_OK;
}

// ------------------------------------------------------------------ packer

struct PackArgs {
  const int32_t* plan;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* blob;
  int T_old, C, d;
};

__device__ __forceinline__ uint32_t code_of(float x, float zf, float sf, float levels) {
  if (sf == 0.0f) return 0u;
  const float t = (x - zf) / sf;
  return static_cast<uint32_t>(fminf(fmaxf(rintf(t), 0.0f), levels));
}

// Zero-fill (the blob's padding bytes are defined as zero).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t n_words) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (; i < n_words; i += stride) p[i] = 0u;
}

// One workgroup (d threads) per (unit, group); the extra group index
// `total_groups` copies zone C.
__global__ __launch_bounds__(128) void zoned_pack_kernel(PackArgs a) {
  __shared__ uint16_t lds_k[kGroup][128];   // the group's key rows (fp16, original order)
  __shared__ uint8_t lds_c[kGroup][128];    // codes by permuted channel
  __shared__ int lds_tok[kGroup];
  const int d = a.d;
  const int unit = blockIdx.y;
  const int grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* P = a.plan;
  const int32_t* U = P + P[H_UNIT_OFF] + unit * kUnitWords;
  const int32_t* perm = P + P[H_PERM_OFF] + unit * d;
  const int32_t* tokmap = P + P[H_TOK_OFF] + unit * a.T_old;
  const size_t base = static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_LO])) |
                      (static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_HI])) << 32);
  uint8_t* ub = a.blob + base;
  const size_t src_unit = static_cast<size_t>(unit) * a.T_old * d;
  const int total = U[U_TOTAL_GROUPS];
  if (grp > total) return;
  if (grp == total) {                      // zone C: fp16 copies
    uint16_t* zc = reinterpret_cast<uint16_t*>(ub + U[U_ZC]);
    const size_t n = static_cast<size_t>(a.C) * d;
    const size_t src = static_cast<size_t>(unit) * a.C * d;
    for (size_t i = tid; i < n; i += blockDim.x) {
      zc[i] = a.k_new[src + i];
      zc[n + i] = a.v_new[src + i];
    }
    return;
  }
  // locate the segment of this group
  int seg = 0, g = grp;
  while (g >= U[U_GROUPS + seg]) {
    g -= U[U_GROUPS + seg];
    ++seg;
  }
  const int w = kSegW[seg];
  const int n_seg = U[U_N + seg];
  const int n_valid = min(kGroup, n_seg - g * kGroup);
  uint8_t* gb = ub + U[U_SEG_OFF + seg] + static_cast<size_t>(g) * U[U_GRP_B + seg];
  if (tid < kGroup) lds_tok[tid] = tid < n_valid ? tokmap[U[U_TOK_PREFIX + seg] + g * kGroup + tid] : -1;
  __syncthreads();
  for (int e = tid; e < kGroup * d; e += blockDim.x) {
    const int s = e / d, c = e % d;
    lds_k[s][c] = lds_tok[s] >= 0 ? a.k[src_unit + static_cast<size_t>(lds_tok[s]) * d + c] : 0;
  }
  __syncthreads();

  // ---- keys: thread = permuted channel position pc
  const int m2 = U[U_M + 0], m4 = U[U_M + 1], m8 = U[U_M + 2];
  const int n_kq = U[U_NKQ];
  if (tid < d) {
    const int pc = tid;
    const int ch = perm[pc];
    if (pc < n_kq) {
      const int bits = pc < m2 ? 2 : (pc < m2 + m4 ? 4 : 8);
      float mn = INFINITY, mx = -INFINITY;
      for (int s = 0; s < n_valid; ++s) {
        const float x = h2f(lds_k[s][ch]);
        mn = fminf(mn, x);
        mx = fmaxf(mx, x);
      }
      const float levels = static_cast<float>((1 << bits) - 1);
      const uint16_t s16 = f2h((mx - mn) / levels);
      const float sf = h2f(s16);
      uint16_t* ks = reinterpret_cast<uint16_t*>(gb + U[U_KCODES_B]);
      uint16_t* kz = reinterpret_cast<uint16_t*>(gb + U[U_KCODES_B] + U[U_KSZ_B]);
      ks[pc] = s16;
      kz[pc] = f2h(mn);
      for (int s = 0; s < kGroup; ++s)
        lds_c[s][pc] = s < n_valid ? static_cast<uint8_t>(code_of(h2f(lds_k[s][ch]), mn, sf, levels)) : 0;
    }
  }
  __syncthreads();
  // key rows: word (slot, wi) of each class block
  const int kw2 = U[U_KWORDS + 0], kw4 = U[U_KWORDS + 1], kw8 = U[U_KWORDS + 2];
  const int W_K = U[U_WK];
  uint32_t* krow = reinterpret_cast<uint32_t*>(gb);
  for (int e = tid; e < kGroup * W_K; e += blockDim.x) {
    const int s = e / W_K, wi = e % W_K;
    uint32_t word = 0;
    if (s < n_valid) {
      int cls_bits, first, count, wl;
      if (wi < kw2) { cls_bits = 2; first = 0; count = m2; wl = wi; }
      else if (wi < kw2 + kw4) { cls_bits = 4; first = m2; count = m4; wl = wi - kw2; }
      else if (wi < kw2 + kw4 + kw8) { cls_bits = 8; first = m2 + m4; count = m8; wl = wi - kw2 - kw4; }
      else { cls_bits = 16; first = n_kq; count = U[U_M + 3]; wl = wi - kw2 - kw4 - kw8; }
      const int per = 32 / cls_bits;
      for (int j = 0; j < per; ++j) {
        const int idx = wl * per + j;
        if (idx >= count) break;
        const int pc = first + idx;
        const uint32_t field = cls_bits == 16 ? static_cast<uint32_t>(lds_k[s][perm[pc]])
                                              : static_cast<uint32_t>(lds_c[s][pc]);
        word |= field << (j * cls_bits);
      }
    }
    krow[e] = word;
  }

  // ---- values
  if (w < 16) {
    const int vwpt = d * w / 32;                 // value words per slot
    uint8_t* vbase = gb + U[U_KCODES_B] + 2 * U[U_KSZ_B];
    uint32_t* vcodes = reinterpret_cast<uint32_t*>(vbase);
    const size_t vsz_b = pad(static_cast<size_t>(kGroup) * (d / kGroup) * 2, 16);
    uint16_t* vs = reinterpret_cast<uint16_t*>(vbase + kGroup * vwpt * 4);
    uint16_t* vz = reinterpret_cast<uint16_t*>(vbase + kGroup * vwpt * 4 + vsz_b);
    for (int e = tid; e < kGroup * (d / kGroup); e += blockDim.x) {
      const int s = e / (d / kGroup), vg = e % (d / kGroup);
      uint32_t* dst = vcodes + s * vwpt + vg * w;
      if (s >= n_valid) {
        for (int i = 0; i < w; ++i) dst[i] = 0u;
        vs[e] = 0;
        vz[e] = 0;
        continue;
      }
      const uint16_t* src = a.v + src_unit + static_cast<size_t>(lds_tok[s]) * d + vg * kGroup;
      float x[kGroup];
      float mn = INFINITY, mx = -INFINITY;
      for (int i = 0; i < kGroup; ++i) {
        x[i] = h2f(src[i]);
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
      }
      const float levels = static_cast<float>((1 << w) - 1);
      const uint16_t s16 = f2h((mx - mn) / levels);
      const float sf = h2f(s16);
      vs[e] = s16;
      vz[e] = f2h(mn);
      const int per = 32 / w;
      for (int i = 0; i < w; ++i) {
        uint32_t word = 0;
        for (int j = 0; j < per; ++j) word |= code_of(x[i * per + j], mn, sf, levels) << (j * w);
        dst[i] = word;
      }
    }
  } else {
    // zone B rows of this group's slots
    uint16_t* zb = reinterpret_cast<uint16_t*>(ub + U[U_ZB]) + static_cast<size_t>(g) * kGroup * d;
    for (int e = tid; e < kGroup * d; e += blockDim.x) {
      const int s = e / d, c = e % d;
      zb[e] = lds_tok[s] >= 0 ? a.v[src_unit + static_cast<size_t>(lds_tok[s]) * d + c] : 0;
    }
  }
}


// ------------------------------------------------------------------ reader

constexpr int kZWaves = 4;
constexpr int kStageBytes = 16384;   // >= the largest group (d = 128): 13312 B

struct ZDecodeArgs {
  const int32_t* plan;
  const uint8_t* blob;
  const uint16_t* q;
  float* out;
  float* partials;
  int Hq, Hkv, C, items_per_split, splits;
  float q_scale;
};

// Decode over one unit's groups (zone A segments, then zone C chunks of 32).
template <int D, int G>
__global__ __launch_bounds__(256) void zoned_decode_kernel(ZDecodeArgs a) {
  constexpr int CV = D / 64;                        // value channels per lane
  __shared__ __attribute__((aligned(16))) uint8_t lds_stage[kZWaves][kStageBytes];
  __shared__ float lds_qp[G][D], lds_qn[G][D];      // query: permuted / natural order
  __shared__ float lds_p[kZWaves][kGroup][G];
  __shared__ float lds_m[kZWaves][G], lds_l[kZWaves][G], lds_o[kZWaves][G][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, unit = blockIdx.y;
  const int b = unit / a.Hkv, kvh = unit % a.Hkv;
  const int32_t* P = a.plan;
  const int32_t* U = P + P[H_UNIT_OFF] + unit * kUnitWords;
  const int32_t* perm = P + P[H_PERM_OFF] + unit * D;
  const size_t base = static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_LO])) |
                      (static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_HI])) << 32);
  const uint8_t* ub = a.blob + base;
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + h) * D;
    lds_qn[h][c] = h2f(qh[c]) * a.q_scale;
    lds_qp[h][c] = h2f(qh[perm[c]]) * a.q_scale;
  }
  __syncthreads();

  const int m2 = U[U_M], m4 = U[U_M + 1], m8 = U[U_M + 2];
  const int n_kq = U[U_NKQ];
  const int kw2 = U[U_KWORDS], kw4 = U[U_KWORDS + 1], kw8 = U[U_KWORDS + 2];
  const int W_K = U[U_WK];
  const int total = U[U_TOTAL_GROUPS];
  const int items = total + (a.C + kGroup - 1) / kGroup;
  const int s_slot = lane & 31, hf = lane >> 5;
  uint8_t* st = lds_stage[wave];

  float m[G], l[G], acc[G][CV], zacc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
    zacc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < CV; ++c) acc[h][c] = 0.0f;
  }

  const int ib = split * a.items_per_split;
  const int ie = min(items, ib + a.items_per_split);
  for (int item = ib + wave; item < ie; item += kZWaves) {
    const bool zone_c = item >= total;
    int seg = 3, g = 0, n_valid;
    const uint8_t* gb = nullptr;
    const uint16_t* zck = nullptr;
    const uint16_t* zcv = nullptr;
    if (!zone_c) {
      seg = 0;
      g = item;
      while (g >= U[U_GROUPS + seg]) {
        g -= U[U_GROUPS + seg];
        ++seg;
      }
      n_valid = min(kGroup, U[U_N + seg] - g * kGroup);
      gb = ub + U[U_SEG_OFF + seg] + static_cast<size_t>(g) * U[U_GRP_B + seg];
      // stage the group's contiguous bytes
      const int nb = U[U_GRP_B + seg];
      const uint4* src = reinterpret_cast<const uint4*>(gb);
      uint4* dst = reinterpret_cast<uint4*>(st);
      for (int i = lane; i < nb / 16; i += 64) dst[i] = src[i];
    } else {
      const int cg = item - total;
      n_valid = min(kGroup, a.C - cg * kGroup);
      zck = reinterpret_cast<const uint16_t*>(ub + U[U_ZC]) + static_cast<size_t>(cg) * kGroup * D;
      zcv = zck + static_cast<size_t>(a.C) * D;
    }
    const int w = kSegW[seg];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- logits: lane = (slot, half of the channels)
    const bool valid = s_slot < n_valid;
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.0f;
    if (valid) {
      if (!zone_c) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(st) + s_slot * W_K;
        const uint16_t* ks = reinterpret_cast<const uint16_t*>(st + U[U_KCODES_B]);
        const uint16_t* kz = reinterpret_cast<const uint16_t*>(st + U[U_KCODES_B] + U[U_KSZ_B]);
        for (int pc = hf * (D / 2); pc < (hf + 1) * (D / 2); ++pc) {
          float kv;
          if (pc < n_kq) {
            int bits, idx, woff;
            if (pc < m2) { bits = 2; idx = pc; woff = 0; }
            else if (pc < m2 + m4) { bits = 4; idx = pc - m2; woff = kw2; }
            else { bits = 8; idx = pc - m2 - m4; woff = kw2 + kw4; }
            const int bit = idx * bits;
            const uint32_t code = (row[woff + bit / 32] >> (bit % 32)) & ((1u << bits) - 1u);
            kv = fmaf(static_cast<float>(code), h2f(ks[pc]), h2f(kz[pc]));
          } else {
            const int idx = pc - n_kq;
            const uint32_t word = row[kw2 + kw4 + kw8 + idx / 2];
            kv = h2f(static_cast<uint16_t>((idx & 1) ? (word >> 16) : (word & 0xFFFFu)));
          }
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] = fmaf(lds_qp[h][pc], kv, part[h]);
        }
      } else {
        const uint16_t* kr = zck + static_cast<size_t>(s_slot) * D;
        for (int c = hf * (D / 2); c < (hf + 1) * (D / 2); ++c) {
          const float kv = h2f(kr[c]);
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] = fmaf(lds_qn[h][c], kv, part[h]);
        }
      }
    }
    float lg[G];
    bool grow = false;
    float mnew[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lg[h] = part[h] + __shfl_xor(part[h], 32, 64);
      const float t = max_strided<1>(valid ? lg[h] : -INFINITY);
      mnew[h] = fmaxf(m[h], t);
      grow |= mnew[h] > m[h];
    }
    if (grow) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = merge_weight(m[h], mnew[h]);
        l[h] *= sc;
        zacc[h] *= sc;
#pragma unroll
        for (int c = 0; c < CV; ++c) acc[h][c] *= sc;
        m[h] = mnew[h];
      }
    }
    if (hf == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = valid ? exp2f(lg[h] - m[h]) : 0.0f;
        lds_p[wave][s_slot][h] = p;
        l[h] += p;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- values: lane = CV consecutive channels
    const int c0 = lane * CV;
    if (!zone_c && w < 16) {
      const int vwpt = D * w / 32;
      const uint8_t* vb = st + U[U_KCODES_B] + 2 * U[U_KSZ_B];
      const uint32_t* vcodes = reinterpret_cast<const uint32_t*>(vb);
      const int vsz_b = (kGroup * (D / kGroup) * 2 + 15) / 16 * 16;
      const uint16_t* vs = reinterpret_cast<const uint16_t*>(vb + kGroup * vwpt * 4);
      const uint16_t* vz = reinterpret_cast<const uint16_t*>(vb + kGroup * vwpt * 4 + vsz_b);
      const int vg = c0 / kGroup;
      for (int s = 0; s < n_valid; ++s) {
        const float sc = h2f(vs[s * (D / kGroup) + vg]);
        const float zr = h2f(vz[s * (D / kGroup) + vg]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = lds_p[wave][s][h];
          const float ps = p * sc;
          zacc[h] = fmaf(p, zr, zacc[h]);
#pragma unroll
          for (int c = 0; c < CV; ++c) {
            const int bit = (c0 + c) * w;
            const uint32_t code = (vcodes[s * vwpt + bit / 32] >> (bit % 32)) & ((1u << w) - 1u);
            acc[h][c] = fmaf(ps, static_cast<float>(code), acc[h][c]);
          }
        }
      }
    } else {
      const uint16_t* vrows = zone_c ? zcv
                                     : reinterpret_cast<const uint16_t*>(ub + U[U_ZB]) +
                                           static_cast<size_t>(g) * kGroup * D;
      for (int s = 0; s < n_valid; ++s) {
        float vv[CV];
#pragma unroll
        for (int c = 0; c < CV; ++c) vv[c] = h2f(vrows[static_cast<size_t>(s) * D + c0 + c]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = lds_p[wave][s][h];
#pragma unroll
          for (int c = 0; c < CV; ++c) acc[h][c] = fmaf(p, vv[c], acc[h][c]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave state -> LDS (l summed over the 32 slot lanes of half 0)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = sum_strided<1>(l[h]);
#pragma unroll
    for (int c = 0; c < CV; ++c) lds_o[wave][h][lane * CV + c] = acc[h][c] + zacc[h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = m[h];
      lds_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  write_split_state<D, G, kZWaves>(a.partials, a.out, a.Hq, static_cast<size_t>(unit), b, kvh, split, a.splits,
                                   lds_m, lds_l, lds_o);
}

struct ZGeometry {
  int G, units, items_max, ips, splits;
  size_t ws_bytes;
};

int zoned_geometry(const int32_t* p, int Hq, ZGeometry* g) {
  int st = check_plan(p);
  if (st != DQA_OK) return st;
  const int Hkv = p[H_HKV];
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return DQA_ERR_SHAPE;
  g->G = Hq / Hkv;
  if (g->G != 1 && g->G != 2 && g->G != 4) return DQA_ERR_UNSUPPORTED;
  g->units = p[H_UNITS];
  g->items_max = p[H_MAX_GROUPS] + (p[H_C] + kGroup - 1) / kGroup;
  long long s = (kTargetWorkgroups + g->units - 1) / (g->units > 0 ? g->units : 1);
  if (s > g->items_max) s = g->items_max;
  if (s > kMaxSplitsMerge - 1) s = kMaxSplitsMerge - 1;
  if (s < 1) s = 1;
  g->ips = g->items_max > 0 ? static_cast<int>((g->items_max + s - 1) / s) : 1;
  g->splits = g->items_max > 0 ? (g->items_max + g->ips - 1) / g->ips : 1;
  g->ws_bytes = partial_state_bytes(static_cast<size_t>(g->units), g->splits, g->G, p[H_D]);
  return DQA_OK;
}

template <int D>
int zlaunch(const ZDecodeArgs& a, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((zoned_decode_kernel<D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((zoned_decode_kernel<D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((zoned_decode_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
    default: return DQA_ERR_UNSUPPORTED;
  }
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

}  // namespace
}  // namespace dqa

using namespace dqa;

extern "C" size_t zoned_plan_words(int B, int Hkv, int T_old, int d) {
  return plan_words(B, Hkv, T_old, d);
}

extern "C" int zoned_plan(const int8_t* v_bits, const int8_t* k_bits, int B, int Hkv, int T_old,
                          int C_new, int d, int32_t* plan, size_t n_words, size_t* blob_bytes) {
  const size_t need = plan_words(B, Hkv, T_old, d);
  if (need == 0 || C_new < 0 || C_new > 256) return DQA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * Hkv > (1 << 20) || T_old > (1 << 24)) return DQA_ERR_SHAPE;
  if (!plan || !blob_bytes) return DQA_ERR_NULL;
  if (static_cast<int64_t>(B) * Hkv * T_old > 0 && !v_bits) return DQA_ERR_NULL;
  if (static_cast<int64_t>(B) * Hkv > 0 && !k_bits) return DQA_ERR_NULL;
  if (n_words < need) return DQA_ERR_WORKSPACE;
  const int units = B * Hkv;
  for (size_t i = 0; i < static_cast<size_t>(units) * T_old; ++i) {
    const int w = v_bits[i];
    if (w != 0 && w != 2 && w != 4 && w != 8 && w != 16) return DQA_ERR_BITS;
  }
  for (size_t i = 0; i < static_cast<size_t>(units) * d; ++i) {
    const int w = k_bits[i];
    if (w != 2 && w != 4 && w != 8 && w != 16) return DQA_ERR_BITS;
  }
  for (size_t i = 0; i < need; ++i) plan[i] = 0;
  plan[H_MAGIC] = kPlanMagic;
  plan[H_VERSION] = 1;
  plan[H_B] = B;
  plan[H_HKV] = Hkv;
  plan[H_TOLD] = T_old;
  plan[H_C] = C_new;
  plan[H_D] = d;
  plan[H_UNITS] = units;
  plan[H_UNIT_OFF] = kHeaderWords;
  plan[H_PERM_OFF] = kHeaderWords + units * kUnitWords;
  plan[H_TOK_OFF] = kHeaderWords + units * (kUnitWords + d);
  size_t base = 0;
  int max_groups = 0;
  for (int u = 0; u < units; ++u) {
    int32_t* U = plan + kHeaderWords + u * kUnitWords;
    int32_t* perm = plan + plan[H_PERM_OFF] + static_cast<size_t>(u) * d;
    int32_t* tok = plan + plan[H_TOK_OFF] + static_cast<size_t>(u) * T_old;
    const int8_t* vb = v_bits + static_cast<size_t>(u) * T_old;
    const int8_t* kb = k_bits + static_cast<size_t>(u) * d;
    int np = 0;
    for (int ci = 0; ci < 4; ++ci) {
      int m = 0;
      for (int c = 0; c < d; ++c)
        if (kb[c] == kSegW[ci]) {
          perm[np++] = c;
          ++m;
        }
      U[U_M + ci] = m;
      U[U_KWORDS + ci] = (m * kSegW[ci] + 31) / 32;
    }
    int nt = 0;
    for (int si = 0; si < 4; ++si) {
      U[U_TOK_PREFIX + si] = nt;
      int n = 0;
      for (int t = 0; t < T_old; ++t)
        if (vb[t] == kSegW[si]) {
          tok[nt++] = t;
          ++n;
        }
      U[U_N + si] = n;
      U[U_GROUPS + si] = (n + kGroup - 1) / kGroup;
    }
    const int W_K = U[U_KWORDS] + U[U_KWORDS + 1] + U[U_KWORDS + 2] + U[U_KWORDS + 3];
    const int n_kq = U[U_M] + U[U_M + 1] + U[U_M + 2];
    U[U_WK] = W_K;
    U[U_NKQ] = n_kq;
    U[U_KCODES_B] = kGroup * W_K * 4;
    U[U_KSZ_B] = static_cast<int32_t>(pad(static_cast<size_t>(n_kq) * 2, 16));
    size_t off = 0;
    int total = 0;
    for (int si = 0; si < 4; ++si) {
      size_t gbytes = static_cast<size_t>(U[U_KCODES_B]) + 2 * static_cast<size_t>(U[U_KSZ_B]);
      if (kSegW[si] < 16)
        gbytes += static_cast<size_t>(kGroup) * (d * kSegW[si] / 32) * 4 +
                  2 * pad(static_cast<size_t>(kGroup) * (d / kGroup) * 2, 16);
      U[U_SEG_OFF + si] = static_cast<int32_t>(off);
      U[U_GRP_B + si] = static_cast<int32_t>(gbytes);
      off += gbytes * U[U_GROUPS + si];
      total += U[U_GROUPS + si];
    }
    U[U_ZB] = static_cast<int32_t>(off);
    off += static_cast<size_t>(U[U_GROUPS + 3]) * kGroup * d * 2;
    U[U_ZC] = static_cast<int32_t>(off);
    off += 2 * static_cast<size_t>(C_new) * d * 2;
    const size_t size = pad(off, 256);
    if (size > 0x7FFFFFFFu) return DQA_ERR_SHAPE;
    U[U_SIZE] = static_cast<int32_t>(size);
    U[U_BASE_LO] = static_cast<int32_t>(base & 0xFFFFFFFFu);
    U[U_BASE_HI] = static_cast<int32_t>(base >> 32);
    U[U_TOTAL_GROUPS] = total;
    if (total > max_groups) max_groups = total;
    base += size;
  }
  plan[H_BLOB_LO] = static_cast<int32_t>(base & 0xFFFFFFFFu);
  plan[H_BLOB_HI] = static_cast<int32_t>(base >> 32);
  plan[H_MAX_GROUPS] = max_groups;
  *blob_bytes = base;
  return DQA_OK;
}

extern "C" int zoned_pack(const int32_t* plan_host, const int32_t* plan_dev, const uint16_t* k,
                          const uint16_t* v, const uint16_t* k_new, const uint16_t* v_new, void* blob,
                          void* stream) {
  int st = check_plan(plan_host);
  if (st != DQA_OK) return st;
  if (!plan_dev) return DQA_ERR_NULL;
  const int units = plan_host[H_UNITS];
  const size_t blob_bytes = static_cast<size_t>(static_cast<uint32_t>(plan_host[H_BLOB_LO])) |
                            (static_cast<size_t>(static_cast<uint32_t>(plan_host[H_BLOB_HI])) << 32);
  if (units == 0 || blob_bytes == 0) return DQA_OK;
  if (!blob) return DQA_ERR_NULL;
  if (plan_host[H_TOLD] > 0 && (!k || !v)) return DQA_ERR_NULL;
  if (plan_host[H_C] > 0 && (!k_new || !v_new)) return DQA_ERR_NULL;
  if (units > 65535) return DQA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n_words = blob_bytes / 4;
  size_t fb = (n_words + 255) / 256;
  if (fb > 16384) fb = 16384;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(fb)), dim3(256), 0, s,
                     static_cast<uint32_t*>(blob), n_words);
  DQA_CHECK_LAUNCH();
  PackArgs a{plan_dev, k, v, k_new, v_new, static_cast<uint8_t*>(blob), plan_host[H_TOLD],
             plan_host[H_C], plan_host[H_D]};
  const dim3 grid(plan_host[H_MAX_GROUPS] + 1, units);
  hipLaunchKernelGGL(zoned_pack_kernel, grid, dim3(128), 0, s, a);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

extern "C" size_t decode_attention_zoned_workspace_bytes(const int32_t* plan_host, int Hq) {
  ZGeometry g;
  if (zoned_geometry(plan_host, Hq, &g) != DQA_OK) return 0;
  return g.ws_bytes;
}

extern "C" int decode_attention_zoned(const uint16_t* q, int Hq, const int32_t* plan_host,
                                      const int32_t* plan_dev, const void* blob, float sm_scale,
                                      void* ws, size_t ws_bytes, float* out, void* stream) {
  ZGeometry g;
  int st = zoned_geometry(plan_host, Hq, &g);
  if (st != DQA_OK) return st;
  if (g.units == 0) return DQA_OK;
  if (!q || !out || !plan_dev || !blob) return DQA_ERR_NULL;
  if (!ws || ws_bytes < g.ws_bytes) return DQA_ERR_WORKSPACE;
  if (g.units > 65535) return DQA_ERR_SHAPE;
  ZDecodeArgs a;
  a.plan = plan_dev;
  a.blob = static_cast<const uint8_t*>(blob);
  a.q = q;
  a.out = out;
  a.partials = static_cast<float*>(ws);
  a.Hq = Hq;
  a.Hkv = plan_host[H_HKV];
  a.C = plan_host[H_C];
  a.items_per_split = g.ips;
  a.splits = g.splits;
  a.q_scale = sm_scale * 1.4426950408889634f;
  const dim3 grid(g.splits, g.units);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int B = plan_host[H_B];
  if (plan_host[H_D] == 128) {
    st = zlaunch<128>(a, g.G, grid, s);
    return st != DQA_OK ? st : launch_split_merge<128>(a.partials, g.splits, B, Hq, a.Hkv, out, s);
  }
  st = zlaunch<64>(a, g.G, grid, s);
  return st != DQA_OK ? st : launch_split_merge<64>(a.partials, g.splits, B, Hq, a.Hkv, out, s);
}
