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
//   zone B = [P_16][d] fp16 value rows of segment 16; zone C = keys
//   [S + C][d], then values [S + C][d], fp16: the S sink tokens, then the
//   C new tokens.
// Sink window ([P1 para 11]: high-precision windows for the attention sinks
// as well as the recent tokens): the first S old tokens stay whole, whatever
// their widths, at the front of zone C.
// Outlier side list ([P1 para 9]: a small share of key outliers isolated
// from the quantized groups): in every key quantization group up to k_out
// entries are taken out one at a time -- the smallest or largest remaining
// value, whichever lies farther from the float32 mean of the remaining
// values (summed in slot order; the largest on a tie; the lowest slot among
// equal values) -- while more than two values remain and they are not all
// equal.  The group is quantized over the rest; a removed entry keeps code 0
// and its fp16 value goes to the group's side list, placed after the key
// zeros: slot offsets [33] uint16, class positions [n_kq*k_out] uint16,
// values [n_kq*k_out] fp16 (16-byte aligned blocks, sorted by slot then
// position).  The reader adds q.(value - zero) to the logit of that slot.
#include "common.h"
#include "merge.h"

namespace dqa {
namespace {

constexpr int kSegW[4] = {2, 4, 8, 16};
constexpr int32_t kPlanMagic = 0x5A4F4E45;  // "ZONE"
constexpr int kHeaderWords = 16;
constexpr int kUnitWords = 40;

constexpr int kPlanVersion = 2;
constexpr int kMaxOutliers = 4;             // side-list entries per key group, at most
constexpr int kMaxZoneC = 256;              // sink + new tokens in zone C, at most
constexpr int kOffsBytes = 80;              // 33 uint16 slot offsets, padded to 16 bytes

// Header word indices.
enum { H_MAGIC, H_VERSION, H_B, H_HKV, H_TOLD, H_C, H_D, H_UNITS, H_BLOB_LO, H_BLOB_HI,
       H_MAX_GROUPS, H_UNIT_OFF, H_PERM_OFF, H_TOK_OFF, H_SINK, H_KOUT };
// Unit record word indices.
enum { U_N = 0,        // [4] kept tokens per segment
       U_M = 4,        // [4] channels per key class
       U_GROUPS = 8,   // [4] groups per segment
       U_KWORDS = 12,  // [4] key-row words per class
       U_WK = 16, U_NKQ = 17, U_KCODES_B = 18, U_KSZ_B = 19,
       U_SEG_OFF = 20, // [4] byte offset of each segment (relative to unit base)
       U_GRP_B = 24,   // [4] bytes per group of each segment
       U_ZB = 28, U_ZC = 29, U_BASE_LO = 30, U_BASE_HI = 31, U_SIZE = 32,
       U_TOTAL_GROUPS = 33, U_TOK_PREFIX = 34 /* [4] token-map start per segment */,
       U_OUT_B = 38 /* bytes of a group's outlier side list (0 without) */ };

__host__ __device__ inline size_t pad(size_t n, size_t a) { return (n + a - 1) / a * a; }

size_t plan_words(int B, int Hkv, int T_old, int d) {
  if (B < 0 || Hkv < 0 || T_old < 0 || (d != 64 && d != 128)) return 0;
  return kHeaderWords + static_cast<size_t>(B) * Hkv * (kUnitWords + d + T_old);
}

// Unit record of a unit whose kept old tokens number n[si] per value segment
// (widths 2, 4, 8, 16) and whose quantized-or-raw key channels number m[ci]
// per key class, placed at byte offset `base` of the blob.  Returns the
// unit's region size in bytes (a multiple of 256), or -1 when it does not fit
// the 31-bit size field.  zoned_plan builds every record with it, and
// check_plan re-derives every record with it.
long long fill_unit(int32_t* U, const int* n, const int* m, int d, int sink, int C_new, int k_out, size_t base) {
  for (int w = 0; w < kUnitWords; ++w) U[w] = 0;
  int nt = 0;
  for (int i = 0; i < 4; ++i) {
    U[U_N + i] = n[i];
    U[U_M + i] = m[i];
    U[U_GROUPS + i] = (n[i] + kGroup - 1) / kGroup;
    U[U_KWORDS + i] = (m[i] * kSegW[i] + 31) / 32;
    U[U_TOK_PREFIX + i] = nt;
    nt += n[i];
  }
  const int W_K = U[U_KWORDS] + U[U_KWORDS + 1] + U[U_KWORDS + 2] + U[U_KWORDS + 3];
  const int n_kq = m[0] + m[1] + m[2];
  U[U_WK] = W_K;
  U[U_NKQ] = n_kq;
  U[U_KCODES_B] = kGroup * W_K * 4;
  U[U_KSZ_B] = static_cast<int32_t>(pad(static_cast<size_t>(n_kq) * 2, 16));
  U[U_OUT_B] = k_out > 0 ? kOffsBytes + 2 * static_cast<int32_t>(pad(static_cast<size_t>(n_kq) * k_out * 2, 16))
                         : 0;
  size_t off = 0;
  int total = 0;
  for (int si = 0; si < 4; ++si) {
    size_t gbytes = static_cast<size_t>(U[U_KCODES_B]) + 2 * static_cast<size_t>(U[U_KSZ_B]) + U[U_OUT_B];
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
  off += 2 * static_cast<size_t>(sink + C_new) * d * 2;
  const size_t size = pad(off, 256);
  if (size > 0x7FFFFFFFu) return -1;
  U[U_SIZE] = static_cast<int32_t>(size);
  U[U_BASE_LO] = static_cast<int32_t>(base & 0xFFFFFFFFu);
  U[U_BASE_HI] = static_cast<int32_t>(base >> 32);
  U[U_TOTAL_GROUPS] = total;
  return static_cast<long long>(size);
}

// A plan as zoned_plan writes it, checked before any launch: the header,
// every unit record (re-derived from its token and channel counts), the blob
// size and the per-unit channel permutation (each channel once); anything
// else is DQA_ERR_PLAN.  The token map (T_old words per unit, the bulk of the
// plan) is not read here: the packer clamps its entries into [0, T_old).
int check_plan(const int32_t* p) {
  if (!p) return DQA_ERR_NULL;
  if (p[H_MAGIC] != kPlanMagic || p[H_VERSION] != kPlanVersion) return DQA_ERR_PLAN;
  const int d = p[H_D], T_old = p[H_TOLD], sink = p[H_SINK], C_new = p[H_C], k_out = p[H_KOUT];
  if (d != 64 && d != 128) return DQA_ERR_PLAN;
  if (p[H_B] < 0 || p[H_HKV] < 0 || C_new < 0 || sink < 0 || T_old < 0 || sink > T_old) return DQA_ERR_PLAN;
  if (C_new + sink > kMaxZoneC || k_out < 0 || k_out > kMaxOutliers) return DQA_ERR_PLAN;
  if (static_cast<int64_t>(p[H_B]) * p[H_HKV] != p[H_UNITS]) return DQA_ERR_PLAN;
  const int units = p[H_UNITS];
  if (units > (1 << 20) || T_old > (1 << 24)) return DQA_ERR_PLAN;
  if (p[H_UNIT_OFF] != kHeaderWords || p[H_PERM_OFF] != kHeaderWords + units * kUnitWords ||
      static_cast<int64_t>(p[H_TOK_OFF]) != static_cast<int64_t>(p[H_PERM_OFF]) + static_cast<int64_t>(units) * d)
    return DQA_ERR_PLAN;
  size_t base = 0;
  int max_groups = 0;
  int32_t rec[kUnitWords];
  for (int u = 0; u < units; ++u) {
    const int32_t* U = p + kHeaderWords + static_cast<size_t>(u) * kUnitWords;
    int n[4], m[4];
    long long sn = 0, sm = 0;
    for (int i = 0; i < 4; ++i) {
      n[i] = U[U_N + i];
      m[i] = U[U_M + i];
      if (n[i] < 0 || m[i] < 0) return DQA_ERR_PLAN;
      sn += n[i];
      sm += m[i];
    }
    if (sn > T_old - sink || sm > d) return DQA_ERR_PLAN;
    const long long size = fill_unit(rec, n, m, d, sink, C_new, k_out, base);
    if (size < 0) return DQA_ERR_PLAN;
    for (int w = 0; w < kUnitWords; ++w)
      if (rec[w] != U[w]) return DQA_ERR_PLAN;
    base += static_cast<size_t>(size);
    if (rec[U_TOTAL_GROUPS] > max_groups) max_groups = rec[U_TOTAL_GROUPS];
    const int32_t* perm = p + p[H_PERM_OFF] + static_cast<size_t>(u) * d;
    uint64_t seen[2] = {0, 0};                    // d <= 128 channels
    for (int c = 0; c < d; ++c) {
      const int32_t ch = perm[c];
      if (ch < 0 || ch >= d || ((seen[ch >> 6] >> (ch & 63)) & 1u)) return DQA_ERR_PLAN;
      seen[ch >> 6] |= uint64_t{1} << (ch & 63);
    }
  }
  const size_t blob = static_cast<size_t>(static_cast<uint32_t>(p[H_BLOB_LO])) |
                      (static_cast<size_t>(static_cast<uint32_t>(p[H_BLOB_HI])) << 32);
  if (blob != base || p[H_MAX_GROUPS] != max_groups) return DQA_ERR_PLAN;
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
  int T_old, C, d, sink, k_out;
};

// code = clamp(rint((x - z) / s), 0, levels) with the IEEE quotient (0 for a
// zero scale).  rcp = 1/s within 1 ulp (0 when s == 0): t * rcp and t / s
// differ by at most 2^-22 of t / s < 2^9, i.e. less than 2^-13, so unless
// t * rcp lies within 2^-12 of a half-integer both round alike; there the
// IEEE division decides.
__device__ __forceinline__ uint32_t code_of(float x, float zf, float sf, float rcp, float levels) {
  const float t = x - zf;
  const float y = t * rcp;
  float q = rintf(y);
  if (__builtin_expect(__builtin_fabsf(y - q) >= 0.499755859375f, 0) && sf != 0.0f) q = rintf(t / sf);
  return static_cast<uint32_t>(__builtin_amdgcn_fmed3f(q, 0.0f, levels));
}
__device__ __forceinline__ float rcp_or_zero(float sf) { return sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(sf); }


// n16 16-byte pieces from src to dst by a 128-thread workgroup, four loads
// in flight per thread (dst and src 16-byte aligned).
__device__ __forceinline__ void copy16(uint16_t* dst, const uint16_t* src, size_t n16, int tid) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (size_t i0 = tid; i0 < n16; i0 += 4 * 128) {
    uint32_t u[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t e = i0 + 128 * i;
      const uint4 x = s4[e < n16 ? e : n16 - 1];
      u[i][0] = x.x;
      u[i][1] = x.y;
      u[i][2] = x.z;
      u[i][3] = x.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(u[i][0]), "+v"(u[i][1]), "+v"(u[i][2]), "+v"(u[i][3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t e = i0 + 128 * i;
      if (e < n16) d4[e] = uint4{u[i][0], u[i][1], u[i][2], u[i][3]};
    }
  }
}

// Packed fp16 min / max of two words (both halves at once), and min / max of
// the two halves of one word (in both halves of the result).
__device__ __forceinline__ uint32_t pk_min_h2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_h2(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ uint32_t pk_min_halves(uint32_t w) {
  uint32_t r;
  asm("v_pk_min_f16 %0, %1, %1 op_sel:[1,0] op_sel_hi:[0,1]" : "=v"(r) : "v"(w));
  return r;
}
__device__ __forceinline__ uint32_t pk_max_halves(uint32_t w) {
  uint32_t r;
  asm("v_pk_max_f16 %0, %1, %1 op_sel:[1,0] op_sel_hi:[0,1]" : "=v"(r) : "v"(w));
  return r;
}
// x - z for the fp16 value in half H of word w, by one mixed-precision FMA
// (x * 1 - z, one rounding): the fp32 subtraction of the widened value.
template <int H>
__device__ __forceinline__ float minus_zero(uint32_t w, float zf) {
  return __builtin_fmaf(half_of<H>(w), opaque_const(1.0f), -zf);
}

// Value codes of one slot's value group (32 channels, fp16 pairs in v[16])
// into W words, fields from the low bits up; code_of's arithmetic with the
// subtraction done by minus_zero.
template <int W>
__device__ __forceinline__ void pack_value_words(const uint32_t (&v)[16], float zf, float sf, float rcp,
                                                 uint32_t* dst) {
  constexpr int per = 32 / W;
  const float levels = static_cast<float>((1 << W) - 1);
#pragma unroll
  for (int i = 0; i < W; ++i) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int e = i * per + j;
      const float t = (e & 1) ? minus_zero<1>(v[e >> 1], zf) : minus_zero<0>(v[e >> 1], zf);
      const float y = t * rcp;
      float q = rintf(y);
      if (__builtin_expect(__builtin_fabsf(y - q) >= 0.499755859375f, 0) && sf != 0.0f) q = rintf(t / sf);
      word |= static_cast<uint32_t>(__builtin_amdgcn_fmed3f(q, 0.0f, levels)) << (j * W);
    }
    dst[i] = word;
  }
}

constexpr int kCodeStride = 130;   // lds_c row stride (halves): a column read by slot hits distinct banks

// Key words of one width class: word wl of slot s packs class positions
// first + wl per .. (per = 32 / BITS), read from lds_c; written to the
// slot-major word rows in LDS (row stride ws).  Thread = (slot, word) with
// the slot fastest, so a column read touches 32 distinct banks.
template <int BITS>
__device__ __forceinline__ void pack_key_class(uint32_t* lds_w, int ws, int col, int first, int count, int nw,
                                               const uint16_t (*lds_c)[kCodeStride], int tid) {
  constexpr int per = 32 / BITS;
  for (int e = tid; e < kGroup * nw; e += 128) {
    const int s = e & (kGroup - 1), wl = e >> 5;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) {
      const int idx = wl * per + j;
      const uint32_t f = lds_c[s][min(first + idx, 127)];
      word |= (idx < count ? f : 0u) << (j * BITS);
    }
    lds_w[s * ws + col + wl] = word;
  }
}

// One workgroup (128 threads) per (unit, group); the extra group index
// `total_groups` copies zone C.  Every global load of a group (its key rows
// and this thread's value pieces) is issued at once, before any of the
// group's arithmetic.
template <int D>
__global__ __launch_bounds__(128) void zoned_pack_kernel(PackArgs a) {
  constexpr int kPR = D / 8;                   // 16-byte pieces per row
  constexpr int kKP = kGroup * kPR / 128;      // key (and zone-B) pieces per thread
  constexpr int kVPT = D / kGroup;             // value groups per slot
  // the group's key rows (fp16, row stride D); after the side list, the
  // packed key words (row stride W_K | 1)
  __shared__ __attribute__((aligned(16))) uint32_t lds_kw[kGroup * (D / 2 + 1)];
  __shared__ uint16_t lds_c[kGroup][kCodeStride];   // by class position: codes, or raw fp16 bits of the 16-bit class
  __shared__ int lds_tok[kGroup];
  __shared__ unsigned long long lds_sm[2][kGroup];  // per wave: class positions whose outlier sits in slot s
  __shared__ int lds_off[kGroup + 1];               // slot offsets in the side list, then its entry count
  uint16_t (*lds_k)[D] = reinterpret_cast<uint16_t (*)[D]>(lds_kw);
  const int unit = blockIdx.y;
  const int grp = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t* P = a.plan;
  const int32_t* U = P + P[H_UNIT_OFF] + unit * kUnitWords;
  const int32_t* perm = P + P[H_PERM_OFF] + unit * D;
  const int32_t* tokmap = P + P[H_TOK_OFF] + unit * a.T_old;
  const size_t base = static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_LO])) |
                      (static_cast<size_t>(static_cast<uint32_t>(U[U_BASE_HI])) << 32);
  uint8_t* ub = a.blob + base;
  const size_t src_unit = static_cast<size_t>(unit) * a.T_old * D;
  const int total = U[U_TOTAL_GROUPS];
  if (grp > total) return;
  if (grp == total) {                      // zone C: fp16 copies, sink tokens first
    uint16_t* zc = reinterpret_cast<uint16_t*>(ub + U[U_ZC]);
    const size_t ns = static_cast<size_t>(a.sink) * D;
    const size_t n = ns + static_cast<size_t>(a.C) * D;
    const size_t src = static_cast<size_t>(unit) * a.C * D;
    // 16-byte pieces (rows are multiples of 16 bytes, every block 16-byte
    // aligned), four loads in flight per thread
    copy16(zc, a.k + src_unit, ns / 8, tid);
    copy16(zc + n, a.v + src_unit, ns / 8, tid);
    copy16(zc + ns, a.k_new + src, (n - ns) / 8, tid);
    copy16(zc + n + ns, a.v_new + src, (n - ns) / 8, tid);
    // the unit's tail padding (every block is a multiple of 16 bytes)
    const size_t end = static_cast<size_t>(U[U_ZC]) + 4 * n;
    const int tail16 = static_cast<int>((static_cast<size_t>(U[U_SIZE]) - end) / 16);
    if (tid < tail16) reinterpret_cast<uint4*>(ub + end)[tid] = uint4{0u, 0u, 0u, 0u};
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
  // token-map entries are clamped into [0, T_old): a map zoned_plan did not
  // write gives an unspecified blob, but every read stays in bounds
  if (tid < kGroup)
    lds_tok[tid] = tid < n_valid ? min(max(tokmap[U[U_TOK_PREFIX + seg] + g * kGroup + tid], 0), a.T_old - 1) : -1;
  const int pc = tid;                      // class position of this thread's key channel
  const int ch = pc < D ? perm[pc] : 0;
  __syncthreads();

  // ---- loads: key rows in 16-byte pieces (piece e: slot e / kPR, channels
  // 8 (e % kPR) ..), and either this thread's value group (code segments:
  // slot tid / kVPT, channels 32 (tid % kVPT) ..) or zone-B pieces laid out
  // like the key pieces.  Masked slots read row 0 and are zeroed below.
  uint32_t kr[kKP][4], vr[4][4] = {};
#pragma unroll
  for (int i = 0; i < kKP; ++i) {
    const int e = tid + 128 * i, s = e / kPR;
    const uint4 x = *reinterpret_cast<const uint4*>(a.k + src_unit + static_cast<size_t>(max(lds_tok[s], 0)) * D +
                                                    8 * (e % kPR));
    kr[i][0] = x.x; kr[i][1] = x.y; kr[i][2] = x.z; kr[i][3] = x.w;
  }
  if (w < 16) {
    const int e = min(tid, D - 1), s = e / kVPT;
    const uint4* src = reinterpret_cast<const uint4*>(a.v + src_unit + static_cast<size_t>(max(lds_tok[s], 0)) * D +
                                                      (e % kVPT) * kGroup);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 x = src[i];
      vr[i][0] = x.x; vr[i][1] = x.y; vr[i][2] = x.z; vr[i][3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      const int e = tid + 128 * i, s = e / kPR;
      const uint4 x = *reinterpret_cast<const uint4*>(a.v + src_unit + static_cast<size_t>(max(lds_tok[s], 0)) * D +
                                                      8 * (e % kPR));
      vr[i][0] = x.x; vr[i][1] = x.y; vr[i][2] = x.z; vr[i][3] = x.w;
    }
  }
#pragma unroll
  for (int i = 0; i < kKP; ++i) asm volatile("" : "+v"(kr[i][0]), "+v"(kr[i][1]), "+v"(kr[i][2]), "+v"(kr[i][3]));
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(vr[i][0]), "+v"(vr[i][1]), "+v"(vr[i][2]), "+v"(vr[i][3]));
#pragma unroll
  for (int i = 0; i < kKP; ++i) {
    const int e = tid + 128 * i, s = e / kPR;
    const bool keep = lds_tok[s] >= 0;
    *reinterpret_cast<uint4*>(&lds_k[s][8 * (e % kPR)]) =
        keep ? uint4{kr[i][0], kr[i][1], kr[i][2], kr[i][3]} : uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // ---- keys: thread = class position pc (rows of masked slots are zero)
  const int m2 = U[U_M + 0], m4 = U[U_M + 1], m8 = U[U_M + 2];
  const int n_kq = U[U_NKQ];
  const uint32_t valid = n_valid >= kGroup ? 0xFFFFFFFFu : ((1u << n_valid) - 1u);
  uint32_t out = 0u;                       // slots moved to the side list (bit s)
  uint16_t* ks = reinterpret_cast<uint16_t*>(gb + U[U_KCODES_B]);
  uint16_t* kz = reinterpret_cast<uint16_t*>(gb + U[U_KCODES_B] + U[U_KSZ_B]);
  if (pc >= n_kq && pc < U[U_KSZ_B] / 2) {   // padding of the scale and zero blocks
    ks[pc] = 0;
    kz[pc] = 0;
  }
  if (pc < n_kq) {
    const int bits = pc < m2 ? 2 : (pc < m2 + m4 ? 4 : 8);
    float x[kGroup];
#pragma unroll
    for (int s = 0; s < kGroup; ++s) x[s] = h2f(lds_k[s][ch]);
    // outliers: each round takes the live slot farthest from the live mean
    // (the first slot of the largest or of the smallest value)
    for (int i = 0; i < a.k_out; ++i) {
      const uint32_t live = valid & ~out;
      float sum = 0.0f, vhi = -INFINITY, vlo = INFINITY;
      int hi = -1, lo = -1;
#pragma unroll
      for (int s = 0; s < kGroup; ++s) {
        const bool l = live >> s & 1u;
        sum = l ? sum + x[s] : sum;            // slot order, float32
        const bool gh = l && x[s] > vhi, gl = l && x[s] < vlo;
        vhi = gh ? x[s] : vhi;
        hi = gh ? s : hi;
        vlo = gl ? x[s] : vlo;
        lo = gl ? s : lo;
      }
      const int count = __builtin_popcount(live);
      if (count <= 2 || vhi == vlo || hi < 0 || lo < 0) break;
      const float mean = sum / static_cast<float>(count);
      out |= 1u << (fabsf(vhi - mean) >= fabsf(vlo - mean) ? hi : lo);
    }
    const uint32_t live = valid & ~out;
    float mn = INFINITY, mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      const bool l = live >> s & 1u;
      mn = fminf(mn, l ? x[s] : INFINITY);
      mx = fmaxf(mx, l ? x[s] : -INFINITY);
    }
    const float levels = static_cast<float>((1 << bits) - 1);
    const uint16_t s16 = f2h((mx - mn) / levels);
    const float sf = h2f(s16), rcp = rcp_or_zero(sf);
    ks[pc] = s16;
    kz[pc] = f2h(mn);
#pragma unroll
    for (int s = 0; s < kGroup; ++s)
      lds_c[s][pc] = live >> s & 1u ? static_cast<uint16_t>(code_of(x[s], mn, sf, rcp, levels)) : 0;
  } else if (pc < D) {
#pragma unroll
    for (int s = 0; s < kGroup; ++s) lds_c[s][pc] = lds_k[s][ch];
  }
  if (a.k_out > 0) {
    // slot s's entries, in class-position order: wave-wide masks of the
    // positions that moved slot s
    const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      const unsigned long long m = __ballot(out >> s & 1u);
      if (lane == s) lds_sm[wv][s] = m;
    }
  }
  __syncthreads();
  // side list: slot offsets, then each position writes its own entries
  if (a.k_out > 0) {
    const int cap = n_kq * a.k_out;
    uint8_t* ob = gb + U[U_KCODES_B] + 2 * U[U_KSZ_B];
    uint16_t* offs = reinterpret_cast<uint16_t*>(ob);
    uint16_t* opc = reinterpret_cast<uint16_t*>(ob + kOffsBytes);
    uint16_t* oval = reinterpret_cast<uint16_t*>(ob + kOffsBytes + pad(static_cast<size_t>(cap) * 2, 16));
    if (tid < kGroup) {
      int o = 0;
#pragma unroll
      for (int s = 0; s < kGroup; ++s)
        if (s < tid) o += __popcll(lds_sm[0][s]) + __popcll(lds_sm[1][s]);
      lds_off[tid] = o;
      offs[tid] = static_cast<uint16_t>(o);
      if (tid == kGroup - 1) {
        lds_off[kGroup] = o + __popcll(lds_sm[0][tid]) + __popcll(lds_sm[1][tid]);
        offs[kGroup] = static_cast<uint16_t>(lds_off[kGroup]);
      }
    } else if (tid > kGroup && tid < kOffsBytes / 2) {
      offs[tid] = 0;                             // padding after the 33 offsets
    }
    __syncthreads();
    // unused entries up to the padded capacity are zero
    const int cap16 = static_cast<int>(pad(static_cast<size_t>(cap) * 2, 16) / 2);
    for (int i = lds_off[kGroup] + tid; i < cap16; i += blockDim.x) {
      opc[i] = 0;
      oval[i] = 0;
    }
    const int wv = tid >> 6;
    for (uint32_t rest = out; rest != 0u; rest &= rest - 1u) {
      const int s = __builtin_ctz(rest);
      const unsigned long long m = lds_sm[wv][s];
      const int rank = static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u))) +
                       (wv ? __popcll(lds_sm[0][s]) : 0);
      const int o = lds_off[s] + rank;
      opc[o] = static_cast<uint16_t>(pc);
      oval[o] = lds_k[s][ch];
    }
  }
  __syncthreads();                               // lds_k is reused for the key words below
  // key rows: class blocks of W_K words per slot, built in LDS (row stride
  // W_K | 1), then copied out as 16-byte pieces
  const int kw2 = U[U_KWORDS + 0], kw4 = U[U_KWORDS + 1], kw8 = U[U_KWORDS + 2], kw16 = U[U_KWORDS + 3];
  const int W_K = U[U_WK];
  const int ws = W_K | 1;
  pack_key_class<2>(lds_kw, ws, 0, 0, m2, kw2, lds_c, tid);
  pack_key_class<4>(lds_kw, ws, kw2, m2, m4, kw4, lds_c, tid);
  pack_key_class<8>(lds_kw, ws, kw2 + kw4, m2 + m4, m8, kw8, lds_c, tid);
  pack_key_class<16>(lds_kw, ws, kw2 + kw4 + kw8, n_kq, U[U_M + 3], kw16, lds_c, tid);

  // ---- values (from registers; no LDS)
  if (w < 16) {
    if (tid < D) {                              // value group (slot s, vg)
      const int vwpt = D * w / 32;              // value words per slot
      uint8_t* vbase = gb + U[U_KCODES_B] + 2 * U[U_KSZ_B] + U[U_OUT_B];
      uint32_t* vcodes = reinterpret_cast<uint32_t*>(vbase);
      constexpr size_t kVszB = static_cast<size_t>(kGroup) * kVPT * 2;   // a multiple of 16
      uint16_t* vs = reinterpret_cast<uint16_t*>(vbase + kGroup * vwpt * 4);
      uint16_t* vz = reinterpret_cast<uint16_t*>(vbase + kGroup * vwpt * 4 + kVszB);
      const int e = tid, s = e / kVPT, vg = e % kVPT;
      uint32_t* dst = vcodes + s * vwpt + vg * w;
      if (s >= n_valid) {
        for (int i = 0; i < w; ++i) dst[i] = 0u;
        vs[e] = 0;
        vz[e] = 0;
      } else {
        uint32_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = vr[i >> 2][i & 3];
        uint32_t pmn = pk_min_h2(v[0], v[1]), pmx = pk_max_h2(v[0], v[1]);
#pragma unroll
        for (int i = 2; i < 16; ++i) {
          pmn = pk_min_h2(pmn, v[i]);
          pmx = pk_max_h2(pmx, v[i]);
        }
        const float mn = h2f(static_cast<uint16_t>(pk_min_halves(pmn) & 0xFFFFu));
        const float mx = h2f(static_cast<uint16_t>(pk_max_halves(pmx) & 0xFFFFu));
        const float levels = static_cast<float>((1 << w) - 1);
        const uint16_t s16 = f2h((mx - mn) / levels);
        const float sf = h2f(s16), rcp = rcp_or_zero(sf);
        vs[e] = s16;
        vz[e] = f2h(mn);
        if (w == 2) pack_value_words<2>(v, mn, sf, rcp, dst);
        else if (w == 4) pack_value_words<4>(v, mn, sf, rcp, dst);
        else pack_value_words<8>(v, mn, sf, rcp, dst);
      }
    }
  } else {
    // zone B rows of this group's slots (masked slots store zeros)
    uint4* zb = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(ub + U[U_ZB]) + static_cast<size_t>(g) * kGroup * D);
#pragma unroll
    for (int i = 0; i < kKP; ++i) {
      const int e = tid + 128 * i;
      const bool keep = lds_tok[e / kPR] >= 0;
      zb[e] = keep ? uint4{vr[i][0], vr[i][1], vr[i][2], vr[i][3]} : uint4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  // key words out: 32 W_K words, contiguous in the blob
  uint4* krow = reinterpret_cast<uint4*>(gb);
  for (int e = tid; e < kGroup * W_K / 4; e += 128) {
    int s = (4 * e) / W_K, c = 4 * e - s * W_K;          // slot and word of the piece's first word
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {                          // a piece may cross rows (W_K < 4 or not a multiple of 4)
      q[j] = lds_kw[s * ws + c];
      if (++c == W_K) {
        c = 0;
        ++s;
      }
    }
    krow[e] = uint4{q[0], q[1], q[2], q[3]};
  }
}


// ------------------------------------------------------------------ reader

constexpr int kZWaves = 8;
// Workgroups per launch: one resident round (one workgroup of eight waves,
// two per SIMD, per compute unit on 256 CUs), so every wave pays its
// start-up once and a (batch, KV head) has half as many splits to merge as
// with two workgroups of four waves per CU.
constexpr int kZoneWorkgroups = 256;
// Staging bytes per wave: a zone-A group's key block (at most 8,480 B for
// d = 128: 32 key rows of at most 66 words, then scales and zeros), or a
// zone-C chunk's fp16 keys (8 KiB).  The host checks every unit against it.
constexpr int kStageBytes = 8704;

struct ZDecodeArgs {
  const int32_t* plan;
  const uint8_t* blob;
  const uint16_t* q;
  float* out;
  float* partials;
  uint32_t* counters;                         // merge counters, one per (batch, KV head)
  int Hq, Hkv, C, items_per_split, splits;   // C: zone-C rows (sink + new tokens)
  int k_out;                                  // side-list entries per key group (0: none)
  float q_scale;
};

// Logit contributions of one key class: the lane's words [wlo, whi) of its
// key row, `rot` rotating the visiting order (conflict-free LDS rows for
// the fp16 rows of zone C).  Entry e of `tab` holds q_h * s (or q_h) of the
// channel that sits at code position e of the class.
template <int W, int G>
__device__ __forceinline__ void key_class(const uint32_t* words, int wlo, int whi, int rot,
                                          const float4* tab, float (&part)[G]) {
  constexpr int CPW = 32 / W;           // codes per word
  const int n = whi - wlo;
  int r = n > 0 ? rot % n : 0;
  for (int it = 0; it < n; ++it) {
    const int wi = wlo + r;
    r = (r + 1 == n) ? 0 : r + 1;
    const uint32_t x = words[wi];
    const float4* e = tab + wi * CPW;
    float code[CPW];
    if constexpr (W == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t bts = (x >> (2 * k)) & 0x03030303u;   // codes 4m + k in byte m
#pragma unroll
        for (int m = 0; m < 4; ++m) code[4 * m + k] = static_cast<float>((bts >> (8 * m)) & 0xFFu);
      }
    } else if constexpr (W == 4) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t bts = (x >> (4 * k)) & 0x0F0F0F0Fu;   // codes 2m + k in byte m
#pragma unroll
        for (int m = 0; m < 4; ++m) code[2 * m + k] = static_cast<float>((bts >> (8 * m)) & 0xFFu);
      }
    } else if constexpr (W == 8) {
#pragma unroll
      for (int m = 0; m < 4; ++m) code[m] = static_cast<float>((x >> (8 * m)) & 0xFFu);
    } else {
      code[0] = h2f(static_cast<uint16_t>(x & 0xFFFFu));
      code[1] = h2f(static_cast<uint16_t>(x >> 16));
    }
#pragma unroll
    for (int p = 0; p < CPW; ++p) {
      const float4 t = e[p];
      const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
      for (int h = 0; h < G; ++h) part[h] = fmaf(tv[h], code[p], part[h]);
      // table reads in batches of four (bounded register use)
      if ((p & 3) == 3) asm volatile("" ::: "memory");
    }
  }
}

// Copy n16 16-byte pieces (at most kStageBytes) into the wave's LDS slice:
// every load is issued before the first store, so the wave waits for one
// memory round trip per item rather than one per piece.
// Pieces past n16 reload the last piece (in bounds, n16 >= 1) and are not
// stored.  The empty asm statements take every loaded value before the first
// store, so the compiler cannot move each load next to its (conditional)
// store.
__device__ __forceinline__ void stage_block(const uint4* src, uint4* dst, int n16, int lane) {
  constexpr int kIters = (kStageBytes / 16 + kWave - 1) / kWave;
  uint32_t t[kIters][4];
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const uint4 u = src[min(lane + kWave * k, n16 - 1)];
    t[k][0] = u.x;
    t[k][1] = u.y;
    t[k][2] = u.z;
    t[k][3] = u.w;
  }
#pragma unroll
  for (int k = 0; k < kIters; ++k) asm volatile("" : "+v"(t[k][0]), "+v"(t[k][1]), "+v"(t[k][2]), "+v"(t[k][3]));
#pragma unroll
  for (int k = 0; k < kIters; ++k) {
    const int i = lane + kWave * k;
    if (i < n16) dst[i] = uint4{t[k][0], t[k][1], t[k][2], t[k][3]};
  }
}

// Decode over one unit's items (zone-A groups in segment order, then zone-C
// chunks of 32 tokens); each wave takes whole items.
//
// Per item: the group's bytes are staged in the wave's LDS slice with
// 16-byte loads.  Keys: logit_h(t) = sum_c q_h,c (s_c code_t,c + z_c)
//   = sum_c (q_h,c s_c) code_t,c + sum_c q_h,c z_c;
// the wave builds the table q_h,c s_c for the group once, and the bias
// sum_c q_h,c z_c once.  Lane (slot t = lane % 32, half) walks half of the
// words of every key class of t's row (both halves of the wave at the same
// class, so the code width is uniform), converting codes to floats and
// accumulating the G heads.  Values: lane = CV consecutive channels;
// out_h,c += sum_t (p_h,t s_t,g) code_t,c, and the zero-point term
// sum_t p_h,t z_t,g is kept per lane (one product per slot, head and value
// group) and summed over lanes once at the end.  fp16 value rows (zone B,
// zone C) are loaded into registers while the keys are staged.
template <int D, int G>
__global__ __launch_bounds__(64 * kZWaves, 1) void zoned_decode_kernel(ZDecodeArgs a) {
  constexpr int CV = D / 64;                        // value channels per lane
  constexpr int NG = D / kGroup;                    // value groups per token
  constexpr int NGH = NG / 2;                       // value groups per lane half
  constexpr int kEntries = D + 26;                  // table entries: classes padded to whole words
  static_assert(kZWaves * G * D * 4 <= kZWaves * kStageBytes, "wave states fit in the staging area");
  __shared__ __attribute__((aligned(16))) uint8_t lds_stage[kZWaves][kStageBytes];
  __shared__ __attribute__((aligned(16))) float4 lds_tab[kZWaves][kEntries];
  __shared__ __attribute__((aligned(16))) float4 lds_ps[kZWaves][kGroup][NG];
  __shared__ float lds_qp[G][D], lds_qn[G][D];      // query: permuted / natural channel order
  __shared__ float lds_m[kZWaves][G], lds_l[kZWaves][G];
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

  // key classes of the unit: channels, words, first channel, first table entry
  int cm[4], ckw[4], cch[4], cent[4];
  {
    int ch = 0, en = 0;
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) {
      cm[ci] = U[U_M + ci];
      ckw[ci] = U[U_KWORDS + ci];
      cch[ci] = ch;
      cent[ci] = en;
      ch += cm[ci];
      en += ckw[ci] * (32 / kSegW[ci]);
    }
  }
  const int n_ent = cent[3] + ckw[3] * 2;
  const int n_kq = U[U_NKQ];
  const int W_K = U[U_WK];
  const int kcodes_b = U[U_KCODES_B], ksz_b = U[U_KSZ_B], out_b = U[U_OUT_B];
  const int total = U[U_TOTAL_GROUPS];
  const int items = total + (a.C + kGroup - 1) / kGroup;
  const int j = lane & 31, hf = lane >> 5;
  const int c0 = lane * CV;
  uint8_t* st = lds_stage[wave];
  float4* tab = lds_tab[wave];

  float m[G], l[G], acc[G][CV], zp[G][NGH];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < CV; ++c) acc[h][c] = 0.0f;
#pragma unroll
    for (int gi = 0; gi < NGH; ++gi) zp[h][gi] = 0.0f;
  }

  const int ib = split * a.items_per_split;
  const int ie = min(items, ib + a.items_per_split);
  for (int item = ib + wave; item < ie; item += kZWaves) {
    const bool zone_c = item >= total;
    int seg = 3, g = 0, n_valid;
    const uint16_t* vrows = nullptr;          // fp16 value rows (zone B / zone C), else null
    const uint8_t* gb = nullptr;              // zone-A group
    const uint4* stage_src;                   // the item's key block / zone-C keys, staged below
    int stage_n16;
    if (!zone_c) {
      seg = 0;
      g = item;
      while (g >= U[U_GROUPS + seg]) {
        g -= U[U_GROUPS + seg];
        ++seg;
      }
      n_valid = min(kGroup, U[U_N + seg] - g * kGroup);
      gb = ub + U[U_SEG_OFF + seg] + static_cast<size_t>(g) * U[U_GRP_B + seg];
      const int nb = kcodes_b + 2 * ksz_b + out_b;  // the key block (with its side list)
      stage_src = reinterpret_cast<const uint4*>(gb);
      stage_n16 = nb / 16;
      if (seg == 3)
        vrows = reinterpret_cast<const uint16_t*>(ub + U[U_ZB]) + static_cast<size_t>(g) * kGroup * D;
    } else {
      const int cg = item - total;
      n_valid = min(kGroup, a.C - cg * kGroup);
      const uint16_t* zck = reinterpret_cast<const uint16_t*>(ub + U[U_ZC]) + static_cast<size_t>(cg) * kGroup * D;
      stage_src = reinterpret_cast<const uint4*>(zck);
      stage_n16 = n_valid * D * 2 / 16;
      vrows = zck + static_cast<size_t>(a.C) * D;
    }
    const int w = kSegW[seg];
    // The lane's value bits of every slot straight into registers (slots
    // past n_valid read 0): fp16 rows (zone B, zone C), or the code word
    // holding its CV channels; with codes, the slot's scales and zeros of
    // the lane's value groups.
    uint32_t vr[kGroup];
    uint32_t vsz[2] = {0u, 0u};
    const int vwpt = D * w / 32;
    const int widx = (c0 * w) >> 5, sh = (c0 * w) & 31;
    const int vsz_b = (kGroup * NG * 2 + 15) / 16 * 16;
    // slots past n_valid reload the last valid slot (in bounds) and are zeroed
    const bool fp16v = zone_c || seg == 3;         // wave-uniform
    if (fp16v) {
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        const int te = min(t, n_valid - 1);
        uint32_t x;
        if constexpr (CV == 2)
          x = *reinterpret_cast<const uint32_t*>(vrows + static_cast<size_t>(te) * D + c0);
        else
          x = vrows[static_cast<size_t>(te) * D + c0];
        vr[t] = t < n_valid ? x : 0u;
      }
    } else {
      const uint8_t* vb = gb + kcodes_b + 2 * ksz_b + out_b;
      const uint32_t* vcodes = reinterpret_cast<const uint32_t*>(vb);
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        const uint32_t x = vcodes[min(t, n_valid - 1) * vwpt + widx];
        vr[t] = t < n_valid ? x : 0u;
      }
      const uint16_t* vs = reinterpret_cast<const uint16_t*>(vb + kGroup * vwpt * 4);
      const uint16_t* vz = reinterpret_cast<const uint16_t*>(vb + kGroup * vwpt * 4 + vsz_b);
      if constexpr (NGH == 2) {
        vsz[0] = *reinterpret_cast<const uint32_t*>(vs + j * NG + 2 * hf);
        vsz[1] = *reinterpret_cast<const uint32_t*>(vz + j * NG + 2 * hf);
      } else {
        vsz[0] = vs[j * NG + hf];
        vsz[1] = vz[j * NG + hf];
      }
    }
    // the key block's loads follow the value loads, so both are in flight
    // together (one memory round trip per item)
    stage_block(stage_src, reinterpret_cast<uint4*>(st), stage_n16, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- table of q*s (and the bias sum q*z) for this item
    float bias[G];
#pragma unroll
    for (int h = 0; h < G; ++h) bias[h] = 0.0f;
    if (!zone_c) {
      const uint16_t* ks = reinterpret_cast<const uint16_t*>(st + kcodes_b);
      const uint16_t* kz = reinterpret_cast<const uint16_t*>(st + kcodes_b + ksz_b);
      for (int e = lane; e < n_ent; e += 64) {
        const int ci = (e >= cent[1]) + (e >= cent[2]) + (e >= cent[3]);
        const int local = e - (ci == 0 ? cent[0] : ci == 1 ? cent[1] : ci == 2 ? cent[2] : cent[3]);
        const int mm = ci == 0 ? cm[0] : ci == 1 ? cm[1] : ci == 2 ? cm[2] : cm[3];
        const int pc = local + (ci == 0 ? cch[0] : ci == 1 ? cch[1] : ci == 2 ? cch[2] : cch[3]);
        float tv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (local < mm) {
          const bool quant = pc < n_kq;
          const float sc = quant ? h2f(ks[pc]) : 1.0f;
          const float zr = quant ? h2f(kz[pc]) : 0.0f;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float qv = lds_qp[h][pc];
            tv[h] = qv * sc;
            bias[h] = fmaf(qv, zr, bias[h]);
          }
        }
        tab[e] = make_float4(tv[0], tv[1], tv[2], tv[3]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) bias[h] = wave_sum(bias[h]);
    } else {
      for (int e = lane; e < D; e += 64) {
        float tv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < G; ++h) tv[h] = lds_qn[h][e];
        tab[e] = make_float4(tv[0], tv[1], tv[2], tv[3]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- logits: lane = (slot j, half of every class's words)
    const bool valid = j < n_valid;
    float part[G];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h] = 0.0f;
    if (valid) {
      if (!zone_c) {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(st) + j * W_K;
        int wb = 0;
#pragma unroll
        for (int ci = 0; ci < 4; ++ci) {
          const int kw = ckw[ci], h0 = (kw + 1) >> 1;
          const int wlo = hf ? h0 : 0, whi = hf ? kw : h0;
          const float4* tb = tab + cent[ci];
          if (ci == 0) key_class<2, G>(row + wb, wlo, whi, 0, tb, part);
          else if (ci == 1) key_class<4, G>(row + wb, wlo, whi, 0, tb, part);
          else if (ci == 2) key_class<8, G>(row + wb, wlo, whi, 0, tb, part);
          else key_class<16, G>(row + wb, wlo, whi, 0, tb, part);
          wb += kw;
        }
        if (a.k_out > 0) {
          // side-list entries of slot j (the two halves take alternate
          // entries): the key there is the stored value, not the code-0
          // dequantization z
          const uint16_t* offs = reinterpret_cast<const uint16_t*>(st + kcodes_b + 2 * ksz_b);
          const uint16_t* opc = offs + kOffsBytes / 2;
          const uint16_t* oval = opc + (n_kq * a.k_out * 2 + 15) / 16 * 8;
          const uint16_t* kz = reinterpret_cast<const uint16_t*>(st + kcodes_b + ksz_b);
          const int e_end = min(static_cast<int>(offs[j + 1]), n_kq * a.k_out);
          for (int e = offs[j] + hf; e < e_end; e += 2) {
            const int pc = min(static_cast<int>(opc[e]), n_kq - 1);
            const float dv = h2f(oval[e]) - h2f(kz[pc]);
#pragma unroll
            for (int h = 0; h < G; ++h) part[h] = fmaf(dv, lds_qp[h][pc], part[h]);
          }
        }
      } else {
        const uint32_t* row = reinterpret_cast<const uint32_t*>(st) + j * (D / 2);
        const int wlo = hf ? D / 4 : 0, whi = hf ? D / 2 : D / 4;
        key_class<16, G>(row, wlo, whi, j, tab, part);
      }
    }
    float lg[G], mnew[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lg[h] = swap_rows<false>(part[h], true) + bias[h];   // the two halves of slot j
      const float t = wave_max(valid ? lg[h] : -INFINITY);
      mnew[h] = fmaxf(m[h], t);
      grow |= mnew[h] > m[h];
    }
    if (grow) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = merge_weight(m[h], mnew[h]);
        l[h] *= sc;
#pragma unroll
        for (int c = 0; c < CV; ++c) acc[h][c] *= sc;
#pragma unroll
        for (int gi = 0; gi < NGH; ++gi) zp[h][gi] *= sc;
        m[h] = mnew[h];
      }
    }
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = valid ? exp2f(lg[h] - m[h]) : 0.0f;
      if (hf == 0) l[h] += p[h];
    }

    // ---- values
    if (!fp16v) {
      // p * scale per (slot, value group) into LDS; zero-point products kept
      // per lane
#pragma unroll
      for (int gi = 0; gi < NGH; ++gi) {
        const int gg = hf * NGH + gi;
        const float sc = h2f(static_cast<uint16_t>(vsz[0] >> (16 * gi)));
        const float zr = h2f(static_cast<uint16_t>(vsz[1] >> (16 * gi)));
        float tv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < G; ++h) {
          tv[h] = p[h] * sc;
          zp[h][gi] = fmaf(p[h], zr, zp[h][gi]);
        }
        lds_ps[wave][j][gg] = make_float4(tv[0], tv[1], tv[2], tv[3]);
      }
    } else if (hf == 0) {
      float tv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < G; ++h) tv[h] = p[h];
      lds_ps[wave][j][0] = make_float4(tv[0], tv[1], tv[2], tv[3]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint32_t mask = (1u << w) - 1u;
    auto accumulate = [&](const float4 p4, const float (&vv)[CV]) {
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < CV; ++c) acc[h][c] = fmaf(pv[h], vv[c], acc[h][c]);
    };
    if (fp16v) {
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        float vv[CV];
        if constexpr (CV == 2) {
          vv[0] = h2f(static_cast<uint16_t>(vr[t] & 0xFFFFu));
          vv[1] = h2f(static_cast<uint16_t>(vr[t] >> 16));
        } else {
          vv[0] = h2f(static_cast<uint16_t>(vr[t]));
        }
        accumulate(lds_ps[wave][t][0], vv);
      }
    } else {
      const int vg = c0 / kGroup;
#pragma unroll
      for (int t = 0; t < kGroup; ++t) {
        float vv[CV];
#pragma unroll
        for (int c = 0; c < CV; ++c) vv[c] = static_cast<float>((vr[t] >> (sh + c * w)) & mask);
        accumulate(lds_ps[wave][t][vg], vv);
      }
    }
    // the next item overwrites the staging area and the tables
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- wave state -> LDS: l over all lanes; the zero-point products over
  // the 32 lanes of each half, where lane c0 / 32 = its value group
  float zsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = wave_sum(l[h]);
    float zs[NGH];
#pragma unroll
    for (int gi = 0; gi < NGH; ++gi) zs[gi] = half_sum(zp[h][gi]);
    zsum[h] = zs[0];
    if constexpr (NGH == 2) zsum[h] = ((c0 / kGroup) & 1) ? zs[1] : zs[0];
  }
  __syncthreads();                                  // staging area becomes the wave states
  float (*lds_o)[G][D] = reinterpret_cast<float (*)[G][D]>(&lds_stage[0][0]);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < CV; ++c) lds_o[wave][h][c0 + c] = acc[h][c] + zsum[h];
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = m[h];
      lds_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  write_split_state<D, G, kZWaves>(a.partials, a.counters + unit, a.out, a.Hq, static_cast<size_t>(unit), b, kvh,
                                   split, a.splits, lds_m, lds_l, lds_o);
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
  // every key block fits one staging slice
  for (int u = 0; u < g->units; ++u) {
    const int32_t* U = p + p[H_UNIT_OFF] + static_cast<size_t>(u) * kUnitWords;
    if (U[U_KCODES_B] + 2 * U[U_KSZ_B] + U[U_OUT_B] > kStageBytes) return DQA_ERR_PLAN;
  }
  g->items_max = p[H_MAX_GROUPS] + (p[H_C] + p[H_SINK] + kGroup - 1) / kGroup;
  long long s = (kZoneWorkgroups + g->units - 1) / (g->units > 0 ? g->units : 1);
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
    case 1: hipLaunchKernelGGL((zoned_decode_kernel<D, 1>), grid, dim3(64 * kZWaves), 0, s, a); break;
    case 2: hipLaunchKernelGGL((zoned_decode_kernel<D, 2>), grid, dim3(64 * kZWaves), 0, s, a); break;
    case 4: hipLaunchKernelGGL((zoned_decode_kernel<D, 4>), grid, dim3(64 * kZWaves), 0, s, a); break;
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
                          int C_new, int d, int sink, int k_out, int32_t* plan, size_t n_words,
                          size_t* blob_bytes) {
  const size_t need = plan_words(B, Hkv, T_old, d);
  if (need == 0 || C_new < 0 || sink < 0 || sink > T_old || C_new + sink > kMaxZoneC) return DQA_ERR_SHAPE;
  if (k_out < 0 || k_out > kMaxOutliers) return DQA_ERR_SHAPE;
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
    if (w != 0 && w != 2 && w != 4 && w != 8 && w != 16) return DQA_ERR_BITS;
  }
  for (size_t i = 0; i < need; ++i) plan[i] = 0;
  plan[H_MAGIC] = kPlanMagic;
  plan[H_VERSION] = kPlanVersion;
  plan[H_B] = B;
  plan[H_HKV] = Hkv;
  plan[H_TOLD] = T_old;
  plan[H_C] = C_new;
  plan[H_D] = d;
  plan[H_UNITS] = units;
  plan[H_UNIT_OFF] = kHeaderWords;
  plan[H_PERM_OFF] = kHeaderWords + units * kUnitWords;
  plan[H_TOK_OFF] = kHeaderWords + units * (kUnitWords + d);
  plan[H_SINK] = sink;
  plan[H_KOUT] = k_out;
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
    }
    // evicted key channels (width 0) close the permutation; they are stored
    // nowhere and read by no product
    for (int c = 0; c < d; ++c)
      if (kb[c] == 0) perm[np++] = c;
    int nt = 0;
    for (int si = 0; si < 4; ++si) {
      int n = 0;
      for (int t = sink; t < T_old; ++t)          // sink tokens live in zone C
        if (vb[t] == kSegW[si]) {
          tok[nt++] = t;
          ++n;
        }
      U[U_N + si] = n;
    }
    int n[4], m[4];
    for (int i = 0; i < 4; ++i) {
      n[i] = U[U_N + i];
      m[i] = U[U_M + i];
    }
    const long long size = fill_unit(U, n, m, d, sink, C_new, k_out, base);
    if (size < 0) return DQA_ERR_SHAPE;
    const int total = U[U_TOTAL_GROUPS];
    if (total > max_groups) max_groups = total;
    base += static_cast<size_t>(size);
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
  if ((plan_host[H_TOLD] > 0 || plan_host[H_SINK] > 0) && (!k || !v)) return DQA_ERR_NULL;
  if (plan_host[H_C] > 0 && (!k_new || !v_new)) return DQA_ERR_NULL;
  if (units > 65535) return DQA_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(blob))
    return DQA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PackArgs a{plan_dev, k, v, k_new, v_new, static_cast<uint8_t*>(blob), plan_host[H_TOLD],
             plan_host[H_C], plan_host[H_D], plan_host[H_SINK], plan_host[H_KOUT]};
  const dim3 grid(plan_host[H_MAX_GROUPS] + 1, units);
  if (plan_host[H_D] == 64)
    hipLaunchKernelGGL(zoned_pack_kernel<64>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(zoned_pack_kernel<128>, grid, dim3(128), 0, s, a);
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
  if (!aligned16(blob) || !aligned16(ws) || !aligned16(out)) return DQA_ERR_ALIGN;
  ZDecodeArgs a;
  a.plan = plan_dev;
  a.blob = static_cast<const uint8_t*>(blob);
  a.q = q;
  a.out = out;
  a.partials = merge_partials(ws, static_cast<size_t>(g.units));
  a.counters = merge_counters(ws);
  a.Hq = Hq;
  a.Hkv = plan_host[H_HKV];
  a.C = plan_host[H_C] + plan_host[H_SINK];
  a.k_out = plan_host[H_KOUT];
  a.items_per_split = g.ips;
  a.splits = g.splits;
  a.q_scale = sm_scale * 1.4426950408889634f;
  const dim3 grid(g.splits, g.units);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (plan_host[H_D] == 128) return zlaunch<128>(a, g.G, grid, s);
  return zlaunch<64>(a, g.G, grid, s);
}
