// RDKV bit allocation: distortion weights of the cache units and the
// Lagrangian width assignment that produces the zoned cache's width maps.
//
// [P3 sec 2.1, theoretical formulation]: a value-cache unit is a token, its
// weight the attention it receives summed over every query position; a
// key-cache unit is a channel, its weight the product of the query and key
// column norms divided by sqrt(d).  The widths b in {0, 2, 4, 8, 16} minimize
// sum w 2^(-b) under a total-bit budget, by Lagrangian relaxation ([P3 sec
// 2.2, bit-allocation pipeline]); weights come from the full prefill cache;
// token widths are assigned first, channel widths over the kept tokens.
//
// Token weights (the dense part) are causal-attention column sums, done in
// two passes over the logits on v_mfma_f32_16x16x32_f16 (fp16 inputs are
// exact, fp32 accumulation):
//   1. per query row, the log-sum-exp of its causal logits (base 2);
//   2. per key tile, sum over rows and over the G heads of a KV head of
//      exp2(logit - lse).  A workgroup owns its 256 keys (4 waves x 64,
//      sharing each query tile), so the sums are written without atomics
//      and repeat bit for bit.  Each query fragment read from LDS feeds the
//      products of a wave's four key blocks (with two, the LDS reads took
//      as long as the products and the pass 15% longer).  Wider workgroups
//      (8 or 16 waves) stream the query rows fewer times but measured
//      slower: the caches already serve most re-reads, and the wider
//      barrier costs more.
// Both passes see identical logits (same operands, same order).  Pass 1
// walks key tiles from 0 upward and pass 2 query tiles from the last one
// downward, so the workgroups of one KV head that run together read the
// same tiles; block ids are laid out so that one KV head stays on one XCD
// when the head count is a multiple of 8.
//
// Channel weights are sums of squares over positions (HBM-bound), reduced
// per chunk and then in a fixed order.
//
// Allocation: with breakpoints w*f for f in {3/8, 3/32, 15/1024, 255/2^19}
// a unit's width at multiplier lam is 2[lam < 3w/8] + 2[lam < 3w/32]
// + 4[lam < 15w/1024] + 8[lam < 255w/2^19] (its Lagrangian minimizer, ties
// to the smaller width), and the smallest lam meeting the budget is the
// breakpoint where the mass of breakpoints (2, 2, 4, 8 bits each), counted
// from the largest down, first exceeds the budget (0 if the total fits).  A
// float32 weight times one factor is exact in float64, so that breakpoint is
// found exactly by a radix select on its float64 bit pattern: six passes of
// a per-chunk histogram (11, ..., 11, 8 bits) and a per-row selection.
#include "common.h"

#include <type_traits>

namespace dqa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // promotable (HIP's uint4 is a struct)

constexpr int kLseRows = 128;   // query rows per workgroup in pass 1 (4 waves x 32)
constexpr int kLseKeys = 64;    // keys per LDS tile in pass 1
constexpr int kSumWaves = 4;    // waves per workgroup in pass 2, sharing one query tile
constexpr int kSumNB = 4;       // 16-key blocks per wave in pass 2 (keys in registers)
constexpr int kSumRB = 4;       // 16-row blocks per query tile in pass 2
constexpr int kSumKeys = 16 * kSumNB * kSumWaves;  // keys per workgroup in pass 2
constexpr int kSumRows = 16 * kSumRB;               // query rows per LDS tile in pass 2
constexpr int kChanRows = 256;  // positions per workgroup of the channel sums
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescale = 0x1p100f;  // a row sum at or above this moves its reference

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ pass 1: lse

template <int D>
__global__ __launch_bounds__(256) void rdkv_lse_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k, int B, int Hq,
                                                       int Hkv, int T, float c,
                                                       float* __restrict__ lse) {
  constexpr int KS = D / 32, PAD = D + 8, CH = D / 8;
  constexpr int LOADS = kLseKeys * CH / 256;
  __shared__ __align__(16) _Float16 lds_k[kLseKeys * PAD];

  const int G = Hq / Hkv;
  const int heads = B * Hq;
  const int nqt = (T + kLseRows - 1) / kLseRows;
  const int hu = blockIdx.x % heads;
  const int qt = nqt - 1 - static_cast<int>(blockIdx.x / heads);  // longest rows first
  const int kv = hu % Hkv, rest = hu / Hkv, g = rest % G, b = rest / G;
  const int h = kv * G + g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 15, grp = lane >> 4;
  const int q0 = qt * kLseRows + wave * 32;

  const uint16_t* qh = q + (static_cast<size_t>(b) * Hq + h) * static_cast<size_t>(T) * D;
  const uint16_t* kh = k + (static_cast<size_t>(b) * Hkv + kv) * static_cast<size_t>(T) * D;

  half8 a[2][KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = min(q0 + 16 * rb + col, T - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      a[rb][s] = *reinterpret_cast<const half8*>(qh + static_cast<size_t>(row) * D + 32 * s + 8 * grp);
  }

  float mc[2][4], l[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mc[rb][r] = 0.0f;
      l[rb][r] = 0.0f;
    }

  const int last_row = min(qt * kLseRows + kLseRows, T) - 1;
  const int nkt = last_row / kLseKeys + 1;

  u32x4 pre[LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int cidx = tid + 256 * j, r = cidx / CH, ch = cidx % CH;
      const int key = min(kt * kLseKeys + r, T - 1);
      pre[j] = *reinterpret_cast<const u32x4*>(kh + static_cast<size_t>(key) * D + ch * 8);
    }
  };

  gload(0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int cidx = tid + 256 * j, r = cidx / CH, ch = cidx % CH;
      *reinterpret_cast<u32x4*>(&lds_k[r * PAD + ch * 8]) = pre[j];
    }
    __syncthreads();
    gload(min(kt + 1, nkt - 1));  // unconditional: keeps the prefetch in registers
    const int kbase = kt * kLseKeys;
    if (kbase > q0 + 31) continue;  // every key of the tile follows every row of the wave

    float4v acc[2][4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      acc[0][nb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
      acc[1][nb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8 bf = *reinterpret_cast<const half8*>(&lds_k[(16 * nb + col) * PAD + 32 * s + 8 * grp]);
        acc[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0][s], bf, acc[0][nb], 0, 0, 0);
        acc[1][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1][s], bf, acc[1][nb], 0, 0, 0);
      }
    }
    // Per lane and row: l = sum of exp2(c x - mc) against a reference mc
    // (log2 units).  A tile's terms are first added against the current
    // reference; only if that sum is not below kRescale (a large logit, an
    // overflow to infinity: a uniform branch, rare after the first tile) is
    // the tile redone with the reference moved up to the tile's maximum
    // (moving it by any delta, mc += delta, l *= 2^-delta, leaves the sum
    // exact).  Key tile 0 always takes that branch: a lane with nothing
    // accumulated yet takes its own maximum as the reference.  Every wave
    // that reaches a later tile holds rows >= 64, all of which saw a valid
    // key in tile 0, so no lane starts its sum after tile 0.
    auto update = [&](auto masked) {
      float t[2][4][4], ls[2][4];
      bool need = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float sum = l[rb][r];
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            t[rb][r][nb] = fmaf(acc[rb][nb][r], c, -mc[rb][r]);
            if constexpr (decltype(masked)::value)
              if (kbase + 16 * nb + col > q0 + 16 * rb + 4 * grp + r) t[rb][r][nb] = -INFINITY;
            sum += fast_exp2(t[rb][r][nb]);
          }
          ls[rb][r] = sum;
          need |= !(sum < kRescale);
        }
      if (kt == 0 || __builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float tm = fmaxf(fmaxf(t[rb][r][0], t[rb][r][1]), fmaxf(t[rb][r][2], t[rb][r][3]));
            const bool fresh = l[rb][r] == 0.0f;
            float delta = fresh ? tm : fmaxf(tm, 0.0f);
            delta = delta > -INFINITY ? delta : 0.0f;  // no valid key in this lane yet
            mc[rb][r] += delta;
            float sum = fresh ? 0.0f : l[rb][r] * fast_exp2(-delta);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) sum += fast_exp2(t[rb][r][nb] - delta);
            l[rb][r] = sum;
          }
      } else {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) l[rb][r] = ls[rb][r];
      }
    };
    if (kbase + kLseKeys - 1 > q0)
      update(std::true_type{});
    else
      update(std::false_type{});
  }

  float* lrow = lse + (static_cast<size_t>(b) * Hq + h) * static_cast<size_t>(T);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool has = l[rb][r] > 0.0f;  // lanes that saw no valid key carry nothing
      const float M = max_adjacent<16>(has ? mc[rb][r] : -INFINITY);
      const float L = sum_adjacent<16>(has ? l[rb][r] * fast_exp2(mc[rb][r] - M) : 0.0f);
      const int row = q0 + 16 * rb + 4 * grp + r;
      if (col == 0 && row < T) lrow[row] = M + __builtin_amdgcn_logf(L);
    }
}

// ----------------------------------------------------- pass 2: column sums

template <int D>
__global__ __launch_bounds__(64 * kSumWaves) void rdkv_colsum_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k, int B,
                                                          int Hq, int Hkv, int T, float c,
                                                          const float* __restrict__ lse,
                                                          float* __restrict__ w) {
  constexpr int KS = D / 32, PAD = D + 8, CH = D / 8;
  constexpr int NT = 64 * kSumWaves;
  constexpr int LOADS = (kSumRows * CH + NT - 1) / NT;
  __shared__ __align__(16) _Float16 lds_q[kSumRows * PAD];
  __shared__ __align__(16) float lds_lse[kSumRows];

  const int G = Hq / Hkv;
  const int units = B * Hkv;
  const int u = blockIdx.x % units;
  const int kt = static_cast<int>(blockIdx.x / units);  // most rows first
  const int b = u / Hkv, kv = u % Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 15, grp = lane >> 4;
  const int k0 = kt * kSumKeys + wave * 16 * kSumNB;

  const uint16_t* kh = k + static_cast<size_t>(u) * T * D;
  half8 bk[kSumNB][KS];
#pragma unroll
  for (int nb = 0; nb < kSumNB; ++nb) {
    const int key = min(k0 + 16 * nb + col, T - 1);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bk[nb][s] = *reinterpret_cast<const half8*>(kh + static_cast<size_t>(key) * D + 32 * s + 8 * grp);
  }

  const int nqt = (T + kSumRows - 1) / kSumRows;
  const int qt_first = (kt * kSumKeys) / kSumRows;
  const int iters = (nqt - qt_first) * G;

  u32x4 pre[LOADS];
  float pre_lse = 0.0f;
  auto gload = [&](int i) {
    const int qt = nqt - 1 - i / G, h = kv * G + i % G;
    const size_t hb = (static_cast<size_t>(b) * Hq + h) * static_cast<size_t>(T);
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int cidx = min(tid + NT * j, kSumRows * CH - 1), r = cidx / CH, ch = cidx % CH;
      const int row = min(qt * kSumRows + r, T - 1);
      pre[j] = *reinterpret_cast<const u32x4*>(q + (hb + row) * D + ch * 8);
    }
    if (tid < kSumRows) pre_lse = lse[hb + min(qt * kSumRows + tid, T - 1)];
  };

  float cs[kSumNB];
#pragma unroll
  for (int nb = 0; nb < kSumNB; ++nb) cs[nb] = 0.0f;
  gload(0);
  for (int i = 0; i < iters; ++i) {
    const int r0 = (nqt - 1 - i / G) * kSumRows;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int cidx = tid + NT * j, r = cidx / CH, ch = cidx % CH;
      if (cidx < kSumRows * CH) *reinterpret_cast<u32x4*>(&lds_q[r * PAD + ch * 8]) = pre[j];
    }
    if (tid < kSumRows) lds_lse[tid] = pre_lse;
    __syncthreads();
    gload(min(i + 1, iters - 1));  // unconditional: keeps the prefetch in registers
    if (r0 + kSumRows - 1 < k0) continue;  // every row of the tile precedes the wave's keys

    float4v acc[kSumRB][kSumNB];
#pragma unroll
    for (int rb = 0; rb < kSumRB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < kSumNB; ++nb) acc[rb][nb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const half8 af = *reinterpret_cast<const half8*>(&lds_q[(16 * rb + col) * PAD + 32 * s + 8 * grp]);
#pragma unroll
        for (int nb = 0; nb < kSumNB; ++nb)
          acc[rb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bk[nb][s], acc[rb][nb], 0, 0, 0);
      }
    }
    auto accumulate = [&](auto masked) {
#pragma unroll
      for (int rb = 0; rb < kSumRB; ++rb) {
        const float4 ls = *reinterpret_cast<const float4*>(&lds_lse[16 * rb + 4 * grp]);
        const float lsr[4] = {ls.x, ls.y, ls.z, ls.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int nb = 0; nb < kSumNB; ++nb) {
            float p = fast_exp2(fmaf(acc[rb][nb][r], c, -lsr[r]));
            if constexpr (decltype(masked)::value) {
              const int row = r0 + 16 * rb + 4 * grp + r;
              if (k0 + 16 * nb + col > row || row >= T) p = 0.0f;
            }
            cs[nb] += p;
          }
        }
      }
    };
    if (r0 < k0 + 16 * kSumNB - 1 || r0 + kSumRows > T)  // a key after a row, or rows past the end
      accumulate(std::true_type{});
    else
      accumulate(std::false_type{});
  }

  float* wu = w + static_cast<size_t>(u) * T;
#pragma unroll
  for (int nb = 0; nb < kSumNB; ++nb) {
    const float v = swap_rows<false>(swap_rows<false>(cs[nb], true), false);
    const int key = k0 + 16 * nb + col;
    if (grp == 0 && key < T) wu[key] = v;
  }
}

// -------------------------------------------------------- channel weights

template <int D>
__global__ __launch_bounds__(256) void rdkv_chan_partial_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k,
                                                                const int8_t* __restrict__ keep,
                                                                int Hq, int Hkv, int T,
                                                                float* __restrict__ part) {
  constexpr int CH = D / 8, RP = 256 / CH;
  __shared__ float red[2][RP][D];
  const int chunk = blockIdx.x, u = blockIdx.y, units = gridDim.y;
  const int b = u / Hkv, kv = u % Hkv, G = Hq / Hkv;
  const int tid = threadIdx.x, c8 = tid % CH, rp = tid / CH;
  const int t0 = chunk * kChanRows, t1 = min(t0 + kChanRows, T);

  float sq[8], sk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sq[e] = sk[e] = 0.0f;
  // four rows' loads are issued before their products (accumulated in row
  // order, as one row at a time would)
  constexpr int kIn = 4;
  auto accum4 = [&](float (&acc)[8], const uint16_t* base, const int8_t* kp) {
    for (int t = t0 + rp; t < t1; t += kIn * RP) {
      uint4 v[kIn];
      bool use[kIn];
#pragma unroll
      for (int i = 0; i < kIn; ++i) {
        const int ti = min(t + i * RP, t1 - 1);           // in bounds; rows past t1 unused
        v[i] = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(ti) * D + c8 * 8);
        use[i] = t + i * RP < t1 && (kp == nullptr || kp[ti] != 0);
      }
#pragma unroll
      for (int i = 0; i < kIn; ++i) {
        if (!use[i]) continue;
        const unsigned wds[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = h2f(static_cast<uint16_t>(wds[e] & 0xFFFFu));
          const float hi = h2f(static_cast<uint16_t>(wds[e] >> 16));
          acc[2 * e] = fmaf(lo, lo, acc[2 * e]);
          acc[2 * e + 1] = fmaf(hi, hi, acc[2 * e + 1]);
        }
      }
    }
  };
  for (int g = 0; g < G; ++g)
    accum4(sq, q + (static_cast<size_t>(b) * Hq + kv * G + g) * static_cast<size_t>(T) * D, nullptr);
  accum4(sk, k + static_cast<size_t>(u) * T * D, keep + static_cast<size_t>(u) * T);

#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[0][rp][c8 * 8 + e] = sq[e];
    red[1][rp][c8 * 8 + e] = sk[e];
  }
  __syncthreads();
  if (tid < 2 * D) {
    const int which = tid / D, ch = tid % D;
    float s = 0.0f;
    for (int r = 0; r < RP; ++r) s += red[which][r][ch];
    part[(static_cast<size_t>(chunk) * units + u) * 2 * D + which * D + ch] = s;
  }
}

__global__ __launch_bounds__(128) void rdkv_chan_finish_kernel(const float* __restrict__ part, int chunks,
                                                               int units, int D, float* __restrict__ w) {
  const int u = blockIdx.x, ch = threadIdx.x;
  if (ch >= D) return;
  double sq = 0.0, sk = 0.0;
  for (int c0 = 0; c0 < chunks; c0 += 8) {   // eight chunks in flight, summed in chunk order
    float a[8], b[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float* p = part + (static_cast<size_t>(min(c0 + k, chunks - 1)) * units + u) * 2 * D;
      a[k] = p[ch];
      b[k] = p[D + ch];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (c0 + k < chunks) {
        sq += a[k];
        sk += b[k];
      }
  }
  w[static_cast<size_t>(u) * D + ch] = static_cast<float>(sqrt(sq) * sqrt(sk) / sqrt(static_cast<double>(D)));
}

// ------------------------------------------------------------- allocation

constexpr int kBins = 2048;        // histogram bins (11-bit digits)
constexpr int kAllocChunk = 4096;  // weights per histogram workgroup
constexpr int kPasses = 6;
constexpr int kShift[kPasses] = {52, 41, 30, 19, 8, 0};
constexpr int kBits[kPasses] = {11, 11, 11, 11, 11, 8};

struct AllocState {
  unsigned long long prefix;  // bit pattern of the multiplier found so far
  long long remaining;        // budget left below the mass above the prefix
  int done;                   // 1: the whole row fits at multiplier 0
  int pad[3];
};

__device__ __forceinline__ double weight_of(float x) { return x > 0.0f ? static_cast<double>(x) : 0.0; }

// i-th breakpoint of a unit of weight x, and the bits it separates
__device__ __forceinline__ double breakpoint(double x, int i) {
  return i == 0 ? x * 0.375 : i == 1 ? x * 0.09375 : i == 2 ? x * (15.0 / 1024.0) : x * (255.0 / 524288.0);
}
__device__ __forceinline__ int breakpoint_bits(int i) { return i < 2 ? 2 : i == 2 ? 4 : 8; }

__global__ void rdkv_alloc_init_kernel(AllocState* st, int rows, long long budget) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  AllocState s;
  s.prefix = 0ull;
  s.remaining = budget;
  s.done = 0;
  s.pad[0] = s.pad[1] = s.pad[2] = 0;
  st[r] = s;
}

__global__ __launch_bounds__(256) void rdkv_hist_kernel(const float* __restrict__ w, int n, int chunks,
                                                        const AllocState* __restrict__ st, int shift,
                                                        int bits, unsigned* __restrict__ hist) {
  __shared__ unsigned h[kBins];
  const int chunk = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const unsigned long long prefix = st[row].prefix;
  if (st[row].done) return;
  for (int i = tid; i < kBins; i += 256) h[i] = 0u;
  __syncthreads();
  const int top = shift + bits;
  const unsigned long long hi_mask = top >= 64 ? 0ull : ~((1ull << top) - 1ull);
  const unsigned dmask = (1u << bits) - 1u;
  const float* wr = w + static_cast<size_t>(row) * n;
  const int e1 = min(chunk * kAllocChunk + kAllocChunk, n);
  for (int e = chunk * kAllocChunk + tid; e < e1; e += 256) {
    const double x = weight_of(wr[e]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned long long key = __builtin_bit_cast(unsigned long long, breakpoint(x, i));
      if ((key & hi_mask) == prefix)
        atomicAdd(&h[static_cast<unsigned>(key >> shift) & dmask], static_cast<unsigned>(breakpoint_bits(i)));
    }
  }
  __syncthreads();
  unsigned* out = hist + (static_cast<size_t>(row) * chunks + chunk) * kBins;
  for (int i = tid; i < kBins; i += 256) out[i] = h[i];
}

constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void rdkv_select_kernel(const unsigned* __restrict__ hist,
                                                                     int chunks, AllocState* __restrict__ st,
                                                                     int shift, int bits, int first_pass) {
  __shared__ unsigned long long suf[kSelectThreads];
  const int row = blockIdx.x, tid = threadIdx.x;
  if (st[row].done) return;
  const unsigned long long prefix = st[row].prefix;
  const unsigned long long rem = static_cast<unsigned long long>(st[row].remaining);
  // thread t holds bins [per t, per t + per): 2 of 2048, or 1 of 256 for
  // t < 256; each bin summed over the chunks in chunk order
  const int nbins = 1 << bits;
  const int per = nbins >= kSelectThreads ? nbins / kSelectThreads : 1;
  const bool has = tid * per < nbins;
  unsigned long long bin[2] = {0, 0};
  unsigned long long t = 0;
  if (has) {
    for (int j = 0; j < per; ++j) {
      const unsigned* hp = hist + static_cast<size_t>(row) * chunks * kBins + tid * per + j;
      for (int c0 = 0; c0 < chunks; c0 += 8) {   // eight loads in flight, summed in chunk order
        unsigned v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = c0 + k < chunks ? hp[static_cast<size_t>(c0 + k) * kBins] : 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) bin[j] += v[k];
      }
      t += bin[j];
    }
  }
  // inclusive suffix sums over the threads (Hillis-Steele in LDS)
  suf[tid] = t;
  __syncthreads();
  for (int off = 1; off < kSelectThreads; off <<= 1) {
    const unsigned long long v = tid + off < kSelectThreads ? suf[tid + off] : 0ull;
    __syncthreads();
    suf[tid] += v;
    __syncthreads();
  }
  const unsigned long long total = suf[0];
  const unsigned long long above = suf[tid] - t;   // mass of the bins above this thread's
  if (first_pass && total <= rem) {
    if (tid == 0) st[row].done = 1;
    return;
  }
  // the thread whose bins hold the breakpoint where the mass counted from
  // the top first exceeds the remaining budget
  if (has && above <= rem && rem < above + t) {
    unsigned long long acc = above;
    for (int j = per - 1; j >= 0; --j) {
      if (acc + bin[j] > rem) {
        st[row].prefix = prefix | (static_cast<unsigned long long>(tid * per + j) << shift);
        st[row].remaining = static_cast<long long>(rem - acc);
        break;
      }
      acc += bin[j];
    }
  }
}

__global__ __launch_bounds__(256) void rdkv_widths_kernel(const float* __restrict__ w, int n,
                                                          const AllocState* __restrict__ st,
                                                          int8_t* __restrict__ out) {
  const int row = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const double lam = __builtin_bit_cast(double, st[row].prefix);
  const double x = weight_of(w[static_cast<size_t>(row) * n + e]);
  int b = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) b += lam < breakpoint(x, i) ? breakpoint_bits(i) : 0;
  out[static_cast<size_t>(row) * n + e] = static_cast<int8_t>(b);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t alloc_ws(int rows, int n) {
  const size_t chunks = (static_cast<size_t>(n) + kAllocChunk - 1) / kAllocChunk;
  return align256(static_cast<size_t>(rows) * sizeof(AllocState)) +
         static_cast<size_t>(rows) * chunks * kBins * sizeof(unsigned);
}

int alloc_run(const float* w, int rows, int n, long long budget, int8_t* widths, void* ws, hipStream_t s) {
  AllocState* st = static_cast<AllocState*>(ws);
  unsigned* hist = reinterpret_cast<unsigned*>(static_cast<char*>(ws) +
                                               align256(static_cast<size_t>(rows) * sizeof(AllocState)));
  const int chunks = static_cast<int>((static_cast<size_t>(n) + kAllocChunk - 1) / kAllocChunk);
  hipLaunchKernelGGL(rdkv_alloc_init_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, st, rows, budget);
  DQA_CHECK_LAUNCH();
  for (int p = 0; p < kPasses; ++p) {
    hipLaunchKernelGGL(rdkv_hist_kernel, dim3(chunks, rows), dim3(256), 0, s, w, n, chunks, st, kShift[p],
                       kBits[p], hist);
    DQA_CHECK_LAUNCH();
    hipLaunchKernelGGL(rdkv_select_kernel, dim3(rows), dim3(kSelectThreads), 0, s, hist, chunks, st, kShift[p],
                       kBits[p], p == 0 ? 1 : 0);
    DQA_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(rdkv_widths_kernel, dim3((n + 255) / 256, rows), dim3(256), 0, s, w, n, st, widths);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}


int check_heads(int B, int Hq, int Hkv, int T, int d) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || T < 0 || Hq % Hkv != 0) return DQA_ERR_SHAPE;
  if (B > 65535 || Hq > 65535 || static_cast<size_t>(B) * Hkv > 65535) return DQA_ERR_SHAPE;
  if (d != 64 && d != 128) return DQA_ERR_UNSUPPORTED;
  const size_t heads = static_cast<size_t>(B) * Hq;
  if (heads * ((static_cast<size_t>(T) + kLseRows - 1) / kLseRows) > 0x7FFFFFFFull) return DQA_ERR_SHAPE;
  if (static_cast<size_t>(B) * Hkv * ((static_cast<size_t>(T) + kSumKeys - 1) / kSumKeys) > 0x7FFFFFFFull)
    return DQA_ERR_SHAPE;
  return DQA_OK;
}

template <int D>
void launch_token(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv, int T, float c, float* lse,
                  float* w, hipStream_t s) {
  const unsigned g1 = static_cast<unsigned>(static_cast<size_t>(B) * Hq * ((T + kLseRows - 1) / kLseRows));
  hipLaunchKernelGGL(rdkv_lse_kernel<D>, dim3(g1), dim3(256), 0, s, q, k, B, Hq, Hkv, T, c, lse);
  const unsigned g2 = static_cast<unsigned>(static_cast<size_t>(B) * Hkv * ((T + kSumKeys - 1) / kSumKeys));
  hipLaunchKernelGGL(rdkv_colsum_kernel<D>, dim3(g2), dim3(64 * kSumWaves), 0, s, q, k, B, Hq, Hkv, T, c, lse, w);
}

template <int D>
void launch_chan(const uint16_t* q, const uint16_t* k, const int8_t* keep, int B, int Hq, int Hkv, int T,
                 float* part, float* w, hipStream_t s) {
  const int chunks = (T + kChanRows - 1) / kChanRows;
  if (chunks > 0)
    hipLaunchKernelGGL(rdkv_chan_partial_kernel<D>, dim3(chunks, B * Hkv), dim3(256), 0, s, q, k, keep, Hq, Hkv,
                       T, part);
  hipLaunchKernelGGL(rdkv_chan_finish_kernel, dim3(B * Hkv), dim3(128), 0, s, part, chunks, B * Hkv, D, w);
}

size_t lse_bytes(int B, int Hq, int T) { return align256(static_cast<size_t>(B) * Hq * T * sizeof(float)); }
size_t chan_bytes(int B, int Hkv, int T, int d) {
  return align256(static_cast<size_t>((T + kChanRows - 1) / kChanRows) * B * Hkv * 2 * d * sizeof(float));
}

int token_weights(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv, int T, int d, float sm_scale,
                  float* w, float* lse, hipStream_t s) {
  const float c = sm_scale * kLog2e;
  if (d == 64)
    launch_token<64>(q, k, B, Hq, Hkv, T, c, lse, w, s);
  else
    launch_token<128>(q, k, B, Hq, Hkv, T, c, lse, w, s);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

int channel_weights(const uint16_t* q, const uint16_t* k, const int8_t* keep, int B, int Hq, int Hkv, int T,
                    int d, float* w, float* part, hipStream_t s) {
  if (d == 64)
    launch_chan<64>(q, k, keep, B, Hq, Hkv, T, part, w, s);
  else
    launch_chan<128>(q, k, keep, B, Hq, Hkv, T, part, w, s);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

bool scale_ok(float sm_scale) { return sm_scale > 0.0f && sm_scale < 3.0e38f; }

}  // namespace
}  // namespace dqa

using namespace dqa;

extern "C" size_t rdkv_token_weights_workspace_bytes(int B, int Hq, int T) {
  if (B < 0 || Hq < 0 || T < 0) return 0;
  return lse_bytes(B, Hq, T);
}

extern "C" int rdkv_token_weights(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv, int T, int d,
                                  float sm_scale, float* w, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_heads(B, Hq, Hkv, T, d);
  if (st != DQA_OK) return st;
  if (!scale_ok(sm_scale)) return DQA_ERR_SHAPE;
  if (B == 0 || T == 0) return DQA_OK;
  if (!q || !k || !w) return DQA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k)) return DQA_ERR_ALIGN;
  if (!ws || ws_bytes < lse_bytes(B, Hq, T)) return DQA_ERR_WORKSPACE;
  return token_weights(q, k, B, Hq, Hkv, T, d, sm_scale, w, static_cast<float*>(ws),
                       static_cast<hipStream_t>(stream));
}

extern "C" size_t rdkv_channel_weights_workspace_bytes(int B, int Hkv, int T, int d) {
  if (B < 0 || Hkv < 0 || T < 0 || (d != 64 && d != 128)) return 0;
  return chan_bytes(B, Hkv, T, d);
}

extern "C" int rdkv_channel_weights(const uint16_t* q, const uint16_t* k, const int8_t* keep, int B, int Hq,
                                    int Hkv, int T, int d, float* w, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_heads(B, Hq, Hkv, T, d);
  if (st != DQA_OK) return st;
  if (B == 0) return DQA_OK;
  if (!w || (T > 0 && (!q || !k || !keep))) return DQA_ERR_NULL;
  if (T > 0 && (!aligned16(q) || !aligned16(k))) return DQA_ERR_ALIGN;
  const size_t need = chan_bytes(B, Hkv, T, d);
  if (need > 0 && (!ws || ws_bytes < need)) return DQA_ERR_WORKSPACE;
  return channel_weights(q, k, keep, B, Hq, Hkv, T, d, w, static_cast<float*>(ws),
                         static_cast<hipStream_t>(stream));
}

extern "C" size_t rdkv_allocate_workspace_bytes(int rows, int n) {
  if (rows < 0 || n < 0) return 0;
  return alloc_ws(rows, n);
}

extern "C" int rdkv_allocate(const float* w, int rows, int n, long long budget, int8_t* widths, void* ws,
                             size_t ws_bytes, void* stream) {
  if (rows < 0 || n < 0 || budget < 0 || rows > 65535) return DQA_ERR_SHAPE;
  if (rows == 0 || n == 0) return DQA_OK;
  if (!w || !widths) return DQA_ERR_NULL;
  if (!ws || ws_bytes < alloc_ws(rows, n)) return DQA_ERR_WORKSPACE;
  return alloc_run(w, rows, n, budget, widths, ws, static_cast<hipStream_t>(stream));
}

namespace {
struct WidthsLayout {
  size_t lse, w_tok, w_ch, scratch, total;
};
WidthsLayout widths_layout(int B, int Hq, int Hkv, int T, int d) {
  WidthsLayout L;
  L.lse = 0;
  L.w_tok = L.lse + lse_bytes(B, Hq, T);
  L.w_ch = L.w_tok + align256(static_cast<size_t>(B) * Hkv * T * sizeof(float));
  L.scratch = L.w_ch + align256(static_cast<size_t>(B) * Hkv * d * sizeof(float));
  size_t s = chan_bytes(B, Hkv, T, d);
  s = s > alloc_ws(B, Hkv * T) ? s : alloc_ws(B, Hkv * T);
  s = s > alloc_ws(B, Hkv * d) ? s : alloc_ws(B, Hkv * d);
  L.total = L.scratch + align256(s);
  return L;
}
}  // namespace

extern "C" size_t rdkv_widths_workspace_bytes(int B, int Hq, int Hkv, int T, int d) {
  if (check_heads(B, Hq, Hkv, T, d) != DQA_OK) return 0;
  if (static_cast<size_t>(Hkv) * T > 0x7FFFFFFFull) return 0;
  return widths_layout(B, Hq, Hkv, T, d).total;
}

extern "C" int rdkv_widths(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv, int T, int d,
                           float sm_scale, long long v_budget, long long k_budget, int8_t* v_bits,
                           int8_t* k_bits, void* ws, size_t ws_bytes, void* stream) {
  const int st = check_heads(B, Hq, Hkv, T, d);
  if (st != DQA_OK) return st;
  if (!scale_ok(sm_scale) || v_budget < 0 || k_budget < 0) return DQA_ERR_SHAPE;
  if (static_cast<size_t>(Hkv) * T > 0x7FFFFFFFull) return DQA_ERR_SHAPE;
  if (B == 0) return DQA_OK;
  if (!k_bits || (T > 0 && (!q || !k || !v_bits))) return DQA_ERR_NULL;
  if (T > 0 && (!aligned16(q) || !aligned16(k))) return DQA_ERR_ALIGN;
  const WidthsLayout L = widths_layout(B, Hq, Hkv, T, d);
  if (!ws || ws_bytes < L.total) return DQA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* lse = reinterpret_cast<float*>(base + L.lse);
  float* w_tok = reinterpret_cast<float*>(base + L.w_tok);
  float* w_ch = reinterpret_cast<float*>(base + L.w_ch);
  void* scratch = base + L.scratch;
  int r;
  if (T > 0) {
    // phase 1 (token weights) and phase 2: one problem per sequence over
    // all its KV heads' tokens
    if ((r = token_weights(q, k, B, Hq, Hkv, T, d, sm_scale, w_tok, lse, s)) != DQA_OK) return r;
    if ((r = alloc_run(w_tok, B, Hkv * T, v_budget, v_bits, scratch, s)) != DQA_OK) return r;
  }
  // phase 1 (channel weights over the kept tokens) and phase 3
  if ((r = channel_weights(q, k, v_bits, B, Hq, Hkv, T, d, w_ch, static_cast<float*>(scratch), s)) != DQA_OK)
    return r;
  return alloc_run(w_ch, B, Hkv * d, k_budget, k_bits, scratch, s);
}
