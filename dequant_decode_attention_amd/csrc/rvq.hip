// Residual vector quantization: nearest-codeword encoder on the matrix cores,
// and decode attention that rebuilds keys/values from their indices.
//
// [P2 sec 2, key components]: a cache vector is matched to the nearest entry
// of a codebook, the residual (vector minus that entry) goes to the next
// codebook, N times; only the N indices are kept (prefill phase); at decode
// time the vectors are rebuilt on demand inside attention.  [P2 sec 2,
// computational optimization]: quantization is parallelized over blocks of
// cache vectors.
//
// Encoder (the one dense contraction of the path): for a block of 256
// vectors and one stage, the keys |c|^2 - 2 r.c of all Kc codewords are a
// [256 x 128] x [128 x Kc] product.  It runs on v_mfma_f32_16x16x32_f16:
// the residual r (fp32) is split as -2r = hi + lo with hi = fp16(-2r) and
// lo = fp16(-2r - hi) (exact products with fp16 codewords, fp32
// accumulation; stage 0 has lo = 0 exactly and skips it), the accumulator
// starts at |c|^2.  Codebook tiles of 64 codewords are staged in LDS, double
// buffered, shared by the 8 waves of the workgroup.  Each lane keeps a
// running (key, index) minimum for its output rows (strict < over
// increasing codeword index, then a lexicographic cross-lane reduction), so
// exact ties go to the lowest index.  The fp32 residual is rebuilt in the
// MFMA A-operand layout at the start of each stage.
#include "common.h"
#include "merge.h"

#include <type_traits>

namespace dqa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kEncMB = 2;            // MFMA row blocks (16 vectors each) per wave
constexpr int kEncWaves = 8;         // waves per workgroup
constexpr int kEncRows = 16 * kEncMB * kEncWaves;   // vectors per workgroup
constexpr int kTileCW = 64;          // codewords per LDS tile
constexpr int kRowPad = kD + 8;      // LDS row stride in halves (bank spread)
constexpr int kMaxStages = 8;        // codebooks per vector at most

__global__ __launch_bounds__(256) void rvq_norms_kernel(const uint16_t* __restrict__ cb, size_t n_cw,
                                                        float* __restrict__ norms) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_cw) return;
  const uint16_t* c = cb + i * kD;
  float s = 0.0f;
  for (int k = 0; k < kD; ++k) {
    const float v = h2f(c[k]);
    s = fmaf(v, v, s);
  }
  norms[i] = s;
}

__device__ __forceinline__ void split_neg2(const float* r, half8& hi, half8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float t = -2.0f * r[j];
    const _Float16 h = static_cast<_Float16>(t);
    hi[j] = h;
    lo[j] = static_cast<_Float16>(t - static_cast<float>(h));
  }
}

template <int MB, int NW>
__global__ __launch_bounds__(NW * 64) void rvq_encode_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                         const uint16_t* __restrict__ cbs,
                                                         const float* __restrict__ norms, int N,
                                                         int Kc, int16_t* __restrict__ idx_out) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_cb[2][kTileCW][kRowPad];
  constexpr int RW = 16 * MB;          // vectors per wave
  constexpr int NT = NW * 64;          // threads
  constexpr int CPT = kTileCW * kD / 8 / NT;   // 16-byte chunks of a codeword tile per thread
  static_assert(CPT * NT == kTileCW * kD / 8, "a tile's chunks split evenly over the threads");
  __shared__ int16_t lds_idx[NW][kMaxStages][RW];   // chosen indices, per stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * (NW * RW) + wave * RW;

  // The residual of stage s is rebuilt at the start of the stage from x and
  // the codewords chosen at stages 0..s-1, subtracted in stage order -- the
  // same fp32 operations, in the same order, as one running update -- so it
  // holds no registers while the codeword tiles stream through.  Layout is
  // the MFMA A operand's: row = row_base + 16*mb + col, channels
  // 32*ks + 8*grp + 0..7.
  const int n_tiles = Kc / kTileCW;
  for (int s = 0; s < N; ++s) {
    const uint16_t* cb = cbs + static_cast<size_t>(s) * Kc * kD;
    const float* nrm = norms + static_cast<size_t>(s) * Kc;
    half8 ahi[MB][4], alo[MB][4];
    {
      // all of a stage's loads of x (or of one earlier stage's codewords)
      // are issued together: one memory round trip per earlier stage
      float r[MB][4][8];
      auto add_chunks = [&](const uint16_t* const (&rows)[MB], bool subtract) {
        uint4 u[MB][4];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) u[mb][ks] = *reinterpret_cast<const uint4*>(rows[mb] + 32 * ks + 8 * grp);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const uint32_t w[4] = {u[mb][ks].x, u[mb][ks].y, u[mb][ks].z, u[mb][ks].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float c = h2f(static_cast<uint16_t>(j & 1 ? w[j >> 1] >> 16 : w[j >> 1] & 0xFFFFu));
              r[mb][ks][j] = subtract ? r[mb][ks][j] - c : c;
            }
          }
      };
      // rows past the end of x read row 0 and are zeroed (their indices are
      // never stored)
      bool valid[MB];
      const uint16_t* xr[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        valid[mb] = row_base + 16 * mb + col < n;
        xr[mb] = x + (valid[mb] ? row_base + 16 * mb + col : 0) * kD;
      }
      add_chunks(xr, false);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        if (!valid[mb])
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) r[mb][ks][j] = 0.0f;
      for (int sp = 0; sp < s; ++sp) {
        const uint16_t* cbp = cbs + static_cast<size_t>(sp) * Kc * kD;
        const uint16_t* cr[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) cr[mb] = cbp + static_cast<size_t>(lds_idx[wave][sp][16 * mb + col]) * kD;
        add_chunks(cr, true);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) split_neg2(r[mb][ks], ahi[mb][ks], alo[mb][ks]);
    }
    float bestk[MB][4];
    int besti[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bestk[mb][r] = INFINITY;
        besti[mb][r] = 0;
      }

    // codeword tiles: thread tid moves 16-byte chunks tid, tid + NT, ... of
    // a 64-codeword tile (global -> registers -> LDS buffer; consecutive
    // threads store consecutive chunks, free of bank conflicts); the
    // tile after next is in flight while the current tile is consumed.  The
    // norms |c|^2 of the lane's 4 codeword columns come straight from global
    // memory, one tile ahead.
    auto gchunks = [&](int t, uint4 (&u)[CPT]) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c = tid + NT * k;
        u[k] = *reinterpret_cast<const uint4*>(cb + (static_cast<size_t>(t) * kTileCW + c / 16) * kD + (c % 16) * 8);
      }
    };
    auto lstore = [&](int buf, const uint4 (&u)[CPT]) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c = tid + NT * k;
        *reinterpret_cast<uint4*>(&lds_cb[buf][c / 16][(c % 16) * 8]) = u[k];
      }
    };
    auto gnorms = [&](int t, float (&nv)[4]) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) nv[nb] = nrm[t * kTileCW + 16 * nb + col];
    };
    {
      uint4 u[CPT];
      gchunks(0, u);
      lstore(0, u);
    }
    __syncthreads();
    // A codeword tile is consumed in two halves of 32 codewords (4 output
    // blocks: 2 row blocks x 2 codeword blocks).  Keys are |c|^2 - 2 r.c,
    // the accumulator starting at |c|^2.  The running minimum of one half
    // (plain VALU) sits beside the matrix-core products of the next half in
    // one straight-line block, so the two overlap; each half's codeword
    // fragments are read from LDS one half ahead; one barrier per tile
    // guards the double-buffered LDS tile.
    // Stage 0 (exact fp16 residual) has no low part.
    auto read_half = [&](half8 (&bf)[2][4], int buf, int h) {
#pragma unroll
      for (int nh = 0; nh < 2; ++nh)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          bf[nh][ks] = *reinterpret_cast<const half8*>(&lds_cb[buf][16 * (2 * h + nh) + col][32 * ks + 8 * grp]);
    };
    auto init_acc = [&](float4v (&acc)[MB][2], const float (&nv)[4], int h) {
#pragma unroll
      for (int nh = 0; nh < 2; ++nh)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float v = nv[2 * h + nh];
          acc[mb][nh] = float4v{v, v, v, v};
        }
    };
    auto products = [&](float4v (&acc)[MB][2], const half8 (&bf)[2][4], auto lo_tag) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int nh = 0; nh < 2; ++nh)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[mb][nh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[mb][ks], bf[nh][ks], acc[mb][nh], 0, 0, 0);
        if constexpr (decltype(lo_tag)::value) {
#pragma unroll
          for (int nh = 0; nh < 2; ++nh)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
              acc[mb][nh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[mb][ks], bf[nh][ks], acc[mb][nh], 0, 0, 0);
        }
      }
    };
    // codewords visited in increasing index order per (row, lane): strict <
    // keeps the lowest index of equal keys
    auto running_min = [&](const float4v (&acc)[MB][2], int cw0) {
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {
        const int cw = cw0 + 16 * nh + col;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float key = acc[mb][nh][r];
            const bool better = key < bestk[mb][r];
            besti[mb][r] = better ? cw : besti[mb][r];
            bestk[mb][r] = better ? key : bestk[mb][r];
          }
      }
    };
    auto tiles = [&](auto lo_tag) {
      half8 bf0[2][4], bf1[2][4];
      float4v acc0[MB][2], acc1[MB][2];
      float nv[4];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) acc1[mb][nh] = float4v{INFINITY, INFINITY, INFINITY, INFINITY};
      gnorms(0, nv);
      uint4 u[CPT];
      gchunks(min(1, n_tiles - 1), u);
      read_half(bf0, 0, 0);
      for (int t = 0; t < n_tiles; ++t) {
        const int buf = t & 1;
        const int tn = min(t + 1, n_tiles - 1), t2 = min(t + 2, n_tiles - 1);
        read_half(bf1, buf, 1);
        init_acc(acc0, nv, 0);
        products(acc0, bf0, lo_tag);
        // before tile 0, acc1 holds +inf: no update
        running_min(acc1, (t - 1) * kTileCW + 32);
        lstore(buf ^ 1, u);                        // tile t+1 (the final tile rewrites a dead buffer)
        gchunks(t2, u);
        init_acc(acc1, nv, 1);
        gnorms(tn, nv);
        products(acc1, bf1, lo_tag);
        running_min(acc0, t * kTileCW);
        __syncthreads();
        if (t + 1 < n_tiles) read_half(bf0, buf ^ 1, 0);
      }
      running_min(acc1, (n_tiles - 1) * kTileCW + 32);
    };
    if (s == 0) tiles(std::false_type{});
    else tiles(std::true_type{});

    // lexicographic (key, index) minimum across the 16 lanes of a row group
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float k = bestk[mb][r];
        int i = besti[mb][r];
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
          const float ko = __shfl_xor(k, m, 64);
          const int io = __shfl_xor(i, m, 64);
          if (ko < k || (ko == k && io < i)) {
            k = ko;
            i = io;
          }
        }
        besti[mb][r] = i;
      }
    if (col == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) lds_idx[wave][s][16 * mb + 4 * grp + r] = static_cast<int16_t>(besti[mb][r]);
    }
    // the next stage (and the final store) read this stage's indices from
    // LDS (same wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // lane l < RW stores the N indices of row row_base + l
  if (lane < RW && row_base + lane < n) {
    int16_t* dst = idx_out + (row_base + lane) * N;
    for (int s = 0; s < N; ++s) dst[s] = lds_idx[wave][s][lane];
  }
}

// ------------------------------------------------------------------ decode

constexpr int kDecWaves = 8;     // one workgroup per compute unit, two waves per SIMD
// Key logits through a table: q . k_hat = sum_s q . Ck_s[k_idx[s]], so a
// table T[h][s][c] = q_h . Ck_s[c] (scaled into the log2 domain) turns each
// key logit into N lookups instead of N gathered codewords.  Used when the
// table of one (batch, KV head) fits this many floats of LDS.
constexpr int kLutFloats = 16384;   // 64 KB
constexpr int kLutWorkgroups = 256; // table-path workgroups resident at once (one per compute unit)
// polls of a unit's table flags before a workgroup builds the whole table
// itself (the pieces come from workgroups that do not wait for anything, so
// this bound is only reached when they cannot all be resident)
constexpr int kTablePolls = 1 << 18;
// per-(batch, KV head) synchronization words: the call epoch, a table-piece
// flag per split, the merge counter
constexpr int kSyncWords = 2 + kMaxSplitsMerge;

// floats between the tables of consecutive units (16-byte aligned rows)
__host__ __device__ inline int lut_stride(int G, int N, int Kc) { return (G * N * Kc + 63) / 64 * 64; }

struct RvqDecArgs {
  const uint16_t* q;
  const int16_t* k_idx;
  const int16_t* v_idx;
  const uint16_t* k_cb;
  const uint16_t* v_cb;
  float* out;
  float* partials;      // [units][splits][G][D + 2] partial softmax states
  float* lut;           // [units][G][N][Kc] key-logit tables (table path only)
  uint32_t* sync;       // [units][kSyncWords]
  int Hq, Hkv, T, N, Kc, n_tiles, tiles_per_split, splits;
  int vidx_words;       // N == 4 and v_idx 8-byte aligned: a token's value indices are two words
  int table_polls;      // polls of the table flags before building the table alone
  float q_scale;
};

// polls of the table flags per workgroup (rvq_decode_set_table_polls)
int g_table_polls = kTablePolls;

// One 16-codeword tile of a unit's key-logit table on the matrix cores:
// codewords [base, base + 16) of the unit's N * Kc (A operand rows, exact
// fp16) against the fp16 query of its G heads (qb: B operand columns, exact;
// columns >= G are zero), fp32 accumulation over the 128 channels.  Lane l
// gets codewords base + 4 (l >> 4) + r, r < 4, for head l & 15.
__device__ __forceinline__ float4v table_tile(const uint16_t* k_cb, const half8 (&qb)[4], int base, int n_cw,
                                              int lane) {
  const int col = lane & 15, grp = lane >> 4;
  const uint16_t* row = k_cb + static_cast<size_t>(min(base + col, n_cw - 1)) * kD + 8 * grp;
  half8 av[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) av[ks] = *reinterpret_cast<const half8*>(row + 32 * ks);
  float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[ks], qb[ks], acc, 0, 0, 0);
  return acc;
}

// The lane's 16 channels: [8 ck, 8 ck + 8) and [64 + 8 ck, 64 + 8 ck + 8),
// so that the 8 lanes of a token read whole 128-byte halves of a codeword
// row with one instruction.
__device__ __forceinline__ int lane_channel(int ck, int c) { return c < 8 ? 8 * ck + c : 64 + 8 * ck + (c - 8); }

// Add one codeword row's 16 channels (as loaded: two 16-byte pieces) to the
// lane's fp32 sums: h * 1 + x is one mixed-precision FMA with the rounding of
// h + x.
__device__ __forceinline__ void add_row16(const uint4& ra, const uint4& rb, float* out) {
  const float one = opaque_const(1.0f);
  const uint32_t w[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[2 * i] = __builtin_fmaf(half_of<0>(w[i]), one, out[2 * i]);
    out[2 * i + 1] = __builtin_fmaf(half_of<1>(w[i]), one, out[2 * i + 1]);
  }
}

// Sum over stages of the lane's 16 channels of the indexed codewords (fp32,
// stage order).  The rows of up to four stages are requested before any is
// summed, so a token costs one memory round trip per four stages.
__device__ __forceinline__ void rebuild16(const uint16_t* cb, const int16_t* idx, int N, int Kc,
                                          int ck, float* out) {
#pragma unroll
  for (int c = 0; c < 16; ++c) out[c] = 0.0f;
  for (int s0 = 0; s0 < N; s0 += 4) {
    uint4 ra[4], rb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // indices are in [0, Kc) when produced by rvq_encode; clamp so that a
      // corrupt index cannot read outside the codebook (stages past N read
      // row 0 of the last stage and are not summed)
      const int s = min(s0 + k, N - 1);
      const uint32_t ci = min(static_cast<uint32_t>(static_cast<uint16_t>(idx[s])), static_cast<uint32_t>(Kc - 1));
      const uint4* row = reinterpret_cast<const uint4*>(cb + (static_cast<size_t>(s) * Kc + ci) * kD);
      ra[k] = row[ck];
      rb[k] = row[8 + ck];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (s0 + k >= N) break;
      add_row16(ra[k], rb[k], out);
    }
  }
}

// Lane = (token j of 8, channel chunk ck of 8); 32-token tiles of four
// 8-token sub-tiles; online softmax per tile; each split writes its partial
// state, and the last split of a (batch, KV head) to finish merges them in
// split order (merge.h).
//
// With at most four stages the value codeword rows of RB sub-tiles are in
// flight at any time (all four of a tile when the registers allow it): a
// ring that runs on across tiles, each slot refilled as soon as it has been
// summed.  The value indices that address the ring are loaded two tiles
// ahead (four 16-bit indices in two words per sub-tile), the key indices
// one tile ahead; the first tile's rows are requested while the table is
// staged.
template <int G, bool LUT, bool VPRE>
__global__ __launch_bounds__(64 * kDecWaves) void rvq_decode_kernel(RvqDecArgs a) {
  constexpr int NCK = 8, TL = 8, IT = 4;
  constexpr int RB = (LUT && G <= 3) ? 4 : 2;
  static_assert(IT % RB == 0, "ring slots map onto fixed sub-tiles");
  __shared__ float lds_m[kDecWaves][G], lds_l[kDecWaves][G];
  __shared__ __attribute__((aligned(16))) float lds_o[kDecWaves][G][kD];
  __shared__ __attribute__((aligned(16))) float lds_lut[LUT ? kLutFloats : 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane / NCK, ck = lane % NCK;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * a.Hkv + kvh;
  const int tb = split * a.tiles_per_split;
  const int te = min(a.n_tiles, tb + a.tiles_per_split);
  constexpr bool vpre = VPRE;   // N <= 4: the value rows through the ring
  // index words of tile ti for this lane, per sub-tile; positions past T
  // read the last token (in bounds)
  auto load_kidx = [&](int ti, uint32_t (&kc)[IT]) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = min(ti * kGroup + it * TL + j, a.T - 1);
      kc[it] = static_cast<uint16_t>(a.k_idx[(unit * a.T + t) * a.N + min(ck, a.N - 1)]);
    }
  };
  auto load_vidx = [&](int ti, uint32_t (&vp)[IT][2]) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = min(ti * kGroup + it * TL + j, a.T - 1);
      const int16_t* vix = a.v_idx + (unit * a.T + t) * a.N;
      if (a.vidx_words) {   // four stages, 8-byte aligned rows
        const uint2 w = *reinterpret_cast<const uint2*>(vix);
        vp[it][0] = w.x;
        vp[it][1] = w.y;
      } else {
        uint32_t e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e[k] = static_cast<uint16_t>(vix[min(k, a.N - 1)]);
        vp[it][0] = e[0] | (e[1] << 16);
        vp[it][1] = e[2] | (e[3] << 16);
      }
    }
  };
  // the 4 stages' codeword rows (the lane's 16 channels) of one sub-tile;
  // stages past N re-read the last stage and are not summed
  // (32-bit byte offsets from the codebook base: at most 8 x 32768 rows of
  // 256 bytes)
  const char* const vcb = reinterpret_cast<const char*>(a.v_cb);
  auto issue = [&](const uint32_t (&vp)[2], uint4 (&r)[4][2]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t st = static_cast<uint32_t>(min(k, a.N - 1));
      const uint32_t ci = min((vp[k >> 1] >> (16 * (k & 1))) & 0xFFFFu, static_cast<uint32_t>(a.Kc - 1));
      const uint32_t off = (st * static_cast<uint32_t>(a.Kc) + ci) * (kD * 2) + 16 * ck;
      r[k][0] = *reinterpret_cast<const uint4*>(vcb + off);
      r[k][1] = *reinterpret_cast<const uint4*>(vcb + off + 128);
    }
  };
  // this call's epoch: one more than the previous call's (flags of this
  // call that equal it are set)
  uint32_t* const sync = a.sync + unit * kSyncWords;
  const uint32_t epoch = __hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
  uint32_t kc[IT] = {}, vcur[IT][2] = {}, vnx[IT][2] = {}, vnn[IT][2] = {};
  uint4 rows[RB][4][2];
  const int t0 = tb + wave;
  if (t0 < te) {
    if (LUT) load_kidx(t0, kc);
    if (vpre) load_vidx(t0, vcur);
  }
  if (vpre && t0 + kDecWaves < te) load_vidx(t0 + kDecWaves, vnx);
  auto issue_first = [&]() {
    if (vpre && t0 < te) {
#pragma unroll
      for (int s = 0; s < RB; ++s) issue(vcur[s], rows[s]);
    }
  };
  if constexpr (LUT) {
    // ---- the unit's key-logit table, built by the unit's workgroups
    // together: split p writes tiles [p per, (p + 1) per) of the N * Kc
    // codewords (device-scope write-through stores), then sets its table
    // flag to the epoch; each workgroup then waits for every split's flag
    // and stages the table into LDS with device-scope loads.  A workgroup
    // never waits before its own flag is set, so the wait ends once the
    // unit's workgroups have started; should it not end within table_polls
    // polls (workgroups of the unit not resident together), the workgroup
    // builds the whole table itself.
    const int n_cw = a.N * a.Kc;
    const int n16 = (n_cw + 15) / 16;
    float* const tab = a.lut + unit * static_cast<size_t>(lut_stride(G, a.N, a.Kc));
    const int col = lane & 15, grp = lane >> 4;
    half8 qb[4];
    {
      const uint16_t* qh = a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + min(col, G - 1)) * kD + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qb[ks] = col < G ? *reinterpret_cast<const half8*>(qh + 32 * ks) : half8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    {
      const int per = (n16 + a.splits - 1) / a.splits;
      const int p0 = split * per, p1 = min(n16, p0 + per);
      // two tiles per wave at a time, both tiles' operands in flight
      for (int t = p0 + wave; t < p1; t += 2 * kDecWaves) {
        float4v r4[2];
        r4[0] = table_tile(a.k_cb, qb, 16 * t, n_cw, lane);
        r4[1] = table_tile(a.k_cb, qb, 16 * min(t + kDecWaves, p1 - 1), n_cw, lane);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int tu = t + u * kDecWaves;
          if (col < G && tu < p1) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int e = 16 * tu + 4 * grp + r;
              if (e < n_cw)
                __hip_atomic_store(tab + col * n_cw + e, r4[u][r] * a.q_scale, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      // the piece's stores (device-scope, write-through) have completed
      // before its flag is set, as the partial states before the merge
      // counter: a device-scope release fence (an L2 write-back) here cost
      // 4.7 us per step
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_store(sync + 1 + split, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the first tile's value rows are requested while the flags are polled
    // and the table is staged (with a shared counter in place of the flags,
    // these gathers held back the neighbouring workgroup's counter update)
    issue_first();
    __shared__ int s_table;
    if (wave == 0) {
      bool done = false;
      for (int n = 0; n < a.table_polls; ++n) {
        bool missing = false;
#pragma unroll
        for (int k = 0; k < kMaxSplitsMerge / 64; ++k) {
          const int i = lane + 64 * k;
          if (i < a.splits)
            missing |= __hip_atomic_load(sync + 1 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch;
        }
        done = __builtin_amdgcn_ballot_w64(missing) == 0;
        if (done) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane == 0) s_table = done;
    }
    __syncthreads();
    if (s_table) {
      // at most kLutFloats / 2 8-byte words: 16 per thread, all in flight
      constexpr int kWords = kLutFloats / 2 / (64 * kDecWaves);
      const int n8 = lut_stride(G, a.N, a.Kc) / 2;
      const uint64_t* src = reinterpret_cast<const uint64_t*>(tab);
      uint64_t* dst = reinterpret_cast<uint64_t*>(lds_lut);
      uint64_t w[kWords];
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const int i = 64 * kDecWaves * k + static_cast<int>(threadIdx.x);
        w[k] = i < n8 ? __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
      }
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        const int i = 64 * kDecWaves * k + static_cast<int>(threadIdx.x);
        if (i < n8) dst[i] = w[k];
      }
    } else {
      for (int t = wave; t < n16; t += kDecWaves) {
        const float4v r4 = table_tile(a.k_cb, qb, 16 * t, n_cw, lane);
        if (col < G) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 16 * t + 4 * grp + r;
            if (e < n_cw) lds_lut[col * n_cw + e] = r4[r] * a.q_scale;
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (!LUT) issue_first();
  float qr[G][16];
  if constexpr (!LUT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint16_t* qp = a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + h) * kD;
#pragma unroll
      for (int c = 0; c < 16; ++c) qr[h][c] = h2f(qp[lane_channel(ck, c)]) * a.q_scale;
    }
  }
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[h][c] = 0.0f;
  }
  for (int ti = t0; ti < te; ti += kDecWaves) {
    const bool has_next = ti + kDecWaves < te;
    float lg[IT][G];
    bool valid[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = ti * kGroup + it * TL + j;
      valid[it] = t < a.T;
      if constexpr (LUT) {
        // lane ck looks up stage ck (N <= 8 = NCK); the 8 lanes of token j sum
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = 0.0f;
        if (valid[it] && ck < a.N) {
          const int ci = min(static_cast<int>(kc[it]), a.Kc - 1);
#pragma unroll
          for (int h = 0; h < G; ++h) part[h] = lds_lut[(h * a.N + ck) * a.Kc + ci];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) lg[it][h] = sum_adjacent<NCK>(part[h]);
      } else {
        float kh[16];
        if (valid[it]) {
          rebuild16(a.k_cb, a.k_idx + (unit * a.T + t) * a.N, a.N, a.Kc, ck, kh);
        } else {
#pragma unroll
          for (int c = 0; c < 16; ++c) kh[c] = 0.0f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < 16; ++c) s = fmaf(qr[h][c], kh[c], s);
          lg[it][h] = sum_adjacent<NCK>(s);
        }
      }
    }
    if (LUT && has_next) load_kidx(ti + kDecWaves, kc);
    if (vpre && ti + 2 * kDecWaves < te) load_vidx(ti + 2 * kDecWaves, vnn);
    bool grow = false;
    float mnew[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = -INFINITY;
#pragma unroll
      for (int it = 0; it < IT; ++it) t = valid[it] ? fmaxf(t, lg[it][h]) : t;
      t = max_strided<NCK>(t);
      mnew[h] = fmaxf(m[h], t);
      grow |= mnew[h] > m[h];
    }
    if (grow) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = merge_weight(m[h], mnew[h]);
        l[h] *= sc;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[h][c] *= sc;
        m[h] = mnew[h];
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float vh[16];
      if (vpre) {
        const int slot = it % RB;
#pragma unroll
        for (int c = 0; c < 16; ++c) vh[c] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (k >= a.N) break;
          add_row16(rows[slot][k][0], rows[slot][k][1], vh);
        }
        // refill the slot: sub-tile it + RB of this tile, else of the next
        if (it + RB < IT) {
          issue(vcur[it + RB], rows[slot]);
        } else if (has_next) {
          issue(vnx[it + RB - IT], rows[slot]);
        }
      } else if (valid[it]) {
        const int t = ti * kGroup + it * TL + j;
        rebuild16(a.v_cb, a.v_idx + (unit * a.T + t) * a.N, a.N, a.Kc, ck, vh);
      }
      if (!valid[it]) continue;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = exp2f(lg[it][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[h][c] = fmaf(p, vh[c], acc[h][c]);
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        vcur[it][w] = vnx[it][w];
        vnx[it][w] = vnn[it][w];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = sum_strided<NCK>(l[h]);
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[h][c] = sum_strided<NCK>(acc[h][c]);
  }
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 16; ++c) lds_o[wave][h][lane_channel(ck, c)] = acc[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = m[h];
      lds_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  // the merge: the last split to finish, found with the unit's counter
  // (the per-split flags that find the table's pieces complete are not
  // used to elect a merging split: with the workgroups of a unit in two
  // resident rounds, a split so elected read another split's state before
  // it had arrived, one head in some runs)
  write_split_state<kD, G, kDecWaves>(a.partials, sync + kSyncWords - 1, a.out, a.Hq, unit, b, kvh, split, a.splits,
                                      lds_m, lds_l, lds_o, sync, epoch);
  if (a.splits == 1 && threadIdx.x == 0)
    __hip_atomic_store(sync, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct RvqGeometry {
  int G, n_tiles, tps, splits;
  size_t units, ws_bytes, lut_off, sync_bytes;
};

int rvq_geometry(int B, int Hq, int Hkv, int T, int d, RvqGeometry* g) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || T < 0 || Hq % Hkv != 0) return DQA_ERR_SHAPE;
  if (d != kD) return DQA_ERR_SHAPE;
  if (B > 65535 || Hkv > 65535) return DQA_ERR_SHAPE;
  g->G = Hq / Hkv;
  if (g->G < 1 || g->G > 4) return DQA_ERR_UNSUPPORTED;
  g->units = static_cast<size_t>(B) * Hkv;
  g->n_tiles = (T + kGroup - 1) / kGroup;
  long long s = (kTargetWorkgroups + static_cast<long long>(g->units) - 1) /
                static_cast<long long>(g->units > 0 ? g->units : 1);
  if (s > g->n_tiles) s = g->n_tiles;
  if (s > kMaxSplitsMerge - 1) s = kMaxSplitsMerge - 1;
  if (s < 1) s = 1;
  g->tps = g->n_tiles > 0 ? static_cast<int>((g->n_tiles + s - 1) / s) : 1;
  g->splits = g->n_tiles > 0 ? (g->n_tiles + g->tps - 1) / g->tps : 1;
  // the synchronization words first, at offsets that do not depend on the
  // shape (one block per (batch, KV head), for at least 16384 of them, as the
  // merge counters of the other decode paths), so that one workspace serves
  // calls of any shape without being cleared again; then the partial states
  // (none with one split) and the key-logit table of every unit
  const size_t sync_units = g->units > kMergeCountersMin ? g->units : kMergeCountersMin;
  g->sync_bytes = (sync_units * kSyncWords * sizeof(uint32_t) + 255) / 256 * 256;
  const size_t part = g->splits > 1 ? g->units * g->splits * g->G * (kD + 2) * sizeof(float) : 0;
  g->lut_off = g->sync_bytes + (part + 255) / 256 * 256;
  g->ws_bytes = g->lut_off + g->units * kLutFloats * sizeof(float);
  return DQA_OK;
}

}  // namespace
}  // namespace dqa

using namespace dqa;

extern "C" size_t rvq_encode_workspace_bytes(int N, int Kc) {
  if (N < 1 || N > kMaxStages || Kc < kTileCW || Kc > 32768 || Kc % kTileCW != 0) return 0;
  return static_cast<size_t>(N) * Kc * sizeof(float);
}

extern "C" int rvq_encode(const uint16_t* x, int64_t n, int d, const uint16_t* codebooks, int N,
                          int Kc, int16_t* idx, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || d != kD) return DQA_ERR_SHAPE;
  if (N < 1 || N > kMaxStages || Kc < kTileCW || Kc > 32768 || Kc % kTileCW != 0) return DQA_ERR_SHAPE;
  if (n == 0) return DQA_OK;
  if (!x || !codebooks || !idx) return DQA_ERR_NULL;
  if (!ws || ws_bytes < rvq_encode_workspace_bytes(N, Kc)) return DQA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(codebooks) || !aligned16(ws)) return DQA_ERR_ALIGN;
  const int64_t blocks = (n + kEncRows - 1) / kEncRows;
  if (blocks > 0x7FFFFFFF) return DQA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* norms = static_cast<float*>(ws);
  const size_t n_cw = static_cast<size_t>(N) * Kc;
  hipLaunchKernelGGL(rvq_norms_kernel, dim3(static_cast<unsigned>((n_cw + 255) / 256)), dim3(256), 0, s,
                     codebooks, n_cw, norms);
  DQA_CHECK_LAUNCH();
  hipLaunchKernelGGL((rvq_encode_kernel<kEncMB, kEncWaves>), dim3(static_cast<unsigned>(blocks)), dim3(kEncWaves * 64), 0, s,
                     x, n, codebooks, norms, N, Kc, idx);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

extern "C" size_t rvq_decode_attention_workspace_bytes(int B, int Hq, int Hkv, int T, int d) {
  RvqGeometry g;
  if (rvq_geometry(B, Hq, Hkv, T, d, &g) != DQA_OK) return 0;
  return g.ws_bytes;
}

extern "C" int rvq_decode_attention(const uint16_t* q, int B, int Hq, int Hkv, int T, int d,
                                    const int16_t* k_idx, const int16_t* v_idx, const uint16_t* k_cb,
                                    const uint16_t* v_cb, int N, int Kc, float sm_scale, void* ws,
                                    size_t ws_bytes, float* out, void* stream) {
  RvqGeometry g;
  int st = rvq_geometry(B, Hq, Hkv, T, d, &g);
  if (st != DQA_OK) return st;
  if (N < 1 || N > kMaxStages || Kc < 1 || Kc > 32768) return DQA_ERR_SHAPE;
  if (g.units == 0) return DQA_OK;
  if (!q || !out) return DQA_ERR_NULL;
  if (T > 0 && (!k_idx || !v_idx || !k_cb || !v_cb)) return DQA_ERR_NULL;
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (!a16(q) || (T > 0 && (!a16(k_cb) || !a16(v_cb)))) return DQA_ERR_ALIGN;
  if (!ws || ws_bytes < g.ws_bytes) return DQA_ERR_WORKSPACE;
  RvqDecArgs a;
  a.q = q;
  a.k_idx = k_idx;
  a.v_idx = v_idx;
  a.k_cb = k_cb;
  a.v_cb = v_cb;
  a.out = out;
  a.sync = static_cast<uint32_t*>(ws);
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + g.sync_bytes);
  a.lut = reinterpret_cast<float*>(static_cast<char*>(ws) + g.lut_off);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T = T;
  a.N = N;
  a.Kc = Kc;
  a.n_tiles = g.n_tiles;
  a.tiles_per_split = g.tps;
  a.splits = g.splits;
  a.vidx_words = N == 4 && (reinterpret_cast<uintptr_t>(v_idx) & 7u) == 0;
  a.table_polls = g_table_polls;
  const bool use_lut = T > 0 && static_cast<long long>(g.G) * N * Kc <= kLutFloats && N <= 8;
  if (use_lut) {
    // one table-holding workgroup of eight waves per compute unit (the
    // table once in its LDS): one resident round of them, so that each
    // stages its table once for more tiles
    long long sp = kLutWorkgroups / static_cast<long long>(g.units);
    if (sp > g.splits) sp = g.splits;
    if (sp < 1) sp = 1;
    a.tiles_per_split = static_cast<int>((g.n_tiles + sp - 1) / sp);
    a.splits = (g.n_tiles + a.tiles_per_split - 1) / a.tiles_per_split;
  }
  a.q_scale = sm_scale * 1.4426950408889634f;
  const dim3 grid(a.splits, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the table path: the unit's table in LDS, one stage per lookup lane
  const bool vpre = N <= 4;
  switch (g.G * 4 + (use_lut ? 2 : 0) + (vpre ? 1 : 0)) {
#define DQA_RVQ_CASE(G_, L_, V_) \
  case G_ * 4 + (L_ ? 2 : 0) + (V_ ? 1 : 0): \
    hipLaunchKernelGGL((rvq_decode_kernel<G_, L_, V_>), grid, dim3(64 * kDecWaves), 0, s, a); \
    break;
#define DQA_RVQ_CASES(G_) DQA_RVQ_CASE(G_, false, false) DQA_RVQ_CASE(G_, false, true) \
  DQA_RVQ_CASE(G_, true, false) DQA_RVQ_CASE(G_, true, true)
    DQA_RVQ_CASES(1)
    DQA_RVQ_CASES(2)
    DQA_RVQ_CASES(3)
    DQA_RVQ_CASES(4)
#undef DQA_RVQ_CASES
#undef DQA_RVQ_CASE
    default: return DQA_ERR_UNSUPPORTED;
  }
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

extern "C" int rvq_decode_set_table_polls(int polls) {
  if (polls < 0) return -1;
  const int prev = g_table_polls;
  g_table_polls = polls;
  return prev;
}
