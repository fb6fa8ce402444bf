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
// Work decomposition (one GPU): grid = (splits, KV heads, batch); a
// workgroup of 4 waves owns a contiguous run of 32-token tiles of one
// (batch, KV head), each wave a contiguous quarter of it.  The two
// contractions run on the matrix cores (v_mfma_f32_16x16x32_f16): at G query
// heads per KV head, q.k and p.v are G-row dense products whose VALU cost
// (2*G*d multiply-adds per token) would exceed the HBM time several times.
//   * logits: A = the query (fp16, exact; rows = heads), B = the dequantized
//     and rotated keys of 16 tokens (fp32 split exactly enough as fp16 hi +
//     lo, two products), fp32 accumulation;
//   * values: A = the value codes of 16 channels x 32 tokens (small integers,
//     exact in fp16), B = p * scale per (token, head) in fp16; the zero
//     point enters as sum(p * zero) in fp32.
// Dequantization, RoPE and the hi/lo split run on the VALU per (token,
// channel); the online softmax is updated once per 32-token tile.  The fp16
// recent zone is handled by a second, VALU kernel launched after the first;
// both write partial softmax states into one workspace, and the last
// workgroup of a (batch, KV head) -- found with a device-scope ticket --
// merges all partials in a fixed order and writes the output.
#include "common.h"

namespace dqa {
namespace {

constexpr int kWavesPerWG = 4;
// the final merge keeps one weight per (split, head) in the workgroup's LDS
// wave-output area (kWavesPerWG * G * D floats)
constexpr int kMaxSplitsMerge = 255;

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
  unsigned* tickets;
  int Hq, Hkv, T_q, R;
  int n_qtiles;         // T_q / 32
  int tile_begin;       // tiles of this launch: [tile_begin, tile_end)
  int tile_end;
  int tiles_per_split;
  int split_base;       // first partial-state slot of this launch
  int total_splits;     // partial-state slots per (batch, KV head), all launches
  float q_scale;        // sm_scale * log2(e): logits in the log2 domain
  float rope_theta;
};

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

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

// Load 16 consecutive fp16 values as fp32.
__device__ __forceinline__ void load16h(const uint16_t* p, float* x) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  const uint4 a = v[0], b = v[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
    x[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
  }
}

// Code of channel c (0..15) from the lane's BITS/2 words (little-endian bit
// stream, channel c at bit c*BITS).
template <int BITS>
__device__ __forceinline__ float code_at(const uint32_t* w, int c) {
  constexpr int kPerWord = 32 / BITS;
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  return static_cast<float>((w[c / kPerWord] >> ((c % kPerWord) * BITS)) & kMask);
}

// All 16 codes of the lane's chunk as fp32.  Codes are first spread one
// per byte with shift+mask, so each conversion is a single byte-to-float
// instruction.
template <int BITS>
__device__ __forceinline__ void codes16(const uint32_t* w, float* out) {
  if constexpr (BITS == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = (w[0] >> (2 * j)) & 0x03030303u;
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * k + j] = static_cast<float>((m >> (8 * k)) & 0xFFu);
    }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int wd = 0; wd < 2; ++wd)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t m = (w[wd] >> (4 * j)) & 0x0F0F0F0Fu;
#pragma unroll
        for (int k = 0; k < 4; ++k) out[8 * wd + 2 * k + j] = static_cast<float>((m >> (8 * k)) & 0xFFu);
      }
  } else {
#pragma unroll
    for (int wd = 0; wd < 4; ++wd)
#pragma unroll
      for (int k = 0; k < 4; ++k) out[4 * wd + k] = static_cast<float>((w[wd] >> (8 * k)) & 0xFFu);
  }
}

// fp16 half `hi` (0 = low, 1 = high) of a packed pair, widened to fp32.
__device__ __forceinline__ float half_of(uint32_t w, int hi) {
  return h2f(static_cast<uint16_t>(hi ? (w >> 16) : (w & 0xFFFFu)));
}

// Load 16 consecutive fp16 values as 8 packed pairs.
__device__ __forceinline__ void load16p(const uint16_t* p, uint32_t* w) {
  const uint4* v = reinterpret_cast<const uint4*>(p);
  const uint4 a = v[0], b = v[1];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <int D, int G, bool ROPE>
struct WaveState {
  static constexpr int NCK = D / 16;
  static constexpr int TL = kWave / NCK;
  static constexpr int IT = kGroup / TL;
  static constexpr int NP = 8;
  uint32_t q2[G][8];                  // query slice, packed fp16 (exact)
  float acc[G][16], zacc[G], l[G], m[G];
  float st_c[NP], st_s[NP];           // rotation step between lane tokens
  double omega;                       // frequency of pair `lane` (anchors)

  // Dot products of the lane's 16 dequantized (and rotated) key channels
  // with the G query slices, completed across the chunk lanes.
  __device__ __forceinline__ void logits(const float* kh, float q_scale, float* out) const {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) s = fmaf(half_of(q2[h][c / 2], c & 1), kh[c], s);
      out[h] = sum_adjacent<NCK>(s) * q_scale;
    }
  }

  // Rotate the lane's 8 channel pairs by (fc, fs) and advance the rotation
  // by one lane step (TL tokens).
  __device__ __forceinline__ void rotate(float* kh, float* fc, float* fs) const {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const float x0 = kh[2 * p], x1 = kh[2 * p + 1];
      kh[2 * p] = x0 * fc[p] - x1 * fs[p];
      kh[2 * p + 1] = x0 * fs[p] + x1 * fc[p];
      const float nc = fc[p] * st_c[p] - fs[p] * st_s[p];
      const float ns = fc[p] * st_s[p] + fs[p] * st_c[p];
      fc[p] = nc;
      fs[p] = ns;
    }
  }

  // Tile-wide max per head, rescale of the running state when it grows.
  __device__ __forceinline__ void update_max(const float (*lg)[G], const bool* valid) {
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
        zacc[h] *= sc;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[h][c] *= sc;
        m[h] = mnew[h];
      }
    }
  }
};

// Rotation of the lane's first token in a tile: the tile anchor e^{i pos w}
// (one pair per lane, exact, shared through LDS) times the lane offset E_j.
template <int D, int G>
__device__ __forceinline__ void tile_rotation(const WaveState<D, G, true>& S, float (*anchor)[2],
                                              const float (*ej)[2], int lane, int c0, int tile_pos,
                                              float* fc, float* fs) {
  if (lane < D / 2) {
    float ac, as;
    rope_unit(static_cast<double>(tile_pos), S.omega, ac, as);
    anchor[lane][0] = ac;
    anchor[lane][1] = as;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const float ac = anchor[c0 / 2 + p][0];
    const float as = anchor[c0 / 2 + p][1];
    const float ec = ej[p][0], es = ej[p][1];
    fc[p] = ac * ec - as * es;
    fs[p] = ac * es + as * ec;
  }
  __builtin_amdgcn_wave_barrier();
}

// Merge the 4 wave states of a workgroup (in LDS), write the split's partial
// state, and let the last workgroup of the (batch, KV head) merge all
// partials in slot order and write the output.  Called by every thread.
template <int D, int G>
__device__ __forceinline__ void finish_workgroup(const KiviArgs& a, size_t unit, int b, int kvh,
                                                 int slot, const float (*lm)[G],
                                                 const float (*ll)[G], const float (*lo)[G][D],
                                                 int* last) {
  float* part = a.partials + (unit * a.total_splits + slot) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, lm[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) {
      const float wt = merge_weight(lm[w][h], M);
      L = fmaf(ll[w][h], wt, L);
      O = fmaf(lo[w][h][c], wt, O);
    }
    if (a.total_splits == 1) {
      a.out[(static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c] = (L > 0.0f) ? O / L : 0.0f;
    } else {
      if (c == 0) {
        part[h * (D + 2) + 0] = M;
        part[h * (D + 2) + 1] = L;
      }
      part[h * (D + 2) + 2 + c] = O;
    }
  }
  if (a.total_splits == 1) return;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(a.tickets + unit, 1u);
    *last = (prev == static_cast<unsigned>(a.total_splits - 1));
  }
  __syncthreads();
  if (!*last) return;
  __threadfence();
  const float* parts = a.partials + unit * a.total_splits * G * (D + 2);
  // per-head merge weights of every split, computed once into LDS (reusing
  // lds_o, whose wave states are no longer needed); loads are independent
  // so they are issued back to back
  float* wts = &const_cast<float(*)[G][D]>(lo)[0][0][0];
  float* scal = wts + kMaxSplitsMerge * G;
  const int ns = a.total_splits;
  for (int e = threadIdx.x; e < G; e += blockDim.x) {
    float M = -INFINITY;
#pragma unroll 8
    for (int sl = 0; sl < ns; ++sl) M = fmaxf(M, parts[(sl * G + e) * (D + 2)]);
    float L = 0.0f;
#pragma unroll 8
    for (int sl = 0; sl < ns; ++sl) {
      const float* ps = parts + (sl * G + e) * (D + 2);
      const float wt = merge_weight(ps[0], M);
      wts[sl * G + e] = wt;
      L = fmaf(ps[1], wt, L);
    }
    scal[e] = (L > 0.0f) ? 1.0f / L : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float O = 0.0f;
#pragma unroll 8
    for (int sl = 0; sl < ns; ++sl) O = fmaf(parts[(sl * G + h) * (D + 2) + 2 + c], wts[sl * G + h], O);
    a.out[(static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c] = O * scal[h];
  }
  if (threadIdx.x == 0) a.tickets[unit] = 0u;
}

// ------------------------------------------------------------ recent zone
// fp16 recent tokens (keys stored before RoPE), VALU: lane = (token j,
// 16-channel chunk); tiles of 32 tokens, waves round-robin.
template <int D, int G, bool ROPE>
__global__ __launch_bounds__(256) void recent_decode_kernel(KiviArgs a) {
  using State = WaveState<D, G, ROPE>;
  constexpr int NCK = State::NCK;
  constexpr int TL = State::TL;
  constexpr int IT = State::IT;
  constexpr int NP = State::NP;
  __shared__ float lds_anchor[kWavesPerWG][D / 2][2];
  __shared__ float lds_ej[ROPE ? kWavesPerWG * kWave : 1][8][2];
  __shared__ float lds_m[kWavesPerWG][G], lds_l[kWavesPerWG][G];
  __shared__ float lds_o[kWavesPerWG][G][D];
  __shared__ int lds_last;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int j = lane / NCK, ck = lane % NCK;
  const int c0 = ck * 16;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * a.Hkv + kvh;

  State S;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    load16p(a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c0, S.q2[h]);
    S.m[h] = -INFINITY;
    S.l[h] = 0.0f;
    S.zacc[h] = 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c) S.acc[h][c] = 0.0f;
  }
  if constexpr (ROPE) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const double om = pow(static_cast<double>(a.rope_theta), -2.0 * (c0 / 2 + p) / D);
      rope_unit(static_cast<double>(j), om, lds_ej[threadIdx.x][p][0], lds_ej[threadIdx.x][p][1]);
      rope_unit(static_cast<double>(TL), om, S.st_c[p], S.st_s[p]);
    }
    S.omega = (lane < D / 2) ? pow(static_cast<double>(a.rope_theta), -2.0 * lane / D) : 0.0;
  }

  bool valid[IT];
  const int tb = a.tile_begin + split * a.tiles_per_split;
  const int te = min(a.tile_end, tb + a.tiles_per_split);
  for (int ti = tb + wave; ti < te; ti += kWavesPerWG) {
    const int tile_pos = ti * kGroup;
    float fc[NP], fs[NP];
    if constexpr (ROPE) tile_rotation<D, G>(S, lds_anchor[wave], lds_ej[ROPE ? threadIdx.x : 0], lane, c0, tile_pos, fc, fs);
    float lg[IT][G];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = tile_pos - a.T_q + it * TL + j;
      valid[it] = r < a.R;
      float kh[16];
      if (valid[it]) {
        load16h(a.k_recent + (unit * a.R + r) * D + c0, kh);
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) kh[c] = 0.0f;
      }
      if constexpr (ROPE) S.rotate(kh, fc, fs);
      S.logits(kh, a.q_scale, lg[it]);
    }
    S.update_max(lg, valid);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = tile_pos - a.T_q + it * TL + j;
      if (!valid[it]) continue;
      float v[16];
      load16h(a.v_recent + (unit * a.R + r) * D + c0, v);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = __builtin_amdgcn_exp2f(lg[it][h] - S.m[h]);
        S.l[h] += p;
#pragma unroll
        for (int c = 0; c < 16; ++c) S.acc[h][c] = fmaf(p, v[c], S.acc[h][c]);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    S.l[h] = sum_strided<NCK>(S.l[h]);
#pragma unroll
    for (int c = 0; c < 16; ++c) S.acc[h][c] = sum_strided<NCK>(S.acc[h][c]);
  }
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 16; ++c) lds_o[wave][h][c0 + c] = S.acc[h][c];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = S.m[h];
      lds_l[wave][h] = S.l[h];
    }
  }
  __syncthreads();
  finish_workgroup<D, G>(a, unit, b, kvh, a.split_base + split, lds_m, lds_l, lds_o, &lds_last);
}

// --------------------------------------------------- quantized tiles (MFMA)

// The lane's 8-code chunk: 8 consecutive channels of one key row, or 8
// consecutive tokens of one value channel; BITS bytes at `p`.
template <int BITS>
__device__ __forceinline__ uint64_t load_chunk(const uint8_t* p) {
  if constexpr (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
  else if constexpr (BITS == 4) return *reinterpret_cast<const uint32_t*>(p);
  else return *reinterpret_cast<const uint64_t*>(p);
}

// Key chunk -> 8 fp32 codes, channel order.
template <int BITS>
__device__ __forceinline__ void key_codes8(uint64_t chunk, float* f) {
  if constexpr (BITS == 2) {
    const uint32_t v = static_cast<uint32_t>(chunk);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t m = (v >> (2 * j)) & 0x0303u;
      f[j] = static_cast<float>(m & 0xFFu);
      f[j + 4] = static_cast<float>(m >> 8);
    }
  } else if constexpr (BITS == 4) {
    const uint32_t w = static_cast<uint32_t>(chunk);
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = static_cast<float>((lo >> (8 * k)) & 0xFFu);
      f[2 * k + 1] = static_cast<float>((hi >> (8 * k)) & 0xFFu);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = static_cast<float>((chunk >> (8 * k)) & 0xFFu);
  }
}

// Value chunk (8 tokens of one channel) -> exact fp16 codes.  Element 2i
// holds token i, element 2i+1 token i+4 (the same order is used for the
// probabilities).  1024 + code is built in the fp16 bit pattern and 1024
// subtracted with a packed half add.
template <int BITS>
__device__ __forceinline__ half8 value_codes8(uint64_t chunk) {
  uint32_t r[4];
  if constexpr (BITS == 2) {
    const uint32_t v = static_cast<uint32_t>(chunk);
    const uint32_t u = v | (v << 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ((u >> (2 * i)) & 0x00030003u) | 0x64006400u;
  } else if constexpr (BITS == 4) {
    const uint32_t w = static_cast<uint32_t>(chunk);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
  } else {
    const uint32_t lo = static_cast<uint32_t>(chunk), hi = static_cast<uint32_t>(chunk >> 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = __builtin_amdgcn_perm(hi, lo, static_cast<uint32_t>(i | (0x0C << 8) | ((4 + i) << 16) | (0x0C << 24))) |
             0x64006400u;
  }
  half8 out;
  const half2v k1024 = {static_cast<_Float16>(1024.0f), static_cast<_Float16>(1024.0f)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2v h = __builtin_bit_cast(half2v, r[i]) - k1024;
    out[2 * i] = h[0];
    out[2 * i + 1] = h[1];
  }
  return out;
}

// token order of the value operand's element e (see value_codes8)
__device__ __forceinline__ constexpr int vtok(int e) { return (e >> 1) + 4 * (e & 1); }

// Max over the 16 lanes of each DPP row (every lane receives its row's max).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppRowMirror>(v));
}

template <int D, int BITS, int G, bool ROPE>
__global__ __launch_bounds__(256) void kivi_mfma_kernel(KiviArgs a) {
  constexpr int KS = D / 32;          // channel blocks of the logit product
  constexpr int MB = D / 16;          // channel blocks of the value product
  constexpr int NVG = D / kGroup;     // value groups per token
  constexpr int NP = 4 * KS;          // RoPE pairs per lane
  constexpr int KROW = D * BITS / 8;  // bytes per key row
  constexpr int VBLK = 4 * D * BITS;  // bytes per 32-token value block
  constexpr int NE = ROPE ? 16 * (D / 2) : 1;

  __shared__ float lds_anchor[kWavesPerWG][2][ROPE ? D / 2 : 1][2];
  __shared__ float lds_E[NE][2];                 // e^{i c w_i}, c = 0..15
  __shared__ double lds_omega[ROPE ? D / 2 : 1];
  __shared__ __attribute__((aligned(16))) float lds_p[kWavesPerWG][4][kGroup];
  __shared__ float lds_m[kWavesPerWG][G], lds_l[kWavesPerWG][G];
  __shared__ float lds_o[kWavesPerWG][G][D];
  __shared__ int lds_last;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * a.Hkv + kvh;

  // wave's contiguous tile range
  const int tb = a.tile_begin + split * a.tiles_per_split;
  const int te = min(a.tile_end, tb + a.tiles_per_split);
  const int tpw = (te - tb + kWavesPerWG - 1) / kWavesPerWG;
  const int wb = tb + wave * tpw;
  const int we = min(te, wb + tpw);

  // RoPE tables shared by the workgroup: omega_i, E[c][i] = e^{i c omega_i}
  float an_c = 1.0f, an_s = 0.0f, w16c = 1.0f, w16s = 0.0f, w32c = 1.0f, w32s = 0.0f;
  if constexpr (ROPE) {
    for (int i = tid; i < D / 2; i += blockDim.x)
      lds_omega[i] = pow(static_cast<double>(a.rope_theta), -2.0 * i / D);
    __syncthreads();
    for (int e = tid; e < 16 * (D / 2); e += blockDim.x)
      rope_unit(static_cast<double>(e / (D / 2)), lds_omega[e % (D / 2)], lds_E[e][0], lds_E[e][1]);
    __syncthreads();
    if (lane < D / 2 && wb < we) {
      const double om = lds_omega[lane];
      rope_unit(static_cast<double>(wb) * kGroup, om, an_c, an_s);
      rope_unit(16.0, om, w16c, w16s);
      rope_unit(32.0, om, w32c, w32s);
    }
  }

  // the query as the A operand of the logit product (rows = heads)
  half8 aq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (col < G) {
      const uint4 u = *reinterpret_cast<const uint4*>(
          a.q + (static_cast<size_t>(b) * a.Hq + kvh * G + col) * D + 32 * ks + 8 * grp);
      aq[ks] = __builtin_bit_cast(half8, u);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) aq[ks][e] = static_cast<_Float16>(0.0f);
    }
  }

  float4v acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  float m[G], lsum[G], zacc[NVG];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.0f;
  }
#pragma unroll
  for (int g = 0; g < NVG; ++g) zacc[g] = 0.0f;

  // key code chunks of a tile: [half][K-step]
  auto load_kchunks = [&](int ti, uint64_t (*kc)[KS]) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint8_t* row = reinterpret_cast<const uint8_t*>(a.k_codes) +
                           (unit * a.T_q + static_cast<size_t>(ti) * kGroup + 16 * sub + col) * KROW;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kc[sub][ks] = load_chunk<BITS>(row + (32 * ks + 8 * grp) * BITS / 8);
    }
  };
  uint64_t kcur[2][KS];
  if (wb < we) load_kchunks(wb, kcur);

  for (int ti = wb; ti < we; ++ti) {
    const int tile_pos = ti * kGroup;
    // value code chunks of this tile, and the key codes of the next one,
    // are requested before this tile's key arithmetic
    uint64_t vch[MB];
    {
      const uint8_t* blk = reinterpret_cast<const uint8_t*>(a.v_codes) + (unit * a.n_qtiles + ti) * VBLK;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) vch[mb] = load_chunk<BITS>(blk + (32 * (16 * mb + col) + 8 * grp) * BITS / 8);
    }
    uint64_t knext[2][KS];
    if (ti + 1 < we) load_kchunks(ti + 1, knext);
    if constexpr (ROPE) {
      if (lane < D / 2) {
        lds_anchor[wave][0][lane][0] = an_c;
        lds_anchor[wave][0][lane][1] = an_s;
        lds_anchor[wave][1][lane][0] = an_c * w16c - an_s * w16s;
        lds_anchor[wave][1][lane][1] = an_c * w16s + an_s * w16c;
        const float nc = an_c * w32c - an_s * w32s;
        const float ns = an_c * w32s + an_s * w32c;
        an_c = nc;
        an_s = ns;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- logits of the tile's two 16-token halves
    uint4 ks4[KS], kz4[KS];
    const size_t tz = (unit * a.n_qtiles + ti) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ks4[ks] = *reinterpret_cast<const uint4*>(a.k_scale + tz + 32 * ks + 8 * grp);
      kz4[ks] = *reinterpret_cast<const uint4*>(a.k_zero + tz + 32 * ks + 8 * grp);
    }
    float4v sacc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      sacc[sub] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float kh[8];
        key_codes8<BITS>(kcur[sub][ks], kh);
        const half8 sh = __builtin_bit_cast(half8, ks4[ks]);
        const half8 zh = __builtin_bit_cast(half8, kz4[ks]);
#pragma unroll
        for (int e = 0; e < 8; ++e) kh[e] = fmaf(kh[e], static_cast<float>(sh[e]), static_cast<float>(zh[e]));
        if constexpr (ROPE) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int i = 16 * ks + 4 * grp + p;
            const float ac = lds_anchor[wave][sub][i][0], as = lds_anchor[wave][sub][i][1];
            const float ec = lds_E[col * (D / 2) + i][0], es = lds_E[col * (D / 2) + i][1];
            const float fc = ac * ec - as * es;
            const float fs = ac * es + as * ec;
            const float x0 = kh[2 * p], x1 = kh[2 * p + 1];
            kh[2 * p] = x0 * fc - x1 * fs;
            kh[2 * p + 1] = x0 * fs + x1 * fc;
          }
        }
        half8 bh, bl;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(kh[2 * p], kh[2 * p + 1]));
          const half2v lo = __builtin_bit_cast(
              half2v, __builtin_amdgcn_cvt_pkrtz(kh[2 * p] - static_cast<float>(hi[0]),
                                                 kh[2 * p + 1] - static_cast<float>(hi[1])));
          bh[2 * p] = hi[0];
          bh[2 * p + 1] = hi[1];
          bl[2 * p] = lo[0];
          bl[2 * p + 1] = lo[1];
        }
        sacc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[ks], bh, sacc[sub], 0, 0, 0);
        sacc[sub] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[ks], bl, sacc[sub], 0, 0, 0);
      }
    }

    // ---- online softmax; heads are rows 0..G-1, held by the lanes of row 0
    float s0[G], s1[G];
    bool grow = false;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s0[h] = sacc[0][h] * a.q_scale;
      s1[h] = sacc[1][h] * a.q_scale;
      const float t = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, row_max16(fmaxf(s0[h], s1[h]))));
      const float tm = __builtin_bit_cast(float, static_cast<int>(t));
      const float mn = fmaxf(m[h], tm);
      sc[h] = merge_weight(m[h], mn);
      grow |= mn > m[h];
      m[h] = mn;
    }
    if (grow) {
      float my = 1.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        lsum[h] *= sc[h];
        my = (col == h) ? sc[h] : my;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= my;
#pragma unroll
      for (int g = 0; g < NVG; ++g) zacc[g] *= my;
    }
    if (grp == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p0 = __builtin_amdgcn_exp2f(s0[h] - m[h]);
        const float p1 = __builtin_amdgcn_exp2f(s1[h] - m[h]);
        lsum[h] += p0 + p1;
        lds_p[wave][h][col] = p0;
        lds_p[wave][h][col + 16] = p1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value product: B = p * scale (lanes col < G), A = value codes
    half8 bv[NVG];
    if (col < G) {
      const float4 p4a = *reinterpret_cast<const float4*>(&lds_p[wave][col][8 * grp]);
      const float4 p4b = *reinterpret_cast<const float4*>(&lds_p[wave][col][8 * grp + 4]);
      const float pt[8] = {p4a.x, p4a.y, p4a.z, p4a.w, p4b.x, p4b.y, p4b.z, p4b.w};
      const size_t tok0 = unit * a.T_q + tile_pos + 8 * grp;
      const uint16_t* vsp = a.v_scale + tok0 * NVG;
      const uint16_t* vzp = a.v_zero + tok0 * NVG;
#pragma unroll
      for (int g = 0; g < NVG; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = vtok(e);
          const float pv = pt[t];
          bv[g][e] = static_cast<_Float16>(pv * h2f(vsp[t * NVG + g]));
          zacc[g] = fmaf(pv, h2f(vzp[t * NVG + g]), zacc[g]);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < NVG; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[g][e] = static_cast<_Float16>(0.0f);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const half8 av = value_codes8<BITS>(vch[mb]);
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv[mb / 2], acc[mb], 0, 0, 0);
    }
    if (ti + 1 < we) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kcur[sub][ks] = knext[sub][ks];
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave state -> LDS: l over the 16 token lanes of row 0; zero-point
  // sums over the 4 row groups of each head lane
  float l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float v = lsum[h];
    v += dpp<kDppQuadXor1>(v);
    v += dpp<kDppQuadXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    v += dpp<kDppRowMirror>(v);
    l[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
  }
#pragma unroll
  for (int g = 0; g < NVG; ++g) {
    zacc[g] += __shfl_xor(zacc[g], 16, kWave);
    zacc[g] += __shfl_xor(zacc[g], 32, kWave);
  }
  if (col < G) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) lds_o[wave][col][16 * mb + 4 * grp + r] = acc[mb][r] + zacc[mb / 2];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = m[h];
      lds_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  finish_workgroup<D, G>(a, unit, b, kvh, a.split_base + split, lds_m, lds_l, lds_o, &lds_last);
}

// ---------------------------------------------------------------- host side

struct Plan {
  int G, n_qtiles, n_rtiles;
  int tps_q, splits_q, splits_r, total;
  size_t units, ticket_bytes, ws_bytes;
};

int make_plan(const dqa_kivi_cache* c, Plan* p) {
  if (!c) return DQA_ERR_NULL;
  if (c->B < 0 || c->Hq <= 0 || c->Hkv <= 0 || c->T_q < 0 || c->R < 0) return DQA_ERR_SHAPE;
  if (c->d != 64 && c->d != 128) return DQA_ERR_SHAPE;
  if (c->bits != 2 && c->bits != 4 && c->bits != 8) return DQA_ERR_BITS;
  if (c->Hq % c->Hkv != 0) return DQA_ERR_SHAPE;
  if (c->T_q % kGroup != 0 || c->R > kMaxRecent) return DQA_ERR_SHAPE;
  if (c->B > 65535 || c->Hkv > 65535) return DQA_ERR_SHAPE;
  p->G = c->Hq / c->Hkv;
  if (p->G != 1 && p->G != 2 && p->G != 4) return DQA_ERR_UNSUPPORTED;
  p->units = static_cast<size_t>(c->B) * c->Hkv;
  p->n_qtiles = c->T_q / kGroup;
  p->n_rtiles = (c->R + kGroup - 1) / kGroup;
  // quantized tiles: enough workgroups to fill the chip, at least one tile
  // per wave when the cache is long enough
  long long want = (kTargetWorkgroups + static_cast<long long>(p->units) - 1) /
                   static_cast<long long>(p->units > 0 ? p->units : 1);
  long long cap = (p->n_qtiles + 3) / 4;
  if (want > cap) want = cap;
  if (want > kMaxSplitsMerge - 1) want = kMaxSplitsMerge - 1;
  if (want < 1) want = 1;
  p->tps_q = p->n_qtiles > 0 ? static_cast<int>((p->n_qtiles + want - 1) / want) : 0;
  p->splits_q = p->n_qtiles > 0 ? (p->n_qtiles + p->tps_q - 1) / p->tps_q : 0;
  // recent tiles (at most 4): one workgroup
  p->splits_r = (p->n_rtiles > 0 || p->n_qtiles == 0) ? 1 : 0;
  p->total = p->splits_q + p->splits_r;
  p->ticket_bytes = (p->units * sizeof(unsigned) + 255) / 256 * 256;
  p->ws_bytes = p->ticket_bytes +
                p->units * static_cast<size_t>(p->total) * p->G * (c->d + 2) * sizeof(float);
  return DQA_OK;
}

template <int D, int BITS, int G>
void launch_q(const KiviArgs& a, bool rope, dim3 grid, hipStream_t s) {
  if (rope)
    hipLaunchKernelGGL((kivi_mfma_kernel<D, BITS, G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kivi_mfma_kernel<D, BITS, G, false>), grid, dim3(256), 0, s, a);
}

template <int D, int G>
void launch_q_bits(const KiviArgs& a, int bits, bool rope, dim3 grid, hipStream_t s) {
  if (bits == 2) launch_q<D, 2, G>(a, rope, grid, s);
  else if (bits == 4) launch_q<D, 4, G>(a, rope, grid, s);
  else launch_q<D, 8, G>(a, rope, grid, s);
}

template <int D>
void launch_quantized(const KiviArgs& a, int G, int bits, bool rope, dim3 grid, hipStream_t s) {
  if (G == 1) launch_q_bits<D, 1>(a, bits, rope, grid, s);
  else if (G == 2) launch_q_bits<D, 2>(a, bits, rope, grid, s);
  else launch_q_bits<D, 4>(a, bits, rope, grid, s);
}

template <int D, int G>
void launch_r(const KiviArgs& a, bool rope, dim3 grid, hipStream_t s) {
  if (rope)
    hipLaunchKernelGGL((recent_decode_kernel<D, G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((recent_decode_kernel<D, G, false>), grid, dim3(256), 0, s, a);
}

template <int D>
void launch_recent(const KiviArgs& a, int G, bool rope, dim3 grid, hipStream_t s) {
  if (G == 1) launch_r<D, 1>(a, rope, grid, s);
  else if (G == 2) launch_r<D, 2>(a, rope, grid, s);
  else launch_r<D, 4>(a, rope, grid, s);
}

}  // namespace
}  // namespace dqa

using namespace dqa;

extern "C" size_t decode_attention_workspace_bytes(const dqa_kivi_cache* cache) {
  Plan p;
  if (make_plan(cache, &p) != DQA_OK) return 0;
  return p.ws_bytes;
}

extern "C" int decode_attention_qkv(const uint16_t* q, const dqa_kivi_cache* c,
                                    float sm_scale, void* ws, size_t ws_bytes,
                                    float* out, void* stream) {
  Plan p;
  int st = make_plan(c, &p);
  if (st != DQA_OK) return st;
  if (p.units == 0) return DQA_OK;
  if (!q || !out) return DQA_ERR_NULL;
  if (c->T_q > 0 && (!c->k_codes || !c->k_scale || !c->k_zero || !c->v_codes ||
                     !c->v_scale || !c->v_zero))
    return DQA_ERR_NULL;
  if (c->R > 0 && (!c->k_recent || !c->v_recent)) return DQA_ERR_NULL;
  if (!ws) return DQA_ERR_WORKSPACE;
  if (ws_bytes < p.ws_bytes) return DQA_ERR_WORKSPACE;
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
  a.tickets = static_cast<unsigned*>(ws);
  a.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + p.ticket_bytes);
  a.Hq = c->Hq;
  a.Hkv = c->Hkv;
  a.T_q = c->T_q;
  a.R = c->R;
  a.n_qtiles = p.n_qtiles;
  a.total_splits = p.total;
  a.q_scale = sm_scale * 1.4426950408889634f;
  a.rope_theta = c->rope_theta;
  const bool rope = c->rope_theta > 0.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.splits_q > 0) {
    a.tile_begin = 0;
    a.tile_end = p.n_qtiles;
    a.tiles_per_split = p.tps_q;
    a.split_base = 0;
    const dim3 grid(p.splits_q, c->Hkv, c->B);
    if (c->d == 128) launch_quantized<128>(a, p.G, c->bits, rope, grid, s);
    else launch_quantized<64>(a, p.G, c->bits, rope, grid, s);
    DQA_CHECK_LAUNCH();
  }
  if (p.splits_r > 0) {
    a.tile_begin = p.n_qtiles;
    a.tile_end = p.n_qtiles + p.n_rtiles;
    a.tiles_per_split = p.n_rtiles;
    a.split_base = p.splits_q;
    const dim3 grid(1, c->Hkv, c->B);
    if (c->d == 128) launch_recent<128>(a, p.G, rope, grid, s);
    else launch_recent<64>(a, p.G, rope, grid, s);
    DQA_CHECK_LAUNCH();
  }
  return DQA_OK;
}
