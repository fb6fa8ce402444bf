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
// (batch, KV head); its waves take the run's tiles round-robin.  Inside a
// wave, lane = (token j, 16-channel chunk ck): a 32-token tile is covered in
// 32/TL iterations of TL tokens; each lane dequantizes 16 channels of one
// token, so code loads are contiguous across the wave (token-major rows).
// The K scale/zero of the tile are loaded once per lane and reused for all
// of the lane's tokens.  Logit partial sums are combined across the chunk
// lanes with DPP; softmax state is updated once per tile (online softmax,
// log2 domain); V codes are consumed with the per-token scale folded into
// the probability (acc += (p*s) * code, zacc += p * z).  The workgroup
// merges its 4 wave states in LDS, writes one partial state per split, and
// the last workgroup of a (batch, KV head) -- found with a device-scope
// ticket -- merges the splits in fixed order and writes the output.
#include "common.h"

namespace dqa {
namespace {

constexpr int kWavesPerWG = 4;

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
  int n_tiles;          // quantized tiles + ceil(R / 32)
  int tiles_per_split;
  int splits;
  float q_scale;        // sm_scale * log2(e): logits in the log2 domain
  float rope_theta;
};

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

template <int D, int BITS, int G, bool ROPE>
__global__ __launch_bounds__(256) void kivi_decode_kernel(KiviArgs a) {
  using State = WaveState<D, G, ROPE>;
  constexpr int NCK = State::NCK;    // channel chunks per token
  constexpr int TL = State::TL;      // tokens per wave iteration
  constexpr int IT = State::IT;      // iterations per 32-token tile
  constexpr int WPC = BITS / 2;      // code words per 16-channel chunk
  constexpr int WPT = D * BITS / 32; // code words per token
  constexpr int NP = State::NP;      // RoPE pairs per lane

  __shared__ float lds_anchor[kWavesPerWG][D / 2][2];
  // per-lane rotation offsets E_j = e^{i j w} of the lane's 8 pairs
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
  // RoPE constants of the lane: its 8 pairs i = c0/2 + p; E_j = e^{i j w}
  // (offset of the lane's first token in a tile), step e^{i TL w} (between
  // the lane's successive tokens).
  if constexpr (ROPE) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const double om = pow(static_cast<double>(a.rope_theta), -2.0 * (c0 / 2 + p) / D);
      rope_unit(static_cast<double>(j), om, lds_ej[threadIdx.x][p][0], lds_ej[threadIdx.x][p][1]);
      rope_unit(static_cast<double>(TL), om, S.st_c[p], S.st_s[p]);
    }
    S.omega = (lane < D / 2) ? pow(static_cast<double>(a.rope_theta), -2.0 * lane / D) : 0.0;
  }

  const int tb = split * a.tiles_per_split;
  const int te = min(a.n_tiles, tb + a.tiles_per_split);
  const bool all_valid[IT] = {};
  bool valid[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) valid[it] = true;
  (void)all_valid;

  // ---------------- quantized tiles
  const int tq_end = min(te, a.n_qtiles);
  for (int ti = tb + wave; ti < tq_end; ti += kWavesPerWG) {
    const int tile_pos = ti * kGroup;
    float fc[NP], fs[NP];
    if constexpr (ROPE) tile_rotation<D, G>(S, lds_anchor[wave], lds_ej[ROPE ? threadIdx.x : 0], lane, c0, tile_pos, fc, fs);

    // loads of the tile: K scale/zero (packed), K and V codes, V scale/zero
    uint32_t ks2[8], kz2[8], kw[IT][WPC], vw[IT][WPC];
    float vs[IT], vz[IT];
    const size_t tz = (unit * a.n_qtiles + ti) * D + c0;
    load16p(a.k_scale + tz, ks2);
    load16p(a.k_zero + tz, kz2);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const size_t tok = unit * a.T_q + tile_pos + it * TL + j;
      const uint32_t* kp = a.k_codes + tok * WPT + ck * WPC;
      const uint32_t* vp = a.v_codes + tok * WPT + ck * WPC;
#pragma unroll
      for (int w = 0; w < WPC; ++w) {
        kw[it][w] = kp[w];
        vw[it][w] = vp[w];
      }
      vs[it] = h2f(a.v_scale[tok * (D / kGroup) + c0 / kGroup]);
      vz[it] = h2f(a.v_zero[tok * (D / kGroup) + c0 / kGroup]);
    }

    float lg[IT][G];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float kh[16];
#pragma unroll
      for (int c = 0; c < 16; ++c)
        kh[c] = fmaf(code_at<BITS>(kw[it], c), half_of(ks2[c / 2], c & 1), half_of(kz2[c / 2], c & 1));
      if constexpr (ROPE) S.rotate(kh, fc, fs);
      S.logits(kh, a.q_scale, lg[it]);
    }
    S.update_max(lg, valid);

#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float ps[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = exp2f(lg[it][h] - S.m[h]);
        S.l[h] += p;
        ps[h] = p * vs[it];
        S.zacc[h] = fmaf(p, vz[it], S.zacc[h]);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float code = code_at<BITS>(vw[it], c);
#pragma unroll
        for (int h = 0; h < G; ++h) S.acc[h][c] = fmaf(ps[h], code, S.acc[h][c]);
      }
    }
  }

  // ---------------- fp16 recent tiles (keys stored before RoPE)
  for (int ti = max(tb, a.n_qtiles) + wave; ti < te; ti += kWavesPerWG) {
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
        const float p = exp2f(lg[it][h] - S.m[h]);
        S.l[h] += p;
#pragma unroll
        for (int c = 0; c < 16; ++c) S.acc[h][c] = fmaf(p, v[c], S.acc[h][c]);
      }
    }
  }

  // ---- combine the lanes of each chunk (they hold different tokens)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    S.l[h] = sum_strided<NCK>(S.l[h]);
    S.zacc[h] = sum_strided<NCK>(S.zacc[h]);
#pragma unroll
    for (int c = 0; c < 16; ++c) S.acc[h][c] = sum_strided<NCK>(S.acc[h][c]);
  }
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < 16; ++c) lds_o[wave][h][c0 + c] = S.acc[h][c] + S.zacc[h];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lds_m[wave][h] = S.m[h];
      lds_l[wave][h] = S.l[h];
    }
  }
  __syncthreads();

  // ---- merge the workgroup's waves; write the split's partial state
  float* part = a.partials + (unit * a.splits + split) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, lds_m[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kWavesPerWG; ++w) {
      const float wt = merge_weight(lds_m[w][h], M);
      L = fmaf(lds_l[w][h], wt, L);
      O = fmaf(lds_o[w][h][c], wt, O);
    }
    if (a.splits == 1) {
      a.out[(static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c] = (L > 0.0f) ? O / L : 0.0f;
    } else {
      if (c == 0) {
        part[h * (D + 2) + 0] = M;
        part[h * (D + 2) + 1] = L;
      }
      part[h * (D + 2) + 2 + c] = O;
    }
  }
  if (a.splits == 1) return;

  // ---- the last workgroup of this (batch, KV head) merges all splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(a.tickets + unit, 1u);
    lds_last = (prev == static_cast<unsigned>(a.splits - 1));
  }
  __syncthreads();
  if (!lds_last) return;
  __threadfence();
  const float* parts = a.partials + unit * a.splits * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, parts[(s * G + h) * (D + 2)]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < a.splits; ++s) {
      const float* ps = parts + (s * G + h) * (D + 2);
      const float wt = merge_weight(ps[0], M);
      L = fmaf(ps[1], wt, L);
      O = fmaf(ps[2 + c], wt, O);
    }
    a.out[(static_cast<size_t>(b) * a.Hq + kvh * G + h) * D + c] = (L > 0.0f) ? O / L : 0.0f;
  }
  if (threadIdx.x == 0) a.tickets[unit] = 0u;
}

// ---------------------------------------------------------------- host side

struct Plan {
  int G, n_qtiles, n_tiles, tps, splits;
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
  p->n_tiles = p->n_qtiles + (c->R + kGroup - 1) / kGroup;
  const long long want = (kTargetWorkgroups + static_cast<long long>(p->units) - 1) /
                         static_cast<long long>(p->units > 0 ? p->units : 1);
  long long s = want < 1 ? 1 : want;
  if (s > p->n_tiles) s = p->n_tiles > 0 ? p->n_tiles : 1;
  p->tps = p->n_tiles > 0 ? static_cast<int>((p->n_tiles + s - 1) / s) : 1;
  p->splits = p->n_tiles > 0 ? (p->n_tiles + p->tps - 1) / p->tps : 1;
  p->ticket_bytes = (p->units * sizeof(unsigned) + 255) / 256 * 256;
  p->ws_bytes = p->ticket_bytes +
                p->units * static_cast<size_t>(p->splits) * p->G * (c->d + 2) * sizeof(float);
  return DQA_OK;
}

template <int D, int BITS, int G>
int launch_g(const KiviArgs& a, bool rope, dim3 grid, hipStream_t s) {
  if (rope)
    hipLaunchKernelGGL((kivi_decode_kernel<D, BITS, G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kivi_decode_kernel<D, BITS, G, false>), grid, dim3(256), 0, s, a);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

template <int D, int BITS>
int launch_bits(const KiviArgs& a, int G, bool rope, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: return launch_g<D, BITS, 1>(a, rope, grid, s);
    case 2: return launch_g<D, BITS, 2>(a, rope, grid, s);
    case 4: return launch_g<D, BITS, 4>(a, rope, grid, s);
    default: return DQA_ERR_UNSUPPORTED;
  }
}

template <int D>
int launch_d(const KiviArgs& a, int bits, int G, bool rope, dim3 grid, hipStream_t s) {
  switch (bits) {
    case 2: return launch_bits<D, 2>(a, G, rope, grid, s);
    case 4: return launch_bits<D, 4>(a, G, rope, grid, s);
    case 8: return launch_bits<D, 8>(a, G, rope, grid, s);
    default: return DQA_ERR_BITS;
  }
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
  a.n_tiles = p.n_tiles;
  a.tiles_per_split = p.tps;
  a.splits = p.splits;
  a.q_scale = sm_scale * 1.4426950408889634f;
  a.rope_theta = c->rope_theta;
  const bool rope = c->rope_theta > 0.0f;
  const dim3 grid(p.splits, c->Hkv, c->B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->d == 128) return launch_d<128>(a, c->bits, p.G, rope, grid, s);
  return launch_d<64>(a, c->bits, p.G, rope, grid, s);
}
