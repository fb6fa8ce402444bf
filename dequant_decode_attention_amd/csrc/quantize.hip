// Quantize + bit-pack kernels for the uniform (KIVI) cache layout.
//
// [P1 para 3] uniform integer quantization: a group's range is split into the
// 2^b levels of the format.  [P1 para 1] each group has a scale factor and a
// zero point; groups of 32.  [P1 para 4] keys are grouped per channel over
// tokens; [P1 para 5] values per token over channels.
//
// Arithmetic (must match the reference bit for bit): min/max exact; scale =
// fp16_rne(fp32(max - min) / fp32(2^b - 1)); zero = min; codes =
// clamp(rint((x - z) / s), 0, 2^b - 1) with IEEE fp32 subtraction and
// division against the stored fp16 scale/zero; scale 0 -> codes 0.  No
// multiply-add appears in this arithmetic, so floating-point contraction
// cannot change it; divisions are IEEE-correct (the library is built without
// fast-math or reciprocal approximations).
#include "common.h"

namespace dqa {
namespace {

struct GroupParams {
  float sf, zf, levels;
  uint16_t s16, z16;
};

__device__ __forceinline__ GroupParams group_params(float mn, float mx, int bits) {
  GroupParams p;
  p.levels = static_cast<float>((1 << bits) - 1);
  const float s32 = (mx - mn) / p.levels;
  p.s16 = f2h(s32);                 // round to nearest even
  p.z16 = f2h(mn);                  // exact: mn is an fp16 value
  p.sf = h2f(p.s16);
  p.zf = mn;
  return p;
}

__device__ __forceinline__ uint32_t quant_code(float x, const GroupParams& p) {
  if (p.sf == 0.0f) return 0u;
  const float t = (x - p.zf) / p.sf;
  const float q = fminf(fmaxf(rintf(t), 0.0f), p.levels);
  return static_cast<uint32_t>(q);
}

// Keys: one workgroup per (32-token tile, KV head, batch); thread c owns
// channel c.  Codes are staged in LDS as bytes and re-read to build the
// token-major packed words.
// Source rows: src_T per (batch, KV head); destination: dst_tiles 32-token
// tiles of capacity per (batch, KV head), this launch's tiles starting at
// tile0 (quantize_pack_k: src_T = T, dst_tiles = T/32, tile0 = 0).
template <int D>
__global__ __launch_bounds__(D) void quantize_k_kernel(
    const uint16_t* __restrict__ k, int src_T, int Hkv, int bits,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0) {
  __shared__ uint8_t lds_codes[kGroup][D];
  const int c = threadIdx.x;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const size_t dtile = unit * dst_tiles + tile0 + tile;        // destination tile
  const uint16_t* src = k + (unit * src_T + static_cast<size_t>(tile) * kGroup) * D;

  float x[kGroup];
#pragma unroll
  for (int t = 0; t < kGroup; ++t) x[t] = h2f(src[t * D + c]);
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int t = 1; t < kGroup; ++t) {
    mn = fminf(mn, x[t]);
    mx = fmaxf(mx, x[t]);
  }
  const GroupParams p = group_params(mn, mx, bits);
  const size_t sz_off = dtile * D + c;
  scale[sz_off] = p.s16;
  zero[sz_off] = p.z16;
#pragma unroll
  for (int t = 0; t < kGroup; ++t) lds_codes[t][c] = static_cast<uint8_t>(quant_code(x[t], p));
  __syncthreads();

  // Packed words of the tile: 32 tokens x (D*bits/32) words, contiguous.
  const int words_per_token = D * bits / 32;
  const int per_word = 32 / bits;
  uint32_t* dst = codes + dtile * kGroup * words_per_token;
  for (int w = c; w < kGroup * words_per_token; w += D) {
    const int t = w / words_per_token;
    const int c0 = (w % words_per_token) * per_word;
    uint32_t word = 0;
    for (int j = 0; j < per_word; ++j) word |= static_cast<uint32_t>(lds_codes[t][c0 + j]) << (j * bits);
    dst[w] = word;
  }
}

// Values: one workgroup per (32-token block, KV head, batch); thread
// (token t, 32-channel group g) reduces its group's min/max in registers and
// stages its codes in LDS; the block is then written channel-major (for each
// channel, the 32 tokens' codes in token order), the layout in which the
// decode kernel's matrix-core operands read 8 consecutive tokens of one
// channel.
// Source rows and destination tiles as quantize_k_kernel.
template <int D>
__global__ __launch_bounds__(D) void quantize_v_kernel(
    const uint16_t* __restrict__ v, int src_T, int Hkv, int bits,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[D][kGroup];   // [channel][token]
  const int tid = threadIdx.x;
  const int t = tid % kGroup, g = tid / kGroup;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const size_t tok = unit * src_T + static_cast<size_t>(blk) * kGroup + t;          // source row
  const size_t dtok = (unit * dst_tiles + tile0 + blk) * kGroup + t;                  // destination token
  const uint4* src = reinterpret_cast<const uint4*>(v + tok * D + g * kGroup);
  float x[kGroup];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = src[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[i * 8 + 2 * j] = h2f(static_cast<uint16_t>(w[j] & 0xFFFFu));
      x[i * 8 + 2 * j + 1] = h2f(static_cast<uint16_t>(w[j] >> 16));
    }
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < kGroup; ++i) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const GroupParams p = group_params(mn, mx, bits);
  scale[dtok * (D / kGroup) + g] = p.s16;
  zero[dtok * (D / kGroup) + g] = p.z16;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) lds_codes[g * kGroup + i][t] = static_cast<uint8_t>(quant_code(x[i], p));
  __syncthreads();
  // channel-major block: stream index c*32 + t, `per_word` codes per word
  const int per_word = 32 / bits;
  uint32_t* dst = codes + (unit * dst_tiles + tile0 + blk) * static_cast<size_t>(D * bits);
  for (int w = tid; w < D * bits; w += D) {
    const int f0 = w * per_word;
    const int c = f0 / kGroup, t0 = f0 % kGroup;
    uint32_t word = 0;
    for (int j = 0; j < per_word; ++j) word |= static_cast<uint32_t>(lds_codes[c][t0 + j]) << (j * bits);
    dst[w] = word;
  }
}

int check_common(const void* in, int B, int Hkv, int T, int d, int bits,
                 const void* codes, const void* scale, const void* zero) {
  if (B < 0 || Hkv < 0 || T < 0) return DQA_ERR_SHAPE;
  if (d != 64 && d != 128) return DQA_ERR_SHAPE;
  if (bits != 2 && bits != 4 && bits != 8) return DQA_ERR_BITS;
  if (static_cast<long long>(B) * Hkv * T == 0) return DQA_OK;
  if (!in || !codes || !scale || !zero) return DQA_ERR_NULL;
  if (static_cast<long long>(B) * Hkv * T * d >= (1LL << 40)) return DQA_ERR_SHAPE;
  return DQA_OK;
}

}  // namespace
}  // namespace dqa

using namespace dqa;

extern "C" int quantize_pack_k(const uint16_t* k, int B, int Hkv, int T, int d,
                               int bits, uint32_t* codes, uint16_t* scale,
                               uint16_t* zero, void* stream) {
  int st = check_common(k, B, Hkv, T, d, bits, codes, scale, zero);
  if (st != DQA_OK) return st;
  if (T % kGroup != 0) return DQA_ERR_SHAPE;
  if (static_cast<long long>(B) * Hkv * T == 0) return DQA_OK;
  if (B > 65535 || Hkv > 65535) return DQA_ERR_SHAPE;
  dim3 grid(T / kGroup, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 128)
    hipLaunchKernelGGL(quantize_k_kernel<128>, grid, dim3(128), 0, s, k, T, Hkv, bits, codes, scale, zero,
                       T / kGroup, 0);
  else
    hipLaunchKernelGGL(quantize_k_kernel<64>, grid, dim3(64), 0, s, k, T, Hkv, bits, codes, scale, zero,
                       T / kGroup, 0);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

extern "C" int quantize_pack_v(const uint16_t* v, int B, int Hkv, int T, int d,
                               int bits, uint32_t* codes, uint16_t* scale,
                               uint16_t* zero, void* stream) {
  int st = check_common(v, B, Hkv, T, d, bits, codes, scale, zero);
  if (st != DQA_OK) return st;
  if (T % kGroup != 0) return DQA_ERR_SHAPE;
  if (static_cast<long long>(B) * Hkv * T == 0) return DQA_OK;
  if (B > 65535 || Hkv > 65535) return DQA_ERR_SHAPE;
  dim3 grid(T / kGroup, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 128)
    hipLaunchKernelGGL(quantize_v_kernel<128>, grid, dim3(128), 0, s, v, T, Hkv, bits, codes, scale, zero,
                       T / kGroup, 0);
  else
    hipLaunchKernelGGL(quantize_v_kernel<64>, grid, dim3(64), 0, s, v, T, Hkv, bits, codes, scale, zero,
                       T / kGroup, 0);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

// ------------------------------------------------------------ streaming append
//
// [P1 para 8]: the newest tokens stay in fp16 (up to 128) because a key
// channel's group statistics need tokens not generated yet; groups are
// quantized once enough tokens are there.  kivi_append stages the recent
// rows followed by the new ones in the workspace, quantizes the oldest 32
// rows of the staged sequence per flush with the kernels above (into the
// quantized buffers' capacity, after the T_q tokens already there), and
// copies the rows that stay in fp16 back to the front of the recent
// buffers.

namespace dqa {
namespace {

// Rows [0, R) of src_a (R_cap rows per unit) followed by rows [0, n) of
// src_b (n rows per unit) into dst (R + n rows per unit), 16 bytes per
// thread; d / 8 chunks per row.
__global__ __launch_bounds__(256) void stage_rows_kernel(const uint16_t* __restrict__ src_a, int R, int R_cap,
                                                         const uint16_t* __restrict__ src_b, int n,
                                                         uint16_t* __restrict__ dst, size_t units, int d) {
  const int cpr = d / 8;
  const size_t rows = static_cast<size_t>(R) + n;
  const size_t total = units * rows * cpr;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t u = i / (rows * cpr);
    const size_t rem = i % (rows * cpr);
    const int r = static_cast<int>(rem / cpr), ch = static_cast<int>(rem % cpr);
    const uint16_t* s = r < R ? src_a + (u * R_cap + r) * d : src_b + (u * n + (r - R)) * d;
    reinterpret_cast<uint4*>(dst + (u * rows + r) * d)[ch] = reinterpret_cast<const uint4*>(s)[ch];
  }
}

// Rows [skip, skip + keep) of src (rows per unit) to rows [0, keep) of dst
// (R_cap rows per unit).
__global__ __launch_bounds__(256) void unstage_rows_kernel(const uint16_t* __restrict__ src, int rows, int skip,
                                                           int keep, uint16_t* __restrict__ dst, int R_cap,
                                                           size_t units, int d) {
  const int cpr = d / 8;
  const size_t total = units * static_cast<size_t>(keep) * cpr;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t u = i / (static_cast<size_t>(keep) * cpr);
    const size_t rem = i % (static_cast<size_t>(keep) * cpr);
    const int r = static_cast<int>(rem / cpr), ch = static_cast<int>(rem % cpr);
    reinterpret_cast<uint4*>(dst + (u * R_cap + r) * d)[ch] =
        reinterpret_cast<const uint4*>(src + (u * rows + skip + r) * d)[ch];
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Flushes (groups of 32 quantized) when `rows` tokens sit in the recent zone
// bounded by R_max: while more than R_max and at least 32 remain.
int flush_count(int rows, int R_max) {
  int f = 0;
  while (rows > R_max && rows >= kGroup) {
    rows -= kGroup;
    ++f;
  }
  return f;
}

int append_shape(const dqa_kivi_cache* c, int n_new) {
  if (!c) return DQA_ERR_NULL;
  if (c->B < 0 || c->Hkv < 0 || n_new < 0) return DQA_ERR_SHAPE;
  if (c->d != 64 && c->d != 128) return DQA_ERR_SHAPE;
  if (c->bits != 2 && c->bits != 4 && c->bits != 8) return DQA_ERR_BITS;
  if (c->T_q < 0 || c->T_q % kGroup != 0 || c->R < 0 || c->R > kMaxRecent) return DQA_ERR_SHAPE;
  if (c->T_cap < 0 || c->T_cap % kGroup != 0 || (c->T_cap > 0 && c->T_cap < c->T_q)) return DQA_ERR_SHAPE;
  if (c->R_cap < 0 || (c->R_cap > 0 && c->R_cap < c->R)) return DQA_ERR_SHAPE;
  if (static_cast<long long>(c->R) + n_new > (1 << 24)) return DQA_ERR_SHAPE;
  if (c->B > 65535 || c->Hkv > 65535) return DQA_ERR_SHAPE;
  return DQA_OK;
}

size_t append_ws_bytes(const dqa_kivi_cache* c, int n_new) {
  const size_t rows = static_cast<size_t>(c->R) + n_new;
  const size_t n = 2 * static_cast<size_t>(c->B) * c->Hkv * rows * c->d * sizeof(uint16_t);
  return n < 256 ? 256 : n;
}

unsigned copy_blocks(size_t chunks) {
  size_t b = (chunks + 255) / 256;
  if (b > 4096) b = 4096;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace
}  // namespace dqa

extern "C" size_t kivi_append_workspace_bytes(const dqa_kivi_cache* cache, int n_new) {
  if (append_shape(cache, n_new) != DQA_OK) return 0;
  return append_ws_bytes(cache, n_new);
}

extern "C" int kivi_append(dqa_kivi_cache* c, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                           int R_max, void* ws, size_t ws_bytes, void* stream) {
  int st = append_shape(c, n_new);
  if (st != DQA_OK) return st;
  if (R_max < 0 || R_max > kMaxRecent) return DQA_ERR_SHAPE;
  const int rows = c->R + n_new;
  const int f = flush_count(rows, R_max);
  const int R_new = rows - f * kGroup;
  const int T_new = c->T_q + f * kGroup;
  const int T_cap = c->T_cap > 0 ? c->T_cap : c->T_q;
  const int R_cap = c->R_cap > 0 ? c->R_cap : c->R;
  if (T_new > T_cap || R_new > R_cap) return DQA_ERR_SHAPE;
  const size_t units = static_cast<size_t>(c->B) * c->Hkv;
  if (units == 0 || rows == 0) {
    c->T_q = T_new;
    c->R = R_new;
    return DQA_OK;
  }
  if (n_new > 0 && (!k_new || !v_new)) return DQA_ERR_NULL;
  if (c->R > 0 || R_new > 0) {
    if (!c->k_recent || !c->v_recent) return DQA_ERR_NULL;
    if (!aligned16(c->k_recent) || !aligned16(c->v_recent)) return DQA_ERR_ALIGN;
  }
  if (f > 0) {
    if (!c->k_codes || !c->k_scale || !c->k_zero || !c->v_codes || !c->v_scale || !c->v_zero) return DQA_ERR_NULL;
    if (!aligned16(c->k_codes) || !aligned16(c->v_codes) || !aligned16(c->k_scale) || !aligned16(c->k_zero) ||
        !aligned16(c->v_scale) || !aligned16(c->v_zero))
      return DQA_ERR_ALIGN;
  }
  if (n_new > 0 && (!aligned16(k_new) || !aligned16(v_new))) return DQA_ERR_ALIGN;
  if (!ws || ws_bytes < append_ws_bytes(c, n_new)) return DQA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DQA_ERR_ALIGN;

  const int d = c->d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint16_t* wk = static_cast<uint16_t*>(ws);
  uint16_t* wv = wk + units * static_cast<size_t>(rows) * d;
  const size_t chunks = units * static_cast<size_t>(rows) * (d / 8);
  hipLaunchKernelGGL(stage_rows_kernel, dim3(copy_blocks(chunks)), dim3(256), 0, s, c->k_recent, c->R, R_cap, k_new,
                     n_new, wk, units, d);
  hipLaunchKernelGGL(stage_rows_kernel, dim3(copy_blocks(chunks)), dim3(256), 0, s, c->v_recent, c->R, R_cap, v_new,
                     n_new, wv, units, d);
  DQA_CHECK_LAUNCH();
  if (f > 0) {
    uint32_t* kc = const_cast<uint32_t*>(c->k_codes);
    uint16_t* ks = const_cast<uint16_t*>(c->k_scale);
    uint16_t* kz = const_cast<uint16_t*>(c->k_zero);
    uint32_t* vc = const_cast<uint32_t*>(c->v_codes);
    uint16_t* vs = const_cast<uint16_t*>(c->v_scale);
    uint16_t* vz = const_cast<uint16_t*>(c->v_zero);
    const dim3 grid(f, c->Hkv, c->B);
    const int dst_tiles = T_cap / kGroup, tile0 = c->T_q / kGroup;
    if (d == 128) {
      hipLaunchKernelGGL(quantize_k_kernel<128>, grid, dim3(128), 0, s, wk, rows, c->Hkv, c->bits, kc, ks, kz,
                         dst_tiles, tile0);
      hipLaunchKernelGGL(quantize_v_kernel<128>, grid, dim3(128), 0, s, wv, rows, c->Hkv, c->bits, vc, vs, vz,
                         dst_tiles, tile0);
    } else {
      hipLaunchKernelGGL(quantize_k_kernel<64>, grid, dim3(64), 0, s, wk, rows, c->Hkv, c->bits, kc, ks, kz,
                         dst_tiles, tile0);
      hipLaunchKernelGGL(quantize_v_kernel<64>, grid, dim3(64), 0, s, wv, rows, c->Hkv, c->bits, vc, vs, vz,
                         dst_tiles, tile0);
    }
    DQA_CHECK_LAUNCH();
  }
  if (R_new > 0) {
    const size_t kchunks = units * static_cast<size_t>(R_new) * (d / 8);
    hipLaunchKernelGGL(unstage_rows_kernel, dim3(copy_blocks(kchunks)), dim3(256), 0, s, wk, rows, f * kGroup, R_new,
                       const_cast<uint16_t*>(c->k_recent), R_cap, units, d);
    hipLaunchKernelGGL(unstage_rows_kernel, dim3(copy_blocks(kchunks)), dim3(256), 0, s, wv, rows, f * kGroup, R_new,
                       const_cast<uint16_t*>(c->v_recent), R_cap, units, d);
    DQA_CHECK_LAUNCH();
  }
  c->T_q = T_new;
  c->R = R_new;
  return DQA_OK;
}
