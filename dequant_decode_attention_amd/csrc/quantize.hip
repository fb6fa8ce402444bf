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
template <int D>
__global__ __launch_bounds__(D) void quantize_k_kernel(
    const uint16_t* __restrict__ k, int T, int Hkv, int bits,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero) {
  __shared__ uint8_t lds_codes[kGroup][D];
  const int c = threadIdx.x;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const uint16_t* src = k + (unit * T + static_cast<size_t>(tile) * kGroup) * D;

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
  const size_t sz_off = (unit * (T / kGroup) + tile) * D + c;
  scale[sz_off] = p.s16;
  zero[sz_off] = p.z16;
#pragma unroll
  for (int t = 0; t < kGroup; ++t) lds_codes[t][c] = static_cast<uint8_t>(quant_code(x[t], p));
  __syncthreads();

  // Packed words of the tile: 32 tokens x (D*bits/32) words, contiguous.
  const int words_per_token = D * bits / 32;
  const int per_word = 32 / bits;
  uint32_t* dst = codes + (unit * T + static_cast<size_t>(tile) * kGroup) * words_per_token;
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
template <int D>
__global__ __launch_bounds__(D) void quantize_v_kernel(
    const uint16_t* __restrict__ v, int T, int Hkv, int bits,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[D][kGroup];   // [channel][token]
  const int tid = threadIdx.x;
  const int t = tid % kGroup, g = tid / kGroup;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const size_t tok = unit * T + static_cast<size_t>(blk) * kGroup + t;
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
  scale[tok * (D / kGroup) + g] = p.s16;
  zero[tok * (D / kGroup) + g] = p.z16;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) lds_codes[g * kGroup + i][t] = static_cast<uint8_t>(quant_code(x[i], p));
  __syncthreads();
  // channel-major block: stream index c*32 + t, `per_word` codes per word
  const int per_word = 32 / bits;
  uint32_t* dst = codes + (unit * (T / kGroup) + blk) * static_cast<size_t>(D * bits);
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
    hipLaunchKernelGGL(quantize_k_kernel<128>, grid, dim3(128), 0, s, k, T, Hkv, bits, codes, scale, zero);
  else
    hipLaunchKernelGGL(quantize_k_kernel<64>, grid, dim3(64), 0, s, k, T, Hkv, bits, codes, scale, zero);
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
    hipLaunchKernelGGL(quantize_v_kernel<128>, grid, dim3(128), 0, s, v, T, Hkv, bits, codes, scale, zero);
  else
    hipLaunchKernelGGL(quantize_v_kernel<64>, grid, dim3(64), 0, s, v, T, Hkv, bits, codes, scale, zero);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}
