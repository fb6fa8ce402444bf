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
  float sf, zf, levels, rcp;
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
  // approximate reciprocal for the fast quotient (0 for a zero scale, whose
  // codes are all 0)
  p.rcp = p.sf == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(p.sf);
  return p;
}

// Packed fp16 minimum / maximum of two pairs (exact; the inputs are finite
// fp16 values, so the plain instructions are used without the canonicalizing
// moves the compiler would add for signalling NaNs), and a DPP lane exchange
// of a 32-bit register.  A lane permute (DPP or row swap) may read a
// register only two wait states after a vector instruction wrote it; the
// compiler ensures that only for instructions it generates, so the
// permutes below take their input through `settled`.
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
__device__ __forceinline__ uint32_t settled(uint32_t v) {
  asm("s_nop 1" : "+v"(v));
  return v;
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(settled(v)), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128;   // row_ror:8 (lane i <- lane (i + 8) mod 16 within its row)
// Packed min (MAX = false) or max of lane L and lane L ^ 32 (rows32) or
// L ^ 16, through the row-swap permutes; every lane gets the result.  The
// permute's two results are copied into scalars before use.
template <bool MAX>
__device__ __forceinline__ uint32_t pk_swap_rows(uint32_t x, bool rows32) {
  x = settled(x);
  uint32_t r0, r1;
  if (rows32) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return MAX ? pk_max_h2(r0, r1) : pk_min_h2(r0, r1);
}

// x - z for the fp16 value in half H of word w: one mixed-precision FMA
// (x * 1 - z, a single rounding), which equals the fp32 subtraction of the
// widened value.
template <int H>
__device__ __forceinline__ float minus_zero(uint32_t w, float zf) {
  return __builtin_fmaf(half_of<H>(w), opaque_const(1.0f), -zf);
}

// code = clamp(rint((x - z) / s), 0, 2^b - 1) with the IEEE quotient, for
// the fp16 value x in half H of word w, from its group's zero, reciprocal
// and (only on the exact path) scale, read from `sf`.  The quotient is first
// approximated as t * rcp(s): rcp is within 1 ulp of 1/s, so t * rcp(s) and
// the IEEE quotient t / s differ by at most 2^-22 of t / s, and t / s < 2^9
// (t <= max - min, and s is (max - min) / (2^b - 1) rounded to fp16, at
// worst halved by subnormal rounding) -- less than 2^-13.  Unless the
// approximation lies within 2^-12 of a half-integer, both round to the same
// integer (and neither is a tie); otherwise the IEEE division decides.  The
// result is the IEEE-division code in every case.
template <int BITS, int H>
__device__ __forceinline__ float quant_code_w(uint32_t w, float zf, float rcp, const float* sf) {
  const float t = minus_zero<H>(w, zf);
  const float y = t * rcp;
  float q = rintf(y);
  // |y - rint(y)| >= 0.5 - 2^-12: y within 2^-12 of a half-integer
  if (__builtin_expect(__builtin_fabsf(y - q) >= 0.499755859375f, 0)) q = rintf(t / *sf);
  return __builtin_amdgcn_fmed3f(q, 0.0f, static_cast<float>((1 << BITS) - 1));
}
template <int BITS>
__device__ __forceinline__ float quant_code_e(uint32_t w, int e, float zf, float rcp, const float* sf) {
  return (e & 1) ? quant_code_w<BITS, 1>(w, zf, rcp, sf) : quant_code_w<BITS, 0>(w, zf, rcp, sf);
}

// Both halves of the result hold min (or max) of the two halves of w.
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

// Tile of 32 tokens x D channels, thread (token quad tq, channel octet co):
// tokens 4 tq .. 4 tq + 3, channels 8 co .. 8 co + 7, read as four 16-byte
// loads.  w[r][j] = token 4 tq + r, channels 8 co + 2 j (low half) and
// 8 co + 2 j + 1 (high half).
template <int D>
__device__ __forceinline__ void load_quad_octet(const uint16_t* rows, int tq, int co, uint32_t (*w)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint4 u = *reinterpret_cast<const uint4*>(rows + static_cast<size_t>(4 * tq + r) * D + 8 * co);
    w[r][0] = u.x;
    w[r][1] = u.y;
    w[r][2] = u.z;
    w[r][3] = u.w;
  }
}

// Keys: one workgroup per (32-token tile, KV head, batch), D threads; thread
// tid = (D/8) tq + co holds tokens 4 tq .. 4 tq + 3 of channels 8 co ..
// 8 co + 7, so a wave's 16-byte loads cover whole rows.  A channel's group
// spans the 8 threads of equal co: their partial min/max (packed fp16, exact)
// combine across the wave's 16-lane rows with the row-swap permutes and, at
// head dim 128, across the two waves through LDS (at 64, one wave holds all
// 8 token quads and a DPP rotation combines the two halves of each row).
// Each thread assembles its (token, octet) pieces of the token-major code
// rows in LDS, and the tile is then copied out contiguously; thread
// (tq, co) also writes the scale and zero of channel 8 co + tq.
// Source rows: src_T per (batch, KV head); destination: dst_tiles 32-token
// tiles of capacity per (batch, KV head), this launch's tiles starting at
// tile0 (quantize_pack_k: src_T = T, dst_tiles = T/32, tile0 = 0).
template <int D, int BITS>
__device__ __forceinline__ void quantize_k_tile(
    const uint16_t* __restrict__ k, int src_T, int Hkv,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0, int tile, int h, int b) {
  constexpr int NCO = D / 8;             // channel octets per token
  // per channel: zero, reciprocal of the scale, scale (fp32)
  __shared__ __attribute__((aligned(16))) float lds_par[3][NCO][8];
  const int tid = threadIdx.x, tq = tid / NCO, co = tid % NCO;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const size_t dtile = unit * dst_tiles + tile0 + tile;        // destination tile
  const uint16_t* src = k + (unit * src_T + static_cast<size_t>(tile) * kGroup) * D;

  // min/max per channel pair in packed fp16 (exact: the inputs are fp16),
  // over the thread's 4 tokens and then over the channel's 8 adjacent lanes
  uint32_t w[4][4];
  load_quad_octet<D>(src, tq, co, w);
  uint32_t mnp[4], mxp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mnp[j] = pk_min_h2(pk_min_h2(w[0][j], w[1][j]), pk_min_h2(w[2][j], w[3][j]));
    mxp[j] = pk_max_h2(pk_max_h2(w[0][j], w[1][j]), pk_max_h2(w[2][j], w[3][j]));
    if constexpr (D == 64) {   // token quads tq and tq ^ 1 share a 16-lane row
      mnp[j] = pk_min_h2(mnp[j], dpp_u32<kDppRowRor8>(mnp[j]));
      mxp[j] = pk_max_h2(mxp[j], dpp_u32<kDppRowRor8>(mxp[j]));
    }
    mnp[j] = pk_swap_rows<false>(pk_swap_rows<false>(mnp[j], true), false);
    mxp[j] = pk_swap_rows<true>(pk_swap_rows<true>(mxp[j], true), false);
  }
  if constexpr (D == 128) {   // the other wave's four token quads
    __shared__ __attribute__((aligned(16))) uint32_t lds_red[2][NCO][8];
    const int wave = tid / kWave;
    if ((tid % kWave) < NCO) {
      *reinterpret_cast<uint4*>(&lds_red[wave][co][0]) = uint4{mnp[0], mnp[1], mnp[2], mnp[3]};
      *reinterpret_cast<uint4*>(&lds_red[wave][co][4]) = uint4{mxp[0], mxp[1], mxp[2], mxp[3]};
    }
    __syncthreads();
    const uint4 omn = *reinterpret_cast<const uint4*>(&lds_red[1 - wave][co][0]);
    const uint4 omx = *reinterpret_cast<const uint4*>(&lds_red[1 - wave][co][4]);
    mnp[0] = pk_min_h2(mnp[0], omn.x);
    mnp[1] = pk_min_h2(mnp[1], omn.y);
    mnp[2] = pk_min_h2(mnp[2], omn.z);
    mnp[3] = pk_min_h2(mnp[3], omn.w);
    mxp[0] = pk_max_h2(mxp[0], omx.x);
    mxp[1] = pk_max_h2(mxp[1], omx.y);
    mxp[2] = pk_max_h2(mxp[2], omx.z);
    mxp[3] = pk_max_h2(mxp[3], omx.w);
  }
  // per token: the octet's codes, accumulated as exact integers in fp32
  // (code e times 2^(BITS e); two halves of 4 codes each above 2 bits) or,
  // at 8 bits, converted into the bytes of two words
  float acc[4][2] = {{0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}, {0.0f, 0.0f}};
  uint32_t w8[4][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};
  // thread (tq, co) derives the parameters of channel 8 co + tq, stores its
  // scale and zero, and shares (zero, reciprocal, scale) through LDS
  {
    uint32_t mnw = mnp[0], mxw = mxp[0];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
      mnw = (tq >> 1) == j ? mnp[j] : mnw;
      mxw = (tq >> 1) == j ? mxp[j] : mxw;
    }
    const int sh = (tq & 1) * 16;
    const GroupParams p = group_params(h2f(static_cast<uint16_t>(mnw >> sh)), h2f(static_cast<uint16_t>(mxw >> sh)), BITS);
    scale[dtile * D + 8 * co + tq] = p.s16;
    zero[dtile * D + 8 * co + tq] = p.z16;
    lds_par[0][co][tq] = p.zf;
    lds_par[1][co][tq] = p.rcp;
    lds_par[2][co][tq] = p.sf;
  }
  __syncthreads();
  float pz[8], pr[8];
  *reinterpret_cast<float4*>(&pz[0]) = *reinterpret_cast<const float4*>(&lds_par[0][co][0]);
  *reinterpret_cast<float4*>(&pz[4]) = *reinterpret_cast<const float4*>(&lds_par[0][co][4]);
  *reinterpret_cast<float4*>(&pr[0]) = *reinterpret_cast<const float4*>(&lds_par[1][co][0]);
  *reinterpret_cast<float4*>(&pr[4]) = *reinterpret_cast<const float4*>(&lds_par[1][co][4]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float c = quant_code_e<BITS>(w[r][e >> 1], e, pz[e], pr[e], &lds_par[2][co][e]);
      if constexpr (BITS == 2) acc[r][0] = fmaf(c, static_cast<float>(1u << (2 * e)), acc[r][0]);
      else if constexpr (BITS == 4) acc[r][e >> 2] = fmaf(c, static_cast<float>(1u << (4 * (e & 3))), acc[r][e >> 2]);
      else w8[r][e >> 2] = __builtin_amdgcn_cvt_pk_u8_f32(c, e & 3, w8[r][e >> 2]);
    }
  }
  // The tile's codes (32 token rows of D * BITS / 8 bytes, this octet's at
  // byte co * BITS of a row) are assembled in LDS, then copied out with
  // 4 * BITS contiguous bytes per thread.
  constexpr int RB = D * BITS / 8;
  __shared__ __attribute__((aligned(16))) uint32_t lds_tile[kGroup * RB / 4];
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_tile) + co * BITS;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint8_t* row = lds + (4 * tq + r) * RB;
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint2*>(row) = uint2{w8[r][0], w8[r][1]};
    } else if constexpr (BITS == 4) {
      *reinterpret_cast<uint32_t*>(row) =
          static_cast<uint32_t>(acc[r][0]) | (static_cast<uint32_t>(acc[r][1]) << 16);
    } else {
      *reinterpret_cast<uint16_t*>(row) = static_cast<uint16_t>(static_cast<uint32_t>(acc[r][0]));
    }
  }
  __syncthreads();
  uint32_t* dst = codes + dtile * (kGroup * RB / 4) + tid * BITS;   // 4 * BITS bytes per thread
  const uint32_t* from = lds_tile + tid * BITS;
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(from);
  } else {
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(from)[i];
  }
}

// Values: one workgroup per (32-token block, KV head, batch), D threads;
// thread tid = (D/8) tq + co holds tokens 4 tq .. 4 tq + 3 of channels
// 8 co .. 8 co + 7, so the 4 threads of a (token, 32-channel) group are
// adjacent lanes and combine their partial min/max with DPP.  The block is
// written channel-major (for each channel, the 32 tokens' codes in token
// order, the layout in which the decode kernel's matrix-core operands read
// 8 consecutive tokens of one channel): each thread puts the 4 tokens'
// codes of each of its channels (4 * BITS bits) into LDS, then thread c
// copies channel c's 4 * BITS bytes out.
// Source rows and destination tiles as quantize_k_kernel.
template <int D, int BITS>
__device__ __forceinline__ void quantize_v_tile(
    const uint16_t* __restrict__ v, int src_T, int Hkv,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0, int blk, int h, int b) {
  constexpr int NCO = D / 8;             // channel octets per token
  constexpr int CB = 4 * BITS;           // bytes of one channel in a block
  // LDS byte offset of channel c: 4 bytes of padding per 8 channels put the
  // channels that one store instruction touches in different banks
  __shared__ __attribute__((aligned(16))) uint32_t lds_codes[(D * CB + (D / 8) * 4) / 4];
  const int tid = threadIdx.x, tq = tid / NCO, co = tid % NCO;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const uint16_t* src = v + (unit * src_T + static_cast<size_t>(blk) * kGroup) * D;
  const size_t dtok0 = (unit * dst_tiles + tile0 + blk) * kGroup;   // destination token of row 0

  uint32_t w[4][4];
  load_quad_octet<D>(src, tq, co, w);
  // per channel: the 4 tokens' codes (token r at bit BITS r), accumulated
  // as exact integers in fp32 or, at 8 bits, converted into bytes
  float accv[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  uint32_t w8[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  // min/max of each of the 4 tokens over the group's 4 adjacent lanes; lane
  // co % 4 == r then derives token r's parameters, stores its scale and
  // zero, and the quad shares (zero, reciprocal, scale) by DPP broadcasts
  float mnr = 0.0f, mxr = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t mnw = pk_min_halves(pk_min_h2(pk_min_h2(w[r][0], w[r][1]), pk_min_h2(w[r][2], w[r][3])));
    uint32_t mxw = pk_max_halves(pk_max_h2(pk_max_h2(w[r][0], w[r][1]), pk_max_h2(w[r][2], w[r][3])));
    mnw = pk_min_h2(mnw, dpp_u32<kDppQuadXor1>(mnw));
    mxw = pk_max_h2(mxw, dpp_u32<kDppQuadXor1>(mxw));
    mnw = pk_min_h2(mnw, dpp_u32<kDppQuadXor2>(mnw));
    mxw = pk_max_h2(mxw, dpp_u32<kDppQuadXor2>(mxw));
    mnr = (co & 3) == r ? h2f(static_cast<uint16_t>(mnw)) : mnr;
    mxr = (co & 3) == r ? h2f(static_cast<uint16_t>(mxw)) : mxr;
  }
  const GroupParams pm = group_params(mnr, mxr, BITS);
  scale[(dtok0 + 4 * tq + (co & 3)) * (D / kGroup) + co / 4] = pm.s16;
  zero[(dtok0 + 4 * tq + (co & 3)) * (D / kGroup) + co / 4] = pm.z16;
  float pz[4], pr[4], ps[4];
  pz[0] = dpp<0x00>(pm.zf);
  pz[1] = dpp<0x55>(pm.zf);
  pz[2] = dpp<0xAA>(pm.zf);
  pz[3] = dpp<0xFF>(pm.zf);
  pr[0] = dpp<0x00>(pm.rcp);
  pr[1] = dpp<0x55>(pm.rcp);
  pr[2] = dpp<0xAA>(pm.rcp);
  pr[3] = dpp<0xFF>(pm.rcp);
  ps[0] = dpp<0x00>(pm.sf);
  ps[1] = dpp<0x55>(pm.sf);
  ps[2] = dpp<0xAA>(pm.sf);
  ps[3] = dpp<0xFF>(pm.sf);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = quant_code_e<BITS>(w[r][e >> 1], e, pz[r], pr[r], &ps[r]);
      if constexpr (BITS == 8) w8[e] = __builtin_amdgcn_cvt_pk_u8_f32(c, r, w8[e]);
      else accv[e] = fmaf(c, static_cast<float>(1u << (BITS * r)), accv[e]);
    }
  }
  uint8_t* lds = reinterpret_cast<uint8_t*>(lds_codes);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = 8 * co + e;
    uint8_t* at = lds + c * CB + (c >> 3) * 4 + tq * (BITS / 2);
    if constexpr (BITS == 2) *at = static_cast<uint8_t>(static_cast<uint32_t>(accv[e]));
    else if constexpr (BITS == 4) *reinterpret_cast<uint16_t*>(at) = static_cast<uint16_t>(static_cast<uint32_t>(accv[e]));
    else *reinterpret_cast<uint32_t*>(at) = w8[e];
  }
  __syncthreads();
  // thread c: channel c's CB bytes (4-byte aligned in LDS) to the block
  const int c = tid;
  const uint32_t* from = lds_codes + (c * CB + (c >> 3) * 4) / 4;
  uint32_t* to = codes + (unit * dst_tiles + tile0 + blk) * static_cast<size_t>(D * BITS) + c * (CB / 4);
  if constexpr (BITS == 2) {
    *reinterpret_cast<uint2*>(to) = uint2{from[0], from[1]};
  } else {
#pragma unroll
    for (int i = 0; i < CB / 16; ++i)
      reinterpret_cast<uint4*>(to)[i] = uint4{from[4 * i], from[4 * i + 1], from[4 * i + 2], from[4 * i + 3]};
  }
}

template <int D, int BITS>
__global__ __launch_bounds__(D) void quantize_k_kernel(
    const uint16_t* __restrict__ k, int src_T, int Hkv,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0) {
  quantize_k_tile<D, BITS>(k, src_T, Hkv, codes, scale, zero, dst_tiles, tile0, blockIdx.x, blockIdx.y, blockIdx.z);
}
template <int D, int BITS>
__global__ __launch_bounds__(D) void quantize_v_kernel(
    const uint16_t* __restrict__ v, int src_T, int Hkv,
    uint32_t* __restrict__ codes, uint16_t* __restrict__ scale,
    uint16_t* __restrict__ zero, int dst_tiles, int tile0) {
  quantize_v_tile<D, BITS>(v, src_T, Hkv, codes, scale, zero, dst_tiles, tile0, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Keys and values of the same tiles in one launch (grid z = 2 B: keys for
// z < B, values for z >= B), for the streaming append.
struct QuantizeOut {
  uint32_t* codes;
  uint16_t* scale;
  uint16_t* zero;
};
template <int D, int BITS>
__global__ __launch_bounds__(D) void quantize_kv_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                        int src_T, int Hkv, QuantizeOut ko, QuantizeOut vo,
                                                        int dst_tiles, int tile0, int B) {
  const int z = blockIdx.z;
  if (z < B)
    quantize_k_tile<D, BITS>(k, src_T, Hkv, ko.codes, ko.scale, ko.zero, dst_tiles, tile0, blockIdx.x, blockIdx.y, z);
  else
    quantize_v_tile<D, BITS>(v, src_T, Hkv, vo.codes, vo.scale, vo.zero, dst_tiles, tile0, blockIdx.x, blockIdx.y,
                             z - B);
}

void launch_quantize_kv(int d, int bits, dim3 grid, hipStream_t s, const uint16_t* k, const uint16_t* v, int src_T,
                        int Hkv, QuantizeOut ko, QuantizeOut vo, int dst_tiles, int tile0, int B) {
#define DQA_QKV(D, BITS)                                                                                   \
  hipLaunchKernelGGL((quantize_kv_kernel<D, BITS>), grid, dim3(D), 0, s, k, v, src_T, Hkv, ko, vo, dst_tiles, \
                     tile0, B)
  if (d == 128) {
    if (bits == 2) DQA_QKV(128, 2);
    else if (bits == 4) DQA_QKV(128, 4);
    else DQA_QKV(128, 8);
  } else {
    if (bits == 2) DQA_QKV(64, 2);
    else if (bits == 4) DQA_QKV(64, 4);
    else DQA_QKV(64, 8);
  }
#undef DQA_QKV
}

// Launch the K or V quantizer for head dim d and width bits over grid
// (tiles, Hkv, B).
template <bool KEYS>
void launch_quantize(int d, int bits, dim3 grid, hipStream_t s, const uint16_t* x, int src_T, int Hkv,
                     uint32_t* codes, uint16_t* scale, uint16_t* zero, int dst_tiles, int tile0) {
#define DQA_QLAUNCH(D, BITS)                                                                             \
  hipLaunchKernelGGL((KEYS ? quantize_k_kernel<D, BITS> : quantize_v_kernel<D, BITS>), grid, dim3(D), 0, s, \
                     x, src_T, Hkv, codes, scale, zero, dst_tiles, tile0)
  if (d == 128) {
    if (bits == 2) DQA_QLAUNCH(128, 2);
    else if (bits == 4) DQA_QLAUNCH(128, 4);
    else DQA_QLAUNCH(128, 8);
  } else {
    if (bits == 2) DQA_QLAUNCH(64, 2);
    else if (bits == 4) DQA_QLAUNCH(64, 4);
    else DQA_QLAUNCH(64, 8);
  }
#undef DQA_QLAUNCH
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
  if (!aligned16(k) || !aligned16(codes)) return DQA_ERR_ALIGN;
  dim3 grid(T / kGroup, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_quantize<true>(d, bits, grid, s, k, T, Hkv, codes, scale, zero, T / kGroup, 0);
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
  if (!aligned16(v) || !aligned16(codes)) return DQA_ERR_ALIGN;
  dim3 grid(T / kGroup, Hkv, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch_quantize<false>(d, bits, grid, s, v, T, Hkv, codes, scale, zero, T / kGroup, 0);
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
// Keys and values in one launch: index space [0, 2 total), the second half
// for the values.
struct RowPair {
  const uint16_t* a;   // recent rows (R_cap per unit)
  const uint16_t* b;   // new rows (n per unit)
  uint16_t* dst;       // staged rows (R + n per unit)
};
__global__ __launch_bounds__(256) void stage_rows_kernel(RowPair kp, RowPair vp, int R, int R_cap, int n,
                                                         size_t units, int d) {
  const int cpr = d / 8;
  const size_t rows = static_cast<size_t>(R) + n;
  const size_t total = units * rows * cpr;
  for (size_t i2 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i2 < 2 * total;
       i2 += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const RowPair& p = i2 < total ? kp : vp;
    const size_t i = i2 < total ? i2 : i2 - total;
    const size_t u = i / (rows * cpr);
    const size_t rem = i % (rows * cpr);
    const int r = static_cast<int>(rem / cpr), ch = static_cast<int>(rem % cpr);
    const uint16_t* s = r < R ? p.a + (u * R_cap + r) * d : p.b + (u * n + (r - R)) * d;
    reinterpret_cast<uint4*>(p.dst + (u * rows + r) * d)[ch] = reinterpret_cast<const uint4*>(s)[ch];
  }
}

// Rows [skip, skip + keep) of src (rows per unit) to rows [0, keep) of dst
// (R_cap rows per unit), keys and values in one launch.
__global__ __launch_bounds__(256) void unstage_rows_kernel(const uint16_t* __restrict__ ksrc,
                                                           const uint16_t* __restrict__ vsrc, int rows, int skip,
                                                           int keep, uint16_t* __restrict__ kdst,
                                                           uint16_t* __restrict__ vdst, int R_cap, size_t units,
                                                           int d) {
  const int cpr = d / 8;
  const size_t total = units * static_cast<size_t>(keep) * cpr;
  for (size_t i2 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i2 < 2 * total;
       i2 += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const bool keys = i2 < total;
    const size_t i = keys ? i2 : i2 - total;
    const size_t u = i / (static_cast<size_t>(keep) * cpr);
    const size_t rem = i % (static_cast<size_t>(keep) * cpr);
    const int r = static_cast<int>(rem / cpr), ch = static_cast<int>(rem % cpr);
    reinterpret_cast<uint4*>((keys ? kdst : vdst) + (u * R_cap + r) * d)[ch] =
        reinterpret_cast<const uint4*>((keys ? ksrc : vsrc) + (u * rows + skip + r) * d)[ch];
  }
}

// Append without a flush: new rows [0, n) of each unit to window rows
// [R, R + n) (R_cap rows per unit), keys and values in one launch.
__global__ __launch_bounds__(256) void append_rows_kernel(const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new, int n, int R,
                                                          uint16_t* __restrict__ k_rec, uint16_t* __restrict__ v_rec,
                                                          int R_cap, size_t units, int d) {
  const int cpr = d / 8;
  const size_t total = units * static_cast<size_t>(n) * cpr;
  for (size_t i2 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i2 < 2 * total;
       i2 += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const bool keys = i2 < total;
    const size_t i = keys ? i2 : i2 - total;
    const size_t u = i / (static_cast<size_t>(n) * cpr);
    const size_t rem = i % (static_cast<size_t>(n) * cpr);
    const int r = static_cast<int>(rem / cpr), ch = static_cast<int>(rem % cpr);
    reinterpret_cast<uint4*>((keys ? k_rec : v_rec) + (u * R_cap + R + r) * d)[ch] =
        reinterpret_cast<const uint4*>((keys ? k_new : v_new) + (u * n + r) * d)[ch];
  }
}

// Flush whose f groups are the window's oldest rows (32 f <= R): one
// workgroup per (KV head, batch) and tensor (grid y < B: keys of batch y,
// else values of batch y - B) quantizes the groups straight from the window,
// then moves the window's remaining R - 32 f rows and the n new rows to the
// window start.  Every row of the new window is loaded before the first is
// stored, so the move is safe in place.
template <int D, int BITS>
__global__ __launch_bounds__(D) void flush_window_kernel(const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new, uint16_t* k_rec,
                                                         uint16_t* v_rec, int R_cap, int R, int n, int f, int Hkv,
                                                         QuantizeOut ko, QuantizeOut vo, int dst_tiles, int tile0,
                                                         int B) {
  constexpr int kPR = D / 8;                   // 16-byte pieces per row
  constexpr int kMaxPieces = kMaxRecent * kPR / D;   // per thread: the new window holds at most kMaxRecent rows
  const int h = blockIdx.x;
  const bool keys = static_cast<int>(blockIdx.y) < B;
  const int b = keys ? blockIdx.y : blockIdx.y - B;
  uint16_t* rec = keys ? k_rec : v_rec;
  const size_t unit = static_cast<size_t>(b) * Hkv + h;
  const int keep = R - kGroup * f;
  const int pieces = (keep + n) * kPR;
  const uint16_t* nw = (keys ? k_new : v_new) + unit * n * D;
  uint16_t* win = rec + unit * R_cap * D;
  // the rows to move are loaded first: their sources (window rows 32 f ..
  // and the new rows) are not among the rows being quantized, so both
  // memory round trips overlap
  uint32_t buf[kMaxPieces][4];
  if (pieces > 0) {
#pragma unroll
    for (int i = 0; i < kMaxPieces; ++i) {
      const int e = min(static_cast<int>(threadIdx.x) + D * i, pieces - 1), r = e / kPR, c8 = e % kPR;
      const uint16_t* src =
          r < keep ? win + static_cast<size_t>(kGroup * f + r) * D : nw + static_cast<size_t>(r - keep) * D;
      const uint4 x = reinterpret_cast<const uint4*>(src)[c8];
      buf[i][0] = x.x;
      buf[i][1] = x.y;
      buf[i][2] = x.z;
      buf[i][3] = x.w;
    }
  }
  for (int t = 0; t < f; ++t) {
    if (keys) quantize_k_tile<D, BITS>(rec, R_cap, Hkv, ko.codes, ko.scale, ko.zero, dst_tiles, tile0, t, h, b);
    else quantize_v_tile<D, BITS>(rec, R_cap, Hkv, vo.codes, vo.scale, vo.zero, dst_tiles, tile0, t, h, b);
    __syncthreads();                           // the tile's LDS and its reads of the window are done
  }
  if (pieces == 0) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's rows are in registers
  __syncthreads();                                    // and every thread's: the window may be overwritten
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int e = static_cast<int>(threadIdx.x) + D * i;
    if (e < pieces) reinterpret_cast<uint4*>(win)[e] = uint4{buf[i][0], buf[i][1], buf[i][2], buf[i][3]};
  }
}

void launch_flush_window(int d, int bits, dim3 grid, hipStream_t s, const uint16_t* k_new, const uint16_t* v_new,
                         uint16_t* k_rec, uint16_t* v_rec, int R_cap, int R, int n, int f, int Hkv, QuantizeOut ko,
                         QuantizeOut vo, int dst_tiles, int tile0, int B) {
#define DQA_FW(D, BITS)                                                                                       \
  hipLaunchKernelGGL((flush_window_kernel<D, BITS>), grid, dim3(D), 0, s, k_new, v_new, k_rec, v_rec, R_cap, R, \
                     n, f, Hkv, ko, vo, dst_tiles, tile0, B)
  if (d == 128) {
    if (bits == 2) DQA_FW(128, 2);
    else if (bits == 4) DQA_FW(128, 4);
    else DQA_FW(128, 8);
  } else {
    if (bits == 2) DQA_FW(64, 2);
    else if (bits == 4) DQA_FW(64, 4);
    else DQA_FW(64, 8);
  }
#undef DQA_FW
}

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
  if (c->B > 32767 || c->Hkv > 65535) return DQA_ERR_SHAPE;   // keys and values share one grid z
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
  // A capacity of 0 means "the current count"; the buffers' row strides are
  // fixed by it, so it is written back below and stays put when R shrinks.
  auto commit = [&]() {
    c->T_cap = T_cap;
    c->R_cap = R_cap;
    c->T_q = T_new;
    c->R = R_new;
    return DQA_OK;
  };
  if (units == 0 || rows == 0) return commit();
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
  uint16_t* krec = const_cast<uint16_t*>(c->k_recent);
  uint16_t* vrec = const_cast<uint16_t*>(c->v_recent);
  if (f == 0) {                                // no flush: the new rows go after the window's rows
    if (n_new > 0) {
      const size_t chunks = units * static_cast<size_t>(n_new) * (d / 8);
      hipLaunchKernelGGL(append_rows_kernel, dim3(copy_blocks(2 * chunks)), dim3(256), 0, s, k_new, v_new, n_new,
                         c->R, krec, vrec, R_cap, units, d);
      DQA_CHECK_LAUNCH();
    }
    return commit();
  }
  uint32_t* kc = const_cast<uint32_t*>(c->k_codes);
  uint16_t* ks = const_cast<uint16_t*>(c->k_scale);
  uint16_t* kz = const_cast<uint16_t*>(c->k_zero);
  uint32_t* vc = const_cast<uint32_t*>(c->v_codes);
  uint16_t* vs = const_cast<uint16_t*>(c->v_scale);
  uint16_t* vz = const_cast<uint16_t*>(c->v_zero);
  const int dst_tiles = T_cap / kGroup, tile0 = c->T_q / kGroup;
  if (kGroup * f <= c->R) {                    // the flushed groups are the window's oldest rows
    launch_flush_window(d, c->bits, dim3(c->Hkv, 2 * c->B), s, k_new, v_new, krec, vrec, R_cap, c->R, n_new, f,
                        c->Hkv, QuantizeOut{kc, ks, kz}, QuantizeOut{vc, vs, vz}, dst_tiles, tile0, c->B);
    DQA_CHECK_LAUNCH();
    return commit();
  }
  // general case (the groups reach into the new rows): window and new rows
  // staged in the workspace, quantized from there, the rest moved back
  uint16_t* wk = static_cast<uint16_t*>(ws);
  uint16_t* wv = wk + units * static_cast<size_t>(rows) * d;
  const size_t chunks = units * static_cast<size_t>(rows) * (d / 8);
  hipLaunchKernelGGL(stage_rows_kernel, dim3(copy_blocks(2 * chunks)), dim3(256), 0, s,
                     RowPair{c->k_recent, k_new, wk}, RowPair{c->v_recent, v_new, wv}, c->R, R_cap, n_new, units, d);
  DQA_CHECK_LAUNCH();
  launch_quantize_kv(d, c->bits, dim3(f, c->Hkv, 2 * c->B), s, wk, wv, rows, c->Hkv, QuantizeOut{kc, ks, kz},
                     QuantizeOut{vc, vs, vz}, dst_tiles, tile0, c->B);
  DQA_CHECK_LAUNCH();
  if (R_new > 0) {
    const size_t kchunks = units * static_cast<size_t>(R_new) * (d / 8);
    hipLaunchKernelGGL(unstage_rows_kernel, dim3(copy_blocks(2 * kchunks)), dim3(256), 0, s, wk, wv, rows,
                       f * kGroup, R_new, krec, vrec, R_cap, units, d);
    DQA_CHECK_LAUNCH();
  }
  return commit();
}
