// Partial softmax states of the split-K decode kernels and their merge.
//
// Every decode path (uniform, zoned, residual-VQ) splits the tokens of a
// (batch, KV head) over several workgroups.  A workgroup combines its waves'
// states and writes one partial state per query head, [m, l, o[D]] in the
// log2 domain: m the running maximum of the logits, l the sum of
// 2^(logit - m), o the unnormalized output.  A second, small kernel merges
// the splits of every (batch, KV head) in split order, so the result does
// not depend on scheduling.  (A last-workgroup merge inside the decode
// kernel would need a device-scope fence and a counter atomic per
// workgroup; on this chip, whose L2 is private to each XCD, those cost more
// than the decode work itself.)
//
// Partial-state layout (fp32): [B * Hkv][splits][G][D + 2].
#pragma once

#include "common.h"

namespace dqa {
namespace {

// splits per (batch, KV head) at most (the merge keeps one weight per split)
constexpr int kMaxSplitsMerge = 255;

// Combine the NW wave states of a workgroup (LDS: lm, ll [NW][G], lo
// [NW][G][D]) and write split `slot`'s partial state -- or, with a single
// split, the normalized output out[b][kvh * G + h][c].  Called by every
// thread of the workgroup.
template <int D, int G, int NW>
__device__ __forceinline__ void write_split_state(float* partials, float* out, int Hq, size_t unit, int b,
                                                  int kvh, int slot, int total_splits, const float (*lm)[G],
                                                  const float (*ll)[G], const float (*lo)[G][D]) {
  float* part = partials + (unit * total_splits + slot) * G * (D + 2);
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, lm[w][h]);
    float L = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = merge_weight(lm[w][h], M);
      L = fmaf(ll[w][h], wt, L);
      O = fmaf(lo[w][h][c], wt, O);
    }
    if (total_splits == 1) {
      out[(static_cast<size_t>(b) * Hq + kvh * G + h) * D + c] = (L > 0.0f) ? O / L : 0.0f;
    } else {
      if (c == 0) {
        part[h * (D + 2) + 0] = M;
        part[h * (D + 2) + 1] = L;
      }
      part[h * (D + 2) + 2 + c] = O;
    }
  }
}

// One wave per (64 output channels of one query head, KV head, batch): the
// lanes compute the merge weight of every split (max over splits, then
// exp2 weights and the weighted row sum, combined in a fixed butterfly
// order), then each lane sums its channel over the splits in split order.
// The first 32 splits' outputs are loaded together with the states.
template <int D, int G>
__global__ __launch_bounds__(64) void split_merge_kernel(const float* __restrict__ partials, int total_splits,
                                                         int Hq, int Hkv, float* __restrict__ out) {
  constexpr int kEarly = 32;
  __shared__ float wts[kMaxSplitsMerge];
  __shared__ float inv_l;
  constexpr int CB = D / 64;                 // 64-channel blocks per head
  const int h = blockIdx.x / CB, c = (blockIdx.x % CB) * 64 + threadIdx.x;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const size_t unit = static_cast<size_t>(b) * Hkv + kvh;
  const float* parts = partials + unit * total_splits * G * (D + 2) + h * (D + 2);
  constexpr size_t kSplitStride = static_cast<size_t>(G) * (D + 2);
  float early[kEarly];
#pragma unroll
  for (int i = 0; i < kEarly; ++i) early[i] = (i < total_splits) ? parts[i * kSplitStride + 2 + c] : 0.0f;
  float M = -INFINITY;
  for (int sl = threadIdx.x; sl < total_splits; sl += 64) M = fmaxf(M, parts[sl * kSplitStride]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float L = 0.0f;
  for (int sl = threadIdx.x; sl < total_splits; sl += 64) {
    const float wt = merge_weight(parts[sl * kSplitStride], M);
    wts[sl] = wt;
    L = fmaf(parts[sl * kSplitStride + 1], wt, L);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
  if (threadIdx.x == 0) inv_l = (L > 0.0f) ? 1.0f / L : 0.0f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  float O = 0.0f;
#pragma unroll
  for (int i = 0; i < kEarly; ++i)
    if (i < total_splits) O = fmaf(early[i], wts[i], O);
  for (int sl = kEarly; sl < total_splits; ++sl) O = fmaf(parts[sl * kSplitStride + 2 + c], wts[sl], O);
  out[(static_cast<size_t>(b) * Hq + kvh * G + h) * D + c] = O * inv_l;
}

// Enqueue the merge of `total` splits (nothing for a single split).
template <int D>
int launch_split_merge(const float* partials, int total, int B, int Hq, int Hkv, float* out, hipStream_t s) {
  if (total <= 1) return DQA_OK;
  const int G = Hq / Hkv;
  const dim3 grid(G * (D / 64), Hkv, B);
  switch (G) {
    case 1: hipLaunchKernelGGL((split_merge_kernel<D, 1>), grid, dim3(64), 0, s, partials, total, Hq, Hkv, out); break;
    case 2: hipLaunchKernelGGL((split_merge_kernel<D, 2>), grid, dim3(64), 0, s, partials, total, Hq, Hkv, out); break;
    case 3: hipLaunchKernelGGL((split_merge_kernel<D, 3>), grid, dim3(64), 0, s, partials, total, Hq, Hkv, out); break;
    case 4: hipLaunchKernelGGL((split_merge_kernel<D, 4>), grid, dim3(64), 0, s, partials, total, Hq, Hkv, out); break;
    default: return DQA_ERR_UNSUPPORTED;
  }
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}

// Bytes of partial states for `splits` splits (at least 256, so that a
// workspace query of 0 always means an invalid shape).
inline size_t partial_state_bytes(size_t units, int splits, int G, int D) {
  const size_t n = splits > 1 ? units * static_cast<size_t>(splits) * G * (D + 2) * sizeof(float) : 0;
  return n < 256 ? 256 : n;
}

}  // namespace
}  // namespace dqa
