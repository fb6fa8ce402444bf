// Partial softmax states of the split-K decode kernels and their merge.
//
// Every decode path (uniform, zoned, residual-VQ) splits the tokens of a
// (batch, KV head) over several workgroups.  A workgroup combines its waves'
// states and writes one partial state per query head, [m, l, o[D]] in the
// log2 domain: m the running maximum of the logits, l the sum of
// 2^(logit - m), o the unnormalized output.  The workgroup that finishes
// last among the splits of a (batch, KV head) -- found with one counter per
// (batch, KV head), incremented once per workgroup -- merges all splits in
// split order, so the result does not depend on scheduling, and sets the
// counter back to zero for the next call.
//
// The L2 caches are private to each XCD, and a device-scope release fence
// (an L2 write-back) in every workgroup would cost more than the decode
// work.  So the partial states are written with device-scope (write-through)
// stores and read with device-scope loads, which bypass the non-coherent
// caches; every wave waits for its stores to complete before the workgroup
// barrier that precedes the counter increment.
//
// Workspace layout: uint32 counters [max(B * Hkv, 16384)] (rounded up to 256
// bytes), then fp32 partial states [B * Hkv][splits][G][D + 2].  The
// counters must be zero before the first call on a workspace; every call
// leaves them zero.
#pragma once

#include "common.h"

namespace dqa {
namespace {

// splits per (batch, KV head) at most (their m and l must fit a workgroup's
// output staging, NW * G * D floats, with NW >= 4 and D >= 64; one wave
// reduces a head's maxima over two lanes' worth: 128)
constexpr int kMaxSplitsMerge = 128;

// Counters at the start of a workspace: one per (batch, KV head), at least
// 16384 of them, so that a workspace can serve cache shapes of up to 16384
// (batch, KV head) units without being cleared again.
constexpr size_t kMergeCountersMin = 16384;
inline size_t merge_counter_bytes(size_t units) {
  const size_t n = (units > kMergeCountersMin ? units : kMergeCountersMin) * sizeof(uint32_t);
  return (n + 255) / 256 * 256;
}
inline uint32_t* merge_counters(void* ws) { return static_cast<uint32_t*>(ws); }
inline float* merge_partials(void* ws, size_t units) {
  return reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + merge_counter_bytes(units));
}

// Combine the NW wave states of a workgroup (LDS: lm, ll [NW][G], lo
// [NW][G][D], lo 16-byte aligned).  With a single split: the normalized
// output out[b][kvh * G + h][c], and false.  Otherwise: split `slot`'s
// partial state (device-scope write-through stores, each wave waits for
// its own), and true.  Called by every thread of the workgroup.
template <int D, int G, int NW>
__device__ __forceinline__ bool store_split_state(float* partials, float* out, int Hq, size_t unit, int b, int kvh,
                                                  int slot, int total_splits, const float (*lm)[G],
                                                  const float (*ll)[G], const float (*lo)[G][D]) {
  float* const part = partials + (unit * total_splits + slot) * G * (D + 2);
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
        __hip_atomic_store(part + h * (D + 2) + 0, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(part + h * (D + 2) + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(part + h * (D + 2) + 2 + c, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (total_splits == 1) return false;
  // every wave's partial-state stores have completed before the caller's
  // workgroup barrier
  __builtin_amdgcn_s_waitcnt(0);
  return true;
}

// Merge every split of a (batch, KV head) in split order into out (lo is
// reused as staging for the splits' m and l).  Every phase has a fixed
// shape (no loop over the splits with a memory or LDS round trip per
// split): the output values of the splits are loaded kChunk splits at a time
// with all loads of a chunk in flight (the first chunk together with the
// splits' m and l); m and l are staged head-major in LDS (rows of
// kMaxSplitsMerge, -inf / 0 past the last split); one wave forms each head's
// maximum M; the weights 2^(m_k - M) replace m; each output then reads its
// head's weights and l values kChunk splits at a time.  Called by every
// thread of the workgroup.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_splits(const float* partials, float* out, int Hq, size_t unit, int b, int kvh,
                                             int total_splits, float (*lo)[G][D]) {
  static_assert(2 * kMaxSplitsMerge * G <= NW * G * D, "m and l of every split fit the output staging");
  constexpr int kChunk = 32;
  constexpr int S = kMaxSplitsMerge;
  constexpr int kPer = (G * D + NW * 64 - 1) / (NW * 64);   // outputs per thread
  constexpr int kStage = (G * S + NW * 64 - 1) / (NW * 64);  // staged (m, l) per thread
  __shared__ float s_M[G];
  const float* const parts = partials + unit * total_splits * G * (D + 2);
  constexpr size_t kSplitStride = static_cast<size_t>(G) * (D + 2);
  auto ld = [](const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  float ov[kPer][kChunk];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int e = min(static_cast<int>(threadIdx.x) + r * NW * 64, G * D - 1);
      const int h = e / D, c = e % D;
#pragma unroll
      for (int k = 0; k < kChunk; ++k)   // past the last split: the last split again, weight 0
        ov[r][k] = ld(parts + min(k0 + k, total_splits - 1) * kSplitStride + h * (D + 2) + 2 + c);
    }
  };
  load_chunk(0);
  float* const sw = &lo[0][0][0];   // [G][S]: m, then the weights
  float* const sl = sw + S * G;     // [G][S]: l
  {
    // (m, l) of a split and head as one 8-byte load (8-byte aligned: the
    // state of a head is D + 2 floats, D even)
    uint64_t ml[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = min(static_cast<int>(threadIdx.x) + j * NW * 64, G * S - 1);
      const int h = i / S, k = min(i % S, total_splits - 1);
      ml[j] = __hip_atomic_load(reinterpret_cast<const uint64_t*>(parts + k * kSplitStride + h * (D + 2)),
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = static_cast<int>(threadIdx.x) + j * NW * 64;
      if (i < G * S) {
        const bool in = i % S < total_splits;
        sw[i] = in ? __builtin_bit_cast(float, static_cast<uint32_t>(ml[j])) : -INFINITY;
        sl[i] = in ? __builtin_bit_cast(float, static_cast<uint32_t>(ml[j] >> 32)) : 0.0f;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float M = wave_max(fmaxf(sw[h * S + threadIdx.x], sw[h * S + 64 + threadIdx.x]));
      if (threadIdx.x == 0) s_M[h] = M;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kStage; ++j) {
    const int i = static_cast<int>(threadIdx.x) + j * NW * 64;
    if (i < G * S) sw[i] = merge_weight(sw[i], s_M[i / S]);
  }
  __syncthreads();
  float Lr[kPer], Or[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    Lr[r] = 0.0f;
    Or[r] = 0.0f;
  }
  for (int k0 = 0; k0 < total_splits; k0 += kChunk) {
    if (k0 > 0) load_chunk(k0);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int h = min(static_cast<int>(threadIdx.x) + r * NW * 64, G * D - 1) / D;
      float w[kChunk], l[kChunk];
#pragma unroll
      for (int q = 0; q < kChunk / 4; ++q) {
        const float4 w4 = *reinterpret_cast<const float4*>(&sw[h * S + k0 + 4 * q]);
        const float4 l4 = *reinterpret_cast<const float4*>(&sl[h * S + k0 + 4 * q]);
        w[4 * q] = w4.x, w[4 * q + 1] = w4.y, w[4 * q + 2] = w4.z, w[4 * q + 3] = w4.w;
        l[4 * q] = l4.x, l[4 * q + 1] = l4.y, l[4 * q + 2] = l4.z, l[4 * q + 3] = l4.w;
      }
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        Lr[r] = fmaf(l[k], w[k], Lr[r]);
        Or[r] = fmaf(ov[r][k], w[k], Or[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = threadIdx.x + r * NW * 64;
    if (e >= G * D) break;
    const int h = e / D, c = e % D;
    out[(static_cast<size_t>(b) * Hq + kvh * G + h) * D + c] = (Lr[r] > 0.0f) ? Or[r] / Lr[r] : 0.0f;
  }
}


// The partial state of split `slot` (store_split_state), and the merge of
// all splits (merge_splits) by the workgroup that finishes last among the
// splits of its (batch, KV head), found with the unit's counter, which
// every workgroup increments once; that workgroup sets the counter back to
// zero (and, if epoch_word is given, stores epoch there).  Called by every
// thread of the workgroup.
template <int D, int G, int NW>
__device__ __forceinline__ void write_split_state(float* partials, uint32_t* counter, float* out, int Hq,
                                                  size_t unit, int b, int kvh, int slot, int total_splits,
                                                  const float (*lm)[G], const float (*ll)[G],
                                                  float (*lo)[G][D], uint32_t* epoch_word = nullptr,
                                                  uint32_t epoch = 0u) {
  __shared__ int s_last;
  if (!store_split_state<D, G, NW>(partials, out, Hq, unit, b, kvh, slot, total_splits, lm, ll, lo)) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == static_cast<uint32_t>(total_splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  merge_splits<D, G, NW>(partials, out, Hq, unit, b, kvh, total_splits, lo);
  if (threadIdx.x == 0) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (epoch_word) __hip_atomic_store(epoch_word, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workspace bytes of the merge: the counters, then the partial states of
// `splits` splits (never 0, so that a workspace query of 0 always means an
// invalid shape).
inline size_t partial_state_bytes(size_t units, int splits, int G, int D) {
  const size_t n = splits > 1 ? units * static_cast<size_t>(splits) * G * (D + 2) * sizeof(float) : 0;
  return merge_counter_bytes(units) + n;
}

}  // namespace
}  // namespace dqa
