// Status strings, interface version and the streaming-copy measurement
// kernel.
#include "common.h"

namespace dqa {
namespace {

// Grid-stride 16-byte copy; used to calibrate HBM byte counters and to
// measure the achievable streaming bandwidth next to the method's kernels.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                          u32x4* __restrict__ dst, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (; i < n; i += stride) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace
}  // namespace dqa

extern "C" const char* dqa_status_string(int status) {
  switch (status) {
    case DQA_OK: return "DQA_OK";
    case DQA_ERR_NULL: return "DQA_ERR_NULL: a required pointer is NULL";
    case DQA_ERR_SHAPE: return "DQA_ERR_SHAPE: a size is out of range or inconsistent";
    case DQA_ERR_BITS: return "DQA_ERR_BITS: unsupported bit width";
    case DQA_ERR_WORKSPACE: return "DQA_ERR_WORKSPACE: workspace missing or too small";
    case DQA_ERR_UNSUPPORTED: return "DQA_ERR_UNSUPPORTED: configuration not built";
    case DQA_ERR_HIP: return "DQA_ERR_HIP: a HIP launch failed";
    case DQA_ERR_PLAN: return "DQA_ERR_PLAN: zoned plan malformed or mismatched";
    case DQA_ERR_ALIGN: return "DQA_ERR_ALIGN: a device pointer is not 16-byte aligned";
    default: return "DQA_ERR_UNKNOWN";
  }
}

extern "C" int dqa_abi_version(void) { return 14; }

extern "C" int dqa_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return DQA_OK;
  if (!src || !dst) return DQA_ERR_NULL;
  if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
    return DQA_ERR_SHAPE;
  const size_t n = bytes / 16;
  size_t blocks = (n + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(dqa::stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const dqa::u32x4*>(src),
                     static_cast<dqa::u32x4*>(dst), n);
  DQA_CHECK_LAUNCH();
  return DQA_OK;
}
