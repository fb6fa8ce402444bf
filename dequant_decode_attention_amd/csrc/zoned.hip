// Mixed-bitwidth zoned cache: plan, packer and decode reader (in progress).
#include "common.h"

extern "C" size_t zoned_plan_words(int, int, int, int) { return 0; }
extern "C" int zoned_plan(const int8_t*, const int8_t*, int, int, int, int, int, int32_t*, size_t,
                          size_t*) { return DQA_ERR_UNSUPPORTED; }
extern "C" int zoned_pack(const int32_t*, const int32_t*, const uint16_t*, const uint16_t*,
                          const uint16_t*, const uint16_t*, void*, void*) { return DQA_ERR_UNSUPPORTED; }
extern "C" size_t decode_attention_zoned_workspace_bytes(const int32_t*, int) { return 0; }
extern "C" int decode_attention_zoned(const uint16_t*, int, const int32_t*, const int32_t*, const void*,
                                      float, void*, size_t, float*, void*) { return DQA_ERR_UNSUPPORTED; }
