// Residual VQ encoder and decode attention (in progress).
#include "common.h"

extern "C" size_t rvq_encode_workspace_bytes(int, int) { return 0; }
extern "C" int rvq_encode(const uint16_t*, int64_t, int, const uint16_t*, int, int, int16_t*, void*,
                          size_t, void*) { return DQA_ERR_UNSUPPORTED; }
extern "C" size_t rvq_decode_attention_workspace_bytes(int, int, int, int, int) { return 0; }
extern "C" int rvq_decode_attention(const uint16_t*, int, int, int, int, int, const int16_t*,
                                    const int16_t*, const uint16_t*, const uint16_t*, int, int, float,
                                    void*, size_t, float*, void*) { return DQA_ERR_UNSUPPORTED; }
