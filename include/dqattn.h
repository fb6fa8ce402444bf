/*
 * dqattn -- decode attention over a low-bit KV cache, for AMD MI355X (gfx950).
 *
 * The KV cache is held as low-bit integer codes (or residual-VQ indices) in
 * HBM; each decode step reads the codes back and dequantizes them inside
 * the attention kernel.  Method pages cited below:
 *   [P1] ihal.it/?p=61653 -- article on KV-cache quantization axes (KIVI,
 *        KVQuant, InnerQ); no headings, cited by paragraph number and topic.
 *   [P2] "VQKV: High-Fidelity and High-Ratio Cache Compression via
 *        Vector-Quantization", gist.science/it/paper/2603.16435.
 *   [P3] "Riepilogo Tecnico: RDKV - Allocazione dei Bit per
 *        Distorsione-Rate ...", gist.science/it/paper/2605.08317; its two
 *        sections numbered 2.2 are cited by title ("bit-allocation
 *        pipeline", "TriZone packed decoding").
 *
 * Conventions shared by every entry point:
 *   - Pointers marked (device) are device memory owned by the caller; the
 *     library never allocates, frees or synchronizes.  Pointers marked
 *     (host) are host memory read synchronously during the call.
 *   - fp16 tensors travel as raw IEEE binary16 bit patterns (uint16_t).
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     All device work is enqueued on it, in stream order.
 *   - Every argument is validated on the host before any HIP call; a
 *     non-zero return means nothing was enqueued and outputs are untouched.
 *     DQA_ERR_HIP means a launch failed (the HIP error is left pending).
 *     Device faults surface at the caller's next synchronization.
 *   - Tensors are dense, row-major, in the layouts stated per argument.
 *   - Thread safety: entry points are stateless and may be called from
 *     several host threads; calls that share a workspace must be ordered by
 *     the caller (same stream or events).
 *   - Decode workspaces (decode_attention_qkv, decode_attention_zoned,
 *     rvq_decode_attention) start with one uint32 counter per (batch, KV
 *     head), at least 16384 of them: the workgroup that finishes a (batch,
 *     KV head) last merges the partial states of its splits and sets the
 *     counter back to zero.  Zero a decode workspace once before its first
 *     use (e.g. hipMemset after hipMalloc); every completed call leaves the
 *     counters zero.  A workspace first used for more than 16384 (batch,
 *     KV head) units must be zeroed again before a call with a different
 *     B * Hkv.
 */
#ifndef DQATTN_H
#define DQATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point that returns int. */
enum {
  DQA_OK = 0,
  DQA_ERR_NULL = 1,        /* a required pointer is NULL */
  DQA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  DQA_ERR_BITS = 3,        /* unsupported bit width */
  DQA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required */
  DQA_ERR_UNSUPPORTED = 5, /* valid by the method but not built (e.g. head ratio) */
  DQA_ERR_HIP = 6,         /* a HIP launch failed */
  DQA_ERR_PLAN = 7,        /* a zoned plan is malformed or does not match */
  DQA_ERR_ALIGN = 8        /* a device pointer is not 16-byte aligned */
};

/* Human-readable name of a status code; never NULL. */
const char* dqa_status_string(int status);

/* Version of this interface (increments on any signature or layout change). */
int dqa_abi_version(void);  /* 14: rvq_decode_attention's workspace starts
                              with its synchronization words;
                              13: rvq_decode_set_table_polls;
                              12: rvq_decode_attention is one launch
                              (the key-logit tables are built in it) and
                              its workspace ends with synchronization
                              words (a larger workspace);
                              11: dqa_kivi_cache ends with an optional
                              rope_table; kivi_rope_table(_words);
                              10: decode workspaces hold merge counters
                              and must be zeroed before first use; the
                              split kernel merges its splits itself
                              (decode_attention_qkv_merge enqueues
                              nothing);
                              9: decode_attention_qkv_noalloc;
                              8: decode_attention_zoned and rvq_encode check
                              16-byte alignment; zoned plans are validated in
                              full; kivi_append writes back zero capacities;
                              7: quantize_pack_k/v and zoned_pack check
                              16-byte alignment; kivi_append takes
                              B <= 32767;
                              6: zoned_plan takes a sink length and the
                              outlier entries per key group;
                              5: RDKV allocation entry points (rdkv_*);
                              4: dqa_kivi_cache carries buffer capacities
                              (T_cap, R_cap) and kivi_append exists;
                              3: 16-byte pointer alignment checked */

/* ------------------------------------------------------------------------
 * Quantize + bit-pack  ([P1 para 1, 3, 4, 5])
 *
 * Asymmetric uniform quantization in groups of 32: the group's range
 * [min, max] is split into 2^bits levels.  scale s = fp16_rne((max - min) /
 * (2^bits - 1)) computed in IEEE fp32; zero z = min (fp16, exact); code
 * q = clamp(rint_half_even((x - z) / s), 0, 2^bits - 1) with IEEE fp32
 * subtraction and division against the stored fp16 s and z; a group with
 * s == 0 gets all-zero codes.  Dequantized value: q * s + z.
 *
 * Packing: codes form little-endian bit streams; stream element f occupies
 * bits [f*bits, f*bits + bits), i.e. uint32 word (f*bits)/32 at bit
 * (f*bits)%32.  Keys: the [B][Hkv][T][d] tensor in row-major order (element
 * (t, c) of a unit at t*d + c).  Values: blocks of 32 tokens, channel-major
 * inside a block (element (t, c) of a unit at (t/32)*32*d + c*32 + t%32).
 * ------------------------------------------------------------------------ */

/* Keys grouped per channel over 32 consecutive tokens ([P1 para 4]); keys are
 * quantized before RoPE ([P1 para 7]).
 *   k      (device) fp16 [B][Hkv][T][d]
 *   T      multiple of 32, >= 0;  d in {64, 128};  bits in {2, 4, 8}
 *   codes  (device) uint32 [B*Hkv*T*d*bits/32]
 *   scale, zero (device) fp16 [B][Hkv][T/32][d]
 * k and codes must be 16-byte aligned (DQA_ERR_ALIGN otherwise).
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_BITS, DQA_ERR_ALIGN,
 * DQA_ERR_HIP. */
int quantize_pack_k(const uint16_t* k, int B, int Hkv, int T, int d, int bits,
                    uint32_t* codes, uint16_t* scale, uint16_t* zero,
                    void* stream);

/* Values grouped per token over 32 consecutive channels ([P1 para 5]).
 *   v      (device) fp16 [B][Hkv][T][d]; T multiple of 32, >= 0; d in {64, 128}
 *   codes  (device) uint32 [B*Hkv*T*d*bits/32]
 *   scale, zero (device) fp16 [B][Hkv][T][d/32]
 * v and codes must be 16-byte aligned.  Errors as quantize_pack_k. */
int quantize_pack_v(const uint16_t* v, int B, int Hkv, int T, int d, int bits,
                    uint32_t* codes, uint16_t* scale, uint16_t* zero,
                    void* stream);

/* ------------------------------------------------------------------------
 * Decode attention over the uniform (KIVI) layout  ([P1 para 2, 6, 7, 8])
 * ------------------------------------------------------------------------ */

/* A quantized cache plus its fp16 recent zone.  All pointers (device). */
typedef struct dqa_kivi_cache {
  int B, Hq, Hkv;         /* batch, query heads, KV heads (Hq % Hkv == 0)       */
  int d;                  /* head dim, 64 or 128                                */
  int bits;               /* 2, 4 or 8                                          */
  int T_q;                /* quantized tokens, multiple of 32, >= 0             */
  int R;                  /* fp16 recent tokens, 0..128 ([P1 para 8])           */
                          /* (the buffers below are laid out with the          */
                          /* capacities T_cap and R_cap at the end)            */
  float rope_theta;       /* > 0: rotate keys after dequantization (interleaved */
                          /* pairs, omega_i = theta^(-2i/d)); <= 0: no RoPE     */
  const uint32_t* k_codes;  /* quantize_pack_k layout, [B][Hkv][T_cap][d]       */
  const uint16_t* k_scale;  /* fp16 [B][Hkv][T_cap/32][d]                       */
  const uint16_t* k_zero;
  const uint32_t* v_codes;  /* quantize_pack_v layout (32-token channel-major)  */
  const uint16_t* v_scale;  /* fp16 [B][Hkv][T_cap][d/32]                       */
  const uint16_t* v_zero;
  const uint16_t* k_recent; /* fp16 [B][Hkv][R_cap][d], keys before RoPE        */
  const uint16_t* v_recent; /* fp16 [B][Hkv][R_cap][d]                          */
  int T_cap;              /* tokens the quantized buffers hold per (batch, KV   */
                          /* head): the arrays above are [B][Hkv][T_cap]...     */
                          /* with T_cap >= T_q, a multiple of 32; 0 means T_q   */
  int R_cap;              /* rows of the recent buffers per (batch, KV head),   */
                          /* >= R; 0 means R                                    */
  const uint32_t* rope_table; /* optional, may be NULL: the in-tile rotation    */
                          /* table kivi_rope_table built for this rope_theta, */
                          /* d and bits (2-/4-bit caches with RoPE); the      */
                          /* decode kernel copies it instead of evaluating   */
                          /* the rotations itself (same values).  A table    */
                          /* whose header names another theta, d or bits is  */
                          /* ignored.  kivi_rope_table_words(d) words,       */
                          /* 16-byte aligned.                                */
} dqa_kivi_cache;

/* In-tile rotation table of a RoPE cache ([P1 para 7]: keys are rotated
 * after dequantization).  For the token at offset j = 0..31 of a 32-token
 * tile and channel pair i it holds e^{i j w_i} (w_i = theta^(-2i/d)) in the
 * split fp16 form the 2- and 4-bit decode kernel multiplies codes with, and
 * e^{i 32 w_i}; the values depend on theta, d and bits only, so a cache
 * builds its table once.
 * kivi_rope_table_words: uint32 words of the table for head dim d (0 unless
 * d is 64 or 128).
 * kivi_rope_table: writes the table (device, kivi_rope_table_words(d) words,
 * 16-byte aligned); enqueues one kernel.  rope_theta > 0, d in {64, 128}
 * (else DQA_ERR_SHAPE), bits in {2, 4} (else DQA_ERR_BITS).
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_BITS, DQA_ERR_ALIGN,
 * DQA_ERR_HIP. */
size_t kivi_rope_table_words(int d);
int kivi_rope_table(float rope_theta, int d, int bits, uint32_t* table,
                    void* stream);

/* Bytes of workspace decode_attention_qkv needs for this cache shape
 * (0 if the shape is invalid; at least 64 KB otherwise).  The workspace
 * holds the merge counters and the per-split partial softmax states; zero
 * it before its first use (see the preamble); every call leaves the counters
 * zero, the rest unspecified.  Calls that share a workspace must
 * not overlap (same stream, or ordered by events). */
size_t decode_attention_workspace_bytes(const dqa_kivi_cache* cache);

/* One decode step: out[b][h] = softmax(sm_scale * q[b][h] . K_hat^T) V_hat,
 * over the dequantized quantized tokens (positions 0..T_q-1) followed by the
 * recent tokens (positions T_q..T_q+R-1).  Query head h reads KV head
 * h / (Hq/Hkv).  With rope_theta > 0 each key is rotated at its position
 * after dequantization ([P1 para 7]); q must already be rotated.
 *   q    (device) fp16 [B][Hq][d]
 *   cache (host) pointer to the descriptor above
 *   ws   (device) workspace of ws_bytes >= decode_attention_workspace_bytes
 *   out  (device) fp32 [B][Hq][d]; zeros when T_q + R == 0
 * Enqueues one kernel.  When the tokens of a (batch, KV head) are split
 * over several workgroups, the workgroup that finishes last merges the
 * splits in a fixed order, so results are bit-reproducible run to run.
 * Every device pointer (q, ws, out and the cache buffers in use) must be
 * 16-byte aligned (hipMalloc returns 256-byte aligned memory).
 * Supported head ratios Hq/Hkv: 1, 2, 4 (else DQA_ERR_UNSUPPORTED).
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_BITS, DQA_ERR_WORKSPACE,
 * DQA_ERR_ALIGN, DQA_ERR_UNSUPPORTED, DQA_ERR_HIP. */
int decode_attention_qkv(const uint16_t* q, const dqa_kivi_cache* cache,
                         float sm_scale, void* ws, size_t ws_bytes, float* out,
                         void* stream);

/* The two phases of decode_attention_qkv; decode_attention_qkv is exactly
 * _partial then _merge on the same stream, with the same cache, workspace
 * and out.  decode_attention_qkv_partial enqueues the split kernel, which
 * also merges the splits (see decode_attention_qkv) and writes out.
 * decode_attention_qkv_merge enqueues nothing: it checks its arguments and
 * returns (kept so that callers of the two-phase form keep working).
 * Arguments, alignment and errors as decode_attention_qkv (the merge checks
 * cache, ws, ws_bytes and out). */
int decode_attention_qkv_partial(const uint16_t* q, const dqa_kivi_cache* cache,
                                 float sm_scale, void* ws, size_t ws_bytes,
                                 float* out, void* stream);
int decode_attention_qkv_merge(const dqa_kivi_cache* cache, const void* ws,
                               size_t ws_bytes, float* out, void* stream);

/* decode_attention_qkv for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the partial softmax states
 * kept in a library-owned device array of decode_attention_noalloc_scratch_bytes()
 * bytes (2 MiB) per GPU, held until the process ends, instead of a caller
 * workspace.  The array of the current device is used (the stream must
 * belong to it); its address is looked up once per device, on the first
 * call there.  The call itself allocates nothing.  Every call on a GPU shares
 * that GPU's array: calls that may overlap on one GPU (different streams,
 * or host threads) race and must be ordered by the caller.  The array needs
 * no clearing: every split writes its whole state before the merge reads it.
 * Arguments as decode_attention_qkv without ws / ws_bytes.
 * Errors: as decode_attention_qkv; DQA_ERR_WORKSPACE when the cache shape
 * needs more partial-state memory than the array holds (before any launch);
 * DQA_ERR_HIP when the array's address cannot be obtained. */
size_t decode_attention_noalloc_scratch_bytes(void);
int decode_attention_qkv_noalloc(const uint16_t* q, const dqa_kivi_cache* cache,
                                 float sm_scale, float* out, void* stream);

/* Streaming append to the cache ([P1 para 8]: per-channel key statistics
 * need tokens not generated yet, so the newest tokens stay in fp16, up to
 * 128 of them, and are quantized a group at a time once enough of them are
 * there).  The n_new tokens are appended after the R recent tokens; then,
 * while the recent zone holds more than R_max tokens and at least 32, its
 * oldest 32 tokens are quantized exactly as quantize_pack_k /
 * quantize_pack_v would quantize them (one key group per channel, one value
 * group per token and 32 channels) into quantized positions T_q..T_q+31,
 * and T_q grows by 32.  The remaining recent tokens move to the front of
 * the recent buffers.  On success cache->T_q and cache->R are updated, and
 * a T_cap or R_cap of 0 is replaced by the capacity the call used (the old
 * T_q or R), so the buffers keep their row strides when R shrinks; the
 * buffers the cache points to must be writable device memory.
 *   cache  (host) descriptor with T_cap >= T_q + 32 * flushes and
 *          R_cap >= the new R (else DQA_ERR_SHAPE and nothing is written)
 *   k_new, v_new (device) fp16 [B][Hkv][n_new][d] (keys before RoPE);
 *          may be null when n_new == 0
 *   R_max  0..128
 *   ws     (device) workspace of ws_bytes >= kivi_append_workspace_bytes
 * B <= 32767.  Enqueues on `stream` (keys and values together in each
 * kernel): without a flush, one copy of the new rows behind the recent rows;
 * with flushes whose groups are all recent rows (32 * flushes <= R), one
 * kernel that quantizes them in place and then moves the rest of the window
 * (every row it moves is loaded before any is stored); otherwise three
 * kernels (stage the window and the new rows in ws, quantize from there,
 * move back).  ws is required in every case.
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_BITS, DQA_ERR_WORKSPACE,
 * DQA_ERR_ALIGN, DQA_ERR_HIP. */
size_t kivi_append_workspace_bytes(const dqa_kivi_cache* cache, int n_new);
int kivi_append(dqa_kivi_cache* cache, const uint16_t* k_new, const uint16_t* v_new,
                int n_new, int R_max, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Mixed-bitwidth zoned cache  ([P3 sec 2.2, bit-allocation pipeline] and
 * [P3 sec 2.2, TriZone packed decoding])
 *
 * Value width per (batch, KV head, token) in {0, 2, 4, 8, 16}; key width
 * per (batch, KV head, channel) in {0, 2, 4, 8, 16}.  Value width 0 evicts
 * the token (key and value); key width 0 evicts the channel from the kept
 * old tokens' keys ([P3 sec 2.1]: a key channel's weight is the logit change
 * of zeroing it), which then read 0 there; the new tokens of zone C keep
 * every channel.  Zone A: kept tokens grouped into segments by value
 * width (2, 4, 8, 16), each cut into 32-slot groups (last one padded with
 * masked slots); per group the key rows (channels grouped into width
 * classes 2, 4, 8, 16; one scale/zero per (group, quantized channel); 16-bit
 * channels raw fp16) and, for widths 2/4/8, the value rows quantized per
 * token in 32-channel groups.  Zone B: fp16 value rows of 16-bit tokens.
 * Zone C: fp16 keys and values of the S sink tokens, then of the C newest
 * tokens.  Sink window ([P1 para 11]: high-precision windows for attention
 * sinks as well as recent tokens): the first S old tokens stay whole
 * (fp16, every channel) whatever their widths.  Outlier side list ([P1
 * para 9]: a small share of key outliers isolated): in every key
 * quantization group up to k_out entries -- each time the smallest or
 * largest remaining value, whichever is farther from the float32 mean of the
 * remaining values (the largest on a tie) -- leave the group's range while
 * more than two distinct values remain; they are stored as fp16 and read
 * back exactly.  The byte layout is fixed and documented with the oracle
 * that reproduces it.
 * ------------------------------------------------------------------------ */

/* int32 words a plan needs for these sizes (0 if invalid). */
size_t zoned_plan_words(int B, int Hkv, int T_old, int d);

/* Build the plan on the host from the width maps.
 *   v_bits (host) int8 [B][Hkv][T_old], values in {0,2,4,8,16}
 *   k_bits (host) int8 [B][Hkv][d], values in {0,2,4,8,16}
 *   C_new  new fp16 tokens per unit;  d in {64, 128}
 *   sink   old tokens kept whole at the front of zone C, 0..T_old, with
 *          sink + C_new <= 256
 *   k_out  side-list entries per key quantization group, 0..4 (0: none)
 *   plan   (host) int32 [plan_words], plan_words >= zoned_plan_words(...)
 *   blob_bytes (host) receives the size of the packed blob
 * The plan is self-describing; the caller copies the same words to device
 * memory for zoned_pack / decode_attention_zoned.  Those two calls validate
 * the host words before any launch (header, every unit record re-derived
 * from its token and channel counts, blob size, channel permutation) and
 * read the device copy in the kernels, so the device words must be an
 * unmodified copy of the host words.  The token map (the bulk of the plan)
 * is not validated on the host; the packer clamps its entries into
 * [0, T_old), so a map zoned_plan did not write gives an unspecified blob
 * but no out-of-bounds read.
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_BITS (a width outside its
 * set), DQA_ERR_WORKSPACE (plan_words too small). */
int zoned_plan(const int8_t* v_bits, const int8_t* k_bits, int B, int Hkv,
               int T_old, int C_new, int d, int sink, int k_out, int32_t* plan,
               size_t plan_words, size_t* blob_bytes);

/* Pack the cache into the blob described by the plan.
 *   plan_host (host) and plan_dev (device): the same words from zoned_plan
 *             (plan_dev a copy of plan_host; a header, unit record or channel
 *             permutation that zoned_plan could not have written is
 *             DQA_ERR_PLAN)
 *   k, v      (device) fp16 [B][Hkv][T_old][d] (the sink tokens are their
 *             first rows)
 *   k_new, v_new (device) fp16 [B][Hkv][C_new][d] (may be NULL if C_new == 0)
 *   blob      (device) blob_bytes bytes (every byte is written)
 * k, v, k_new, v_new and blob must be 16-byte aligned (DQA_ERR_ALIGN).
 * Errors: DQA_ERR_NULL, DQA_ERR_PLAN, DQA_ERR_ALIGN, DQA_ERR_HIP. */
int zoned_pack(const int32_t* plan_host, const int32_t* plan_dev,
               const uint16_t* k, const uint16_t* v, const uint16_t* k_new,
               const uint16_t* v_new, void* blob, void* stream);

/* Workspace bytes for decode_attention_zoned (0 if invalid; at least 64 KB
 * otherwise): merge counters and partial softmax states; zero it before its
 * first use (see the preamble). */
size_t decode_attention_zoned_workspace_bytes(const int32_t* plan_host, int Hq);

/* Decode attention over zones A (kept tokens, masked slots skipped), B and
 * C, with dequantization fused into the products.
 *   q (device) fp16 [B][Hq][d], Hq a multiple of Hkv (ratio as above)
 *   plan_host, plan_dev as for zoned_pack
 *   blob (device) as written by zoned_pack
 *   out (device) fp32 [B][Hq][d]
 * blob, ws and out must be 16-byte aligned (DQA_ERR_ALIGN).
 * Enqueues the split kernel (the last split of each (batch, KV head) to
 * finish merges the splits in split order).
 * Errors: DQA_ERR_NULL, DQA_ERR_PLAN, DQA_ERR_SHAPE, DQA_ERR_WORKSPACE,
 * DQA_ERR_ALIGN, DQA_ERR_UNSUPPORTED, DQA_ERR_HIP. */
int decode_attention_zoned(const uint16_t* q, int Hq, const int32_t* plan_host,
                           const int32_t* plan_dev, const void* blob,
                           float sm_scale, void* ws, size_t ws_bytes,
                           float* out, void* stream);

/* ------------------------------------------------------------------------
 * Residual vector quantization  ([P2 sec 2, key components])
 *
 * Stage s picks the codeword of codebook s nearest (squared Euclidean) to
 * the running fp32 residual, lowest index on exact ties, then subtracts it.
 * Distances are formed on the matrix cores as |c|^2 - 2 r.c with r split
 * into two fp16 halves and fp32 accumulation, so two codewords whose exact
 * distances differ by less than that arithmetic's error bound may come out
 * in either order.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for rvq_encode (codeword norms). */
size_t rvq_encode_workspace_bytes(int N, int Kc);

/* Encode n vectors.
 *   x         (device) fp16 [n][d], d == 128
 *   codebooks (device) fp16 [N][Kc][d], 1 <= N <= 8, 64 <= Kc <= 32768, Kc % 64 == 0
 *   idx       (device) int16 [n][N]
 *   ws        (device) >= rvq_encode_workspace_bytes(N, Kc)
 * x, codebooks and ws must be 16-byte aligned (DQA_ERR_ALIGN).
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_WORKSPACE, DQA_ERR_ALIGN,
 * DQA_ERR_HIP. */
int rvq_encode(const uint16_t* x, int64_t n, int d, const uint16_t* codebooks,
               int N, int Kc, int16_t* idx, void* ws, size_t ws_bytes,
               void* stream);

/* Workspace bytes for rvq_decode_attention (0 if invalid): 130
 * synchronization words per (batch, KV head), for at least 16384 of them,
 * at the start (a call counter, a table-piece flag per split, the merge
 * counter), then partial softmax states and room for the key-logit table
 * (64 KB per (batch, KV head)).  Zero it before its first use; every call
 * leaves the words as the next call on it expects, for any shape of up to
 * 16384 (batch, KV head) units, so it is not cleared again. */
size_t rvq_decode_attention_workspace_bytes(int B, int Hq, int Hkv, int T, int d);

/* Decode attention with keys and values rebuilt on the fly from their
 * indices ([P2 sec 2, decoding phase]): k_hat = sum_s Ck_s[k_idx[s]],
 * v_hat likewise, summed in fp32 in stage order.
 *   q (device) fp16 [B][Hq][d]; k_idx, v_idx (device) int16 [B][Hkv][T][N]
 *   k_codebooks, v_codebooks (device) fp16 [N][Kc][d]
 *   out (device) fp32 [B][Hq][d]
 *   q and the codebooks 16-byte aligned (else DQA_ERR_ALIGN)
 * When G * N * Kc <= 16384 (G = Hq / Hkv) the key logits go through a
 * per-(batch, KV head) table of q_h . Ck_s[c], built by the workgroups of
 * that (batch, KV head) in the same launch (a piece each, through the
 * workspace) and staged in LDS, so each key costs N lookups instead of N
 * gathered codewords; otherwise keys are rebuilt like values.
 * Enqueues one kernel; the last split of each (batch, KV head) to finish
 * merges the splits in split order.  Calls that overlap on one workspace
 * race.
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_ALIGN, DQA_ERR_WORKSPACE,
 * DQA_ERR_UNSUPPORTED, DQA_ERR_HIP. */
int rvq_decode_attention(const uint16_t* q, int B, int Hq, int Hkv, int T,
                         int d, const int16_t* k_idx, const int16_t* v_idx,
                         const uint16_t* k_codebooks,
                         const uint16_t* v_codebooks, int N, int Kc,
                         float sm_scale, void* ws, size_t ws_bytes, float* out,
                         void* stream);

/* Test hook for rvq_decode_attention's table path: the number of polls of a
 * (batch, KV head)'s table flags after which a workgroup stops waiting for
 * the other workgroups' pieces and builds the whole table itself (the path
 * taken when the workgroups of one (batch, KV head) cannot all be resident
 * at once).  Default 262144; 0 sends every workgroup down that path.
 * Applies to later calls in this process (not synchronized with calls on
 * other host threads).  Returns the previous value, or -1 for polls < 0
 * (nothing changed). */
int rvq_decode_set_table_polls(int polls);

/* ------------------------------------------------------------------------
 * RDKV bit allocation ([P3 sec 2.1, theoretical formulation]; [P3 sec 2.2,
 * bit-allocation pipeline]): distortion weights of the cache units, and the
 * widths in {0, 2, 4, 8, 16} that minimize sum_u w_u 2^(-b_u) under a total
 * budget sum_u b_u <= B by Lagrangian relaxation.  The maps feed zoned_plan.
 * Widths at multiplier lam: 2[lam < 3w/8] + 2[lam < 3w/32]
 * + 4[lam < 15w/1024] + 8[lam < 255w/524288] (the minimizer of
 * w 2^(-b) + lam b, ties to the smaller width); lam is the smallest value at
 * which a row's widths fit its budget, found exactly (float64 breakpoints of
 * float32 weights).  Weights that are NaN, negative or -0 count as 0;
 * weights must otherwise be finite.  Supported head dims d: 64 and 128
 * (else DQA_ERR_UNSUPPORTED); sm_scale must be positive and finite.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for rdkv_token_weights: the per-row log-sum-exp. */
size_t rdkv_token_weights_workspace_bytes(int B, int Hq, int T);

/* Token weights w_t = sum over query positions tau >= t of the causal
 * prefill attention a_{tau,t} (logits scaled by sm_scale), summed over the
 * G = Hq/Hkv query heads that read each KV head.
 *   q (device) fp16 [B][Hq][T][d] (every prefill query position),
 *   k (device) fp16 [B][Hkv][T][d] (keys as attention reads them),
 *   both 16-byte aligned; w (device) fp32 [B][Hkv][T].
 * Deterministic (no atomics).  Errors: DQA_ERR_NULL, DQA_ERR_SHAPE,
 * DQA_ERR_UNSUPPORTED, DQA_ERR_ALIGN, DQA_ERR_WORKSPACE, DQA_ERR_HIP. */
int rdkv_token_weights(const uint16_t* q, const uint16_t* k, int B, int Hq,
                       int Hkv, int T, int d, float sm_scale, float* w,
                       void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for rdkv_channel_weights (0 if invalid or T == 0). */
size_t rdkv_channel_weights_workspace_bytes(int B, int Hkv, int T, int d);

/* Channel weights w_c = ||Q_{:,c}|| ||K_{kept,c}|| / sqrt(d): the query
 * column over every position of the KV head's G query heads, the key
 * column over the tokens whose keep entry is nonzero.
 *   q, k as in rdkv_token_weights; keep (device) int8 [B][Hkv][T] (e.g.
 *   the value widths: 0 = evicted); w (device) fp32 [B][Hkv][d].
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_UNSUPPORTED, DQA_ERR_ALIGN,
 * DQA_ERR_WORKSPACE, DQA_ERR_HIP. */
int rdkv_channel_weights(const uint16_t* q, const uint16_t* k,
                         const int8_t* keep, int B, int Hq, int Hkv, int T,
                         int d, float* w, void* ws, size_t ws_bytes,
                         void* stream);

/* Workspace bytes for rdkv_allocate. */
size_t rdkv_allocate_workspace_bytes(int rows, int n);

/* One Lagrangian allocation per row: w (device) fp32 [rows][n] ->
 * widths (device) int8 [rows][n], each row's total <= budget (bits).
 * rows <= 65535, budget >= 0.  Errors: DQA_ERR_NULL, DQA_ERR_SHAPE,
 * DQA_ERR_WORKSPACE, DQA_ERR_HIP. */
int rdkv_allocate(const float* w, int rows, int n, long long budget,
                  int8_t* widths, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for rdkv_widths (0 if the shape is invalid). */
size_t rdkv_widths_workspace_bytes(int B, int Hq, int Hkv, int T, int d);

/* The three phases in one call, one allocation per sequence over all of its
 * KV heads: token weights; value widths v_bits (device) int8 [B][Hkv][T]
 * with sum over a sequence <= v_budget; channel weights over the tokens
 * with nonzero value width; key widths k_bits (device) int8 [B][Hkv][d]
 * with sum over a sequence <= k_budget.  Inputs as in rdkv_token_weights.
 * Errors: those of the three steps. */
int rdkv_widths(const uint16_t* q, const uint16_t* k, int B, int Hq, int Hkv,
                int T, int d, float sm_scale, long long v_budget,
                long long k_budget, int8_t* v_bits, int8_t* k_bits, void* ws,
                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Measurement helper (not part of the method): a plain streaming copy used
 * to calibrate bandwidth counters and to measure the achievable HBM rate.
 *   src, dst (device), bytes a multiple of 16, both 16-byte aligned.
 * Errors: DQA_ERR_NULL, DQA_ERR_SHAPE, DQA_ERR_HIP.
 * ------------------------------------------------------------------------ */
int dqa_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DQATTN_H */
