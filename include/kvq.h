/*
 * kvq — FP8 (OCP e4m3) paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libkvq.so.  Every pointer argument is either a HOST pointer (marked
 * [host]) or a DEVICE pointer (marked [device]); no call takes ownership of any
 * buffer and no call allocates, frees or synchronises device memory.  Device work
 * is enqueued on the caller's HIP stream (`stream` is a hipStream_t; NULL is the
 * default stream) and returns immediately.
 *
 * The method, as the source pages describe vLLM's FP8 KV cache:
 *   - "vLLM FP8 KV-Cache and Attention Quantization Update" (agentlenshq.com):
 *     FP8 e4m3 KV storage halving cache bytes with attention run in FP8
 *     (introduction); two-level accumulation, partial sums flushed to true FP32
 *     registers so long contractions keep their accuracy (section "Two-level
 *     accumulation"); sliding-window layers kept in bf16 (section "Hybrid
 *     attention and layer skipping"); per-KV-head scale arrays and query
 *     quantisation moved into a fusable op (section "Kernel and fusion
 *     optimizations").
 *   - "[vLLM] KV Cache Quantization: KV cache FP8/INT8 quantization"
 *     (blog.secrett2633.cloud): per-tensor vs per-token-head scales, the -1.0
 *     "not loaded" sentinel, the single-kv-scale rule, Q and softmax-probability
 *     scales.
 *
 * Status: every call returns kvq_status.  Host-side argument checks happen before
 * any device work is enqueued; on failure nothing is enqueued and
 * kvq_last_error() (thread-local) describes the problem.  Device-resident inputs
 * (block-table entries, slots, sequence lengths) cannot be checked without a
 * synchronisation: they are preconditions, stated per call.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 1
/* Tokens per cache page.  Fixed: the pages' tests use page size 16. */
#define KVQ_PAGE_SIZE 16
/* Largest finite e4m3 magnitude; the saturation bound of every encoder here. */
#define KVQ_E4M3_MAX 448.0f

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes */
  KVQ_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, group size, dtype combo */
  KVQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  KVQ_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} kvq_status;

typedef enum {
  KVQ_BF16 = 0,     /* bfloat16 */
  KVQ_FP8_E4M3 = 1, /* OCP e4m3 ("float8_e4m3fn"): bias 7, max 448, NaN 0x7F/0xFF */
  KVQ_F32 = 2       /* float32 (attention outputs only) */
} kvq_dtype;

typedef enum {
  /* One K and one V scale for the whole layer (checkpoint value, else 1.0). */
  KVQ_SCALE_PER_TENSOR = 0,
  /* One scale per (token, KV head), computed at cache-store time as amax/448. */
  KVQ_SCALE_PER_TOKEN_HEAD = 1,
  /* One K and one V scale per KV head for the whole layer: FA3-style scale arrays
   * ("vLLM FP8 KV-Cache and Attention Quantization Update", section "Kernel and
   * fusion optimizations": one scale per KV head).  Every row of head h is
   * quantised and read with k_scales[h] / v_scales[h]. */
  KVQ_SCALE_PER_KV_HEAD = 2
} kvq_scale_mode;

/* Resolved per-tensor scales (see kvq_resolve_scales).  All > 0. */
typedef struct {
  float q_scale;
  float k_scale;
  float v_scale;
  float prob_scale;
} kvq_scales;

/*
 * A paged KV cache for one layer.  The pools are caller-owned device buffers with
 * this fixed layout (P = num_pages, H = num_kv_heads, D = head_dim, 16 = page size):
 *
 *   dtype KVQ_FP8_E4M3:
 *     k_pages  uint8 [P][H][16][D]   token-major: one (page, head) tile holds 16
 *                                    key rows of D codes, contiguous
 *     v_pages  uint8 [P][H][D][16]   dim-major: one (page, head) tile holds D rows
 *                                    of 16 codes (one row per channel)
 *     k_scales, v_scales  float [P][H][16]   per-token-head mode
 *                         float [H]          per-KV-head mode: each > 0 and finite
 *                                            (a precondition: device values are not
 *                                            checked); NULL in per-tensor mode
 *   dtype KVQ_BF16 (sliding-window layers kept in bf16):
 *     k_pages  bf16  [P][H][16][D],  v_pages  bf16  [P][H][D][16]; no scales.
 *
 * Slot s of the cache is page s / 16, offset s % 16.  Pool bases must be 256-byte
 * aligned.  Supported: head_dim in {64, 128, 256}, page_size == 16.
 */
typedef struct {
  kvq_dtype dtype;     /* KVQ_FP8_E4M3 or KVQ_BF16 */
  kvq_scale_mode mode; /* fp8 only; ignored for bf16 */
  int32_t num_pages;
  int32_t page_size;   /* must be KVQ_PAGE_SIZE */
  int32_t num_kv_heads;
  int32_t head_dim;
  void* k_pages;       /* [device] */
  void* v_pages;       /* [device] */
  float* k_scales;     /* [device] per-token-head and per-KV-head modes only */
  float* v_scales;     /* [device] per-token-head and per-KV-head modes only */
} kvq_cache_desc;

/* ------------------------------------------------------------------------------
 * Host-only helpers (no device work; callable without a GPU).
 * ----------------------------------------------------------------------------*/

int32_t kvq_abi_version(void);
const char* kvq_status_string(kvq_status s);
/* Description of the last failure on the calling thread ("" if none). */
const char* kvq_last_error(void);

#define KVQ_WARN_UNCALIBRATED_Q_OR_PROB 1u

/*
 * Resolve raw scale parameters as loaded from a checkpoint, where -1.0 (any value
 * <= 0) means "not loaded".  Source: "[vLLM] KV Cache Quantization", sections
 * "BaseKVCacheMethod", "Per-Token-Head vs Per-Tensor quantization", "Scale
 * merging logic" and "Q/Prob scales and FP8 attention":
 *   per-token-head: all four resolved scales are 1.0 (the kernel computes K/V
 *     scales at store time; Q/prob parameters are dropped); no warning;
 *   per-tensor: k > 0 and v > 0 -> (k, v); k < 0 and v < 0 -> (1, 1); otherwise
 *     a single kv scale was loaded into k: k must be > 0 (else
 *     KVQ_ERR_INVALID_ARG) and both become max(k, v);
 *     q > 0 -> q else 1.0; prob > 0 -> prob else 1.0 (the page shows the q rule;
 *     prob follows the same reading);
 *     *warn_flags gets KVQ_WARN_UNCALIBRATED_Q_OR_PROB when q or prob is 1.0;
 *   per-KV-head: the per-tensor rules, applied to one head's (k, v) pair; resolve
 *     each head with its own call and upload the k and v results as the cache's
 *     scale arrays.
 * The platform rule that doubles K/V scales for the FNUZ fp8 variant is never
 * applied: gfx950 uses the OCP e4m3 format.
 * out [host], warn_flags [host] (may be NULL).
 */
kvq_status kvq_resolve_scales(kvq_scale_mode mode, float k_in, float v_in, float q_in,
                              float prob_in, kvq_scales* out, uint32_t* warn_flags);

#define KVQ_SKIP_SLIDING_WINDOW 1u
/*
 * Per-layer KV cache dtype ("vLLM FP8 KV-Cache and Attention Quantization Update",
 * section "Hybrid attention and layer skipping"): KVQ_BF16 when
 * (skip_flags & KVQ_SKIP_SLIDING_WINDOW) and window > 0, else KVQ_FP8_E4M3.
 */
kvq_dtype kvq_layer_kv_dtype(int32_t window, uint32_t skip_flags);

/* ------------------------------------------------------------------------------
 * Device operations.
 * ----------------------------------------------------------------------------*/

/*
 * Quantising cache write ("[vLLM] KV Cache Quantization", section "Per-Token-Head
 * vs Per-Tensor quantization": per-token-head scales are computed by the kernel
 * when the cache is stored).
 *
 * For every token t < num_tokens with slot_mapping[t] >= 0, and every KV head h:
 *   fp8 per-tensor:      s = k_scale (resp. v_scale), s > 0
 *   fp8 per-KV-head:     s = cache->k_scales[h] (resp. v_scales[h])
 *   fp8 per-token-head:  s = fl32(amax / 448), amax = max_d |x[d]| (NaN
 *                        propagates); amax == 0 -> s = 1.0; s is stored in the
 *                        scale pool at (page, h, offset)
 *   code[d] = e4m3_rne_saturating(fl32(x[d] / s)), IEEE float32 division;
 *             a NaN quotient gives 0x7F | sign bit of x[d]
 *   bf16 cache: x is copied unchanged.
 * k, v [device]: bf16, token t / head h / dim d at element t*token_stride + h*D + d
 *   (token_stride in elements, >= H*D; 0 means H*D).
 * slot_mapping [device]: int64 [num_tokens]; negative = skip.  Preconditions:
 *   every non-negative slot < num_pages*16, no slot repeated within one call.
 * k_scale, v_scale: per-tensor fp8 scales (> 0); ignored in the other modes.
 * num_tokens == 0 is a no-op.
 */
kvq_status kvq_cache_write(const kvq_cache_desc* cache, const void* k, const void* v,
                           int64_t token_stride, const int64_t* slot_mapping,
                           int32_t num_tokens, float k_scale, float v_scale,
                           void* stream);

/*
 * Flat quantisation utility (the encoder of kvq_cache_write, exposed for tests and
 * for callers that keep their own layout): codes[i] = e4m3_rne_saturating(
 * fl32(x[i] / scale)) for i < n; NaN quotient -> 0x7F | sign bit of x[i].
 * x [device] bf16 [n]; codes [device] uint8 [n]; scale > 0 (any float accepted).
 */
kvq_status kvq_quantize_fp8(const void* x, int64_t n, float scale, uint8_t* codes,
                            void* stream);

/* Decode workspace layout, fixed for every call so that calls of any shape may share
 * one buffer: bytes [0, KVQ_DECODE_COUNTER_BYTES) hold the int32 completion counter
 * of each (sequence b, KV head g) at index b * num_kv_heads + g; the split-K partial
 * results follow.  A call with more than one split supports at most
 * KVQ_DECODE_MAX_SPLIT_UNITS (sequence, KV head) pairs (KVQ_ERR_UNSUPPORTED beyond). */
#define KVQ_DECODE_MAX_SPLIT_UNITS 65536
#define KVQ_DECODE_COUNTER_BYTES (4 * KVQ_DECODE_MAX_SPLIT_UNITS)

/*
 * Workspace bytes needed by kvq_decode_attention for these arguments: the counter
 * prefix (KVQ_DECODE_COUNTER_BYTES) followed by the split-K partial results; 0 when
 * every sequence fits in one split (then no workspace is read or written).
 * pages_per_split = 0 selects the library's choice, which depends only on the
 * arguments given here (it spreads max_seq_len over about two workgroups per CU);
 * otherwise 1..256.  A batch whose lengths differ widely runs faster with a smaller
 * value chosen from its actual lengths, since the library sees only max_seq_len.
 * bytes [host].
 */
kvq_status kvq_decode_workspace_bytes(const kvq_cache_desc* cache, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_seq_len,
                                      int32_t window, int32_t pages_per_split,
                                      size_t* bytes);

/*
 * Paged GQA decode attention: one new query token per sequence over the cache.
 *
 * For sequence b, query head h (KV head g = h / (num_q_heads / num_kv_heads)), and
 * keys j in [lo, L) with L = seq_lens[b], lo = max(0, L - window) if window > 0
 * else 0 (seq_lens counts the current token, whose K/V are already written):
 *   fp8 cache:  q codes = e4m3_rne_saturating(fl32(q / q_scale)) (the fused query
 *               quantisation), score_j = (q_codes . k_codes_j) * q_scale *
 *               k_scale_j * softmax_scale, where k_scale_j is the per-token-head
 *               scale, cache->k_scales[g] (per-KV-head) or scales->k_scale
 *               (per-tensor); V likewise with v_scale_j.
 *   bf16 cache: score_j = (q . k_j) * softmax_scale on the bf16 values.
 *   out[b][h] = sum_j softmax(score)_j * v_j;  L == 0 gives zeros.
 * Arithmetic: products are exact, sums and the online softmax are float32; the
 * probability weights p_j * v_scale_j enter the P.V dot products rounded to f16;
 * partial results of each split are merged in float32 (the pages' two-level
 * accumulation: level 1 inside a page, level 2 in the split's fp32 registers,
 * level 3 across splits, done by the last split of each (sequence, KV head) to
 * finish; there is a single kernel launch per call).
 *
 * q [device] bf16 [num_seqs][num_q_heads][D];  out [device] [num_seqs][num_q_heads][D]
 *   of out_dtype (KVQ_BF16 or KVQ_F32).
 * block_table [device] int32 [num_seqs][block_table_stride]: physical page of each
 *   logical page.  seq_lens [device] int32 [num_seqs].
 * Preconditions: 0 <= seq_lens[b] <= max_seq_len; entries used are < num_pages.
 *   (A device length above max_seq_len cannot be detected on the host; the kernel
 *   then reads that sequence only up to max_seq_len -- no access past its block-table
 *   row -- so its output is wrong but no memory outside the arguments is touched and
 *   the workspace counters still return to zero.)
 * scales [host]: per-tensor values (q_scale and, in per-tensor mode, k/v scales;
 *   the per-KV-head mode takes k/v from the cache's scale arrays).
 * window: 0 = full attention, > 0 = the last `window` keys.
 * softmax_scale: 0 selects 1/sqrt(D).
 * pages_per_split: 0 = library choice; must match kvq_decode_workspace_bytes.
 * workspace [device], workspace_bytes: at least kvq_decode_workspace_bytes(...).
 *   Its counter prefix must be zero before the first call (allocate it zero-filled);
 *   every call leaves it zero again, so one workspace, sized for the largest call,
 *   serves calls of any shape.  Calls that share one workspace must not overlap in
 *   time (same stream, or ordered by events).
 * Supported: D in {64,128,256}; num_q_heads / num_kv_heads in {1,2,4,8,16}.
 */
kvq_status kvq_decode_attention(const kvq_cache_desc* cache, const void* q,
                                int32_t num_seqs, int32_t num_q_heads,
                                const int32_t* block_table, int32_t block_table_stride,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                const kvq_scales* scales, int32_t window,
                                float softmax_scale, int32_t pages_per_split,
                                void* out, kvq_dtype out_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Size of the device scratch behind kvq_decode_attention_noalloc (per GPU). */
#define KVQ_DECODE_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * kvq_decode_attention without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It calls no allocating routine: the split-K partials and the
 * completion counters live in a library-owned device array of KVQ_DECODE_SCRATCH_BYTES
 * per GPU (the workspace layout above: counter prefix, then partials), held until the
 * process ends.  The first call on a device (the calling thread's current device,
 * which must own `stream`) looks the array up and clears its counters with a small
 * kernel on `stream`.  Every call on one GPU shares that array: calls that overlap in
 * time on one GPU (different streams, or another thread) race and give wrong results;
 * order them on one stream.  Arguments, results and preconditions are those of
 * kvq_decode_attention; KVQ_ERR_WORKSPACE when kvq_decode_workspace_bytes(...) for
 * these arguments exceeds KVQ_DECODE_SCRATCH_BYTES (split the batch or raise
 * pages_per_split).
 */
kvq_status kvq_decode_attention_noalloc(const kvq_cache_desc* cache, const void* q,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        const int32_t* block_table,
                                        int32_t block_table_stride, const int32_t* seq_lens,
                                        int32_t max_seq_len, const kvq_scales* scales,
                                        int32_t window, float softmax_scale,
                                        int32_t pages_per_split, void* out,
                                        kvq_dtype out_dtype, void* stream);

/*
 * Decode step: the cache write of each sequence's new token and the decode attention
 * of kvq_decode_attention, in one launch.  For every sequence b with L = seq_lens[b]
 * > 0 and every KV head h, the row k_new[b][h] / v_new[b][h] is stored at position
 * L - 1, i.e. at slot block_table[b][(L-1)/16] * 16 + (L-1) % 16, exactly as
 * kvq_cache_write would store it (same quantisation and scales: per-tensor
 * scales->k_scale / v_scale, per-KV-head arrays, or per-token-head amax / 448),
 * and attention then runs
 * over positions [lo, L) as in kvq_decode_attention, reading the new row.  Results
 * (cache contents and output) equal kvq_cache_write followed by kvq_decode_attention
 * ("Kernel and fusion optimizations" of "vLLM FP8 KV-Cache and Attention
 * Quantization Update": work around the attention op fused into its launch).
 * k_new, v_new [device]: bf16 [num_seqs][num_kv_heads][D], contiguous, 16-byte
 * aligned.  The other arguments, their preconditions and the workspace rules are
 * those of kvq_decode_attention; the cache is written, so no other call may use it
 * concurrently.  A sequence whose device length exceeds max_seq_len (a precondition
 * violation) gets no new row written.
 */
kvq_status kvq_decode_step(const kvq_cache_desc* cache, const void* q, const void* k_new,
                           const void* v_new, int32_t num_seqs, int32_t num_q_heads,
                           const int32_t* block_table, int32_t block_table_stride,
                           const int32_t* seq_lens, int32_t max_seq_len,
                           const kvq_scales* scales, int32_t window, float softmax_scale,
                           int32_t pages_per_split, void* out, kvq_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked causal prefill over an FP8 cache ("vLLM FP8 KV-Cache and Attention
 * Quantization Update", sections "Two-level accumulation" and "Kernel and fusion
 * optimizations"; prefill of head_dim 256 in section "Per-architecture results").
 *
 * Sequence b owns query rows cu_q_lens[b] .. cu_q_lens[b+1]-1 (n_b rows); its
 * cache already holds all L = seq_lens[b] tokens, the n_b new ones last (write them
 * with kvq_cache_write first).  Query row i sits at absolute position L - n_b + i
 * and, with causal != 0, sees keys 0 .. L - n_b + i (window > 0: only keys
 * > L - n_b + i - window).
 *   S = (q codes . k codes) on FP8 matrix cores, scaled by q_scale * k_scale_j *
 *   softmax_scale (k_scale_j: per-token-head scale, cache->k_scales[g] per-KV-head,
 *   or scales->k_scale per-tensor; V alike); online softmax in float32 against a
 *   reference that puts the largest weight seen at 2^4 (at most 2^8); the weights
 *   quantised to e4m3 with prob_scale (per-token V scales folded in before
 *   rounding) and P.V on FP8 matrix cores, each 64-key chunk's sum added into the
 *   running float32 output (two-level accumulation; the row sum uses the same
 *   rounded weights, so the output is a convex combination of V rows).
 * q [device] bf16 [total_q][num_q_heads][D]; out [device] [total_q][num_q_heads][D].
 * cu_q_lens [device] int32 [num_seqs+1]; seq_lens [device] int32 [num_seqs];
 * block_table as for decode.  max_q_len >= every n_b.
 * bf16 cache (the sliding-window layers' skip path, "Hybrid attention and layer
 *   skipping"): S = q . k on the bf16 values (bf16 matrix cores, exact products,
 *   float32 sums) scaled by softmax_scale, float32 online softmax, weights rounded to
 *   bf16 for P.V and normalised by the sum of the rounded weights; scales unused.
 * Supported: fp8 or bf16 cache, D in {64,128,256}, group size in {1,2,4,8,16}.
 */
kvq_status kvq_prefill_attention(const kvq_cache_desc* cache, const void* q,
                                 const int32_t* cu_q_lens, int32_t num_seqs,
                                 int32_t num_q_heads, const int32_t* block_table,
                                 int32_t block_table_stride, const int32_t* seq_lens,
                                 int32_t max_q_len, const kvq_scales* scales,
                                 int32_t causal, int32_t window, float softmax_scale,
                                 void* out, kvq_dtype out_dtype, void* stream);

/* Level 2 of the FP8 prefill's two-level accumulation ("vLLM FP8 KV-Cache and Attention
 * Quantization Update", section "Two-level accumulation": partial sums flushed to true
 * FP32 registers every chunk; the page's recommendations table offers turning the
 * scheme off for head_dim-256 prefill-heavy work). */
typedef enum {
  /* The matrix core's float32 C operand carries the running output: each 64-key
   * chunk's MFMA adds into it (the default; kvq_prefill_attention). */
  KVQ_ACCUM_MFMA_CHAIN = 0,
  /* Explicit flush: each 64-key chunk's MFMA starts from zero and its result is added
   * into the running output by float32 vector adds (16 extra adds per lane and
   * output block per chunk). */
  KVQ_ACCUM_VALU_ADD = 1
} kvq_accumulation;

/*
 * kvq_prefill_attention with the level-2 accumulation form chosen by `accum` (an
 * ablation of the two-level scheme; both forms keep the running output in float32).
 * Arguments, layouts and errors as kvq_prefill_attention; additionally
 * KVQ_ERR_INVALID_ARG for an unknown `accum` and KVQ_ERR_UNSUPPORTED for
 * KVQ_ACCUM_VALU_ADD over a bf16 cache (its prefill has the chained form only).
 */
kvq_status kvq_prefill_attention_accum(const kvq_cache_desc* cache, const void* q,
                                       const int32_t* cu_q_lens, int32_t num_seqs,
                                       int32_t num_q_heads, const int32_t* block_table,
                                       int32_t block_table_stride, const int32_t* seq_lens,
                                       int32_t max_q_len, const kvq_scales* scales,
                                       int32_t causal, int32_t window, float softmax_scale,
                                       void* out, kvq_dtype out_dtype,
                                       kvq_accumulation accum, void* stream);

/*
 * Workspace for kvq_prefill_attention_ws: 0 where the launch needs no key split (it
 * already has about 1.5 workgroups per CU: roughly num_seqs * num_kv_heads *
 * ceil(max_q_len * G / 128) >= 384, G = num_q_heads / num_kv_heads) and for bf16
 * caches or unsupported shapes; else the bytes of the split's partial results
 * (splits * workgroups * 128 rows * (head_dim + 2) * 4).  Depends only on these
 * arguments.
 */
size_t kvq_prefill_workspace_bytes(const kvq_cache_desc* cache, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_q_len);

/*
 * kvq_prefill_attention for short query chunks on long contexts: the same result
 * (same arguments, layouts and errors), computed with each workgroup's keys split over
 * up to 32 workgroups.  Each split writes unnormalised partial results (O, reference
 * maximum, row sum) to `workspace` [device], and a second kernel on the same stream
 * combines them through their maxima and sums, as the prefill combines its key tiles
 * ("vLLM FP8 KV-Cache and Attention Quantization Update", section "Two-level
 * accumulation").  Used
 * where kvq_prefill_workspace_bytes is non-zero: 16 new tokens on 131,072 cached
 * tokens otherwise run on 8 workgroups.  workspace_bytes must be at least that value
 * (else INVALID_ARG), workspace 16-byte aligned; with a null workspace the call is
 * kvq_prefill_attention.  A bf16 cache ignores the workspace.  The workspace is
 * scratch owned by the caller; calls that share one must not overlap.
 */
kvq_status kvq_prefill_attention_ws(const kvq_cache_desc* cache, const void* q,
                                    const int32_t* cu_q_lens, int32_t num_seqs,
                                    int32_t num_q_heads, const int32_t* block_table,
                                    int32_t block_table_stride, const int32_t* seq_lens,
                                    int32_t max_q_len, const kvq_scales* scales,
                                    int32_t causal, int32_t window, float softmax_scale,
                                    void* out, kvq_dtype out_dtype, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Paged query-key logits for a sparse-attention indexer ("vLLM Qwen3.8-Flash-Next: QSA
 * Indexer ... FP8 support", section on the reference test of the decode/prefill
 * selection: the indexer's top-k selection reads these scores from an FP8 or bf16
 * paged cache, and FP8 scores are compared value by value).
 *
 * Request b owns query rows cu_rows[b] .. cu_rows[b+1]-1; row r sees the first
 * min(row_lens[r], seq_lens[b]) keys of request b's cache (keys through the block
 * table as in kvq_decode_attention).  For query head h (key head g = h / (Hq/Hkv)):
 *   out[r][h][j] = (q codes . k codes) * q_scale * k_scale_j   (FP8 cache: q quantised
 *                  to e4m3 with scales->q_scale; k_scale_j as in attention: per-token-
 *                  head, cache->k_scales[g] per-KV-head, or scales->k_scale per-tensor)
 *   out[r][h][j] = q . k_j                                     (bf16 cache, unscaled)
 * for visible j, and -inf for the other j < out_stride.  Products are exact and sums
 * float32 (e4m3 and bf16 values widened for the matrix cores); no softmax scale and
 * no reduction over heads (the selection rule is the caller's).
 * q [device] bf16 [total_rows][num_q_heads][D], 16-byte aligned; cu_rows [device]
 * int32 [num_seqs+1]; total_rows = cu_rows[num_seqs] (a host value that sizes the
 * launch: the kernel takes the rows themselves from cu_rows, and 0 writes nothing);
 * row_lens [device] int32 [total_rows]; seq_lens [device] int32 [num_seqs]; out
 * [device] float32 [total_rows][num_q_heads][out_stride], 16-byte aligned, out_stride
 * a multiple of 4; every entry is written.  Only the K pool (and K scales) of the cache
 * is read.  Errors: INVALID_ARG for NULL pointers, a negative count, misaligned q/out
 * (16 bytes) or per-token-head k_scales (16 bytes), out_stride not a multiple of 4, Hq
 * not a multiple of Hkv, a grid past 2^31 - 1 workgroups; HIP for a failed launch.
 * Supported: fp8 or bf16 cache, D in {64,128,256}, any group size.
 */
kvq_status kvq_paged_logits(const kvq_cache_desc* cache, const void* q, const int32_t* cu_rows,
                            int32_t num_seqs, int32_t total_rows, int32_t num_q_heads,
                            const int32_t* row_lens, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* seq_lens,
                            const kvq_scales* scales, float* out,
                            int32_t out_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
