// Chunked FP8 prefill attention (placeholder entry point until the MFMA kernel
// lands): reports KVQ_ERR_UNSUPPORTED after validating its arguments.
#include "kvq_device.h"
#include "kvq_host.h"

using namespace kvq;

extern "C" kvq_status kvq_prefill_attention(const kvq_cache_desc* cache, const void* q,
                                            const int32_t* cu_q_lens, int32_t num_seqs,
                                            int32_t num_q_heads, const int32_t* block_table,
                                            int32_t block_table_stride, const int32_t* seq_lens,
                                            int32_t max_q_len, const kvq_scales* scales,
                                            int32_t causal, int32_t window, float softmax_scale,
                                            void* out, kvq_dtype out_dtype, void* stream) {
  clear_error();
  if (kvq_status s = check_cache(cache)) return s;
  return fail(KVQ_ERR_UNSUPPORTED, "prefill kernel not built yet");
}
