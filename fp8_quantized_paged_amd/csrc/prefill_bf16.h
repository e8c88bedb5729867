// Arguments and launcher of the bf16-cache prefill kernel (prefill_bf16.hip), called by
// kvq_prefill_attention (prefill.hip) after its argument checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct PrefillBf16Args {
  const uint16_t* q;          // bf16 [total_q][num_q_heads][D]
  const int32_t* cu_q_lens;   // [num_seqs + 1]
  const int32_t* seq_lens;    // [num_seqs]
  const int32_t* block_table;
  int32_t bt_stride;
  const uint16_t* k_pages;    // bf16 [P][Hkv][16][D]
  const uint16_t* v_pages;    // bf16 [P][Hkv][D][16]
  int32_t num_kv_heads, num_q_heads;
  int32_t tiles;              // 128-position query tiles per (sequence, head)
  int32_t causal, window;
  float sm_log2;              // softmax scale * log2(e)
  void* out;
  int32_t out_f32;
};

// blocks = num_seqs * num_q_heads * tiles
void launch_prefill_bf16(const PrefillBf16Args& args, int head_dim, int64_t blocks,
                         hipStream_t st);

}  // namespace kvq
