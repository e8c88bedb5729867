// Host-side helpers shared by the kvq entry points: error reporting and argument
// checks.  Nothing here touches the device.
#pragma once

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "kvq.h"

namespace kvq {

// Records a formatted message for kvq_last_error() and returns `st`.
kvq_status fail(kvq_status st, const char* fmt, ...);
void clear_error();

inline bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
inline bool supported_group(int g) {
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

// Checks the fields of a cache descriptor that every call relies on.
kvq_status check_cache(const kvq_cache_desc* c);

// Body of kvq_decode_attention (k_new == v_new == nullptr) and kvq_decode_step.
kvq_status decode_impl(const kvq_cache_desc* cache, const void* q, int32_t num_seqs,
                       int32_t num_q_heads, const int32_t* block_table,
                       int32_t block_table_stride, const int32_t* seq_lens,
                       int32_t max_seq_len, const kvq_scales* scales, int32_t window,
                       float softmax_scale, int32_t pages_per_split, void* out,
                       kvq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                       void* stream, const void* k_new, const void* v_new);

}  // namespace kvq
