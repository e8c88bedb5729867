// Host entry points of the chunked prefill: argument checks, then the FP8 kernels
// (prefill_kernel.h, instantiated per head_dim in prefill_d*.hip) or, for a bf16
// cache, the bf16 kernel (prefill_bf16.hip).
#include "kvq_device.h"
#include "kvq_host.h"
#include "prefill_bf16.h"
#include "prefill_kernel.h"


using namespace kvq;

static kvq_status prefill_impl(const kvq_cache_desc* cache, const void* q,
                               const int32_t* cu_q_lens, int32_t num_seqs, int32_t num_q_heads,
                               const int32_t* block_table, int32_t block_table_stride,
                               const int32_t* seq_lens, int32_t max_q_len,
                               const kvq_scales* scales, int32_t causal, int32_t window,
                               float softmax_scale, void* out, kvq_dtype out_dtype,
                               kvq_accumulation accum, void* stream) {
  if (kvq_status s = check_cache(cache)) return s;
  if (accum != KVQ_ACCUM_MFMA_CHAIN && accum != KVQ_ACCUM_VALU_ADD)
    return fail(KVQ_ERR_INVALID_ARG, "accumulation %d", (int)accum);
  if (num_seqs < 0 || num_q_heads <= 0 || max_q_len < 0 || window < 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_seqs %d num_q_heads %d max_q_len %d window %d",
                num_seqs, num_q_heads, max_q_len, window);
  if (num_q_heads % cache->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  const int G = num_q_heads / cache->num_kv_heads;
  if (!supported_group(G))
    return fail(KVQ_ERR_UNSUPPORTED, "group size %d (1, 2, 4, 8, 16 are built)", G);
  if (num_seqs == 0 || max_q_len == 0) return KVQ_OK;
  if (out_dtype != KVQ_BF16 && out_dtype != KVQ_F32)
    return fail(KVQ_ERR_UNSUPPORTED, "out_dtype %d (bf16 or f32)", (int)out_dtype);
  if (!q || !out || !cu_q_lens || !seq_lens || !block_table)
    return fail(KVQ_ERR_INVALID_ARG, "q, out, cu_q_lens, seq_lens or block_table is NULL");
  if (((uintptr_t)q | (uintptr_t)out) & 15u)
    return fail(KVQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (block_table_stride <= 0) return fail(KVQ_ERR_INVALID_ARG, "block_table_stride <= 0");
  if (cache->dtype == KVQ_BF16) {  // the skip path's bf16 cache: prefill_bf16.hip
    if (accum != KVQ_ACCUM_MFMA_CHAIN)
      return fail(KVQ_ERR_UNSUPPORTED, "the bf16-cache prefill has one accumulation form");
    if (!(softmax_scale >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale < 0");
    const int Db = cache->head_dim;
    PrefillBf16Args ba;
    ba.q = static_cast<const uint16_t*>(q);
    ba.cu_q_lens = cu_q_lens;
    ba.seq_lens = seq_lens;
    ba.block_table = block_table;
    ba.bt_stride = block_table_stride;
    ba.k_pages = static_cast<const uint16_t*>(cache->k_pages);
    ba.v_pages = static_cast<const uint16_t*>(cache->v_pages);
    ba.num_kv_heads = cache->num_kv_heads;
    ba.num_q_heads = num_q_heads;
    ba.tiles = (max_q_len + 127) / 128;
    ba.causal = causal != 0;
    ba.window = window;
    const float smb = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)Db);
    ba.sm_log2 = smb * pf::kLog2e;
    ba.out = out;
    ba.out_f32 = out_dtype == KVQ_F32;
    const int64_t bblocks = (int64_t)num_seqs * num_q_heads * ba.tiles;
    if (bblocks > 0x7FFFFFFF) return fail(KVQ_ERR_INVALID_ARG, "grid too large");
    launch_prefill_bf16(ba, Db, bblocks, static_cast<hipStream_t>(stream));
    const hipError_t be = hipGetLastError();
    if (be != hipSuccess) return fail(KVQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(be));
    return KVQ_OK;
  }
  if (!scales) return fail(KVQ_ERR_INVALID_ARG, "scales is NULL");
  if (!(scales->q_scale > 0.0f) || !(scales->prob_scale > 0.0f) ||
      (cache->mode == KVQ_SCALE_PER_TENSOR && !(scales->k_scale > 0.0f && scales->v_scale > 0.0f)))
    return fail(KVQ_ERR_INVALID_ARG, "scales must be > 0");
  if (!(softmax_scale >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "softmax_scale < 0");
  const int D = cache->head_dim;
  const int np = pf::kWgRows / G;
  pf::PrefillArgs args;
  args.q = static_cast<const uint16_t*>(q);
  args.cu_q_lens = cu_q_lens;
  args.num_kv_heads = cache->num_kv_heads;
  args.tiles = (max_q_len + np - 1) / np;
  args.block_table = block_table;
  args.bt_stride = block_table_stride;
  args.seq_lens = seq_lens;
  args.k_pages = static_cast<const uint8_t*>(cache->k_pages);
  args.v_pages = static_cast<const uint8_t*>(cache->v_pages);
  args.k_scales = cache->k_scales;
  args.v_scales = cache->v_scales;
  args.q_scale = scales->q_scale;
  args.k_scale = scales->k_scale;
  args.v_scale = scales->v_scale;
  args.prob_scale = scales->prob_scale;
  args.head_scales = cache->mode == KVQ_SCALE_PER_KV_HEAD;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)D);
  args.sm_log2 = sm * pf::kLog2e;
  args.causal = causal != 0;
  args.window = window;
  args.out = out;
  args.out_f32 = out_dtype == KVQ_F32;
  const int64_t blocks = (int64_t)num_seqs * cache->num_kv_heads * args.tiles;
  if (blocks > 0x7FFFFFFF) return fail(KVQ_ERR_INVALID_ARG, "grid too large");
  auto st = static_cast<hipStream_t>(stream);
  const bool pth = cache->mode == KVQ_SCALE_PER_TOKEN_HEAD;
  const bool valu = accum == KVQ_ACCUM_VALU_ADD;
  switch (D) {
    case 64: pf::launch_prefill_fp8<64>(G, pth, valu, args, (unsigned)blocks, st); break;
    case 128: pf::launch_prefill_fp8<128>(G, pth, valu, args, (unsigned)blocks, st); break;
    case 256: pf::launch_prefill_fp8<256>(G, pth, valu, args, (unsigned)blocks, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}

extern "C" kvq_status kvq_prefill_attention(const kvq_cache_desc* cache, const void* q,
                                            const int32_t* cu_q_lens, int32_t num_seqs,
                                            int32_t num_q_heads, const int32_t* block_table,
                                            int32_t block_table_stride, const int32_t* seq_lens,
                                            int32_t max_q_len, const kvq_scales* scales,
                                            int32_t causal, int32_t window, float softmax_scale,
                                            void* out, kvq_dtype out_dtype, void* stream) {
  clear_error();
  return prefill_impl(cache, q, cu_q_lens, num_seqs, num_q_heads, block_table,
                      block_table_stride, seq_lens, max_q_len, scales, causal, window,
                      softmax_scale, out, out_dtype, KVQ_ACCUM_MFMA_CHAIN, stream);
}

extern "C" kvq_status kvq_prefill_attention_accum(
    const kvq_cache_desc* cache, const void* q, const int32_t* cu_q_lens, int32_t num_seqs,
    int32_t num_q_heads, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, int32_t max_q_len, const kvq_scales* scales, int32_t causal,
    int32_t window, float softmax_scale, void* out, kvq_dtype out_dtype,
    kvq_accumulation accum, void* stream) {
  clear_error();
  return prefill_impl(cache, q, cu_q_lens, num_seqs, num_q_heads, block_table,
                      block_table_stride, seq_lens, max_q_len, scales, causal, window,
                      softmax_scale, out, out_dtype, accum, stream);
}
