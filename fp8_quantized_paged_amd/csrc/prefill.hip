// Host entry points of the chunked prefill: argument checks, then the FP8 kernels
// (prefill_kernel.h, instantiated per head_dim in prefill_d*.hip) or, for a bf16
// cache, the bf16 kernel (prefill_bf16.hip).
#include <algorithm>

#include "kvq_device.h"
#include "kvq_host.h"
#include "prefill_bf16.h"
#include "prefill_kernel.h"


using namespace kvq;

namespace kvq {
namespace pf {

// Key splits for a launch of `blocks` workgroups: none once the launch has about 1.5
// workgroups per CU, else enough for ~512 workgroups, at most kMaxSplits.  A short
// query chunk on a long context otherwise runs on a handful of workgroups (16 new
// tokens at group 4 on 131,072 cached: 8 workgroups, 2.18 ms).  Fewer splits also mean
// fewer partial results for the merge: round-robin A/B over four short-chunk shapes,
// ~512 workgroups / at most 32 splits 4-12% faster than ~768 / 64 and ~1,024 / 64
// (16 new on 131,072: 110.6 against 118.7 and 119.3 us; 8 x 16 on 32,768: 148 against
// 168 and 175 us).
constexpr int kMaxSplits = 32;
static int plan_splits(int64_t blocks) {
  if (blocks >= 384) return 1;
  return (int)std::min<int64_t>(kMaxSplits, (512 + blocks - 1) / blocks);
}
static size_t split_ws_bytes(int nsplit, int64_t blocks, int D) {
  return nsplit <= 1 ? 0 : (size_t)nsplit * blocks * kWgRows * (D + 2) * sizeof(float);
}

// Combines the key splits' partial results of one row (thread: 4 of its D dims; one
// dim per thread, for 4x the waves, measured slower: 139 against 128 us per call):
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the splits that saw keys.
// Rows are decoded from the prefill workgroup index as the prefill kernel decodes them.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(const PrefillArgs a, int G,
                                                            int nblocks) {
  constexpr int TPR = D / 4;       // threads per row
  constexpr int RPB = 256 / TPR;   // rows per merge workgroup
  constexpr int PER = kWgRows / RPB;
  const int blk = (int)blockIdx.x / PER;
  const int wg_row = ((int)blockIdx.x % PER) * RPB + (int)threadIdx.x / TPR;
  const int d0 = 4 * ((int)threadIdx.x % TPR);
  const int hkv = a.num_kv_heads;
  const int g = blk % hkv;
  const int rest = blk / hkv;
  const int tile = a.tiles - 1 - rest % a.tiles;
  const int b = rest / a.tiles;
  const int q0 = a.cu_q_lens[b];
  const int n = a.cu_q_lens[b + 1] - q0;
  const int p_loc = tile * (kWgRows / G) + wg_row / G;
  if (p_loc >= n) return;  // no such row (no barrier in this kernel)
  // The loads are unconditional and the loops unrolled, so several splits' loads are
  // in flight at once (one at a time, behind a branch: 136 against 128 us per call of
  // 16 new tokens on 131,072 with 64 splits, of which the merge took 54 us); a split
  // that saw no key wrote no O, and a select (never a multiplication: the memory may
  // hold NaN) drops what its slot holds.
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < a.nsplit; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(
        a.ws_ml + 2 * (((int64_t)s * nblocks + blk) * kWgRows + wg_row));
    M = ml.y > 0.0f ? fmaxf(M, ml.x) : M;
  }
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float lsum = 0.0f;
#pragma unroll 8
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t r = ((int64_t)s * nblocks + blk) * kWgRows + wg_row;
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + 2 * r);
    float4 o = *reinterpret_cast<const float4*>(a.ws_o + r * D + d0);
    const bool has = ml.y > 0.0f;
    const float w = has ? exp2f(ml.x - M) : 0.0f;
    o = has ? o : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    lsum += has ? w * ml.y : 0.0f;
    acc.x += w * o.x;
    acc.y += w * o.y;
    acc.z += w * o.z;
    acc.w += w * o.w;
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  const int64_t orow = ((int64_t)(q0 + p_loc) * hkv * G + g * G + wg_row % G) * D + d0;
  if (a.out_f32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + orow) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + orow) =
        make_uint2(pack_bf16x2(acc.x * inv, acc.y * inv), pack_bf16x2(acc.z * inv, acc.w * inv));
  }
}

}  // namespace pf
}  // namespace kvq

static kvq_status prefill_impl(const kvq_cache_desc* cache, const void* q,
                               const int32_t* cu_q_lens, int32_t num_seqs, int32_t num_q_heads,
                               const int32_t* block_table, int32_t block_table_stride,
                               const int32_t* seq_lens, int32_t max_q_len,
                               const kvq_scales* scales, int32_t causal, int32_t window,
                               float softmax_scale, void* out, kvq_dtype out_dtype,
                               kvq_accumulation accum, void* workspace,
                               size_t workspace_bytes, void* stream) {
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
  // key splits only where the caller gave a workspace (kvq_prefill_attention_ws)
  args.nsplit = workspace ? pf::plan_splits(blocks) : 1;
  args.ws_o = nullptr;
  args.ws_ml = nullptr;
  if (args.nsplit > 1) {
    const size_t need = pf::split_ws_bytes(args.nsplit, blocks, D);
    if (workspace_bytes < need)
      return fail(KVQ_ERR_INVALID_ARG, "workspace %zu bytes, %zu needed", workspace_bytes, need);
    if ((uintptr_t)workspace & 15u)
      return fail(KVQ_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    args.ws_o = static_cast<float*>(workspace);
    args.ws_ml = args.ws_o + (size_t)args.nsplit * blocks * pf::kWgRows * D;
  }
  auto st = static_cast<hipStream_t>(stream);
  const bool pth = cache->mode == KVQ_SCALE_PER_TOKEN_HEAD;
  const bool valu = accum == KVQ_ACCUM_VALU_ADD;
  const dim3 grid((unsigned)blocks, (unsigned)args.nsplit);
  switch (D) {
    case 64: pf::launch_prefill_fp8<64>(G, pth, valu, args, grid, st); break;
    case 128: pf::launch_prefill_fp8<128>(G, pth, valu, args, grid, st); break;
    case 256: pf::launch_prefill_fp8<256>(G, pth, valu, args, grid, st); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  if (args.nsplit > 1) {
    const unsigned mblocks = (unsigned)(blocks * pf::kWgRows / (256 / (D / 4)));
    switch (D) {
      case 64: pf::prefill_merge_kernel<64><<<mblocks, 256, 0, st>>>(args, G, (int)blocks); break;
      case 128: pf::prefill_merge_kernel<128><<<mblocks, 256, 0, st>>>(args, G, (int)blocks); break;
      case 256: pf::prefill_merge_kernel<256><<<mblocks, 256, 0, st>>>(args, G, (int)blocks); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_ERR_HIP, "prefill merge launch: %s", hipGetErrorString(e));
  }
  return KVQ_OK;
}

extern "C" size_t kvq_prefill_workspace_bytes(const kvq_cache_desc* cache, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_q_len) {
  if (!cache || cache->num_kv_heads <= 0 || num_seqs <= 0 || num_q_heads <= 0 ||
      max_q_len <= 0 || num_q_heads % cache->num_kv_heads || cache->dtype != KVQ_FP8_E4M3)
    return 0;
  const int G = num_q_heads / cache->num_kv_heads;
  if (!supported_group(G)) return 0;
  const int np = pf::kWgRows / G;
  const int64_t blocks = (int64_t)num_seqs * cache->num_kv_heads * ((max_q_len + np - 1) / np);
  return pf::split_ws_bytes(pf::plan_splits(blocks), blocks, cache->head_dim);
}

extern "C" kvq_status kvq_prefill_attention_ws(
    const kvq_cache_desc* cache, const void* q, const int32_t* cu_q_lens, int32_t num_seqs,
    int32_t num_q_heads, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, int32_t max_q_len, const kvq_scales* scales, int32_t causal,
    int32_t window, float softmax_scale, void* out, kvq_dtype out_dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  clear_error();
  return prefill_impl(cache, q, cu_q_lens, num_seqs, num_q_heads, block_table,
                      block_table_stride, seq_lens, max_q_len, scales, causal, window,
                      softmax_scale, out, out_dtype, KVQ_ACCUM_MFMA_CHAIN, workspace,
                      workspace_bytes, stream);
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
                      softmax_scale, out, out_dtype, KVQ_ACCUM_MFMA_CHAIN, nullptr, 0, stream);
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
                      softmax_scale, out, out_dtype, accum, nullptr, 0, stream);
}
