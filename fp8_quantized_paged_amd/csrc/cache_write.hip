// Quantising paged cache write and the flat e4m3 quantiser.
//
// "[vLLM] KV Cache Quantization: KV cache FP8/INT8 quantization"
// (blog.secrett2633.cloud), section "Per-Token-Head vs Per-Tensor quantization":
// per-tensor mode uses one K and one V scale per layer; per-token-head mode has
// the kernel compute a scale for every (token, head) when it stores the cache.
// "vLLM FP8 KV-Cache and Attention Quantization Update", section "Kernel and fusion
// optimizations": per-KV-head mode quantises head h with its own layer scale.
// Scale = amax / 448, code = clamp(round_rne(v / scale), +-448).
//
// Work split: one row = one (token, KV head) of D bf16 values; D/8 lanes own a
// row, 8 consecutive values (one 16-byte load) each.  The row maximum is reduced
// across those lanes; every lane then quantises its 8 values.  K rows are stored
// token-major (8 codes = one 8-byte store per lane), V rows dim-major (one byte per
// channel row of the page tile).
#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

template <int D, bool kFp8, bool kPerTokenHead>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t token_stride,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t num_heads,
    uint8_t* __restrict__ k_pages, uint8_t* __restrict__ v_pages,
    float* __restrict__ k_scales, float* __restrict__ v_scales, float k_scale,
    float v_scale) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int c = threadIdx.x % kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  if (row >= (int64_t)num_tokens * num_heads) return;  // whole rows exit together
  const int t = (int)(row / num_heads);
  const int h = (int)(row % num_heads);
  const int64_t slot = slots[t];
  if (slot < 0) return;
  const int64_t page = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t tile = page * num_heads + h;  // (page, head) tile index

  const int64_t src = (int64_t)t * token_stride + (int64_t)h * D;
  // per-KV-head mode: k_scales / v_scales hold one scale per head (per-tensor: null)
  float ks = k_scale, vs = v_scale;
  if constexpr (kFp8 && !kPerTokenHead) {
    if (k_scales != nullptr) {
      ks = k_scales[h];
      vs = v_scales[h];
    }
  }
  store_token_row<D, kFp8, kPerTokenHead>(k + src, v + src, c, tile, off, k_pages, v_pages,
                                          k_scales, v_scales, ks, vs);
}

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       int64_t n, float scale,
                                                       uint8_t* __restrict__ codes) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const uint4 w = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lo |= e4m3_quantize(bf16_bits_to_float(ww[j] & 0xFFFFu), scale) << (16 * j);
      lo |= e4m3_quantize(bf16_bits_to_float(ww[j] >> 16), scale) << (16 * j + 8);
      hi |= e4m3_quantize(bf16_bits_to_float(ww[2 + j] & 0xFFFFu), scale) << (16 * j);
      hi |= e4m3_quantize(bf16_bits_to_float(ww[2 + j] >> 16), scale) << (16 * j + 8);
    }
    reinterpret_cast<uint2*>(codes)[i] = make_uint2(lo, hi);
  }
  // tail
  const int64_t i = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) codes[i] = (uint8_t)e4m3_quantize(bf16_bits_to_float(x[i]), scale);
}

template <int D>
static void launch_cache_write(const kvq_cache_desc* c, const void* k, const void* v,
                               int64_t stride, const int64_t* slots, int32_t n,
                               float ks, float vs, hipStream_t st) {
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const int64_t rows = (int64_t)n * c->num_kv_heads;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* kp = static_cast<uint8_t*>(c->k_pages);
  auto* vp = static_cast<uint8_t*>(c->v_pages);
  if (c->dtype == KVQ_BF16)
    cache_write_kernel<D, false, false><<<grid, 256, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, nullptr, nullptr, 1.f, 1.f);
  else if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD)
    cache_write_kernel<D, true, true><<<grid, 256, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, c->k_scales, c->v_scales,
        1.f, 1.f);
  else if (c->mode == KVQ_SCALE_PER_KV_HEAD)
    cache_write_kernel<D, true, false><<<grid, 256, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, c->k_scales, c->v_scales,
        1.f, 1.f);
  else
    cache_write_kernel<D, true, false><<<grid, 256, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, nullptr, nullptr, ks, vs);
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_cache_write(const kvq_cache_desc* cache, const void* k,
                                      const void* v, int64_t token_stride,
                                      const int64_t* slot_mapping, int32_t num_tokens,
                                      float k_scale, float v_scale, void* stream) {
  clear_error();
  if (kvq_status s = check_cache(cache)) return s;
  if (num_tokens < 0) return fail(KVQ_ERR_INVALID_ARG, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return KVQ_OK;
  const int row = cache->num_kv_heads * cache->head_dim;
  if (token_stride == 0) token_stride = row;
  if (token_stride < row)
    return fail(KVQ_ERR_INVALID_ARG, "token_stride %lld < num_kv_heads*head_dim %d",
                (long long)token_stride, row);
  if (token_stride % 8)
    return fail(KVQ_ERR_INVALID_ARG, "token_stride %lld is not a multiple of 8",
                (long long)token_stride);
  if (!k || !v || !slot_mapping)
    return fail(KVQ_ERR_INVALID_ARG, "k, v or slot_mapping is NULL");
  if ((((uintptr_t)k) | ((uintptr_t)v)) & 15u)
    return fail(KVQ_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (cache->dtype == KVQ_FP8_E4M3 && cache->mode == KVQ_SCALE_PER_TENSOR &&
      !(k_scale > 0.0f && v_scale > 0.0f))
    return fail(KVQ_ERR_INVALID_ARG, "per-tensor scales must be > 0 (k=%g v=%g)",
                (double)k_scale, (double)v_scale);
  if (cache->num_pages == 0)
    return fail(KVQ_ERR_INVALID_ARG, "cache has no pages");
  auto st = static_cast<hipStream_t>(stream);
  switch (cache->head_dim) {
    case 64: launch_cache_write<64>(cache, k, v, token_stride, slot_mapping, num_tokens, k_scale, v_scale, st); break;
    case 128: launch_cache_write<128>(cache, k, v, token_stride, slot_mapping, num_tokens, k_scale, v_scale, st); break;
    case 256: launch_cache_write<256>(cache, k, v, token_stride, slot_mapping, num_tokens, k_scale, v_scale, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "cache_write launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}

extern "C" kvq_status kvq_quantize_fp8(const void* x, int64_t n, float scale,
                                       uint8_t* codes, void* stream) {
  clear_error();
  if (n < 0) return fail(KVQ_ERR_INVALID_ARG, "n %lld < 0", (long long)n);
  if (n == 0) return KVQ_OK;
  if (!x || !codes) return fail(KVQ_ERR_INVALID_ARG, "x or codes is NULL");
  if ((((uintptr_t)x) & 15u) || (((uintptr_t)codes) & 7u))
    return fail(KVQ_ERR_INVALID_ARG, "x must be 16-byte and codes 8-byte aligned");
  const int64_t nvec = (n + 7) / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  quantize_kernel<<<(unsigned)blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(x), n, scale, codes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return KVQ_OK;
}
