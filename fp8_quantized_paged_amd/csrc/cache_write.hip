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
// Work split: a workgroup owns 16 consecutive tokens of the call and one KV head;
// D/8 lanes own a (token, head) row, 8 consecutive values (one 16-byte load) each.
// The row maxima of K and V are reduced across those lanes together (row_amax_bf16_kv);
// every lane then quantises its 8 values (per-token-head rows: the scale and a
// reciprocal once per row and two fused multiply-adds per value, whose codes equal
// those of the division -- see row_scale and e4m3_quantize4_row).  K rows go token-major (8 codes = one 8-byte store per lane).  V rows go
// dim-major: when the 16 tokens fill one page in order (slots 16 p .. 16 p + 15, the
// usual bulk fill; every wave checks the block's 16 slots itself with scalar loads) the
// codes are transposed through LDS and every channel row of the page tile is written
// with one 16-byte store (32 bytes for bf16).  When the 16 tokens instead end one page
// and start another, each run in order (a chunk that begins mid-page, any page table),
// the same staging feeds each channel row's two parts in aligned pieces of 1, 2, 4 and
// 8 elements (mid-page fill 486 -> 232 us, head_dim-256 8,192 tokens 27.1 -> 15.9 us);
// otherwise each lane stores its bytes where they belong (one byte per channel row).
// The transpose stages the block
// token-major (each lane one 8- or 16-byte LDS write) and each channel's thread gathers
// its 16 values with byte (bf16: 16-bit) reads, which neighbouring lanes share per
// dword; staging channel-major instead took one-byte LDS writes that the 32 (head_dim
// 256) or 16 lanes of a row aimed at one bank (head_dim-256 8,192-token write 20.2 ->
// 10.5 us, 131,072 tokens 265 -> 146 us; Llama-shaped whole-cache fill 188 -> 176 us).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

constexpr int kWriteTokens = 16;  // tokens per workgroup: one page when aligned

template <int D, bool kFp8, bool kPerTokenHead>
__global__ __launch_bounds__(2 * D) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t token_stride,
    const int64_t* __restrict__ slots, int32_t num_tokens, int32_t num_heads,
    uint8_t* __restrict__ k_pages, uint8_t* __restrict__ v_pages,
    float* __restrict__ k_scales, float* __restrict__ v_scales, float k_scale,
    float v_scale) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int EB = kFp8 ? 1 : 2;  // bytes per stored element
  // V codes (bf16: values) of the 16 tokens, token-major: [token][d]
  __shared__ __align__(16) uint8_t vt[D * kWriteTokens * EB];
  const int c = threadIdx.x % kLanesPerRow;
  const int i = threadIdx.x / kLanesPerRow;  // token of the workgroup
  // head fastest: neighbouring workgroups read the neighbouring pieces of the same
  // token rows and write neighbouring (page, head) tiles
  const int h = (int)(blockIdx.x % (unsigned)num_heads);
  const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)num_heads) * kWriteTokens;
  const int64_t t = t0 + i;
  const int64_t slot = t < num_tokens ? slots[t] : -1;
  // the rows do not depend on the slots: their loads go out with the slot loads
  const int64_t src = t * token_stride + (int64_t)h * D;
  uint4 kw = make_uint4(0u, 0u, 0u, 0u), vw = kw;
  if (t < num_tokens) {
    kw = *reinterpret_cast<const uint4*>(k + src + c * 8);
    vw = *reinterpret_cast<const uint4*>(v + src + c * 8);
  }
  // Whole-page fast path: 16 tokens present, slots 16 p + j in order.  Split path: the
  // block starts at offset koff != 0 of a page, its first 16 - koff tokens fill that
  // page's end in order and its last koff tokens start another page in order (a chunk
  // that begins mid-page; the two pages need not be neighbours).  The block's slots are
  // read at uniform addresses (scalar loads), so every wave reaches the same decision
  // on its own, without a workgroup vote.
  int64_t slot0 = -1, slotB = 0;
  int koff = 0;
  bool page_run = false, split_run = false;
  if (t0 + kWriteTokens <= num_tokens) {
    // all 16 loads in one batch, and the whole-page test first: a split test that
    // fetched the second run's first slot on its own put a second scalar round trip on
    // every block (head_dim-256 8,192-token write 10.8 -> 12.3 us)
    int64_t sj[kWriteTokens];
#pragma unroll
    for (int j = 0; j < kWriteTokens; ++j) sj[j] = slots[t0 + j];
    slot0 = sj[0];
    bool in_order = slot0 >= 0 && (slot0 & 15) == 0;
#pragma unroll
    for (int j = 1; j < kWriteTokens; ++j) in_order &= sj[j] == slot0 + j;
    page_run = in_order;
    if (!page_run && slot0 >= 0) {
      // the split check, off the whole-page path: consecutive slots, a page starting
      // only at token 16 - koff
      koff = (int)(slot0 & 15);
      bool run = koff != 0;
#pragma unroll
      for (int j = 1; j < kWriteTokens; ++j) {
        const bool start = (sj[j] & 15) == 0;
        run &= start ? (sj[j] >= 0) & (j == kWriteTokens - koff) : sj[j] == sj[j - 1] + 1;
        slotB = j == kWriteTokens - koff ? sj[j] : slotB;
      }
      split_run = run;
    }
  }
  // per-KV-head mode: k_scales / v_scales hold one scale per head (per-tensor: null)
  float ks = k_scale, vs = v_scale;
  float kr = 0.0f, vr = 0.0f;  // per-token-head: 1 / scale for the fast quotient
  bool kfast = false, vfast = false;
  if constexpr (kFp8 && !kPerTokenHead) {
    if (k_scales != nullptr) {
      ks = k_scales[h];
      vs = v_scales[h];
    }
  }
  if (!page_run && !split_run) {
    // any slot pattern: every (token, head) row on its own (rows of skipped tokens
    // simply do nothing; whole rows of lanes agree)
    if (slot >= 0) {
      store_token_row<D, kFp8, kPerTokenHead>(k + src, v + src, c, (slot >> 4) * num_heads + h,
                                              (int)(slot & 15), k_pages, v_pages, k_scales,
                                              v_scales, ks, vs);
    }
    return;
  }
  // the staged path: K rows and scales to their slots, V through LDS to the page tiles
  auto staged = [&](auto split_tag) {
    constexpr bool kSplit = decltype(split_tag)::value;
    const int64_t tile = (slot0 >> 4) * num_heads + h;  // the page's (page, head) tile
    // K rows and scales: each token's own slot (for a whole page: the page's tile, offset i)
    const int64_t rt = kSplit ? (slot >> 4) * num_heads + h : tile;
    const int ro = kSplit ? (int)(slot & 15) : i;
    if constexpr (!kFp8) {
      // bf16 cache: K row copied, V values staged in LDS
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_pages) + (rt * kPage + ro) * D +
                                c * 8) = kw;
      *reinterpret_cast<uint4*>(vt + (i * D + c * 8) * 2) = vw;
    } else {
      const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
      const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
      float kf[8], vf[8];
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        kf[2 * j] = bf16_bits_to_float(kk[j] & 0xFFFFu);
        kf[2 * j + 1] = bf16_bits_to_float(kk[j] >> 16);
        vf[2 * j] = bf16_bits_to_float(vv[j] & 0xFFFFu);
        vf[2 * j + 1] = bf16_bits_to_float(vv[j] >> 16);
      }
      if constexpr (kPerTokenHead) {
        const uint32_t kv = row_amax_bf16_kv<kLanesPerRow>(kw, vw);
        const uint32_t ka = kv << 16, va = kv & 0xFFFF0000u;  // float32 magnitude bits
        const RowScale krs = row_scale(ka), vrs = row_scale(va);
        ks = krs.s;
        vs = vrs.s;
        kr = krs.r;
        vr = vrs.r;
        kfast = krs.fast;
        vfast = vrs.fast;
        if (c == 0) {
          k_scales[rt * kPage + ro] = ks;
          v_scales[rt * kPage + ro] = vs;
        }
      }
      *reinterpret_cast<uint2*>(k_pages + (rt * kPage + ro) * D + c * 8) =
          make_uint2(e4m3_quantize4_row(kf, ks, kr, kfast), e4m3_quantize4_row(kf + 4, ks, kr, kfast));
      const uint32_t vlo = e4m3_quantize4_row(vf, vs, vr, vfast);
      const uint32_t vhi = e4m3_quantize4_row(vf + 4, vs, vr, vfast);
      *reinterpret_cast<uint2*>(vt + i * D + c * 8) = make_uint2(vlo, vhi);
    }
    __syncthreads();
    if constexpr (kSplit) {
      // elements koff .. 15 of page A's channel row d come from tokens 0 .. 15 - koff,
      // elements 0 .. koff - 1 of page B's from tokens 16 - koff .. 15; each part goes out
      // in aligned pieces of 1, 2, 4 and 8 elements (the bits of koff), leaving the rows'
      // other elements -- other tokens' -- untouched
      if (threadIdx.x < D) {
        const int d = threadIdx.x;
        uint8_t* rowA = v_pages + (((slot0 >> 4) * num_heads + h) * D + d) * kPage * EB;
        uint8_t* rowB = v_pages + (((slotB >> 4) * num_heads + h) * D + d) * kPage * EB;
        auto put = [&](uint8_t* row, int e0, auto w_tag, int tok0) {
          constexpr int W = decltype(w_tag)::value;  // elements
          constexpr int NB = W * EB;                 // bytes
          uint32_t x[NB >= 4 ? NB / 4 : 1] = {};
  #pragma unroll
          for (int u = 0; u < W; ++u) {
            const uint32_t val = kFp8 ? (uint32_t)vt[(tok0 + u) * D + d]
                                      : (uint32_t)reinterpret_cast<const uint16_t*>(vt)[(tok0 + u) * D + d];
            x[(u * EB) / 4] |= val << (8 * ((u * EB) % 4));
          }
          uint8_t* dst = row + e0 * EB;
          if constexpr (NB == 1) *dst = (uint8_t)x[0];
          else if constexpr (NB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)x[0];
          else if constexpr (NB == 4) *reinterpret_cast<uint32_t*>(dst) = x[0];
          else if constexpr (NB == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(x[0], x[1]);
          else *reinterpret_cast<uint4*>(dst) = make_uint4(x[0], x[1], x[2], x[3]);
        };
        using W1 = std::integral_constant<int, 1>;
        using W2 = std::integral_constant<int, 2>;
        using W4 = std::integral_constant<int, 4>;
        using W8 = std::integral_constant<int, 8>;
        int e = koff;  // page A: up to the page's end, smallest pieces first
        if (e & 1) { put(rowA, e, W1{}, e - koff); e += 1; }
        if (e & 2) { put(rowA, e, W2{}, e - koff); e += 2; }
        if (e & 4) { put(rowA, e, W4{}, e - koff); e += 4; }
        if (e & 8) { put(rowA, e, W8{}, e - koff); }
        int f = 0;     // page B: from the page's start, largest pieces first
        if (koff & 8) { put(rowB, f, W8{}, kWriteTokens - koff + f); f += 8; }
        if (koff & 4) { put(rowB, f, W4{}, kWriteTokens - koff + f); f += 4; }
        if (koff & 2) { put(rowB, f, W2{}, kWriteTokens - koff + f); f += 2; }
        if (koff & 1) { put(rowB, f, W1{}, kWriteTokens - koff + f); }
      }
      return;
    }
    // one channel row of the V tile per thread: 16 codes (16 bytes) or 16 bf16 (32 bytes),
    // gathered from the 16 staged tokens
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      uint32_t wd[4 * EB];
      if constexpr (kFp8) {
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t x = 0;
  #pragma unroll
          for (int e = 0; e < 4; ++e) x |= (uint32_t)vt[(4 * q + e) * D + d] << (8 * e);
          wd[q] = x;
        }
      } else {
        const uint16_t* vt16 = reinterpret_cast<const uint16_t*>(vt);
  #pragma unroll
        for (int q = 0; q < 8; ++q)
          wd[q] = (uint32_t)vt16[(2 * q) * D + d] | ((uint32_t)vt16[(2 * q + 1) * D + d] << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(v_pages + (tile * D + d) * kPage * EB);
  #pragma unroll
      for (int w = 0; w < EB; ++w) dst[w] = make_uint4(wd[4 * w], wd[4 * w + 1], wd[4 * w + 2], wd[4 * w + 3]);
    }
  };
  if (split_run) staged(std::true_type{});
  else staged(std::false_type{});
}

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x,
                                                       int64_t n, float scale,
                                                       uint8_t* __restrict__ codes) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const uint4 w = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float f[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[2 * j] = bf16_bits_to_float(ww[j] & 0xFFFFu);
      f[2 * j + 1] = bf16_bits_to_float(ww[j] >> 16);
    }
    reinterpret_cast<uint2*>(codes)[i] = make_uint2(e4m3_quantize4(f, scale),
                                                    e4m3_quantize4(f + 4, scale));
  }
  // tail
  const int64_t i = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float f = bf16_bits_to_float(x[i]);
    codes[i] = (uint8_t)(e4m3_quantize2(f, f, scale) & 0xFFu);
  }
}

template <int D>
static void launch_cache_write(const kvq_cache_desc* c, const void* k, const void* v,
                               int64_t stride, const int64_t* slots, int32_t n,
                               float ks, float vs, hipStream_t st) {
  const dim3 grid((unsigned)(((int64_t)n + kWriteTokens - 1) / kWriteTokens * c->num_kv_heads));
  constexpr int kThreads = 2 * D;  // 16 tokens x D / 8 lanes
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* kp = static_cast<uint8_t*>(c->k_pages);
  auto* vp = static_cast<uint8_t*>(c->v_pages);
  if (c->dtype == KVQ_BF16)
    cache_write_kernel<D, false, false><<<grid, kThreads, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, nullptr, nullptr, 1.f, 1.f);
  else if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD)
    cache_write_kernel<D, true, true><<<grid, kThreads, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, c->k_scales, c->v_scales,
        1.f, 1.f);
  else if (c->mode == KVQ_SCALE_PER_KV_HEAD)
    cache_write_kernel<D, true, false><<<grid, kThreads, 0, st>>>(
        kk, vv, stride, slots, n, c->num_kv_heads, kp, vp, c->k_scales, c->v_scales,
        1.f, 1.f);
  else
    cache_write_kernel<D, true, false><<<grid, kThreads, 0, st>>>(
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
  if (((int64_t)num_tokens + kWriteTokens - 1) / kWriteTokens * cache->num_kv_heads > 0x7FFFFFFF)
    return fail(KVQ_ERR_INVALID_ARG, "num_tokens %d x num_kv_heads %d: grid too large",
                num_tokens, cache->num_kv_heads);
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
