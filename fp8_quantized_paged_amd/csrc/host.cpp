// Host-only entry points of libkvq: version, status strings, last error, scale
// resolution and the per-layer dtype policy.  No HIP calls.
#include <math.h>
#include <string.h>

#include "kvq_host.h"

namespace kvq {

static thread_local char g_last_error[512];

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

kvq_status check_cache(const kvq_cache_desc* c) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->dtype != KVQ_FP8_E4M3 && c->dtype != KVQ_BF16)
    return fail(KVQ_ERR_UNSUPPORTED, "cache dtype %d is not fp8 or bf16", (int)c->dtype);
  if (c->page_size != KVQ_PAGE_SIZE)
    return fail(KVQ_ERR_UNSUPPORTED, "page_size %d (only %d is built)", c->page_size,
                KVQ_PAGE_SIZE);
  if (c->num_pages < 0 || c->num_kv_heads <= 0)
    return fail(KVQ_ERR_INVALID_ARG, "num_pages %d / num_kv_heads %d", c->num_pages,
                c->num_kv_heads);
  if (!supported_head_dim(c->head_dim))
    return fail(KVQ_ERR_UNSUPPORTED, "head_dim %d (64, 128, 256 are built)", c->head_dim);
  if (c->num_pages > 0 && (!c->k_pages || !c->v_pages))
    return fail(KVQ_ERR_INVALID_ARG, "k_pages / v_pages is NULL");
  if ((((uintptr_t)c->k_pages) | ((uintptr_t)c->v_pages)) & 255u)
    return fail(KVQ_ERR_INVALID_ARG, "page pools must be 256-byte aligned");
  if (c->dtype == KVQ_FP8_E4M3) {
    if (c->mode != KVQ_SCALE_PER_TENSOR && c->mode != KVQ_SCALE_PER_TOKEN_HEAD &&
        c->mode != KVQ_SCALE_PER_KV_HEAD)
      return fail(KVQ_ERR_INVALID_ARG, "scale mode %d", (int)c->mode);
    if (c->mode == KVQ_SCALE_PER_TOKEN_HEAD && c->num_pages > 0 &&
        (!c->k_scales || !c->v_scales))
      return fail(KVQ_ERR_INVALID_ARG, "per-token-head cache without scale pools");
    if (c->mode == KVQ_SCALE_PER_KV_HEAD && (!c->k_scales || !c->v_scales))
      return fail(KVQ_ERR_INVALID_ARG, "per-KV-head cache without scale arrays");
    if (c->mode == KVQ_SCALE_PER_KV_HEAD && ((((uintptr_t)c->k_scales) |
                                              ((uintptr_t)c->v_scales)) & 3u))
      return fail(KVQ_ERR_INVALID_ARG, "scale arrays must be 4-byte aligned");
  }
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

#ifndef KVQ_SOURCE_HASH
#define KVQ_SOURCE_HASH "unstamped"
#endif

extern "C" {

// Hash of the sources this library was built from (set by the build script); the
// Python binding compares it with the tree's to refuse a stale library.
extern __attribute__((visibility("default"))) const char kvq_build_source_hash[];
const char kvq_build_source_hash[] = KVQ_SOURCE_HASH;

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* kvq_last_error(void) { return g_last_error; }

kvq_status kvq_resolve_scales(kvq_scale_mode mode, float k_in, float v_in, float q_in,
                              float prob_in, kvq_scales* out, uint32_t* warn_flags) {
  clear_error();
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  uint32_t warn = 0;
  if (mode == KVQ_SCALE_PER_TOKEN_HEAD) {
    *out = kvq_scales{1.0f, 1.0f, 1.0f, 1.0f};
  } else if (mode == KVQ_SCALE_PER_TENSOR || mode == KVQ_SCALE_PER_KV_HEAD) {
    // per-KV-head: the same rules for one head's (k, v) pair
    float k, v;
    if (k_in > 0.0f && v_in > 0.0f) {
      k = k_in;
      v = v_in;
    } else if (k_in < 0.0f && v_in < 0.0f) {
      k = v = 1.0f;
    } else {
      // a single kv scale is loaded into k and duplicated as max(k, v)
      if (!(k_in > 0.0f))
        return fail(KVQ_ERR_INVALID_ARG, "single kv scale must be in k_scale (k=%g v=%g)",
                    (double)k_in, (double)v_in);
      k = v = fmaxf(k_in, v_in);
    }
    const float q = q_in > 0.0f ? q_in : 1.0f;
    const float p = prob_in > 0.0f ? prob_in : 1.0f;
    if (q == 1.0f || p == 1.0f) warn |= KVQ_WARN_UNCALIBRATED_Q_OR_PROB;
    *out = kvq_scales{q, k, v, p};
  } else {
    return fail(KVQ_ERR_INVALID_ARG, "scale mode %d", (int)mode);
  }
  if (warn_flags) *warn_flags = warn;
  return KVQ_OK;
}

kvq_dtype kvq_layer_kv_dtype(int32_t window, uint32_t skip_flags) {
  return ((skip_flags & KVQ_SKIP_SLIDING_WINDOW) && window > 0) ? KVQ_BF16 : KVQ_FP8_E4M3;
}

}  // extern "C"
