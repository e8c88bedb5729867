// kvq_decode_attention_noalloc: kvq_decode_attention for callers that cannot allocate
// (code under HIP graph capture, tight serving loops): the split-K partials and
// completion counters live in a file-scope device array of fixed size instead of a
// caller-provided workspace.  Same kernels, same layout (counter prefix, then
// partials), same results.
#include <atomic>
#include <mutex>

#include "kvq_device.h"
#include "kvq_host.h"

namespace kvq {

// The scratch: KVQ_DECODE_COUNTER_BYTES of completion counters, then split partials.
// Every device the library runs on holds its own copy until the process ends.  On
// the host the array's name is only a stand-in for the symbol, never a device
// address: host code uses the address hipGetSymbolAddress returns per device.
static __device__ __align__(256) uint8_t scratch[KVQ_DECODE_SCRATCH_BYTES];

__global__ void zero_counters_kernel(uint32_t* p, int n) {
  for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n;
       i += (int)(gridDim.x * blockDim.x))
    p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

// Device address of `scratch` on the current device, looked up once per device (with
// that device current).  The first lookup also clears the counter prefix with a fill
// kernel on `st` (kernels leave the counters zero after every call; this covers the
// first one).  A graph capture that records this launch replays a harmless re-clear.
static kvq_status scratch_of_current_device(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVQ_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      const int words = KVQ_DECODE_COUNTER_BYTES / (int)sizeof(uint32_t);
      zero_counters_kernel<<<64, 256, 0, st>>>(static_cast<uint32_t*>(p), words);
      e = hipGetLastError();
      if (e != hipSuccess)
        return fail(KVQ_ERR_HIP, "scratch counter clear: %s", hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVQ_OK;
}

}  // namespace kvq

using namespace kvq;

extern "C" kvq_status kvq_decode_attention_noalloc(
    const kvq_cache_desc* cache, const void* q, int32_t num_seqs, int32_t num_q_heads,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
    int32_t max_seq_len, const kvq_scales* scales, int32_t window, float softmax_scale,
    int32_t pages_per_split, void* out, kvq_dtype out_dtype, void* stream) {
  clear_error();
  size_t need = 0;
  if (kvq_status s = kvq_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_seq_len,
                                                window, pages_per_split, &need))
    return s;
  if (need > (size_t)KVQ_DECODE_SCRATCH_BYTES)
    return fail(KVQ_ERR_WORKSPACE,
                "these arguments need %zu bytes of split partials and counters; the "
                "allocation-free entry point holds %d (split the batch, or raise "
                "pages_per_split)",
                need, KVQ_DECODE_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    if (kvq_status s = scratch_of_current_device(static_cast<hipStream_t>(stream), &ws))
      return s;
  }
  return decode_impl(cache, q, num_seqs, num_q_heads, block_table, block_table_stride,
                     seq_lens, max_seq_len, scales, window, softmax_scale, pages_per_split,
                     out, out_dtype, ws, ws ? (size_t)KVQ_DECODE_SCRATCH_BYTES : 0, stream,
                     nullptr, nullptr);
}
