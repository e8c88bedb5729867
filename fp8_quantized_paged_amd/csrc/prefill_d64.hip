// FP8 chunked prefill kernels of head_dim 64 (prefill_kernel.h), every group size,
// scale mode and accumulation form.
#include "prefill_kernel.h"

namespace kvq {
namespace pf {
KVQ_DEFINE_PREFILL_LAUNCH(64)
}  // namespace pf
}  // namespace kvq
