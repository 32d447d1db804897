// Multi-query attention kernel instances for int4 KV pools (every page size,
// head dim and tile shape).  One file per format so the instances compile in
// parallel.
#include "prefill_kernels.h"

namespace kvp {
template hipError_t launch_prefill_fmt<kI4>(const PrefillArgs&, int, int, int, bool, dim3,
                                          hipStream_t);
}  // namespace kvp
