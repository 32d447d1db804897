// Decode kernel instances for int8 KV pools, uniform split plan:
// decode_mfma_kernel, decode_valu_kernel
// (every page size and head dim).  One file per (format, plan) so the
// instances compile in parallel.
#include "decode_kernels.h"

namespace kvp {
template hipError_t launch_decode_fmt<kI8, false>(const DecodeArgs&, int, int, bool, int,
                                                  dim3, dim3, size_t, hipStream_t);
}  // namespace kvp
