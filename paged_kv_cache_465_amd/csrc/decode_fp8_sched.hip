// Decode kernel instances for fp8 KV pools, balanced schedule:
// decode_mfma_stream_kernel, decode_valu_kernel
// (every page size and head dim).  One file per (format, plan) so the
// instances compile in parallel.
#include "decode_kernels.h"

namespace kvp {
template hipError_t launch_decode_fmt<kFP8, true>(const DecodeArgs&, int, int, bool, int,
                                                  dim3, dim3, size_t, hipStream_t);
}  // namespace kvp
