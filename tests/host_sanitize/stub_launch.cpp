// Launchers that launch nothing: the C-ABI host code (api.hip) linked
// against these runs every check, size computation and parameter fill of
// every entry point on a machine without a GPU, under the host sanitizers.
#include "mz_internal.h"

namespace mz {
hipError_t launch_fwd_plan(const FwdParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd_rotate(const FwdParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_fwd_main(const FwdParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeParams&, hipStream_t) { return hipSuccess; }
}  // namespace mz
