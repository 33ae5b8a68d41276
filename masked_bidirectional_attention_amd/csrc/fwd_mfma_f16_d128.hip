// fwd_mfma_kernel instantiated for f16, head_dim 128 (every mask kind,
// one or two key streams, K rotated in the kernel or by the K pass).
#include "fwd_mfma.h"

namespace mz {

void launch_mfma_f16_d128(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s) {
  launch_mfma_td<F16, 128>(p, nwork, nstr, kr, s);
}

}  // namespace mz
