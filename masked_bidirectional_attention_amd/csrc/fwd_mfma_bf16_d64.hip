// fwd_mfma_kernel instantiated for bf16, head_dim 64 (every mask kind,
// one or two key streams, K rotated in the kernel or by the K pass).
#include "fwd_mfma.h"

namespace mz {

void launch_mfma_bf16_d64(const FwdParams& p, unsigned nwork, int nstr, bool kr, hipStream_t s) {
  launch_mfma_td<BF16, 64>(p, nwork, nstr, kr, s);
}

}  // namespace mz
