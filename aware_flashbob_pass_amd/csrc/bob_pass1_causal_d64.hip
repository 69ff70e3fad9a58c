// The causal d = 64 two-pass sweep of pass 1 for 16-bit inputs, in a translation unit
// of its own: it is compiled with the matrix-core VGPR form (-mllvm -amdgpu-mfma-vgpr-form),
// so the score products write VGPRs that the element-wise work reads directly,
// while the four accumulator tiles stay in AGPRs through inline-assembly products
// (mfma_acc). With the default form a kernel of more than 256 registers puts every
// product in AGPRs, and each step then copies its four score tiles (64 registers)
// out with v_accvgpr_read before the element-wise work (the non-causal sweep still
// does: in this form it would need more than 256 VGPRs).
#include "pass1_kernel.hpp"

namespace fb {

template <class TT>
static hipError_t launch_t(const Pass1Args& a, hipStream_t s) {
  const size_t lds = pass1_lds_bytes<TT, 64>();
  hipError_t e = ensure_lds(&bob_pass1_kernel<TT, 64, true, kTwoPass>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass1_kernel<TT, 64, true, kTwoPass>), dim3(row_tiles(a.N), a.BH, a.nsplit), dim3(kBlock),
                     lds, s, a);
  return hipGetLastError();
}

hipError_t launch_pass1_causal_d64(const Pass1Args& a, DT dt, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_t<BF16>(a, s);
    case DT::F16: return launch_t<F16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fb
