// The non-causal d = 128 BoB sweep of pass 2 (16-bit inputs), in a translation unit of its own
// compiled with -mllvm -amdgpu-mfma-vgpr-form: its score products write VGPRs that the
// element-wise work reads directly, while the two accumulator tiles stay in AGPRs
// through inline-assembly products (mfma_acc). With the default form this one-wave-
// per-SIMD kernel gets every product in AGPRs and copies the score tiles out each step.
// (The causal build of this form spills to scratch memory; it keeps the default form.)
#include "pass2_kernel.hpp"

namespace fb {

template <class TT>
static hipError_t launch_t(const Pass2Args& a, hipStream_t s) {
  const size_t lds = pass2_lds_bytes<TT, 128>();
  hipError_t e = ensure_lds(&bob_pass2_kernel<TT, 128, false>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass2_kernel<TT, 128, false>), dim3(row_tiles(a.N), a.BH, a.nsplit), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_pass2_d128(const Pass2Args& a, DT dt, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_t<BF16>(a, s);
    case DT::F16: return launch_t<F16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fb
