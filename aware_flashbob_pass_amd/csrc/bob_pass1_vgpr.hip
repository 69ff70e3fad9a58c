// The two-pass sweeps of pass 1 for 16-bit inputs at d = 64, in a translation
// unit of their own compiled with -mllvm -amdgpu-mfma-vgpr-form: their score products
// write VGPRs that the element-wise work reads directly, while the four accumulator
// tiles stay in AGPRs through inline-assembly products (mfma_acc). With the default
// form a kernel of more than 256 registers puts every product in AGPRs, and each step
// then copies its four score tiles out with v_accvgpr_read before the element-wise work.
#include <cmath>

#include "pass1_kernel.hpp"

namespace fb {

template <class TT, bool CAUSAL, bool FOLD = false, int ASML = kAsmNone>
static hipError_t launch_64(const Pass1Args& a, hipStream_t s) {
  const size_t lds = (ASML != kAsmNone ? pass1_asm_lds_bytes() : pass1_lds_bytes<TT, 64>()) + pass1_o_lds_bytes();
  hipError_t e = ensure_lds(&bob_pass1_kernel<TT, 64, CAUSAL, kTwoPass, FOLD, ASML>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass1_kernel<TT, 64, CAUSAL, kTwoPass, FOLD, ASML>), dim3(row_tiles(a.N), a.BH, a.nsplit),
                     dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

// tau folds exactly into bf16 operands when it is a positive power of two (bf16 has
// float32's exponent range; 2^-60 .. 2^60 keeps any value above 2^-66 a normal number).
static bool tau_folds(float tau) {
  int e = 0;
  return tau > 0.f && std::frexp(tau, &e) == 0.5f && e >= -59 && e <= 61;
}

// bf16 with a foldable tau runs the scheduled loop: over the whole sweep when no step
// needs a mask (non-causal, N a multiple of 32), else over the steps that need none,
// with compiled steps for the rest; other tau keep the compiled loop.
hipError_t launch_pass1_d64(const Pass1Args& a, DT dt, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16:
      if (!tau_folds(a.tau)) return causal ? launch_64<BF16, true>(a, s) : launch_64<BF16, false>(a, s);
      if (causal) return launch_64<BF16, true, true, kAsmPrefix>(a, s);
      return a.N % 32 == 0 ? launch_64<BF16, false, true, kAsmAll>(a, s) : launch_64<BF16, false, true, kAsmPrefix>(a, s);
    case DT::F16: return causal ? launch_64<F16, true>(a, s) : launch_64<F16, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fb
