// Statistics kernel: one online-softmax forward sweep per query tile.
//
// BoB recomputes every score tile from the forward's row statistics (the
// score-recomputation model of the FlashBoB review page, Strengths: Theorem 4.5),
// so the call starts with a FlashAttention-style forward that produces
//   O = softmax(tau Q K^T) V,  L_i = log sum_j exp(tau q_i . k_j),
// and, fused into its epilogue, D_i = sum_t dO_it O_it formed from the float32
// O before rounding (D = rowsum(P * dP) = rowsum(dO * O) in exact arithmetic).
#include "common.hpp"
#include "kernels.hpp"

namespace fb {

template <class TT, int D, bool CAUSAL, bool WITH_D>
__global__ __launch_bounds__(kBlock) void attn_fwd_kernel(FwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  extern __shared__ __align__(16) unsigned char smem[];
  T* krow = reinterpret_cast<T*>(smem);
  T* vt = krow + G::ROW_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y;
  const size_t base = (size_t)bh * N * D;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* K = reinterpret_cast<const T*>(a.K) + base;
  const T* Vm = reinterpret_cast<const T*>(a.V) + base;
  const int q0 = blockIdx.x * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  V bq[G::DK];
  load_resident<TT, D>(Q, qi, N, g, bq);
  f32x16 acc[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) acc[mb] = zero16();
  float m = -1e30f, l = 0.f;
  const float cs = a.tau * kLog2e;

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (int)(blockIdx.x + 1) * (kBlockRows / kTile));
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kTile;
    __syncthreads();
    stage_tile<TT, D>(K, k0, N, krow, nullptr, tid, kBlock);
    stage_tile<TT, D>(Vm, k0, N, nullptr, vt, tid, kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + kTile - 1) continue;  // every key after every query of this wave

    f32x16 s = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) s = TT::mfma(lds_row_op<TT, D>(krow, n, t, g), bq[t], s);

    float mx = -1e30f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kappa(r, g);
      const bool ok = key < N && (!CAUSAL || key <= qi);
      s[r] = ok ? s[r] * cs : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, xor32(mx));
    const float mnew = fmaxf(m, mx);
    const float sc = fast_exp2(m - mnew);
    l *= sc;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) acc[mb] *= sc;
    V pp[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(s[r] - mnew);
      l += p;
      vset<TT>(pp[r / TT::KPL], r % TT::KPL, p);
    }
    m = mnew;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int t = 0; t < G::NK; ++t) acc[mb] = TT::mfma(lds_t_op<TT, D>(vt, mb * 32 + n, t, g), pp[t], acc[mb]);
  }

  const float lt = l + xor32(l);
  const float inv = 1.f / lt;
  if (qi < N) {
    T* O = reinterpret_cast<T*>(a.O) + base + (size_t)qi * D;
    const T* dO = WITH_D ? reinterpret_cast<const T*>(a.dO) + base + (size_t)qi * D : nullptr;
    float dot = 0.f;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = mb * 32 + kappa(r4 * 4, g);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[mb][r4 * 4 + e] * inv;
        store4<TT>(O + dim, o[0], o[1], o[2], o[3]);
        if constexpr (WITH_D) {
          float x[4];
          load4<TT>(dO + dim, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) dot += x[e] * o[e];
        }
      }
    // lanes n and n + 32 own the same query, so the exchanges below stay paired
    if (g == 0) a.L[(size_t)bh * N + qi] = m * kLn2 + __logf(lt);
    if constexpr (WITH_D) {
      dot += xor32(dot);
      if (g == 0) a.D[(size_t)bh * N + qi] = dot;
    }
  }
}

template <class TT, int D, bool CAUSAL, bool WITH_D>
static hipError_t launch_fwd_t(const FwdArgs& a, int BH, hipStream_t s) {
  using G = Geo<TT, D>;
  const size_t lds = (size_t)(G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem);
  hipError_t e = ensure_lds(&attn_fwd_kernel<TT, D, CAUSAL, WITH_D>, lds);
  if (e != hipSuccess) return e;
  dim3 grid(row_tiles(a.N), BH);
  hipLaunchKernelGGL((attn_fwd_kernel<TT, D, CAUSAL, WITH_D>), grid, dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <class TT, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int BH, hipStream_t s) {
  const bool wd = a.D != nullptr;
  if (causal) return wd ? launch_fwd_t<TT, D, true, true>(a, BH, s) : launch_fwd_t<TT, D, true, false>(a, BH, s);
  return wd ? launch_fwd_t<TT, D, false, true>(a, BH, s) : launch_fwd_t<TT, D, false, false>(a, BH, s);
}

template <class TT>
static hipError_t launch_fwd_tt(const FwdArgs& a, int d, bool causal, int BH, hipStream_t s) {
  return d == 64 ? launch_fwd_d<TT, 64>(a, causal, BH, s) : launch_fwd_d<TT, 128>(a, causal, BH, s);
}

hipError_t launch_attn_fwd(const FwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_fwd_tt<BF16>(a, d, causal, BH, s);
    case DT::F16: return launch_fwd_tt<F16>(a, d, causal, BH, s);
    default: return launch_fwd_tt<F32>(a, d, causal, BH, s);
  }
}

}  // namespace fb
