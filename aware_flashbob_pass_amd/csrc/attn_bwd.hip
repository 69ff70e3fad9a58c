// First backward g(Q, K, V, dO) = (dQ, dK, dV): the map that BoB differentiates
// (FlashBoB review page, Report preview / Scope & Claims).
//   D_i = sum_t dO_it O_it,  dS = P (dO V^T - D),
//   dQ = tau dS K  (query-tile parallel kernel),
//   dK = tau dS^T Q, dV = P^T dO  (key-tile parallel kernel).
// Two launches instead of one with dQ atomics keep the result deterministic.
#include "common.hpp"
#include "kernels.hpp"

namespace fb {

template <class TT, int D>
__global__ __launch_bounds__(kBlock) void bwd_rowdot_kernel(BwdArgs a, int rows) {
  using T = typename TT::elem;
  const int r = blockIdx.x * kBlock + threadIdx.x;
  if (r >= rows) return;
  const T* O = reinterpret_cast<const T*>(a.O) + (size_t)r * D;
  const T* dO = reinterpret_cast<const T*>(a.dO) + (size_t)r * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float o[4], x[4];
    load4<TT>(O + c, o);
    load4<TT>(dO + c, x);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += o[e] * x[e];
  }
  a.D[r] = acc;
}

template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBlock) void bwd_dq_kernel(BwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB;
  extern __shared__ __align__(16) unsigned char smem[];
  T* k_r = reinterpret_cast<T*>(smem);
  T* v_r = k_r + G::ROW_ELEMS;
  T* k_t = v_r + G::ROW_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y;
  const size_t base = (size_t)bh * N * D;
  const T* K = reinterpret_cast<const T*>(a.K) + base;
  const T* Vm = reinterpret_cast<const T*>(a.V) + base;
  const int q0 = blockIdx.x * kBlockRows + wave * kTile;
  const int qi = q0 + n;
  V bq[G::DK], bdo[G::DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.Q) + base, qi, N, g, bq);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.dO) + base, qi, N, g, bdo);
  const size_t rowv = (size_t)bh * N + (qi < N ? qi : 0);
  const float lq = a.L[rowv] * kLog2e;
  const float dq = a.D[rowv];
  const float cs = a.tau * kLog2e;

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (int)(blockIdx.x + 1) * (kBlockRows / kTile));
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kTile;
    __syncthreads();
    stage_tile<TT, D>(K, k0, N, k_r, k_t, tid, kBlock);
    stage_tile<TT, D>(Vm, k0, N, v_r, nullptr, tid, kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + kTile - 1) continue;
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) {
      s = TT::mfma(lds_row_op<TT, D>(k_r, n, t, g), bq[t], s);
      dp = TT::mfma(lds_row_op<TT, D>(v_r, n, t, g), bdo[t], dp);
    }
    V wds[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kappa(r, g);
      const bool ok = key < N && (!CAUSAL || key <= qi);
      const float p = ok ? fast_exp2(s[r] * cs - lq) : 0.f;
      vset<TT>(wds[r / TT::KPL], r % TT::KPL, p * (dp[r] - dq));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < G::NK; ++t) acc[mb] = TT::mfma(lds_t_op<TT, D>(k_t, mb * 32 + n, t, g), wds[t], acc[mb]);
  }
  if (qi >= N) return;
  T* dQ = reinterpret_cast<T*>(a.dQ) + base + (size_t)qi * D;
  const float tau = a.tau;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int r = r4 * 4;
      store4<TT>(dQ + mb * 32 + kappa(r, g), tau * acc[mb][r], tau * acc[mb][r + 1], tau * acc[mb][r + 2],
                 tau * acc[mb][r + 3]);
    }
}

template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBlock) void bwd_dkdv_kernel(BwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB;
  extern __shared__ __align__(16) unsigned char smem[];
  T* q_r = reinterpret_cast<T*>(smem);
  T* do_r = q_r + G::ROW_ELEMS;
  T* q_t = do_r + G::ROW_ELEMS;
  T* do_t = q_t + G::T_ELEMS;
  float* sc = reinterpret_cast<float*>(do_t + G::T_ELEMS);  // [2][32]: L*log2e, D

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y;
  const size_t base = (size_t)bh * N * D;
  const size_t vbase = (size_t)bh * N;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* dO = reinterpret_cast<const T*>(a.dO) + base;
  const int k0w = blockIdx.x * kBlockRows + wave * kTile;
  const int kj = k0w + n;
  V bk[G::DK], bv[G::DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.K) + base, kj, N, g, bk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.V) + base, kj, N, g, bv);
  const float cs = a.tau * kLog2e;

  f32x16 accK[MB], accV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accK[mb] = zero16();
    accV[mb] = zero16();
  }
  const int nqt = (N + kTile - 1) / kTile;
  const int qt_first = CAUSAL ? (int)blockIdx.x * (kBlockRows / kTile) : 0;
  for (int it = qt_first; it < nqt; ++it) {
    const int i0 = it * kTile;
    __syncthreads();
    stage_tile<TT, D>(Q, i0, N, q_r, q_t, tid, kBlock);
    stage_tile<TT, D>(dO, i0, N, do_r, do_t, tid, kBlock);
    if (tid < 2 * kTile) {
      const int which = tid / kTile, qrow = i0 + tid % kTile;
      float v = 0.f;
      if (qrow < N) v = which == 0 ? a.L[vbase + qrow] * kLog2e : a.D[vbase + qrow];
      sc[tid] = v;
    }
    __syncthreads();
    if (CAUSAL && i0 + kTile - 1 < k0w) continue;
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) {
      s = TT::mfma(lds_row_op<TT, D>(q_r, n, t, g), bk[t], s);
      dp = TT::mfma(lds_row_op<TT, D>(do_r, n, t, g), bv[t], dp);
    }
    V wds[G::NK], wp[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = kappa(r, g);
      const int qrow = i0 + qr;
      const bool ok = qrow < N && kj < N && (!CAUSAL || kj <= qrow);
      const float p = ok ? fast_exp2(s[r] * cs - sc[qr]) : 0.f;
      vset<TT>(wds[r / TT::KPL], r % TT::KPL, p * (dp[r] - sc[kTile + qr]));
      vset<TT>(wp[r / TT::KPL], r % TT::KPL, p);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < G::NK; ++t) {
        accK[mb] = TT::mfma(lds_t_op<TT, D>(q_t, mb * 32 + n, t, g), wds[t], accK[mb]);
        accV[mb] = TT::mfma(lds_t_op<TT, D>(do_t, mb * 32 + n, t, g), wp[t], accV[mb]);
      }
  }
  if (kj >= N) return;
  T* dK = reinterpret_cast<T*>(a.dK) + base + (size_t)kj * D;
  T* dV = reinterpret_cast<T*>(a.dV) + base + (size_t)kj * D;
  const float tau = a.tau;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int r = r4 * 4;
      const int dim = mb * 32 + kappa(r, g);
      store4<TT>(dK + dim, tau * accK[mb][r], tau * accK[mb][r + 1], tau * accK[mb][r + 2], tau * accK[mb][r + 3]);
      store4<TT>(dV + dim, accV[mb][r], accV[mb][r + 1], accV[mb][r + 2], accV[mb][r + 3]);
    }
}

template <class TT, int D>
static hipError_t launch_rowdot_t(const BwdArgs& a, int BH, hipStream_t s) {
  const int rows = BH * a.N;
  hipLaunchKernelGGL((bwd_rowdot_kernel<TT, D>), dim3((rows + kBlock - 1) / kBlock), dim3(kBlock), 0, s, a, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_rowdot(const BwdArgs& a, DT dt, int d, int BH, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return d == 64 ? launch_rowdot_t<BF16, 64>(a, BH, s) : launch_rowdot_t<BF16, 128>(a, BH, s);
    case DT::F16: return d == 64 ? launch_rowdot_t<F16, 64>(a, BH, s) : launch_rowdot_t<F16, 128>(a, BH, s);
    default: return d == 64 ? launch_rowdot_t<F32, 64>(a, BH, s) : launch_rowdot_t<F32, 128>(a, BH, s);
  }
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_dq_t(const BwdArgs& a, int BH, hipStream_t s) {
  using G = Geo<TT, D>;
  const size_t lds = (size_t)(2 * G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem);
  hipError_t e = ensure_lds(&bwd_dq_kernel<TT, D, CAUSAL>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<TT, D, CAUSAL>), dim3(row_tiles(a.N), BH), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_dkdv_t(const BwdArgs& a, int BH, hipStream_t s) {
  using G = Geo<TT, D>;
  const size_t lds = (size_t)2 * (G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem) + 2 * kTile * sizeof(float);
  hipError_t e = ensure_lds(&bwd_dkdv_kernel<TT, D, CAUSAL>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<TT, D, CAUSAL>), dim3(row_tiles(a.N), BH), dim3(kBlock), lds, s, a);
  return hipGetLastError();
}

template <class TT>
static hipError_t dq_tt(const BwdArgs& a, int d, bool causal, int BH, hipStream_t s) {
  if (d == 64) return causal ? launch_dq_t<TT, 64, true>(a, BH, s) : launch_dq_t<TT, 64, false>(a, BH, s);
  return causal ? launch_dq_t<TT, 128, true>(a, BH, s) : launch_dq_t<TT, 128, false>(a, BH, s);
}

template <class TT>
static hipError_t dkdv_tt(const BwdArgs& a, int d, bool causal, int BH, hipStream_t s) {
  if (d == 64) return causal ? launch_dkdv_t<TT, 64, true>(a, BH, s) : launch_dkdv_t<TT, 64, false>(a, BH, s);
  return causal ? launch_dkdv_t<TT, 128, true>(a, BH, s) : launch_dkdv_t<TT, 128, false>(a, BH, s);
}

hipError_t launch_bwd_dq(const BwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return dq_tt<BF16>(a, d, causal, BH, s);
    case DT::F16: return dq_tt<F16>(a, d, causal, BH, s);
    default: return dq_tt<F32>(a, d, causal, BH, s);
  }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return dkdv_tt<BF16>(a, d, causal, BH, s);
    case DT::F16: return dkdv_tt<F16>(a, d, causal, BH, s);
    default: return dkdv_tt<F32>(a, d, causal, BH, s);
  }
}

}  // namespace fb
