// BoB pass 2: key-tile parallel. Produces gK and gV.
//
// After pass 1 every query row's scalars L, D, alpha, E are known (review page,
// Summary: only the two length-N vectors alpha and E cross the pass boundary,
// besides the statistics). For key j, summing over queries i:
//   dS   = P (dP - D),
//   Sbar = P (G (dP - D) - alpha dP + H - E),      (cotangent of the scores)
//   dPbar = P (G - alpha),                          (cotangent of dP)
//   gK_j = tau sum_i (dS_ij UQ_i + Sbar_ij Q_i),    gV_j = sum_i dPbar_ij dO_i,
// with G = tau (UQ K^T + Q UK^T), H = dO UV^T, dP = dO V^T, P = exp(tau Q K^T - L).
//
// Each workgroup owns 128 keys (4 waves x 32), keeps K, V, UK, UV rows of its
// keys in registers as matrix-core B operands, and streams 32-query tiles of
// Q, dO, UQ (row-major and transposed copies) and the four row scalars
// through LDS. With splits of the query range, each wave writes raw
// accumulators and a reduce kernel sums them in split order.
//
// This file holds the float32 kernel, the split reduce and the launches; the
// staged 16-bit kernel template is in pass2_kernel.hpp (its non-causal d = 128 BoB
// instances are built in bob_pass2_vgpr.hip).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "pass2_kernel.hpp"

namespace fb {

// Single-buffered variant (transposed LDS copies); used for float32 inputs.
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBlock) void bob_pass2_simple_kernel(Pass2Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB;
  extern __shared__ __align__(16) unsigned char smem[];
  T* q_r = reinterpret_cast<T*>(smem);
  T* do_r = q_r + G::ROW_ELEMS;
  T* uq_r = do_r + G::ROW_ELEMS;
  T* q_t = uq_r + G::ROW_ELEMS;
  T* do_t = q_t + G::T_ELEMS;
  T* uq_t = do_t + G::T_ELEMS;
  float* sc = reinterpret_cast<float*>(uq_t + G::T_ELEMS);  // [4][32]: L*log2e, D, alpha, E

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const size_t vbase = (size_t)bh * N;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* dO = reinterpret_cast<const T*>(a.dO) + base;
  const T* UQ = reinterpret_cast<const T*>(a.UQ) + base;
  const int k0w = blockIdx.x * kBlockRows + wave * kTile;
  const int kj = k0w + n;

  V bk[G::DK], bv[G::DK], buk[G::DK], buv[G::DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.K) + base, kj, N, g, bk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.V) + base, kj, N, g, bv);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.UK) + base, kj, N, g, buk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.UV) + base, kj, N, g, buv);
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x16 accK[MB], accV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accK[mb] = zero16();
    accV[mb] = zero16();
  }

  const int nqt = (N + kTile - 1) / kTile;
  const int qt_first = CAUSAL ? (int)blockIdx.x * (kBlockRows / kTile) : 0;
  const int span = nqt - qt_first;
  const int it_begin = qt_first + (int)((long long)split * span / a.nsplit);
  const int it_end = qt_first + (int)((long long)(split + 1) * span / a.nsplit);

  for (int it = it_begin; it < it_end; ++it) {
    const int i0 = it * kTile;
    __syncthreads();
    stage_tile<TT, D>(Q, i0, N, q_r, q_t, tid, kBlock);
    stage_tile<TT, D>(dO, i0, N, do_r, do_t, tid, kBlock);
    stage_tile<TT, D>(UQ, i0, N, uq_r, uq_t, tid, kBlock);
    if (tid < 4 * kTile) {
      const int which = tid / kTile, rr = tid % kTile;
      const int qrow = i0 + rr;
      float v = 0.f;
      if (qrow < N) {
        if (which == 0) v = a.L[vbase + qrow] * kLog2e;
        else if (which == 1) v = a.D[vbase + qrow];
        else if (which == 2) v = a.alpha[vbase + qrow];
        else v = a.E[vbase + qrow];
      }
      sc[tid] = v;
    }
    __syncthreads();
    if (CAUSAL && i0 + kTile - 1 < k0w) continue;  // every query before every key of this wave

    // score tiles (queries x keys): S, G, dP, H
    f32x16 s = zero16(), gg = zero16(), dp = zero16(), h = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) {
      const V aq = lds_row_op<TT, D>(q_r, n, t, g);
      const V auq = lds_row_op<TT, D>(uq_r, n, t, g);
      const V ado = lds_row_op<TT, D>(do_r, n, t, g);
      s = TT::mfma(aq, bk[t], s);
      gg = TT::mfma(auq, bk[t], gg);
      gg = TT::mfma(aq, buk[t], gg);
      dp = TT::mfma(ado, bv[t], dp);
      h = TT::mfma(ado, buv[t], h);
    }

    V wds[G::NK], wsb[G::NK], wdp[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = kappa(r, g);
      const int qrow = i0 + qr;
      const bool ok = qrow < N && kj < N && (!CAUSAL || kj <= qrow);
      const float lq = sc[qr], dq = sc[kTile + qr], al = sc[2 * kTile + qr], eq = sc[3 * kTile + qr];
      const float p = ok ? fast_exp2(s[r] * cs - lq) : 0.f;
      const float gv = gg[r] * tau;
      const float dpv = dp[r];
      const float t1 = dpv - dq;
      const int kk = r / TT::KPL, ss = r % TT::KPL;
      vset<TT>(wds[kk], ss, p * t1);
      vset<TT>(wsb[kk], ss, p * (gv * t1 - al * dpv + h[r] - eq));
      vset<TT>(wdp[kk], ss, p * (gv - al));
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int dim = mb * 32 + n;
#pragma unroll
      for (int t = 0; t < G::NK; ++t) {
        const V tuq = lds_t_op<TT, D>(uq_t, dim, t, g);
        const V tq = lds_t_op<TT, D>(q_t, dim, t, g);
        const V tdo = lds_t_op<TT, D>(do_t, dim, t, g);
        accK[mb] = TT::mfma(tuq, wds[t], accK[mb]);
        accK[mb] = TT::mfma(tq, wsb[t], accK[mb]);
        accV[mb] = TT::mfma(tdo, wdp[t], accV[mb]);
      }
    }
  }

  if (a.nsplit == 1) {
    pass2_epilogue<TT, D>(accK, accV, kj, g, bh, a);
    return;
  }
  pass2_write_record<TT, D>(accK, accV, split, bh, blockIdx.x, wave, lane, a);
}

// Sum the split records of one wave in split order and write one 32-wide head-dim
// block of gK, gV. A workgroup takes one wave's record and one block (grid x = key
// tile x wave, z = block); thread t sums slots 4 (t / 64) .. 4 (t / 64) + 3 of record
// lane t % 64, so consecutive threads read consecutive 16 bytes of the quad-major
// record tiles and four times as many waves are in flight as with one thread per
// record lane.
template <class TT, int D>
__global__ __launch_bounds__(kBlock) void bob_pass2_reduce_kernel(Pass2Args a) {
  constexpr int MB = Geo<TT, D>::MB;
  const int L = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  const int g = L >> 5, n = L & 31;
  const int kt = blockIdx.x >> 2, wave = blockIdx.x & 3;
  const int bh = blockIdx.y, mb = blockIdx.z;
  const int kj = kt * kBlockRows + wave * kTile + n;
  const int kt_count = row_tiles(a.N);
  f32x4 dK = {0.f, 0.f, 0.f, 0.f}, dV = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = a.part + ((((size_t)sp * a.BH + bh) * kt_count + kt) * 4 + wave) * pass2_record_floats(D);
    const f32x4 k4 = tile_quad(R + (0 * MB + mb) * 1024, L, r4);
    const f32x4 v4 = tile_quad(R + (1 * MB + mb) * 1024, L, r4);
    dK += k4;
    dV += v4;
  }
  pass2_epilogue_quad<TT, D>(dK, dV, kj, g, bh, mb, r4, a);
}

// kReduceAtomic: clear the float32 sums (a fill kernel, so that the call can be
// captured in a HIP graph) ...
__global__ __launch_bounds__(kBlock) void zero_f32_kernel(float* p, size_t n) {
  for (size_t i = ((size_t)blockIdx.x * kBlock + threadIdx.x) * 4; i < n; i += (size_t)gridDim.x * kBlock * 4) {
    if (i + 4 <= n) *reinterpret_cast<f32x4*>(p + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    else
      for (size_t j = i; j < n; ++j) p[j] = 0.f;
  }
}

// ... and convert them afterwards: gK = tau * (sum of dS^T UQ + Sbar^T Q), gV = sum.
template <class TT, int D>
__global__ __launch_bounds__(kBlock) void pass2_convert_kernel(Pass2Args a) {
  using T = typename TT::elem;
  const size_t plane = (size_t)a.BH * a.N * D;
  for (size_t i = ((size_t)blockIdx.x * kBlock + threadIdx.x) * 4; i < plane; i += (size_t)gridDim.x * kBlock * 4) {
    const f32x4 k = *reinterpret_cast<const f32x4*>(a.acc32 + i);
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.acc32 + plane + i);
    store4<TT>(reinterpret_cast<T*>(a.gK) + i, a.tau * k[0], a.tau * k[1], a.tau * k[2], a.tau * k[3]);
    store4<TT>(reinterpret_cast<T*>(a.gV) + i, v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
  const size_t blocks = std::min<size_t>(4096, (n / 4 + kBlock - 1) / kBlock + 1);
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_pass2_convert(const Pass2Args& a, DT dt, int d, hipStream_t s) {
  const size_t plane = (size_t)a.BH * a.N * d;
  const dim3 grid((unsigned)std::min<size_t>(4096, (plane / 4 + kBlock - 1) / kBlock));
  switch (dt) {
    case DT::BF16:
      if (d == 64) hipLaunchKernelGGL((pass2_convert_kernel<BF16, 64>), grid, dim3(kBlock), 0, s, a);
      else hipLaunchKernelGGL((pass2_convert_kernel<BF16, 128>), grid, dim3(kBlock), 0, s, a);
      break;
    case DT::F16:
      if (d == 64) hipLaunchKernelGGL((pass2_convert_kernel<F16, 64>), grid, dim3(kBlock), 0, s, a);
      else hipLaunchKernelGGL((pass2_convert_kernel<F16, 128>), grid, dim3(kBlock), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_p2_t(const Pass2Args& a, hipStream_t s) {
  const size_t lds = pass2_lds_bytes<TT, D>();
  dim3 grid(row_tiles(a.N), a.BH, a.nsplit);
  if constexpr (TT::KPL == 1) {
    hipError_t e = ensure_lds(&bob_pass2_simple_kernel<TT, D, CAUSAL>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass2_simple_kernel<TT, D, CAUSAL>), grid, dim3(kBlock), lds, s, a);
  } else if constexpr (D == 128 && !CAUSAL) {
    return launch_pass2_d128(a, std::is_same_v<TT, BF16> ? DT::BF16 : DT::F16, s);
  } else {
    hipError_t e = ensure_lds(&bob_pass2_kernel<TT, D, CAUSAL>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass2_kernel<TT, D, CAUSAL>), grid, dim3(kBlock), lds, s, a);
  }
  return hipGetLastError();
}

template <class TT>
static hipError_t launch_p2_tt(const Pass2Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_p2_t<TT, 64, true>(a, s) : launch_p2_t<TT, 64, false>(a, s);
  return causal ? launch_p2_t<TT, 128, true>(a, s) : launch_p2_t<TT, 128, false>(a, s);
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_fb_dkdv_t(const Pass2Args& a, hipStream_t s) {
  const size_t lds = pass2_lds_bytes<TT, D>();
  hipError_t e = ensure_lds(&bob_pass2_kernel<TT, D, CAUSAL, true>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass2_kernel<TT, D, CAUSAL, true>), dim3(row_tiles(a.N), a.BH, a.nsplit), dim3(kBlock), lds,
                     s, a);
  return hipGetLastError();
}

template <class TT>
static hipError_t launch_fb_dkdv_tt(const Pass2Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_fb_dkdv_t<TT, 64, true>(a, s) : launch_fb_dkdv_t<TT, 64, false>(a, s);
  return causal ? launch_fb_dkdv_t<TT, 128, true>(a, s) : launch_fb_dkdv_t<TT, 128, false>(a, s);
}

hipError_t launch_first_bwd_dkdv(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_fb_dkdv_tt<BF16>(a, d, causal, s);
    case DT::F16: return launch_fb_dkdv_tt<F16>(a, d, causal, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass2(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_p2_tt<BF16>(a, d, causal, s);
    case DT::F16: return launch_p2_tt<F16>(a, d, causal, s);
    default: return launch_p2_tt<F32>(a, d, causal, s);
  }
}

template <class TT, int D>
static hipError_t launch_r2_t(const Pass2Args& a, hipStream_t s) {
  dim3 grid(row_tiles(a.N) * 4, a.BH, Geo<TT, D>::MB);  // one workgroup per wave record
  hipLaunchKernelGGL((bob_pass2_reduce_kernel<TT, D>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pass2_reduce(const Pass2Args& a, DT dt, int d, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return d == 64 ? launch_r2_t<BF16, 64>(a, s) : launch_r2_t<BF16, 128>(a, s);
    case DT::F16: return d == 64 ? launch_r2_t<F16, 64>(a, s) : launch_r2_t<F16, 128>(a, s);
    default: return d == 64 ? launch_r2_t<F32, 64>(a, s) : launch_r2_t<F32, 128>(a, s);
  }
}

}  // namespace fb
