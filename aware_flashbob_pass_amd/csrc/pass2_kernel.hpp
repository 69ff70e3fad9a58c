// The staged pass-2 kernel template (16-bit inputs) and the pass-2 epilogue helpers.
// Included by bob_pass2.hip (every instance but the VGPR-form ones) and by
// bob_pass2_vgpr.hip (the non-causal d = 128 BoB instances, built with the
// matrix-core VGPR form: see that file).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fb {

// gK_j and gV_j at the 4 head dims of slots 4 r4 .. 4 r4 + 3 of head-dim block mb.
template <class TT, int D>
__device__ inline void pass2_epilogue_quad(const f32x4& dK, const f32x4& dV, int kj, int g, int bh, int mb, int r4,
                                           const Pass2Args& a) {
  using T = typename TT::elem;
  if (kj >= a.N) return;
  const size_t row = (size_t)bh * a.N + kj;
  const int dim = mb * 32 + kappa(r4 * 4, g);
  const float tau = a.tau;
  store4<TT>(reinterpret_cast<T*>(a.gK) + row * D + dim, tau * dK[0], tau * dK[1], tau * dK[2], tau * dK[3]);
  store4<TT>(reinterpret_cast<T*>(a.gV) + row * D + dim, dV[0], dV[1], dV[2], dV[3]);
}

template <class TT, int D>
__device__ inline void pass2_epilogue_block(const f32x16& dK, const f32x16& dV, int kj, int g, int bh, int mb,
                                            const Pass2Args& a) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 k4 = {dK[r4 * 4], dK[r4 * 4 + 1], dK[r4 * 4 + 2], dK[r4 * 4 + 3]};
    const f32x4 v4 = {dV[r4 * 4], dV[r4 * 4 + 1], dV[r4 * 4 + 2], dV[r4 * 4 + 3]};
    pass2_epilogue_quad<TT, D>(k4, v4, kj, g, bh, mb, r4, a);
  }
}

template <class TT, int D>
__device__ inline void pass2_epilogue(const f32x16 (&dK)[Geo<TT, D>::MB], const f32x16 (&dV)[Geo<TT, D>::MB],
                                      int kj, int g, int bh, const Pass2Args& a) {
#pragma unroll
  for (int mb = 0; mb < Geo<TT, D>::MB; ++mb) pass2_epilogue_block<TT, D>(dK[mb], dV[mb], kj, g, bh, mb, a);
}

template <class TT, int D>
__device__ inline void pass2_write_record(const f32x16 (&dK)[Geo<TT, D>::MB], const f32x16 (&dV)[Geo<TT, D>::MB],
                                          int split, int bh, int kt, int wave, int lane, const Pass2Args& a) {
  constexpr int MB = Geo<TT, D>::MB;
  const size_t rec = (((size_t)split * a.BH + bh) * row_tiles(a.N) + kt) * 4 + wave;
  float* R = a.part + rec * pass2_record_floats(D);  // [2][MB] quad-major tiles (store_tile16)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    store_tile16(R + (0 * MB + mb) * 1024, lane, dK[mb]);
    store_tile16(R + (1 * MB + mb) * 1024, lane, dV[mb]);
  }
}

// kReduceAtomic: add one wave's partial sums into the float32 buffers (gK without its
// factor tau, gV) with hardware float32 atomics; the order of the additions from
// different splits is not fixed, so results may differ in the last bits between runs.
template <class TT, int D>
__device__ inline void pass2_atomic_add(const f32x16 (&dK)[Geo<TT, D>::MB], const f32x16 (&dV)[Geo<TT, D>::MB],
                                        int kj, int g, int bh, const Pass2Args& a) {
  if (kj >= a.N) return;
  const size_t plane = (size_t)a.BH * a.N * D;
  float* k32 = a.acc32 + ((size_t)bh * a.N + kj) * D;
  float* v32 = k32 + plane;
#pragma unroll
  for (int mb = 0; mb < Geo<TT, D>::MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dim = mb * 32 + kappa(r, g);
      unsafeAtomicAdd(k32 + dim, dK[mb][r]);
      unsafeAtomicAdd(v32 + dim, dV[mb][r]);
    }
}

// kReduceLastBlock: after a workgroup has written its records, it counts itself in
// the key tile's counter; the workgroup that arrives last sums every split's records
// of the tile in split order (the same order as the merge kernel, so the result is
// bitwise the same as with kReduceRecords), writes gK, gV and resets the counter.
// The records of other workgroups may sit in another XCD's L2, so the writers
// release them at device scope before counting and the last one acquires before
// reading.
template <class TT, int D>
__device__ inline void pass2_last_block_merge(int kt, int bh, int wave, int lane, int kj, int g, const Pass2Args& a) {
  constexpr int MB = Geo<TT, D>::MB;
  __shared__ int last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = a.counters + (size_t)bh * row_tiles(a.N) + kt;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == (unsigned)a.nsplit - 1;
    if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  f32x16 dK[MB], dV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dK[mb] = zero16();
    dV[mb] = zero16();
  }
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R =
        a.part + ((((size_t)sp * a.BH + bh) * row_tiles(a.N) + kt) * 4 + wave) * pass2_record_floats(D);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      dK[mb] += load_tile16(R + (0 * MB + mb) * 1024, lane);
      dV[mb] += load_tile16(R + (1 * MB + mb) * 1024, lane);
    }
  }
  pass2_epilogue<TT, D>(dK, dV, kj, g, bh, a);
}

// Staged variant for 16-bit inputs: three LDS stages of row-major Q, dO, UQ
// tiles plus their four row scalars, copied two steps ahead from inline
// assembly so that the end of a step waits only for the copies of the next one
// (the compiler does not see them and inserts no wait of its own); transposed
// operands come from the transposing LDS load. Each step forms its score tiles,
// its weights and its accumulating products in turn. At d = 64 the kernel fits
// 256 registers, so two waves share each SIMD (two workgroups per CU) and each
// one's matrix-core work overlaps the other's vector work; that beat forming
// the next step's tiles during the current step at one wave per SIMD.
template <class TT, int D, bool CAUSAL, bool FIRST = false>
__global__ __launch_bounds__(kBlock, (D == 64 ? 2 : 1)) void bob_pass2_kernel(Pass2Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB, DK = G::DK, NK = G::NK;
  constexpr int NT = 3, NBUF = 3, AHEAD = NBUF - 1;
  constexpr int STAGE_ELEMS = NT * G::ROW_ELEMS + 4 * kTile * 4 / (int)sizeof(T);  // tiles + 4 x 32 floats
  static_assert(TT::KPL == 8 && NK == 2, "16-bit inputs only");
  // Non-causal d = 128 (one wave per SIMD): AGPR accumulators from inline assembly,
  // everything else in the VGPR form (bob_pass2_vgpr.hip), so no score-tile copies.
  // The causal build of that form spills to scratch memory and keeps the default form.
  constexpr bool ASM_ACC = D == 128 && !FIRST && !CAUSAL;
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  int kt, bh;
  tile_and_head<CAUSAL, false>(kt, bh);
  const int N = a.N, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const size_t vbase = (size_t)bh * N;
  const T* src[NT] = {reinterpret_cast<const T*>(a.Q) + base, reinterpret_cast<const T*>(a.dO) + base,
                      reinterpret_cast<const T*>(a.UQ) + base};
  // FIRST (the first backward g: dK = tau dS^T Q, dV = P^T dO) needs S and dP only:
  // no UQ tile, no UK / UV rows, and only the L and D row scalars.
  constexpr int NSCAL = FIRST ? 2 : 4;
  constexpr int COPIES = (FIRST ? 2 : 3) * stage_copies<D, kBlock / 64>() + 1;  // per wave and stage
  const float* vsrc[4] = {(FIRST ? a.L : a.l2) + vbase, a.D + vbase, FIRST ? nullptr : a.alpha + vbase,
                          FIRST ? nullptr : a.c + vbase};
  const int k0w = kt * kBlockRows + wave * kTile;
  const int kj = k0w + n;

  V bk[DK], bv[DK], buk[DK], buv[DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.K) + base, kj, N, g, bk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.V) + base, kj, N, g, bv);
  if constexpr (!FIRST) {
    load_resident<TT, D>(reinterpret_cast<const T*>(a.UK) + base, kj, N, g, buk);
    load_resident<TT, D>(reinterpret_cast<const T*>(a.UV) + base, kj, N, g, buv);
  }
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x16 accK[MB], accV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accK[mb] = zero16();
    accV[mb] = zero16();
  }

  const int nqt = (N + kTile - 1) / kTile;
  const int qt_first = CAUSAL ? kt * (kBlockRows / kTile) : 0;
  const int span = nqt - qt_first;
  const int it_begin = qt_first + (int)((long long)split * span / a.nsplit);
  const int it_end = qt_first + (int)((long long)(split + 1) * span / a.nsplit);
  const int nsteps = it_end - it_begin;

  auto tile = [&](int j, int t) { return lds + (j % NBUF) * STAGE_ELEMS + t * G::ROW_ELEMS; };
  auto scal = [&](int j) { return reinterpret_cast<float*>(lds + (j % NBUF) * STAGE_ELEMS + NT * G::ROW_ELEMS); };
  auto active = [&](int j) { return !CAUSAL || (it_begin + j) * kTile + kTile - 1 >= k0w; };

  // Each stage also holds the row scalars of its 32 queries (rows >= N repeat row
  // N - 1): L log2(e), D, alpha and c = alpha D + E as pass 1 wrote them, so that
  // Sbar = P (Pbar - E) = dPbar (dP - D) + P (H - c) (Pbar = G (dP - D) - alpha dP
  // + H); the first backward stages L and D and scales L here. Wave w copies
  // scalar w % NSCAL with its lanes 0..31, so every wave issues the same number of
  // copies per stage (with NSCAL = 2 two waves write the same values).
  // Whole 32-row blocks take the scalar-base copies (no per-step address arithmetic);
  // the ragged last block keeps stage_direct and glds4, which repeat row N - 1.
  constexpr int CP = stage_copies<D, kBlock / 64>();
  unsigned coff[CP];
#pragma unroll
  for (int p = 0; p < CP; ++p) coff[p] = stage_lane_offset<D, kBlock / 64>(p, wave, lane);
  const unsigned lds_wave = lds_addr(lds) + (unsigned)wave * 1024u;
  auto issue = [&](int stg, int j) {
    const int i0 = (it_begin + j) * kTile;
    const int which = wave % NSCAL;
    if (i0 + kTile <= N) {
      const unsigned stage_bytes = (unsigned)((stg % NBUF) * STAGE_ELEMS * (int)sizeof(T));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (!FIRST || t < 2)
          stage_block_saddr<D, kBlock / 64>(src[t] + (size_t)i0 * D, coff,
                                            lds_wave + stage_bytes + (unsigned)(t * G::ROW_ELEMS * (int)sizeof(T)));
      if (lane < kTile)
        glds4_saddr(vsrc[which] + i0, (unsigned)lane * 4u, lds_addr(scal(stg) + which * kTile));
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        if (!FIRST || t < 2) stage_direct<TT, D, kBlock / 64, true>(src[t], i0, N, tile(stg, t), wave, lane);
      if (lane < kTile) glds4<true>(vsrc[which] + min(i0 + lane, N - 1), scal(stg) + which * kTile);
    }
  };
  settle_regs(bk, bv);
  if constexpr (!FIRST) settle_regs(buk, buv);
  for (int j = 0; j < AHEAD && j < nsteps; ++j) issue(j, j);
  wait_vmem();
  __syncthreads();

  f32x16 sc, gc, pc, hc;  // score tiles of the current step
  auto scores_kstep = [&](int j, int t, f32x16& s_, f32x16& g_, f32x16& p_, f32x16& h_) {
    const V aq = lds_row_op<TT, D>(tile(j, 0), n, t, g);
    const V ado = lds_row_op<TT, D>(tile(j, 1), n, t, g);
    const V auq = lds_row_op<TT, D>(tile(j, 2), n, t, g);
    s_ = TT::mfma(aq, bk[t], s_);
    if constexpr (!FIRST) {
      g_ = TT::mfma(auq, bk[t], g_);
      g_ = TT::mfma(aq, buk[t], g_);
    }
    p_ = TT::mfma(ado, bv[t], p_);
    if constexpr (!FIRST) h_ = TT::mfma(ado, buv[t], h_);
  };
  auto step = [&](auto S_c, int j) {
    constexpr int S = decltype(S_c)::value;
    constexpr int SC = (S + AHEAD) % NBUF;
    const bool copies = j + AHEAD < nsteps;
    if (copies) issue(SC, j + AHEAD);  // buffer SC was last read in step j - 1
    const int i0 = (it_begin + j) * kTile;
    if (active(j)) {
      sc = zero16();
      gc = zero16();
      pc = zero16();
      hc = zero16();
#pragma unroll
      for (int t = 0; t < DK; ++t) scores_kstep(S, t, sc, gc, pc, hc);
      // Row scalars of the streamed queries: lane group g holds rows kappa(r, g), which
      // for r = 4 r4 .. 4 r4 + 3 are the 4 consecutive rows 8 r4 + 4 g .. + 3.
      const float* sv = scal(S);
      auto row4 = [&](int which, int r4) {
        return *reinterpret_cast<const f32x4*>(sv + which * kTile + r4 * 8 + g * 4);
      };
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = FIRST ? row4(0, r4) * kLog2e : row4(0, r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[r4 * 4 + e] = sc[r4 * 4 + e] * cs - l4[e];
      }
      if (i0 + kTile > N || (CAUSAL && i0 < k0w + kTile - 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i0 + kappa(r, g);
          if (!(qrow < N && (!CAUSAL || kj <= qrow))) sc[r] = -INFINITY;
        }
      }
      V wds[NK], wsb[NK], wdp[NK];
      f32x4 d4, a4, c4;  // D, alpha, c of the current group of 4 rows (loaded at its first row)
      auto elementwise = [&](int r) {
        if ((r & 3) == 0) {
          d4 = row4(1, r >> 2);
          if constexpr (!FIRST) {
            a4 = row4(2, r >> 2);
            c4 = row4(3, r >> 2);
          }
        }
        const float dq = d4[r & 3];
        const float p = fast_exp2(sc[r]);
        const float dpv = pc[r];
        const float t1 = dpv - dq;
        const int kk = r >> 3, ss = r & 7;
        vset<TT>(wds[kk], ss, p * t1);  // dS
        if constexpr (FIRST) {
          vset<TT>(wdp[kk], ss, p);  // P
        } else {
          const float dpb = p * (gc[r] * tau - a4[r & 3]);           // dPbar = P (G - alpha)
          vset<TT>(wsb[kk], ss, fmaf(dpb, t1, p * (hc[r] - c4[r & 3])));  // Sbar
          vset<TT>(wdp[kk], ss, dpb);
        }
      };
#pragma unroll
      for (int t = 0; t < DK; ++t)
#pragma unroll
        for (int r = t * 8 / DK; r < (t + 1) * 8 / DK; ++r) elementwise(r);
#pragma unroll
      for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const V tuq = lds_tr_op<TT, D>(tile(S, 2), mb, t, lane);
          const V tq = lds_tr_op<TT, D>(tile(S, 0), mb, t, lane);
          const V tdo = lds_tr_op<TT, D>(tile(S, 1), mb, t, lane);
          if (t == 0) {
#pragma unroll
            for (int r = 8 + mb * 8 / MB; r < 8 + (mb + 1) * 8 / MB; ++r) elementwise(r);
          }
          if constexpr (ASM_ACC) {  // AGPR accumulators from inline assembly
            mfma_acc<TT>(accK[mb], tuq, wds[t]);  // dS^T UQ
            mfma_acc<TT>(accK[mb], tq, wsb[t]);   // Sbar^T Q
            mfma_acc<TT>(accV[mb], tdo, wdp[t]);  // dPbar^T dO
          } else {
            if constexpr (FIRST) {
              accK[mb] = TT::mfma(tq, wds[t], accK[mb]);  // dS^T Q
            } else {
              accK[mb] = TT::mfma(tuq, wds[t], accK[mb]);  // dS^T UQ
              accK[mb] = TT::mfma(tq, wsb[t], accK[mb]);   // Sbar^T Q
            }
            accV[mb] = TT::mfma(tdo, wdp[t], accV[mb]);    // P^T dO or dPbar^T dO
          }
        }
    }
    if (copies) wait_vmem_keep<COPIES>();  // this step's copies may stay in flight
    else wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + NBUF <= nsteps; j += NBUF) unroll_steps(step, j, std::make_integer_sequence<int, NBUF>{});
  unroll_steps_until(step, j, nsteps, std::make_integer_sequence<int, NBUF - 1>{});

  if constexpr (ASM_ACC) acc_settle<MB>(accK, accV);
  if (a.nsplit == 1) {
    pass2_epilogue<TT, D>(accK, accV, kj, g, bh, a);
    return;
  }
  if constexpr (!FIRST) {
    if (a.reduce == kReduceAtomic) {
      pass2_atomic_add<TT, D>(accK, accV, kj, g, bh, a);
      return;
    }
  }
  pass2_write_record<TT, D>(accK, accV, split, bh, kt, wave, lane, a);
  if constexpr (!FIRST) {
    if (a.reduce == kReduceLastBlock) pass2_last_block_merge<TT, D>(kt, bh, wave, lane, kj, g, a);
  }
}

template <class TT, int D>
inline size_t pass2_lds_bytes() {
  using G = Geo<TT, D>;
  if constexpr (TT::KPL == 1)
    return (size_t)3 * (G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem) + 4 * kTile * sizeof(float);
  return (size_t)3 * (3 * G::ROW_ELEMS * sizeof(typename TT::elem) + 4 * kTile * sizeof(float));
}

}  // namespace fb
