// Pass-1 accumulator epilogue and split records, shared by the pass-1 kernels.
//
// FlashBoB review page (Summary; Strengths on Prop. 4.1): alpha and E enter
// gQ and gdO affinely, so each query row keeps alpha-free sums over the keys
// and applies the two scalars once at the end:
//   gQ_i  = tau [ (W_a UK + W_b K) - alpha_i W_a K - e0_i P K ],
//   gdO_i = (P UV + (P G) V) - alpha_i O_i,
//   e0_i = sum_j W_b,   E_i = e0_i - alpha_i D_i.
// A = W_a UK + W_b K, B = W_a K, C = P K and X = P UV + (P G) V are the four
// float32 register tiles (head dims x 32 queries per wave). With E written out,
// gQ = tau [A - alpha (P dP) K - E P K]; since W_a K = (P dP) K - D P K, taking
// B = W_a K and the e0 coefficient is the same value and lets A and B share the
// weight tile W_a (one weight tile fewer per step).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace fb {

template <class TT, int D>
struct P1 {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  static constexpr int MBA = G::MB;  // accumulated 32-wide head-dim blocks
  // record layout (floats): acc[4][MBA] tiles of [4 quads][64 lanes][4] (store_tile16),
  // alpha_p[64], e0_p[64]
  static constexpr int ACC_FLOATS = 4 * MBA * 16 * 64;
};

// gQ_i and gdO_i at the 4 head dims of slots 4 r4 .. 4 r4 + 3 of the 32-wide
// head-dim block `mbg` from their alpha-free sums, with alpha_i and e0_i already
// summed over the lane pair of the row. orow: the row of O to read (global memory,
// or a copy in LDS), or null for the row in a.O.
template <class TT, int D>
__device__ inline void pass1_epilogue_quad(const f32x4& A, const f32x4& B, const f32x4& C, const f32x4& X,
                                           float alpha, float e0, int qi, int g, int bh, int mbg, int r4,
                                           const Pass1Args& a, const typename TT::elem* orow = nullptr) {
  using T = typename TT::elem;
  const int N = a.N;
  if (qi >= N) return;
  const size_t row = (size_t)bh * N + qi;
  const int dim = mbg * 32 + kappa(r4 * 4, g);
  const float tau = a.tau;
  float o[4], q[4], x[4];
  load4<TT>((orow ? orow : reinterpret_cast<const T*>(a.O) + row * D) + dim, o);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    q[e] = tau * (A[e] - alpha * B[e] - e0 * C[e]);
    x[e] = X[e] - alpha * o[e];
  }
  store4<TT>(reinterpret_cast<T*>(a.gQ) + row * D + dim, q[0], q[1], q[2], q[3]);
  store4<TT>(reinterpret_cast<T*>(a.gdO) + row * D + dim, x[0], x[1], x[2], x[3]);
}

__device__ inline f32x4 quad_of(const f32x16& v, int r4) {
  return f32x4{v[r4 * 4], v[r4 * 4 + 1], v[r4 * 4 + 2], v[r4 * 4 + 3]};
}

// The same over the whole 32-wide head-dim block `mbg` (16 slots of the lane).
template <class TT, int D>
__device__ inline void pass1_epilogue_block(const f32x16& A, const f32x16& B, const f32x16& C, const f32x16& X,
                                            float alpha, float e0, int qi, int g, int bh, int mbg,
                                            const Pass1Args& a, const typename TT::elem* orow = nullptr) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
    pass1_epilogue_quad<TT, D>(quad_of(A, r4), quad_of(B, r4), quad_of(C, r4), quad_of(X, r4), alpha, e0, qi, g,
                               bh, mbg, r4, a, orow);
}

// alpha_i and E_i = e0_i - alpha_i D_i of the row, and for pass 2 L_i log2(e) and
// c_i = alpha_i D_i + E_i (lane group 0 writes).
__device__ inline void pass1_write_scalars(float alpha, float e0, int qi, int g, int bh, const Pass1Args& a) {
  if (qi >= a.N || g != 0) return;
  const size_t row = (size_t)bh * a.N + qi;
  const float dq = a.D[row];
  const float E = e0 - alpha * dq;
  a.alpha[row] = alpha;
  a.E[row] = E;
  a.l2[row] = a.L[row] * kLog2e;
  a.c[row] = fmaf(alpha, dq, E);
}

// The same with L_i log2(e) and D_i of the row already in registers.
__device__ inline void pass1_write_scalars(float alpha, float e0, int qi, int g, int bh, const Pass1Args& a, float l2,
                                           float dq) {
  if (qi >= a.N || g != 0) return;
  const size_t row = (size_t)bh * a.N + qi;
  const float E = e0 - alpha * dq;
  a.alpha[row] = alpha;
  a.E[row] = E;
  a.l2[row] = l2;
  a.c[row] = fmaf(alpha, dq, E);
}

// gQ_i, gdO_i, alpha_i, E_i from the alpha-free sums of one wave.
template <class TT, int D>
__device__ inline void pass1_epilogue(const f32x16 (&A)[P1<TT, D>::MBA], const f32x16 (&B)[P1<TT, D>::MBA],
                                      const f32x16 (&C)[P1<TT, D>::MBA], const f32x16 (&X)[P1<TT, D>::MBA],
                                      float alpha_p, float e0_p, int qi, int g, int bh, const Pass1Args& a) {
  constexpr int MBA = P1<TT, D>::MBA;
  const float alpha = pair_sum32(alpha_p);
  const float e0 = pair_sum32(e0_p);
#pragma unroll
  for (int mbl = 0; mbl < MBA; ++mbl)
    pass1_epilogue_block<TT, D>(A[mbl], B[mbl], C[mbl], X[mbl], alpha, e0, qi, g, bh, mbl, a);
  pass1_write_scalars(alpha, e0, qi, g, bh, a);
}

// The same with the row of O read from `orow` (a copy in LDS) and L_i log2(e), D_i
// from registers: no global load at the end of the sweep.
template <class TT, int D>
__device__ inline void pass1_epilogue(const f32x16 (&A)[P1<TT, D>::MBA], const f32x16 (&B)[P1<TT, D>::MBA],
                                      const f32x16 (&C)[P1<TT, D>::MBA], const f32x16 (&X)[P1<TT, D>::MBA],
                                      float alpha_p, float e0_p, int qi, int g, int bh, const Pass1Args& a,
                                      const typename TT::elem* orow, float l2, float dq) {
  constexpr int MBA = P1<TT, D>::MBA;
  const float alpha = pair_sum32(alpha_p);
  const float e0 = pair_sum32(e0_p);
#pragma unroll
  for (int mbl = 0; mbl < MBA; ++mbl)
    pass1_epilogue_block<TT, D>(A[mbl], B[mbl], C[mbl], X[mbl], alpha, e0, qi, g, bh, mbl, a, orow);
  pass1_write_scalars(alpha, e0, qi, g, bh, a, l2, dq);
}

// Raw accumulators and row partials of one wave for split `split`.
template <class TT, int D>
__device__ inline float* pass1_record(const Pass1Args& a, int split, int bh, int qt, int wave) {
  const size_t rec = (((size_t)split * a.BH + bh) * row_tiles(a.N) + qt) * 4 + wave;
  return a.part + rec * pass1_record_floats(D);
}

template <class TT, int D>
__device__ inline void pass1_write_record(const f32x16 (&A)[P1<TT, D>::MBA], const f32x16 (&B)[P1<TT, D>::MBA],
                                          const f32x16 (&C)[P1<TT, D>::MBA], const f32x16 (&X)[P1<TT, D>::MBA],
                                          float alpha_p, float e0_p, int split, int bh, int qt, int wave, int lane,
                                          const Pass1Args& a) {
  constexpr int MB = P1<TT, D>::MBA;
  float* R = pass1_record<TT, D>(a, split, bh, qt, wave);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    store_tile16(R + (0 * MB + mb) * 1024, lane, A[mb]);
    store_tile16(R + (1 * MB + mb) * 1024, lane, B[mb]);
    store_tile16(R + (2 * MB + mb) * 1024, lane, C[mb]);
    store_tile16(R + (3 * MB + mb) * 1024, lane, X[mb]);
  }
  R[P1<TT, D>::ACC_FLOATS + lane] = alpha_p;
  R[P1<TT, D>::ACC_FLOATS + 64 + lane] = e0_p;
}

}  // namespace fb
