// Shared device helpers for the gfx950 attention BoB kernels.
//
// Tiling convention used by every kernel here. A wave owns 32 "resident" rows
// (queries in the statistics kernel and pass 1, keys in pass 2) and walks the
// other ("streamed") side in steps of 32 rows that the workgroup stages in LDS.
// Each step forms 32x32 score tiles with v_mfma_f32_32x32x{16 bf16|16 f16|2 f32}
// so that lane l owns resident row (l % 32) and, in its 16 accumulator slots
// r = 0..15, the streamed rows kappa(r, l / 32) = 8*(r/4) + 4*(l/32) + r%4.
// That is the matrix cores' own output layout with the resident side on the
// N (column) axis: the score tile is S^T (streamed x resident).
//
// The accumulating contractions (sum over the streamed rows) then reuse each
// lane's slots directly as the B operand: the contraction index k of slot r is
// the streamed row kappa(r, g), and the A operand (streamed-tensor columns)
// is read from a transposed LDS copy whose 32 columns are stored in the order
// pos(k) with pos(kappa(r, g)) = 16*g + r, so that a lane's KPL operand
// elements are contiguous. Outputs come out transposed as well (head dim on
// the M axis, resident row on the N axis): lane l holds dims
// kappa(r, l / 32) of resident row l % 32, so every per-row scalar (LSE, D,
// alpha, E) is a per-lane value after one exchange between lanes l and l ^ 32.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>
#include <stdint.h>

namespace fb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTile = 32;  // resident rows per wave == streamed rows per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- element types and their matrix-core instruction -----------------------
struct BF16 {
  using elem = __bf16;
  using vec = bf16x8;
  static constexpr int KPL = 8;  // operand elements per lane per k-step
  __device__ static inline f32x16 mfma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline elem cvt(float x) { return (elem)x; }
  __device__ static inline float tof(elem x) { return (float)x; }
};
struct F16 {
  using elem = _Float16;
  using vec = f16x8;
  static constexpr int KPL = 8;
  __device__ static inline f32x16 mfma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline elem cvt(float x) { return (elem)x; }
  __device__ static inline float tof(elem x) { return (float)x; }
};
struct F32 {
  using elem = float;
  using vec = float;
  static constexpr int KPL = 1;
  __device__ static inline f32x16 mfma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline elem cvt(float x) { return x; }
  __device__ static inline float tof(elem x) { return x; }
};

template <class TT>
__device__ inline void vset(typename TT::vec& v, int s, float x) {
  if constexpr (TT::KPL == 1) {
    v = x;
  } else {
    v[s] = TT::cvt(x);
  }
}

__host__ __device__ constexpr int kappa(int r, int g) { return ((r >> 2) << 3) + (g << 2) + (r & 3); }
__host__ __device__ constexpr int tpos(int k) { return (((k >> 2) & 1) << 4) + ((k >> 3) << 2) + (k & 3); }

// ---- LDS tile geometry --------------------------------------------------------
// Row-major copy: 32 rows x D, row stride RS elements. For 16-bit types the rows
// are unpadded and the 16-byte chunks of row r are stored XOR-swizzled: chunk c
// at position c ^ swz(r), chosen so that the kernels' LDS reads are free of bank
// conflicts (64 four-byte banks; rocprofv3 SQ_LDS_BANK_CONFLICT reads zero for the
// statistics kernel and both passes at d = 64 and 128):
//  - the 16-byte row reads of the score operands take 16 consecutive rows at one
//    chunk, so the rows sharing a bank offset need distinct swizzles;
//  - the transposing 8-byte reads take 4 aligned consecutive rows x 64 bytes
//    (chunks 4m .. 4m + 3) per 32 lanes, so rows sharing a bank offset need
//    swizzles that differ above bit 1.
// d = 64 (128-byte rows: rows r and r + 1 are 32 banks apart): with h = (r / 2) mod 8,
// swz = ((h & 1) << 2) | (h >> 1). d = 128 (256-byte rows, all at one bank offset):
// swz = ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1), a bijection on 16
// rows whose top two bits differ within every 4 aligned rows. The former swizzles,
// (r / 2) mod 8 and r mod 16, left the transposing reads 2-way and 4-way
// conflicted (23-60% of the LDS-active cycles).
// Layout 1 serves the 16-query d = 128 pass 1, whose reads group lanes differently
// (16-byte row reads: 16 rows x 4 chunks per 64 lanes; transposing reads: 16 rows x
// 32 bytes). No simple bank model predicted its conflicts, so its swizzle was found
// by measurement: of 48 candidates (bit permutations of the row's low four bits,
// with and without their low bits XOR-ed into the high ones), four read both
// patterns without conflicts; this one is XOR-linear in the row bits
// (8 b0 ^ 10 b1 ^ 5 b2 ^ 4 b3). They leave the 32-query kernels' transposing reads
// 2-way conflicted, hence two layouts.
// float32 rows are padded by one element instead.
// Transposed copy (float32 kernels and the first backward): D rows (head dims)
// x 32 columns in tpos() order, row stride TS.
template <int D, int L = 0>
__device__ inline int swz(int row) {
  if constexpr (D == 64) {
    const int h = (row >> 1) & 7;
    return ((h & 1) << 2) | (h >> 1);
  } else if constexpr (L == 1) {
    return ((row & 1) ? 8 : 0) ^ ((row & 2) ? 10 : 0) ^ ((row & 4) ? 5 : 0) ^ ((row & 8) ? 4 : 0);
  } else {
    return ((row & 3) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  }
}

template <class TT, int D>
struct Geo {
  using T = typename TT::elem;
  static constexpr int PAD = (sizeof(T) == 2) ? 8 : 1;
  static constexpr int RS = (sizeof(T) == 2) ? D : D + 1;
  static constexpr int TS = kTile + PAD;
  static constexpr int ROW_ELEMS = kTile * RS;
  static constexpr int T_ELEMS = D * TS;
  static constexpr int DK = D / (2 * TT::KPL);      // k-steps over the head dim
  static constexpr int NK = kTile / (2 * TT::KPL);  // k-steps over 32 streamed rows
  static constexpr int MB = D / 32;                 // 32-wide head-dim blocks
};

// Element offset of (row, col) in a row-major LDS tile (col: 4-element aligned
// within its 16-byte chunk for 16-bit types).
template <class TT, int D, int L = 0>
__device__ inline int roff(int row, int col) {
  if constexpr (sizeof(typename TT::elem) == 2) {
    return row * D + ((((col >> 3) ^ swz<D, L>(row)) << 3) | (col & 7));
  } else {
    return row * Geo<TT, D>::RS + col;
  }
}

// Stage rows [r0, r0 + 32) of a [N][D] tensor into LDS (row-major copy `rowbuf`
// and/or transposed copy `tbuf`, either may be null). Rows >= N read as zero.
// All `nthreads` threads of the block take part; caller brackets with barriers.
template <class TT, int D>
__device__ inline void stage_tile(const typename TT::elem* __restrict__ src, int r0, int N,
                                  typename TT::elem* rowbuf, typename TT::elem* tbuf, int tid,
                                  int nthreads) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / CH;         // chunks per row
  constexpr int NCH = kTile * CPR;
  for (int c = tid; c < NCH; c += nthreads) {
    const int row = c / CPR;
    const int e0 = (c % CPR) * CH;
    const int grow = r0 + row;
    uint4 raw = make_uint4(0u, 0u, 0u, 0u);
    if (grow < N) raw = *reinterpret_cast<const uint4*>(src + (size_t)grow * D + e0);
    const T* v = reinterpret_cast<const T*>(&raw);
    if (rowbuf) {
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(rowbuf + roff<TT, D>(row, e0)) = raw;
      } else {
#pragma unroll
        for (int e = 0; e < CH; ++e) rowbuf[row * G::RS + e0 + e] = v[e];
      }
    }
    if (tbuf) {
      const int p = tpos(row);
#pragma unroll
      for (int e = 0; e < CH; ++e) tbuf[(e0 + e) * G::TS + p] = v[e];
    }
  }
}

// A operand of a score tile: streamed row m = lane % 32, head dims of k-step t.
template <class TT, int D>
__device__ inline typename TT::vec lds_row_op(const typename TT::elem* rowbuf, int m, int t, int g) {
  const typename TT::elem* p = rowbuf + roff<TT, D>(m, t * 2 * TT::KPL + g * TT::KPL);
  return *reinterpret_cast<const typename TT::vec*>(p);
}

// A operand of an accumulating contraction: head dim `dim`, streamed rows of
// k-step t (slots r = t*KPL .. t*KPL + KPL - 1 of lane group g).
template <class TT, int D>
__device__ inline typename TT::vec lds_t_op(const typename TT::elem* tbuf, int dim, int t, int g) {
  using G = Geo<TT, D>;
  const typename TT::elem* p = tbuf + dim * G::TS + g * 16 + t * TT::KPL;
  return *reinterpret_cast<const typename TT::vec*>(p);
}

// B operand held in registers for the whole kernel: resident row `row`
// (zero when row >= N), head dims of every k-step.
template <class TT, int D>
__device__ inline void load_resident(const typename TT::elem* __restrict__ src, int row, int N, int g,
                                     typename TT::vec (&out)[Geo<TT, D>::DK]) {
  using G = Geo<TT, D>;
  using V = typename TT::vec;
#pragma unroll
  for (int t = 0; t < G::DK; ++t) {
    if (row < N) {
      out[t] = *reinterpret_cast<const V*>(src + (size_t)row * D + t * 2 * TT::KPL + g * TT::KPL);
    } else {
      if constexpr (TT::KPL == 1) {
        out[t] = 0.f;
      } else {
#pragma unroll
        for (int s = 0; s < TT::KPL; ++s) out[t][s] = TT::cvt(0.f);
      }
    }
  }
}

// One direct global -> LDS copy: global_load_lds_dwordx4, whose lane L writes
// the 16 bytes at the wave-uniform LDS address `lds` + 16 L (the address goes in
// M0). ASYNC = false uses the compiler builtin; the compiler cannot tell which
// LDS bytes such a copy writes, so it waits for the copy to land before the
// wave's next LDS read. ASYNC = true issues the same instruction from inline
// assembly, invisible to the compiler, so copies stay in flight across LDS reads
// and barriers; the kernel then orders them itself with s_waitcnt vmcnt before
// the barrier that publishes a stage (the s_nop covers the M0 write -> LDS-DMA
// hazard).
template <bool ASYNC>
__device__ inline void glds16(const void* gsrc, void* lds) {
  if constexpr (ASYNC) {
    const unsigned m0 =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) void*)lds);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
  } else {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
  }
}

// The same for 4 bytes per lane: lane l's value lands at lds + 4 l.
template <bool ASYNC>
__device__ inline void glds4(const void* gsrc, void* lds) {
  if constexpr (ASYNC) {
    const unsigned m0 =
        __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) void*)lds);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
  } else {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
  }
}

// Direct global -> LDS staging of one 32-row stage of a [N][D] tensor (16-bit
// types) with glds16. LDS slot s of the tile is row s / (D / 8), physical chunk
// s % (D / 8); its source is the logical chunk (physical chunk ^ swz(row)) of
// that row, which realises the XOR swizzle of roff(). Rows >= N fetch row
// N - 1 (finite values; every consumer masks them out). Each wave issues
// stage_copies<D, NWAVES>() copies. Completion: s_waitcnt vmcnt then a
// workgroup barrier.
template <int D, int NWAVES>
__host__ __device__ constexpr int stage_copies() { return kTile * (D / 8) / (64 * NWAVES); }

template <class TT, int D, int NWAVES, bool ASYNC = false, int L = 0>
__device__ inline void stage_direct(const typename TT::elem* __restrict__ src, int r0, int N,
                                    typename TT::elem* tile, int wave, int lane) {
  static_assert(sizeof(typename TT::elem) == 2, "16-bit types only");
  constexpr int SPR = D / 8;                     // 16-byte slots per row
  constexpr int PER_WAVE = kTile * SPR / (64 * NWAVES);
  static_assert(PER_WAVE * 64 * NWAVES == kTile * SPR, "stage must split evenly over the waves");
#pragma unroll
  for (int p = 0; p < PER_WAVE; ++p) {
    const int blk = p * NWAVES + wave;
    const int slot = blk * 64 + lane;
    const int row = slot / SPR, pc = slot % SPR;
    const int c = pc ^ swz<D, L>(row);
    const int grow = min(r0 + row, N - 1);
    glds16<ASYNC>(src + (size_t)grow * D + c * 8, tile + blk * 64 * 8);
  }
}

// The same copies for a whole 32-row block (every row below N) in the scalar-base form:
// the block's address is wave-uniform and each lane's byte offset within it, which is the
// same for every block, is computed once (stage_lane_offset), so a step spends no vector
// instructions on addresses. lds_tile_wave: the LDS byte address of the tile plus
// 1024 wave (wave-uniform). The s_nop covers the M0 write -> LDS-DMA hazard.
template <int D, int NWAVES, int L = 0>
__device__ inline unsigned stage_lane_offset(int p, int wave, int lane) {
  constexpr int SPR = D / 8;
  const int slot = (p * NWAVES + wave) * 64 + lane, row = slot / SPR;
  return 2u * (unsigned)(row * D + (((slot % SPR) ^ swz<D, L>(row)) << 3));
}
template <int D, int NWAVES>
__device__ inline void stage_block_saddr(const void* block, const unsigned (&off)[stage_copies<D, NWAVES>()],
                                         unsigned lds_tile_wave) {
#pragma unroll
  for (int p = 0; p < stage_copies<D, NWAVES>(); ++p) {
    const unsigned m0 = lds_tile_wave + (unsigned)(p * NWAVES * 1024);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0" ::"v"(off[p]), "s"(block), "{m0}"(m0)
                 : "memory");
  }
}
// 4 bytes per lane in the scalar-base form: lane l's value (at byte off of src) lands at
// LDS byte address lds + 4 l.
__device__ inline void glds4_saddr(const void* src, unsigned off, unsigned lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1 offset:0" ::"v"(off), "s"(src), "{m0}"(lds) : "memory");
}
// The LDS byte address of an LDS pointer, wave-uniform.
template <class P>
__device__ inline unsigned lds_addr(const P* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(__attribute__((address_space(3))) const void*)p);
}

__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Unrolled runs of pipeline steps with compile-time stage indices: unroll_steps
// calls f(integral_constant<int, I>, j0 + I) for every I of the sequence;
// unroll_steps_until does so only while j0 + I < end (a loop's tail).
template <class F, int... I>
__device__ inline void unroll_steps(F& f, int j0, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}, j0 + I), ...);
}
template <class F, int... I>
__device__ inline void unroll_steps_until(F& f, int j0, int end, std::integer_sequence<int, I...>) {
  ((j0 + I < end ? f(std::integral_constant<int, I>{}, j0 + I) : void()), ...);
}

// Make the compiler complete the loads that produced these registers here (an
// empty asm that reads them), before a loop that keeps inline-assembly copies in
// flight across its own s_waitcnt vmcnt(N).
template <class R>
__device__ inline void settle_one(const R& r) {
  asm volatile("" ::"v"(r));
}
template <class... R>
__device__ inline void settle_regs(const R&... r) {
  (settle_one(r), ...);
}
template <class V, int K>
__device__ inline void settle_regs(const V (&r)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) settle_one(r[k]);
}
template <class V, int K, class... R>
__device__ inline void settle_regs(const V (&r)[K], const R&... rest) {
  settle_regs(r);
  settle_regs(rest...);
}

// All but the newest N vector-memory operations of the wave have completed.
template <int N>
__device__ inline void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// A operand of an accumulating contraction (head dims x streamed rows) read from
// the ROW-MAJOR copy with gfx950's transposing LDS load. Within each 16-lane
// group, the load hands destination lane i element (i % 4) of the 8-byte chunk
// addressed by source lane 4e + i / 4, for e = 0..3. Each lane therefore
// addresses streamed row (base + e_src) at head dims 4 * q_src .. + 3 with
// e_src = (lane % 16) / 4, q_src = lane % 4, and receives 4 streamed rows of
// head dim (lane % 16) of its 16-dim group. Two loads (h = 0, 1) give the 8
// k-slots s = 4h + e, which are streamed rows 16t + 8h + 4g + e = kappa(8t + s, g),
// the same rows the score-tile B operand holds in its slots.
template <class TT, int D>
__device__ inline typename TT::vec lds_tr_op(const typename TT::elem* rowbuf, int mb, int t, int lane) {
  static_assert(TT::KPL == 8, "transposing LDS loads are for 16-bit types");
  const int i = lane & 15, g = lane >> 5, half = (lane >> 4) & 1;
  const int col = mb * 32 + half * 16 + (i & 3) * 4;
  const int row0 = t * 16 + g * 4 + (i >> 2);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(rowbuf + roff<TT, D>(row0, col)));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(rowbuf + roff<TT, D>(row0 + 8, col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename TT::vec, v);
}

// Accumulating product into AGPRs, issued from inline assembly: used by the sweeps
// compiled with the matrix-core VGPR form (bob_pass1_vgpr.hip, bob_pass2_vgpr.hip),
// so their accumulator tiles stay in AGPRs and their score tiles in VGPRs with no
// copies between the two files. The compiler does not see these as matrix-core ops,
// so the asm covers the hazards it would otherwise handle: s_nop 1 (2 wait states)
// after the vector instruction that wrote a weight operand; reads of the
// accumulators after the sweep wait in acc_settle.
template <class TT>
__device__ inline void mfma_acc(f32x16& acc, typename TT::vec a, typename TT::vec b) {
  if constexpr (std::is_same_v<TT, BF16>)
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 24 wait states after the last accumulating product before anything reads the
// accumulator tiles (a 16-pass product's result needs 18); the operands tie every
// later read of the tiles to this point.
template <int MB>
__device__ inline void acc_settle(f32x16 (&A)[MB], f32x16 (&B)[MB]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) asm volatile("" : "+a"(A[mb]), "+a"(B[mb]));
}

// The same for 16 x 16 x 32 products on 16 x 16 float32 tiles (four values a lane), and
// the settle of four arrays of such tiles (an 8-pass product's result needs 10 wait states;
// 24 are given).
template <class TT>
__device__ inline void mfma16_acc(f32x4& acc, typename TT::vec a, typename TT::vec b) {
  if constexpr (std::is_same_v<TT, BF16>)
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int M>
__device__ inline void acc16_settle(f32x4 (&A)[M], f32x4 (&B)[M], f32x4 (&C)[M], f32x4 (&X)[M]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int m = 0; m < M; ++m) asm volatile("" : "+a"(A[m]), "+a"(B[m]), "+a"(C[m]), "+a"(X[m]));
}

// Index of the calling wave in its workgroup as a wave-uniform (scalar)
// value, so that branches and offsets derived from it stay scalar.
__device__ inline int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// A wave's 16 accumulator slots per lane as one 1024-float record tile, quad-major:
// slots 4q .. 4q + 3 of lane L at floats 4 (64 q + L). Each of the wave's four 16-byte
// stores (or loads) of a tile then covers 1 KB of contiguous memory; with each lane's
// 16 slots contiguous instead, every store was strided by 64 bytes per lane and the
// split-record writes at the end of pass 1 ran at about a third of HBM's rate.
__device__ inline void store_tile16(float* tile, int lane, const f32x16& v) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<f32x4*>(tile)[q * 64 + lane] = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}
__device__ inline f32x4 tile_quad(const float* tile, int lane, int q) {
  return reinterpret_cast<const f32x4*>(tile)[q * 64 + lane];
}
__device__ inline f32x16 load_tile16(const float* tile, int lane) {
  f32x16 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 x = tile_quad(tile, lane, q);
    v[4 * q] = x[0];
    v[4 * q + 1] = x[1];
    v[4 * q + 2] = x[2];
    v[4 * q + 3] = x[3];
  }
  return v;
}

// Tile and head of a workgroup of a (tiles x heads) grid. Causal grids are
// walked heaviest tile first across all heads (longest-processing-time order):
// the dispatcher issues workgroups by linear id, so tile `heavy_first(lin)`
// for every head comes before the next lighter tile of any head.
template <bool CAUSAL, bool LAST_IS_HEAVIEST>
__device__ inline void tile_and_head(int& tile, int& head) {
  if (!CAUSAL) {
    tile = blockIdx.x;
    head = blockIdx.y;
    return;
  }
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int rank = lin / gridDim.y;
  head = lin % gridDim.y;
  tile = LAST_IS_HEAVIEST ? (int)gridDim.x - 1 - rank : rank;
}

// Maximum of the 16 slots of one lane (balanced tree: depth 4).
__device__ inline float max16(const f32x16& v) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = fmaxf(v[2 * i], v[2 * i + 1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = fmaxf(a[2 * i], a[2 * i + 1]);
  return fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
}

// Sum / maximum of x over the lane pair (l, l ^ 32), returned on both lanes.
// gfx950's v_permlane32_swap exchanges the two 32-lane halves in the vector ALU
// (no LDS round trip): with both operands x, lane i < 32 receives (x[i],
// x[i + 32]) and lane i >= 32 receives (x[i - 32], x[i]) (layout checked with an
// in-bounds probe). Addition and maximum commute, so both lanes of a pair get
// the bitwise-same result.
__device__ inline float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Store 4 consecutive head dims [dim, dim + 4) of one row.
template <class TT>
__device__ inline void store4(typename TT::elem* dst, float a, float b, float c, float d) {
  using T = typename TT::elem;
  if constexpr (sizeof(T) == 2) {
    T v[4] = {TT::cvt(a), TT::cvt(b), TT::cvt(c), TT::cvt(d)};
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(v);
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
}

template <class TT>
__device__ inline void load4(const typename TT::elem* src, float (&o)[4]) {
  using T = typename TT::elem;
  if constexpr (sizeof(T) == 2) {
    uint2 raw = *reinterpret_cast<const uint2*>(src);
    const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = TT::tof(v[e]);
  } else {
    f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = v[e];
  }
}

}  // namespace fb
