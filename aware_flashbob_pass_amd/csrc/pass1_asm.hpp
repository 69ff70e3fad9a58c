// The step loop of pass 1's d = 64 bf16 sweep with tau folded into the resident rows,
// as one inline-assembly block with a fixed schedule (pass1_asm_loop.inc, written by
// gen_pass1_asm.py, whose docstring gives the schedule and the register map). It
// computes what bob_pass1_kernel's pipelined step loop computes for that sweep
// (FlashBoB review page, Summary; Strengths on Prop. 4.1) over steps that need no
// mask: whole 32-key blocks that no query of the workgroup precedes.
//
// Entry state (all set up by the caller, as for the compiled loop): the first stages
// copied and published by a barrier, and the score tiles S, G, dP, H of step 0
// formed. The block runs `nsteps` steps; the copies run ahead to step `nsteps_all`
// of the sweep, so compiled steps can follow it (then nsteps is a multiple of the
// stage count). On exit sc, gc, pc, hc hold the score tiles of step nsteps, the dP
// tile less D when FB_PASS1_ASM_DBIAS is set. The block binds its state to fixed
// registers at entry and exit only; between the two it owns every VGPR, a[0:239] and
// s[40:54].
#pragma once

#include "common.hpp"
#include "pass1_asm_loop.inc"

namespace fb {

__device__ inline void pass1_asm_steps(f32x16& sc, f32x16& gc, f32x16& pc, f32x16& hc, const bf16x8 (&bq)[4],
                                       const bf16x8 (&buq)[4], const bf16x8 (&bdo)[4], f32x16 (&A)[2],
                                       f32x16 (&B)[2], f32x16 (&C)[2], f32x16 (&X)[2], float& alpha, float& e0,
                                       float lq, float dq, const __bf16* k3, const __bf16* v3, const __bf16* uk3,
                                       const __bf16* uv3, const __bf16* lds, int wave, int lane, int nsteps,
                                       int nsteps_all) {
  using LdsPtr = __attribute__((address_space(3))) const void*;
  const unsigned lb = (unsigned)(size_t)(LdsPtr)lds;
  const int n = lane & 31, g = lane >> 5;
  // score operands: streamed row n, head dims 16 t + 8 g .. + 7 (lds_row_op)
  const unsigned r0 = lb + 2u * roff<BF16, 64>(n, 0 * 16 + g * 8);
  const unsigned r1 = lb + 2u * roff<BF16, 64>(n, 1 * 16 + g * 8);
  const unsigned r2 = lb + 2u * roff<BF16, 64>(n, 2 * 16 + g * 8);
  const unsigned r3 = lb + 2u * roff<BF16, 64>(n, 3 * 16 + g * 8);
  // transposing reads of k-step 0 (lds_tr_op): later k-steps are 16 rows (2048 bytes)
  // further on, since the swizzle depends on row bits 1..3 only
  const int i = lane & 15, half = (lane >> 4) & 1;
  const int row0 = g * 4 + (i >> 2);
  const int col0 = half * 16 + (i & 3) * 4, col1 = 32 + col0;
  const unsigned t0 = lb + 2u * roff<BF16, 64>(row0, col0);
  const unsigned t1 = lb + 2u * roff<BF16, 64>(row0 + 8, col0);
  const unsigned t2 = lb + 2u * roff<BF16, 64>(row0, col1);
  const unsigned t3 = lb + 2u * roff<BF16, 64>(row0 + 8, col1);
  // direct copies (stage_direct with one copy per wave and tensor): the lane's source
  // offset within a 32-row block and the wave's LDS destination
  const int slot = wave * 64 + lane, crow = slot >> 3;
  const unsigned coff = 2u * (unsigned)(crow * 64 + (((slot & 7) ^ swz<64>(crow)) << 3));
  const unsigned ldsw = __builtin_amdgcn_readfirstlane(lb + (unsigned)wave * 1024u);
  const unsigned ns = __builtin_amdgcn_readfirstlane((unsigned)nsteps);
  const unsigned ns_all = __builtin_amdgcn_readfirstlane((unsigned)nsteps_all);
  asm volatile(FB_PASS1_ASM_LOOP
               : "+{v[0:15]}"(sc), "+{v[16:31]}"(gc), "+{v[32:47]}"(pc), "+{v[48:63]}"(hc), "+{v254}"(alpha),
                 "+{v255}"(e0), "+{a[0:15]}"(A[0]), "+{a[16:31]}"(A[1]), "+{a[32:47]}"(B[0]), "+{a[48:63]}"(B[1]),
                 "+{a[64:79]}"(C[0]), "+{a[80:95]}"(C[1]), "+{a[96:111]}"(X[0]), "+{a[112:127]}"(X[1]),
                 "+{s[40:41]}"(k3), "+{s[42:43]}"(v3), "+{s[44:45]}"(uk3), "+{s[46:47]}"(uv3)
               : "{a[128:131]}"(bq[0]), "{a[132:135]}"(buq[0]), "{a[136:139]}"(bdo[0]), "{a[140:143]}"(bq[1]),
                 "{a[144:147]}"(buq[1]), "{a[148:151]}"(bdo[1]), "{a[152:155]}"(bq[2]), "{a[156:159]}"(buq[2]),
                 "{a[160:163]}"(bdo[2]), "{a[164:167]}"(bq[3]), "{a[168:171]}"(buq[3]), "{a[172:175]}"(bdo[3]),
                 "{v252}"(lq), "{v253}"(dq), "{v243}"(coff), "{v244}"(r0), "{v245}"(r1), "{v246}"(r2),
                 "{v247}"(r3), "{v248}"(t0), "{v249}"(t1), "{v250}"(t2), "{v251}"(t3), "{s48}"(ldsw),
                 "{s49}"(ns_all), "{s51}"(ns)
               : FB_PASS1_ASM_CLOBBERS);
}

}  // namespace fb
