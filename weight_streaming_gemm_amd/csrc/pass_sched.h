// pass_sched.h — the schedule of the persistent pass kernel (pass.hip) as pure
// integer functions, compiled for host and device.
//
// One launch runs a sequence of GEMMs; every workgroup (one per compute unit, P
// in all) takes part in every GEMM.  A GEMM with NS 16-output sub-tiles and KB
// 256-weight blocks is cut along K into S chunks of kbc = KB / S blocks; a unit
// is one sub-tile over one chunk (kbc block steps).  Chunk c is dealt to the
// workgroups [first_cu(c), first_cu(c + 1)), which share its NS units as
// contiguous runs of whole units (their counts differ by at most one; which
// workgroups get the longer runs rotates from GEMM to GEMM).  So a workgroup
// needs the activations of one chunk only, and a unit is never split between
// workgroups: only the chunks of a sub-tile meet across workgroups.
//
// Inside a workgroup the compute waves split its steps (unit-major: step i is
// block i mod kbc of unit i / kbc) into NC contiguous equal sub-ranges.  A wave
// leaves one piece (its partial 16 x 16 tile) per unit its sub-range touches;
// the pieces of a unit are added in wave order.
#pragma once
#include <stdint.h>

#include "layout.h"

namespace qg {

// chunk of workgroup p (chunk c takes workgroups floor(c P / S) .. floor((c + 1) P / S) - 1)
QG_HD int pass_chunk_of(int p, int S, int P) { return (int)(((int64_t)(p + 1) * S - 1) / P); }
QG_HD int pass_first_cu(int c, int S, int P) { return (int)((int64_t)c * P / S); }

// the units [*ns0, *ns1) of workgroup p in its chunk *c (sub-tiles of that chunk)
QG_HD void pass_units(int p, int S, int P, int NS, int rot, int* c, int* ns0, int* ns1) {
  const int cc = pass_chunk_of(p, S, P);
  const int lo = pass_first_cu(cc, S, P), hi = pass_first_cu(cc + 1, S, P);
  const int pc = hi - lo;                                  // workgroups of the chunk (>= 1 when S <= P)
  const int q = (p - lo + pc - rot % pc) % pc;             // rotated place among them
  const int base = NS / pc, extra = NS % pc;
  const int a = q * base + (q < extra ? q : extra);
  *c = cc;
  *ns0 = a;
  *ns1 = a + base + (q < extra ? 1 : 0);
}

// Share weights of the compute waves: waves w and w + NC/2 run on one SIMD,
// where the older wave (lower index) is issued first and, with equal shares,
// ends 1-5 us before the younger one; the first half of the waves takes
// PASS_W_OLD parts of a workgroup's steps to PASS_W_YOUNG for the second half
// (9 : 7 measured best of 1 : 1, 8 : 7, 11 : 9, 9 : 7, 7 : 5, 10 : 7, 5 : 3).
#ifndef PASS_W_OLD
#define PASS_W_OLD 9
#define PASS_W_YOUNG 7
#endif
// first step of wave w's sub-range when n steps are split over NC waves
QG_HD int pass_wave_first(int w, int NC, int n) {
  const int h = NC / 2;
  const int64_t cum = w <= h ? (int64_t)PASS_W_OLD * w : (int64_t)PASS_W_OLD * h + (int64_t)PASS_W_YOUNG * (w - h);
  const int64_t total = (int64_t)PASS_W_OLD * h + (int64_t)PASS_W_YOUNG * (NC - h);
  return (int)((int64_t)n * cum / total);
}
// the wave whose sub-range holds step i (0 <= i < n): the last wave whose
// sub-range starts at or before i (waves with empty sub-ranges start where the
// next one does)
QG_HD int pass_step_owner(int i, int NC, int n) {
  int w = NC - 1;
  while (w > 0 && pass_wave_first(w, NC, n) > i) --w;
  return w;
}

// LDS layout of one block's activations for R rows (a slot): rows are taken
// in pairs (R2 = R rounded up to even; a missing last row is converted like the
// others and never read).  Row r's 32 binary16 A operands sit at PASS_X_ROW r
// (operand (gg, t) at 16 (8 gg + t); the 16-byte pad per row puts the rows of
// one step on different banks), then the 8 R fp32 sub-block sums at
// PASS_X_ROW R2.  The raw bf16 rows land in the same slot first (row pair q
// at 2 PASS_X_ROW q, row 2 q + h at 512 h further, under its own operands) and
// each pair is converted in place.
constexpr int PASS_X_ROW = 528;
QG_HD int pass_x_rows(int R) { return R + (R & 1); }
QG_HD int pass_x_block_bytes(int R) { return PASS_X_ROW * pass_x_rows(R) + 32 * R; }

// K chunks of a GEMM with KB blocks at R rows over P workgroups: the fewest
// (dividing KB, at most max_chunks and at most P) whose activations fit x_area
// bytes of LDS; 0 when none does
QG_HD int pass_chunks(int KB, int R, int P, int x_area, int max_chunks) {
  for (int S = 1; S <= max_chunks && S <= P && S <= KB; ++S)
    if (KB % S == 0 && (int64_t)(KB / S) * pass_x_block_bytes(R) <= x_area) return S;
  return 0;
}

// Compute wave w of workgroup p in a GEMM (NS sub-tiles, KB blocks, S chunks of
// kbc, rotation rot): its count of steps, its first packed step (sub-tile * KB +
// block) and first block within the chunk
QG_HD void pass_wave_share(int p, int w, int NC, int P, int NS, int KB, int S, int kbc, int rot, int* count,
                           int* step0, int* jj0) {
  int c, ns0, ns1;
  pass_units(p, S, P, NS, rot, &c, &ns0, &ns1);
  const int n = (ns1 - ns0) * kbc;
  const int a = pass_wave_first(w, NC, n), b = pass_wave_first(w + 1, NC, n);
  *count = b - a;
  const int ns = ns0 + a / kbc, jj = a % kbc;
  *step0 = b > a ? ns * KB + c * kbc + jj : 0;
  *jj0 = b > a ? jj : 0;
}

// Gated input: K chunk c (kbc blocks per chunk) of a GEMM whose input column j
// depends on outputs j and half + j of the previous GEMM (half = K / 16 input
// sub-tiles, i.e. the previous GEMM's sub-tiles [16 kbc c, 16 kbc (c + 1)) and
// the same + half).  w[0..3] = bitmask of the workgroups (P <= 256) whose units
// of the previous GEMM (NSp sub-tiles, Sp chunks, rotation rot_p) hold any of
// them: the workgroups the chunk waits for.
QG_HD void pass_gated_mask(int c, int kbc, int half, int P, int NSp, int Sp, int rot_p, uint64_t w[4]) {
  const int lo = 16 * kbc * c, hi = 16 * kbc * (c + 1);
  w[0] = w[1] = w[2] = w[3] = 0;
  for (int q = 0; q < P && q < 256; ++q) {
    int cq, ns0, ns1;
    pass_units(q, Sp, P, NSp, rot_p, &cq, &ns0, &ns1);
    if ((ns0 < hi && ns1 > lo) || (ns0 < hi + half && ns1 > lo + half)) w[q / 64] |= 1ull << (q % 64);
  }
}

}  // namespace qg
