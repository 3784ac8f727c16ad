// prefill_plan.h — the row-tiled kernel's plan and activation-image layout as
// pure integer functions (host and device), shared by the kernels, the host
// library and the CPU replay of the kernel's data flow.
//
// A workgroup covers MT = WM RTW row tiles of 16 rows and WN sub-tile pairs of
// 32 outputs (WM x WN waves, each RTW row tiles x PF_U sub-tiles).  x is
// converted once into an image of 1 KiB chunks, one (row tile group m, block j)
// after another: chunk 8 rt + t holds the binary16 A operands of row tile rt,
// step t (lane 16 g + r at 16 bytes each: row 16 (MT m + rt) + r, k = 256 j + 64 g
// + 32 (e & 1) + 4 t + (e >> 1) for element e), chunk 8 MT + rt the sub-block-sum
// operands of row tile rt.
#pragma once
#include <stdint.h>
#include <stddef.h>

#include "layout.h"

namespace qg {

constexpr int PF_U = 2;                        // output sub-tiles per wave
constexpr int PF_CHUNK = 64 * 16;              // one image chunk: 64 lanes x 16 B

// bytes of one (row tile group, block) of the image for MT row tiles
QG_HD constexpr int pf_buf(int MT) { return 9 * MT * PF_CHUNK; }
// byte offset of chunk c of (row tile group m, block j)
QG_HD int64_t pf_chunk_off(int64_t m, int64_t j, int64_t KB, int MT, int c) {
  return (m * KB + j) * (int64_t)pf_buf(MT) + (int64_t)c * PF_CHUNK;
}
QG_HD int pf_operand_chunk(int rt, int t) { return 8 * rt + t; }
QG_HD int pf_sum_chunk(int MT, int rt) { return 8 * MT + rt; }

// Grid: mt row tile groups (16 wm rtw rows) x nt output tiles (32 wn outputs)
// x S chunks of K (kc blocks each).  The workspace (ws_bytes) holds the image
// (img_bytes) and, with S > 1, the chunks' partial outputs, slices of R x N fp32
// `slice` floats apart, which a last kernel adds in chunk order.
struct PrefillPlan {
  int wm, wn, rtw;
  int64_t mt, nt, S, kc, slice;
  size_t img_bytes, ws_bytes;
};

// The wave grid (WM x WN waves of RTW row tiles: 2 x 4 and 2 x 6 of 4, 1 x 8 of
// 4, or, up to 32 rows, 1 x 8 of 2 with two workgroups per CU) and K in chunks (of at least 8
// blocks) while the grid is below the resident workgroups.  The grid with the
// lowest estimated time is taken: rounds of resident workgroups times the work
// of one (rows x outputs x kc blocks) times the workgroups sharing a CU, over
// the grid's measured relative speed.
inline PrefillPlan prefill_plan(int64_t N, int64_t K, int R, int cus) {
  const int64_t NS = padded_n(N) / TILE_N, KB = K / SB_W;
  PrefillPlan best{};
  double best_cost = 0.0;
  // {WM, WN, RTW, workgroups per CU, relative speed}
  const double grids[4][5] = {{2, 4, 4, 1, 1.0}, {2, 6, 4, 1, 1.12}, {1, 8, 4, 1, 1.0}, {1, 8, 2, 2, 1.0}};
  for (int gi = 0; gi < 4; ++gi) {
    const int wm = (int)grids[gi][0], wn = (int)grids[gi][1], rtw = (int)grids[gi][2], occ = (int)grids[gi][3];
    // two row tiles per wave decode every weight for half the products: only
    // where a 64-row tile would leave at least half its rows idle
    if (rtw == 2 && R > 32) continue;
    PrefillPlan p{};
    p.wm = wm;
    p.wn = wn;
    p.rtw = rtw;
    const int rows = wm * rtw * 16;
    p.mt = (R + rows - 1) / rows;
    p.nt = (NS + wn * PF_U - 1) / (wn * PF_U);
    const int64_t slots = (int64_t)cus * occ;
    int64_t S = 1;
    while (p.mt * p.nt * S * 2 <= slots && KB / (S * 2) >= 8) S *= 2;
    p.kc = (KB + S - 1) / S;
    p.S = (KB + p.kc - 1) / p.kc;
    const int64_t rounds = (p.mt * p.nt * p.S + slots - 1) / slots;
    const double cost = (double)rounds * occ * (double)rows * (wn * PF_U * 16) * (double)p.kc / grids[gi][4];
    if (gi == 0 || cost < best_cost) {
      best = p;
      best_cost = cost;
    }
  }
  best.img_bytes = (size_t)best.mt * (size_t)KB * (size_t)pf_buf(best.wm * best.rtw);
  best.slice = ((int64_t)R * N + 3) / 4 * 4;       // slices rounded up to 16 bytes
  best.ws_bytes = best.img_bytes + (best.S > 1 ? (size_t)best.S * (size_t)best.slice * 4 : 0);
  return best;
}

}  // namespace qg
