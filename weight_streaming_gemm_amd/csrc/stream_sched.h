// stream_sched.h — the stream-K schedule of the streaming GEMM as pure integer
// functions (host and device).
//
// The (tile, block) steps i = t * KB + j, 0 <= i < I = T * KB, are cut into P
// contiguous ranges [first(p), first(p+1)) with first(p) = floor(p I / P);
// P <= I so no range is empty.  A workgroup's part of a tile is a "segment";
// a segment that does not cover the whole tile leaves a partial result in one
// of the workgroup's two partial slots: slot 2p if the segment starts inside
// the tile (it is the workgroup's first segment), else slot 2p + 1 (it ends
// inside the tile: the workgroup's last segment).
#pragma once
#include <stdint.h>

#include "layout.h"

namespace qg {

QG_HD int64_t range_first(int64_t p, int64_t P, int64_t I) { return p * I / P; }

// the workgroup whose range holds step i
QG_HD int64_t range_owner(int64_t i, int64_t P, int64_t I) { return ((i + 1) * P + I - 1) / I - 1; }

// workgroups holding a piece of tile t: q_lo .. q_hi
QG_HD int64_t tile_first_owner(int64_t t, int64_t KB, int64_t P, int64_t I) { return range_owner(t * KB, P, I); }
QG_HD int64_t tile_last_owner(int64_t t, int64_t KB, int64_t P, int64_t I) { return range_owner((t + 1) * KB - 1, P, I); }

// partial slot of workgroup q's segment of tile t (the segment must be partial)
QG_HD int64_t partial_slot(int64_t q, int64_t t, int64_t KB, int64_t P, int64_t I) {
  return (range_first(q, P, I) > t * KB) ? 2 * q : 2 * q + 1;
}

}  // namespace qg
