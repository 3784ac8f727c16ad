// stream_sched.h — the stream-K schedule of the streaming GEMM as pure integer
// functions (host and device).
//
// The (tile, block) steps i = t * KB + j, 0 <= i < I = T * KB, are cut into V
// contiguous ranges [first(v), first(v+1)) with first(v) = floor(v I / V);
// V <= I so no range is empty.  A range's part of a tile is a "segment"; a
// segment that does not cover the whole tile leaves a partial result in one of
// the range's two partial slots: slot 2v if the segment starts inside the tile
// (it is the range's first segment), else slot 2v + 1 (it ends inside the tile:
// the range's last segment).
//
// The functions are templates on the integer type: the host uses int64_t; the
// kernel uses uint32_t, which is exact while V * I < 2^31 (checked by the host).
#pragma once
#include <stdint.h>

#include "layout.h"

namespace qg {

template <class U>
QG_HD U range_first(U v, U V, U I) { return v * I / V; }

// the range holding step i
template <class U>
QG_HD U range_owner(U i, U V, U I) { return ((i + 1) * V + I - 1) / I - 1; }

// ranges holding a piece of tile t: tile_first_owner .. tile_last_owner
template <class U>
QG_HD U tile_first_owner(U t, U KB, U V, U I) { return range_owner<U>(t * KB, V, I); }
template <class U>
QG_HD U tile_last_owner(U t, U KB, U V, U I) { return range_owner<U>((t + 1) * KB - 1, V, I); }

// partial slot of range q's segment of tile t (the segment must be partial)
template <class U>
QG_HD U partial_slot(U q, U t, U KB, U V, U I) {
  return (range_first<U>(q, V, I) > t * KB) ? 2 * q : 2 * q + 1;
}

// Activations of a range of steps [i0, i1) of a matrix with KB blocks per tile
// row: the range touches min(i1 - i0, KB) distinct blocks, and block j sits in
// slot (j - j0) mod KB of the workgroup's activation area, j0 = i0 mod KB.
template <class U>
QG_HD U x_slots(U i0, U i1, U KB) { return (i1 - i0 < KB) ? (i1 - i0) : KB; }

}  // namespace qg
