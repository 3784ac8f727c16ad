// qgemm_kernels.hip — gfx950 kernels of the weight-streaming Q4_K-style GEMM.
//
// The method (OpenJet multi-agent serving page, section on moving the weights
// only once): the quantised weights are streamed from HBM once per decode step
// and every weight that arrives is applied to all R stacked activation rows, so
// a step costs one weight read whatever R is.  Here that is
//
//   y[r, n] = sum_k w[n, k] x[r, k],  w[n, k] = d sc_s q_k - dmin m_s
//
// computed per 256-weight block (d, dmin, sc_s, m_s of output n) as
//
//   y[r, n] += d * sum_k (sc_s q_k) x[r, k]  -  dmin * sum_k m_s x[r, k]
//
// sc_s q_k (<= 945) and m_s (<= 63) are integers, exact in binary16, so both
// sums run on the fp16 matrix cores (v_mfma_f32_16x16x32_f16) with exact
// products and fp32 accumulation; d and dmin are applied in fp32 once per
// block.  x enters the matrix cores as binary16, which holds every bf16 value
// of magnitude in [2^-17, 65504] exactly.
//
// Layouts: layout.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "layout.h"
#include "operand.h"
#include "stream_sched.h"
#include "qgemm_internal.h"

namespace qg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ WConst header_consts(u32x4 h, int g) { return header_consts(h.x, h.y, h.z, h.w, g); }

// ---------------------------------------------------------------------------
// canonical -> packed (one thread per (sub-tile, block, lane))
__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ packed, int64_t N,
            int64_t KB, int64_t NS) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = NS * KB * 64;
  if (tid >= total) return;
  int lane = (int)(tid & 63);
  int64_t pair = tid >> 6;           // ns * KB + j
  int64_t ns = pair / KB, j = pair % KB;
  int g = lane >> 4, nl = lane & 15;
  int64_t n = ns * TILE_N + nl;
  uint8_t blk[SB_CANON];
  if (n < N) {
    const uint8_t* src = canon + (n * KB + j) * SB_CANON;
    // canonical blocks are 16-byte aligned (144 = 9 * 16) when the base is
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    for (int i = 0; i < SB_CANON / 16; ++i) {
      u32x4 v = s4[i];
      for (int b = 0; b < 4; ++b) {
        uint32_t wv = v[b];
        blk[16 * i + 4 * b + 0] = (uint8_t)(wv);
        blk[16 * i + 4 * b + 1] = (uint8_t)(wv >> 8);
        blk[16 * i + 4 * b + 2] = (uint8_t)(wv >> 16);
        blk[16 * i + 4 * b + 3] = (uint8_t)(wv >> 24);
      }
    }
  } else {
    for (int i = 0; i < SB_CANON; ++i) blk[i] = 0;
  }
  uint8_t* qdst = packed + quant_chunk_off(ns, j, KB) + lane * 16;
  for (int h = 0; h < 2; ++h) {
    u32x4 o;
    for (int u = 0; u < 4; ++u) o[u] = pack_quant_dword(blk, g, 4 * h + u);
    *reinterpret_cast<u32x4*>(qdst + h * 1024) = o;
  }
  if (g == 0) {
    uint32_t hd[4];
    pack_header(blk, hd);
    uint8_t* hdst = packed + quant_region_bytes(NS * TILE_N, KB * SB_W) + header_chunk_off(ns, j, KB) + nl * 16;
    *reinterpret_cast<u32x4*>(hdst) = u32x4{hd[0], hd[1], hd[2], hd[3]};
  }
}


// ---------------------------------------------------------------------------
// The streaming kernel.
//
// Work.  The NW waves of a workgroup form an nwn x (NW / nwn) grid: nwn side by
// side along N, NW / nwn along K (nwn is chosen per GEMM).  A tile is nwn * NT
// 16-output sub-tiles; tile t needs KB block steps.  The T * KB (tile, block)
// steps of a GEMM are cut into V = P contiguous ranges, one per workgroup (one
// workgroup per CU): equal ranges (stream-K: every CU streams the same bytes
// whatever the matrix shape), or ranges of whole tiles when the host finds the
// uneven split cheaper than sharing tiles.  When a tile row of activations does
// not fit in LDS, K is cut into S chunks of KB blocks and the ranges hold whole
// tiles of one chunk ("virtual" tiles c * treal + t).  Inside a range, each row
// of nwn waves takes an equal contiguous sub-range, each wave its NT sub-tiles
// of every tile.
//
// Sums.  A wave writes a tile it covers alone straight to y.  The pieces of a
// tile shared by several waves meet in LDS and are added, after the range, in
// wave order.  A tile shared with other ranges leaves the workgroup's sum in a
// global partial slot; the last range to finish the tile adds the slots in
// range order (with K chunks: the chunks' partial tiles, in chunk order).
// Every sum has a fixed order, so results are deterministic.
//
// Min term.  Either eight more matrix-core products per step with B = m_s
// (MSUM = false), or, when a range uses each block for several steps, one
// fp16 product per step of the sub-block sums of x, staged with the
// activations as two binary16 parts of X_s / 256 (MSUM = true).  The
// vector-unit variant (VR = R <= 4 rows) replaces the products by dot products
// on the vector units and always uses the sums, staged in fp32.
//
// Streams.  At the start of a range the workgroup converts the activations of
// the blocks the range touches (R rows x 256 bf16 each) into the matrix-core
// operand layout in LDS; the steps then read only weights from memory: per
// step and sub-tile the 2 KiB quant chunk and the outputs' 16-byte headers,
// with raw buffer loads (streaming hint), RING steps ahead in a register ring
// (each slot refilled right after its step) up to the end of the wave's
// sub-range.  Loads past the end of the work address beyond the buffer and
// return zeros without memory traffic.
#ifndef QG_RING
#define QG_RING 4
#endif
constexpr int RING = QG_RING;                  // weight ring depth, steps (4, 6 or 8)
static_assert(RING == 4 || RING == 6 || RING == 8, "the main loop unrolls 4, 6 or 8 steps");
constexpr uint32_t OOB = 0x80000000u;          // beyond every buffer (sizes < 2^31)
constexpr int SC1 = 16;                        // cache policy: coherent across the device

// aux 2 = streaming (non-temporal) hint for data read once; 0 for shared data
template <class T, int AUX>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(T) == 16)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, AUX));
}
__device__ __forceinline__ void bstore_sc1(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, SC1);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// the sum of four bf16 values (two dwords) in fp32, with two dot products against ones
// The matrix-core min term's sub-block sums: X_s / 256 (in binary16's range for
// |x| <= 65504) in two binary16 parts, hi = f16(X_s / 256) and lo = f16(X_s / 256
// - hi) (the difference exact in fp32): lane group g holds (hi_2g, hi_2g+1,
// lo_2g, lo_2g+1) of its row and B = (m_2g, m_2g+1, m_2g, m_2g+1) of its output,
// so one 16 x 16 x 16 product adds m_s (hi + lo) over the 8 sub-blocks; the 256
// goes back into -dmin (exact).
__device__ __forceinline__ f16x4 sum_parts(float s0, float s1) {
  const float a0 = s0 * (1.0f / 256.0f), a1 = s1 * (1.0f / 256.0f);
  const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
  return f16x4{h0, h1, (_Float16)(a0 - (float)h0), (_Float16)(a1 - (float)h1)};
}
__device__ __forceinline__ f16x4 min_parts_b(const WConst& c) { return f16x4{c.m[0], c.m[1], c.m[0], c.m[1]}; }
__device__ __forceinline__ float sum4_bf16(uint32_t d0, uint32_t d1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  const float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d0), one, 0.0f, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d1), one, s, false);
}

// v from the lane picked by the data-parallel-primitive control CTRL
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// the value of the first active lane: for values that are uniform by
// construction, so that the compiler keeps them (and branches on them) scalar
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int NT>
struct WStage {
  u32x4 qa[NT], qb[NT], hd[NT];
};

// where a wave stands in its sequence of steps (uniform across the wave)
struct Cursor {
  int g;          // 0 for the launch's GEMM; 1 past the end
  int v;          // range index
  int A, B;       // the range's steps
  int it, it1;    // current step and end of this wave's sub-range
  int t, j;       // tile and block of step it
  int tr, jb;     // output tile and first block of tile t's chunk (K in chunks)
  int KB, NS, I, V, T;
  int aligned, S, kbr, treal;
  int nwn, wn, wk, nwk;            // wave grid of GEMM g and this wave's place in it
  __amdgpu_buffer_rsrc_t qr, hr;   // quant and header regions of GEMM g (load cursor)
};

// VR > 0: the vector-unit variant for exactly VR rows (RT = NT = 1, MSUM): dot
// products of the binary16 operands on the vector units instead of the matrix
// cores, one lane per (output, lane group), reduced over the 4 lane groups at
// the end of each segment into the matrix-core accumulator layout.
constexpr int VROWS = 4;

template <int RT, int NT, int NW, bool MSUM, int VR = 0>
__global__ void __launch_bounds__(NW * 64, NW / 4)
stream_kernel(StreamArgs a) {
  constexpr bool VALU = VR > 0;
  static_assert(VR <= VROWS && (!VALU || (RT == 1 && NT == 1 && MSUM)), "vector-unit variant: one row tile");
  constexpr int NTHR = NW * 64;
  constexpr int XAREA = x_area_bytes(RT, NT, NW);
  __shared__ __attribute__((aligned(16))) uint8_t xlds[XAREA];
  __shared__ f32x4 pieces[NW * 2 * NT * RT * 64];
  __shared__ uint32_t s_last[2];
  __shared__ uint8_t s_chunk_last[NTHR];         // K in chunks: last arrivals of a range's tiles

  const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6), g4 = lane >> 4, nl = lane & 15;
  const int p = blockIdx.x, P = a.P, R = a.R;
  constexpr int G = 1;                            // one GEMM per launch
  const int XT = 64 * R + 16;                     // LDS bytes of one step's activations
  const int XS = 8 * XT;                          // offset of a block's sub-block sums
  const int SB = XS + (MSUM ? 8 * 4 * R : 0);     // LDS bytes of one block's activations

  auto get_desc = [&](int) __attribute__((always_inline)) -> GemmDesc { return a.d0; };
  // range v of the cursor's GEMM and this wave's sub-range of it
  auto set_range = [&](Cursor& c) __attribute__((always_inline)) {
    if (c.aligned) {
      c.A = uni(c.KB * (int)range_first<uint32_t>(c.v, c.V, c.T));
      c.B = uni(c.KB * (int)range_first<uint32_t>(c.v + 1, c.V, c.T));
    } else {
      c.A = uni((int)range_first<uint32_t>(c.v, c.V, c.I));
      c.B = uni((int)range_first<uint32_t>(c.v + 1, c.V, c.I));
    }
    c.it = uni(c.A + (int)range_first<uint32_t>(c.wk, c.nwk, c.B - c.A));
    c.it1 = uni(c.A + (int)range_first<uint32_t>(c.wk + 1, c.nwk, c.B - c.A));
    c.t = uni(c.it / c.KB);
    c.j = uni(c.it - c.t * c.KB);
    const int cc = uni(c.t / c.treal);
    c.tr = uni(c.t - cc * c.treal);
    c.jb = uni(cc * c.KB);
  };
  // the cursor's tile advances by one (and into the next chunk after the last tile)
  auto next_tile = [&](Cursor& c) __attribute__((always_inline)) {
    c.t = uni(c.t + 1);
    c.tr = uni(c.tr + 1);
    if (c.tr == c.treal) { c.tr = 0; c.jb = uni(c.jb + c.KB); }
  };
  auto enter = [&](Cursor& c, int g) __attribute__((always_inline)) {
    c.g = g;
    if (g >= G) {
      c.v = 0; c.V = 1; c.A = c.B = 0;
      c.it = 1; c.it1 = 0;
      c.t = 0; c.j = 0; c.KB = 1; c.NS = 0; c.I = 0; c.T = 0; c.aligned = 0;
      c.tr = 0; c.jb = 0; c.S = 1; c.kbr = 1; c.treal = 1;
      c.nwn = 1; c.wn = 0; c.wk = w; c.nwk = NW;
      c.qr = make_rsrc(nullptr, 0);
      c.hr = make_rsrc(nullptr, 0);
      return;
    }
    const GemmDesc d = get_desc(g);
    c.v = p;
    c.V = d.V;
    c.KB = d.KB;
    c.NS = d.NS;
    c.I = d.I;
    c.T = d.T;
    c.aligned = d.aligned;
    c.S = d.S;
    c.kbr = d.kbr;
    c.treal = d.treal;
    c.nwn = d.nwn;
    c.nwk = uni(NW / d.nwn);
    c.wn = uni(w % d.nwn);
    c.wk = uni(w / d.nwn);
    c.qr = make_rsrc(d.packed, d.quant_bytes);
    c.hr = make_rsrc(d.packed + d.quant_bytes, d.hdr_bytes);
    set_range(c);
  };
  // the load cursor's next step: the next one of this wave's sub-range; past its
  // end none (the loads return zeros without memory traffic)
  auto next = [&](Cursor& c) __attribute__((always_inline)) {
    c.it = uni(c.it + 1);
    c.j = uni(c.j + 1);
    if (c.j == c.KB) { c.j = 0; next_tile(c); }
  };

  // ---- weights: RING steps ahead -----------------------------------------------
  auto load_w = [&](WStage<NT>& st, const Cursor& c) __attribute__((always_inline)) {
    for (int u = 0; u < NT; ++u) {
      const int ns = (c.tr * c.nwn + c.wn) * NT + u;
      const bool ok = c.it < c.it1 && ns < c.NS;
      const uint32_t qo = ok ? (uint32_t)(ns * c.kbr + c.jb + c.j) * CHUNK_Q + lane * 16 : OOB;
      const uint32_t ho = ok ? (uint32_t)(ns * c.kbr + c.jb + c.j) * CHUNK_H + nl * 16 : OOB;
      st.qa[u] = bload<u32x4, 2>(c.qr, qo);
      st.qb[u] = bload<u32x4, 2>(c.qr, qo + 1024);
      st.hd[u] = bload<u32x4, 2>(c.hr, ho);
    }
  };

  // ---- activations of a range: block j = (j0 + b) mod KB goes to slot b.  A slot
  // holds 8 steps t of XT = 64 R + 16 bytes (the pad puts consecutive steps on
  // different LDS banks); in step t, lane group gg and row r hold the A operand
  // of lane 16 gg + r % 16 of row tile r / 16, built from x[r, 256 j + 64 gg +
  // 4 t + {0..3}] and the same 32 further on.  32 threads per (slot, row), XB
  // rows in flight per thread, the rows taken in an order rotated by the
  // workgroup index (all workgroups read the same activations).  The loads of
  // the first batch are issued on their own (x_load) so that the kernel can
  // queue them ahead of the weight ring. ---
  constexpr int XGROUPS = NTHR / 32, XB = 16;
  u32x2 xlo[XB], xhi[XB];
  // (slot, row) of this thread's k-th row of the batch at base, rows = nslots R;
  // slots rotated by the workgroup index.  Walked incrementally: one division.
  struct XRow { int b, r; };
  auto x_rows = [&](int nslots, int base, XRow (&o)[XB]) __attribute__((always_inline)) {
    const int qg = XGROUPS / R, mg = XGROUPS - qg * R;
    int b = base / R, r = base - b * R;
    b += p % nslots;
    for (int k = 0; k < XB; ++k) {
      o[k].b = b >= nslots ? b - nslots : b;     // b < 2 nslots while the row is valid
      o[k].r = r;
      r += mg;
      b += qg;
      if (r >= R) { r -= R; ++b; }
    }
  };
  auto x_load = [&](const GemmDesc& d, int jbase, int j0, int nslots, int base) __attribute__((always_inline)) {
    const int sub = tid & 31, gg = sub >> 3, t = sub & 7;
    const int K = d.kbr * SB_W;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(d.x, (uint32_t)(R * K * 2));
    const int rows = nslots * R;
    XRow rw[XB];
    x_rows(nslots, base, rw);
    for (int k = 0; k < XB; ++k) {
      const int rb = base + k * XGROUPS;
      int j = j0 + rw[k].b;
      if (j >= d.KB) j -= d.KB;
      const uint32_t off = (uint32_t)((rw[k].r * K + (jbase + j) * SB_W + 64 * gg + 4 * t) * 2);
      xlo[k] = bload<u32x2, 0>(xr, rb < rows ? off : OOB);
      xhi[k] = bload<u32x2, 0>(xr, rb < rows ? off + 64 : OOB);
    }
  };
  auto x_store = [&](int nslots, int base) __attribute__((always_inline)) {
    const int sub = tid & 31, gg = sub >> 3, t = sub & 7;
    const int rows = nslots * R;
    XRow rw[XB];
    x_rows(nslots, base, rw);
    for (int k = 0; k < XB; ++k) {
      const int rb = base + k * XGROUPS;
      if (rb >= rows) break;
      const f16x8 op = build_a(xlo[k].x, xlo[k].y, xhi[k].x, xhi[k].y);
      *reinterpret_cast<f16x8*>(xlds + rw[k].b * SB + t * XT + (gg * R + rw[k].r) * 16) = op;
      if constexpr (MSUM) {
        // sub-block sums: the 8 threads t of lane group gg (8 consecutive lanes) add
        // their run sums as ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7))
        float s0 = sum4_bf16(xlo[k].x, xlo[k].y), s1 = sum4_bf16(xhi[k].x, xhi[k].y);
        s0 += dpp_f32<0xB1>(s0); s1 += dpp_f32<0xB1>(s1);    // lane ^ 1
        s0 += dpp_f32<0x4E>(s0); s1 += dpp_f32<0x4E>(s1);    // lane ^ 2
        s0 += dpp_f32<0x104>(s0); s1 += dpp_f32<0x104>(s1);  // lane + 4 (for lane t = 0)
        if (t == 0) {
          // fp32 for the vector-unit variant's multiply-adds, two binary16 parts for the matrix cores
          if constexpr (VALU)
            *reinterpret_cast<f32x2*>(xlds + rw[k].b * SB + XS + (gg * R + rw[k].r) * 8) = f32x2{s0, s1};
          else
            *reinterpret_cast<f16x4*>(xlds + rw[k].b * SB + XS + (gg * R + rw[k].r) * 8) = sum_parts(s0, s1);
        }
        // one row at a time: few values live while the weight ring is in flight
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // the rest of a range's conversion once its first batch is loaded
  auto x_convert_rest = [&](const GemmDesc& d, int jbase, int j0, int nslots) __attribute__((always_inline)) {
    const int rows = nslots * R;
    x_store(nslots, tid >> 5);
    for (int base = (tid >> 5) + XB * XGROUPS; base < rows; base += XB * XGROUPS) {
      x_load(d, jbase, j0, nslots, base);
      x_store(nslots, base);
    }
  };
  // this lane's A-operand offsets inside a slot, per row tile.  A row >= R of a
  // row tile takes row R - 1's operand: a row of A only reaches the same row of
  // the product, and rows >= R are never stored.
  int xoff[RT];
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + nl;
    xoff[rt] = (g4 * R + (r < R ? r : R - 1)) * 16;
  }

  f32x4 acc[NT][RT];
  float vacc[VR > 0 ? VR : 1];                    // vector-unit variant: row r of this lane's output
  auto zero_acc = [&]() __attribute__((always_inline)) {
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt) acc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (VALU)
      for (int r = 0; r < VR; ++r) vacc[r] = 0.f;
  };
  // vector-unit variant, end of a segment: add the 4 lane groups' sums of each
  // row ((g0 + g1) + (g2 + g3) in every lane) and take the matrix-core layout:
  // lane (g, n) holds rows 4g .. 4g + 3 of output n
  auto vacc_to_acc = [&]() __attribute__((always_inline)) {
    float tot[VR > 0 ? VR : 1];
    for (int r = 0; r < VR; ++r) {
      float v = vacc[r];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      tot[r] = v;
    }
    for (int i = 0; i < 4; ++i) {
      float v = 0.f;
      for (int r = 0; r < VR; ++r)
        if (r == 4 * g4 + i) v = tot[r];
      acc[0][0][i] = v;
    }
  };

  // the vector-unit step: for each row r < R, the lane's 64 weights (sub-blocks
  // 2g, 2g + 1 of output n) times x as binary16 pairs (v_dot2_f32_f16: exact
  // products, fp32 sums), then d and the min term from the sub-block sums
  auto compute_valu = [&](const WStage<NT>& st, int slot) __attribute__((always_inline)) {
    const WConst c = header_consts(st.hd[0], g4);
    float ds[VR > 0 ? VR : 1];
    for (int r = 0; r < VR; ++r) ds[r] = 0.f;
    const int base = slot * SB;
    for (int t = 0; t < 8; ++t) {
      const uint32_t wd = (t < 4) ? st.qa[0][t] : st.qb[0][t - 4];
      const f16x8 b = build_b(wd, c);
      for (int r = 0; r < VR; ++r) {
        const f16x8 x8 = *reinterpret_cast<const f16x8*>(xlds + base + t * XT + (g4 * R + r) * 16);
        float v = ds[r];
        for (int e = 0; e < 8; e += 2)
          v = __builtin_amdgcn_fdot2(f16x2{b[e], b[e + 1]}, f16x2{x8[e], x8[e + 1]}, v, false);
        ds[r] = v;
      }
    }
    for (int r = 0; r < VR; ++r) {
      // min term of the lane's two sub-blocks: m_2g X_2g + m_2g+1 X_2g+1
      const f32x2 sm = *reinterpret_cast<const f32x2*>(xlds + base + XS + (g4 * R + r) * 8);
      const float mt = __builtin_fmaf(min_operand(c, 0), sm.x, min_operand(c, 1) * sm.y);
      vacc[r] = __builtin_fmaf(c.d, ds[r], vacc[r]);
      vacc[r] = __builtin_fmaf(c.nmin, mt, vacc[r]);
    }
  };

  // MSUM: the min term from the staged sub-block sums (one fp16 product of their two parts),
  // else from the activation operands of the 8 steps (eight products)
  auto compute = [&](const WStage<NT>& st, int slot) __attribute__((always_inline)) {
    constexpr bool msum = MSUM;
    WConst c[NT];
    f16x8 bm[NT];
    f32x4 ds[NT][RT], ms[NT][RT];
    for (int u = 0; u < NT; ++u) {
      c[u] = header_consts(st.hd[u], g4);
      if constexpr (!msum) bm[u] = build_m_full(c[u]);
      for (int rt = 0; rt < RT; ++rt) {
        ds[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        ms[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    const int base = slot * SB;
    for (int t = 0; t < 8; ++t) {
      f16x8 xa[RT];
      for (int rt = 0; rt < RT; ++rt) {
        const int addr = base + t * XT + xoff[rt];
        xa[rt] = *reinterpret_cast<const f16x8*>(xlds + addr);
      }
      for (int u = 0; u < NT; ++u) {
        const uint32_t wd = (t < 4) ? st.qa[u][t] : st.qb[u][t - 4];
        const f16x8 b = build_b(wd, c[u]);
        for (int rt = 0; rt < RT; ++rt) {
          ds[u][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rt], b, ds[u][rt], 0, 0, 0);
          if constexpr (!msum)
            ms[u][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rt], bm[u], ms[u][rt], 0, 0, 0);
        }
      }
    }
    float nmin[NT];
    for (int u = 0; u < NT; ++u) nmin[u] = msum ? c[u].nmin * 256.0f : c[u].nmin;
    if constexpr (msum)
      for (int rt = 0; rt < RT; ++rt) {
        const f16x4 xsum = *reinterpret_cast<const f16x4*>(xlds + base + XS + xoff[rt] / 2);
        for (int u = 0; u < NT; ++u)
          ms[u][rt] = __builtin_amdgcn_mfma_f32_16x16x16f16(xsum, min_parts_b(c[u]), ms[u][rt], 0, 0, 0);
      }
    // acc += d * ds - dmin * ms, two fused multiply-adds per element
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt)
        for (int i = 0; i < 4; ++i) {
          acc[u][rt][i] = __builtin_fmaf(c[u].d, ds[u][rt][i], acc[u][rt][i]);
          acc[u][rt][i] = __builtin_fmaf(nmin[u], ms[u][rt][i], acc[u][rt][i]);
        }
  };

  // ---- outputs ------------------------------------------------------------------
  // sub-tiles (t * nwn + wn) * NT + u of tile t belong to the waves of column wn
  // (through a global-space pointer: a generic store would also count as an LDS
  // access and make every later LDS wait conservative)
  auto write_y = [&](const GemmDesc& d, int t, int wn, const f32x4 (&v)[NT][RT]) __attribute__((always_inline)) {
    typedef float __attribute__((address_space(1))) global_float;
    global_float* const y = (global_float*)d.y;
    for (int u = 0; u < NT; ++u) {
      const int n = ((t * d.nwn + wn) * NT + u) * TILE_N + nl;
      if (n >= d.N) continue;
      for (int rt = 0; rt < RT; ++rt)
        for (int i = 0; i < 4; ++i) {
          const int r = rt * 16 + 4 * g4 + i;
          if (r < R) y[(int64_t)r * d.N + n] = v[u][rt][i];
        }
    }
  };
  // the result of tile t (column wn) of the cursor's GEMM: y, or with K in
  // chunks the chunk's partial result, in slot t of the partial buffer
  auto tile_result = [&](const Cursor& c, const GemmDesc& d, int t, int wn, const f32x4 (&v)[NT][RT])
      __attribute__((always_inline)) {
    if (c.S == 1) {
      write_y(d, t, wn, v);
    } else {
      const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, (uint32_t)(c.T * c.nwn * NT * RT * 1024));
      for (int u = 0; u < NT; ++u)
        for (int rt = 0; rt < RT; ++rt)
          bstore_sc1(v[u][rt], pr, (uint32_t)(((((t * c.nwn + wn) * NT + u) * RT + rt) * 64 + lane) * 16));
    }
  };
  // LDS piece (sub-range wk, slot sl, column wn): one per wave and slot
  auto piece_at = [&](int nwn, int wk, int sl, int wn, int u, int rt) __attribute__((always_inline)) -> f32x4& {
    return pieces[(((((wk * 2 + sl) * nwn + wn) * NT + u) * RT + rt) * 64) + lane];
  };
  // a wave's segment of tile C.t ends: y if it covers the tile, else a piece in
  // LDS slot 0 (the segment starts inside the tile) or 1
  auto finish_segment = [&](const Cursor& c, const GemmDesc& d, int ja, int a_w) __attribute__((always_inline)) {
    if (ja == 0 && c.j == c.KB - 1) {
      tile_result(c, d, c.t, c.wn, acc);
      return;
    }
    const int sl = (a_w > c.t * c.KB) ? 0 : 1;
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt) piece_at(c.nwn, c.wk, sl, c.wn, u, rt) = acc[u][rt];
  };

  // the partial slots of the current GEMM: 2 V of nwn * NT * RT KiB
  auto part_rsrc = [&](const Cursor& c) __attribute__((always_inline)) {
    return make_rsrc(a.part, (uint32_t)(2 * c.V * c.nwn * NT * RT * 1024));
  };
  auto gslot_off = [&](const Cursor& c, int slot, int wn, int u, int rt) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(((((slot * c.nwn + wn) * NT + u) * RT + rt) * 64 + lane) * 16);
  };
  // the last range to arrive at tile t adds the tile's global partial slots in
  // range order and writes y (column wn of the tile)
  auto global_fixup = [&](const Cursor& c, const GemmDesc& d, int t, int wn) __attribute__((always_inline)) {
    const int q_lo = (int)tile_first_owner<uint32_t>(t, c.KB, c.V, c.I);
    const int q_hi = (int)tile_last_owner<uint32_t>(t, c.KB, c.V, c.I);
    const __amdgpu_buffer_rsrc_t pr = part_rsrc(c);
    f32x4 sum[NT][RT];
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt) sum[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // FB slots in flight at a time, added in range order
    constexpr int FB = RT == 1 ? 8 : (RT == 2 ? 4 : 2);
    for (int q0 = q_lo; q0 <= q_hi; q0 += FB) {
      f32x4 v[FB][NT][RT];
      for (int k = 0; k < FB; ++k) {
        const int q = q0 + k;
        const int qs = q <= q_hi ? (int)partial_slot<uint32_t>(q, t, c.KB, c.V, c.I) : 0;
        for (int u = 0; u < NT; ++u)
          for (int rt = 0; rt < RT; ++rt)
            v[k][u][rt] = bload<f32x4, SC1>(pr, q <= q_hi ? gslot_off(c, qs, wn, u, rt) : OOB);
      }
      for (int k = 0; k < FB; ++k)
        if (q0 + k <= q_hi)
          for (int u = 0; u < NT; ++u)
            for (int rt = 0; rt < RT; ++rt) sum[u][rt] += v[k][u][rt];
    }
    write_y(d, t, wn, sum);
  };

  // ---- end of a range: add the pieces of shared tiles (sub-range order), then
  // the tiles shared with other ranges (range order) ------------------------------
  auto close_range = [&](const Cursor& c, const GemmDesc& d) __attribute__((always_inline)) {
    __syncthreads();                              // every piece is in LDS
    const int A = c.A, B = c.B, KB = c.KB, L = B - A, nwn = c.nwn, nwk = c.nwk;
    const int tA = A / KB, tB = (B - 1) / KB;
    const bool cross_a = tA * KB < A, cross_b = (tB + 1) * KB > B;
    // (tile, column) pairs, spread over the waves
    for (int pi = w; pi < (tB - tA + 1) * nwn; pi += NW) {
      const int t = tA + pi / nwn, wn = pi % nwn;
      const int s0 = (t * KB > A ? t * KB : A) - A;                   // the tile's steps in the range,
      const int s1 = ((t + 1) * KB < B ? (t + 1) * KB : B) - A;       // local [s0, s1)
      const int k_lo = (int)range_owner<uint32_t>(s0, nwk, L);
      const int k_hi = (int)range_owner<uint32_t>(s1 - 1, nwk, L);
      const bool crossing = (t == tA && cross_a) || (t == tB && cross_b);
      if (k_lo == k_hi && !crossing) continue;    // one sub-range covered it: already in y
      f32x4 sum[NT][RT];
      for (int u = 0; u < NT; ++u)
        for (int rt = 0; rt < RT; ++rt) sum[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = k_lo; kk <= k_hi; ++kk) {
        const int a_k = A + (int)range_first<uint32_t>(kk, nwk, L);
        const int b_k = A + (int)range_first<uint32_t>(kk + 1, nwk, L);
        if (a_k == b_k) continue;                 // an empty sub-range holds no piece
        const int sl = (a_k > t * KB) ? 0 : 1;
        for (int u = 0; u < NT; ++u)
          for (int rt = 0; rt < RT; ++rt) sum[u][rt] += piece_at(nwn, kk, sl, wn, u, rt);
      }
      if (!crossing) {
        tile_result(c, d, t, wn, sum);
      } else {
        const int gs = (int)partial_slot<uint32_t>(c.v, t, KB, c.V, c.I);
        const __amdgpu_buffer_rsrc_t pr = part_rsrc(c);
        for (int u = 0; u < NT; ++u)
          for (int rt = 0; rt < RT; ++rt) bstore_sc1(sum[u][rt], pr, gslot_off(c, gs, wn, u, rt));
      }
    }
    if (cross_a || cross_b) {
      __builtin_amdgcn_s_waitcnt(0);              // this thread's partial stores are complete
      __syncthreads();
      // lanes 0 and 1 arrive at tiles tA and tB with one atomic instruction
      if (tid < 2) {
        const bool mine = tid == 0 ? cross_a : (cross_b && !(cross_a && tB == tA));
        const int t = tid == 0 ? tA : tB;
        uint32_t is_last = 0;
        if (mine) {
          const uint32_t owners = tile_last_owner<uint32_t>(t, KB, c.V, c.I) - tile_first_owner<uint32_t>(t, KB, c.V, c.I);
          is_last = __hip_atomic_fetch_add(a.cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == owners;
        }
        s_last[tid] = is_last;
      }
      __syncthreads();
      const uint32_t last = s_last[0] | (s_last[1] << 1);
      // the waves of the first nwn columns add the tile's slots (column w)
      if (w < nwn) {
        if (last & 1u) global_fixup(c, d, tA, w);
        if (last & 2u) global_fixup(c, d, tB, w);
      }
      // re-arm the counters for the next launch, after every column has read
      __syncthreads();
      if (tid == 0) {
        if (last & 1u) __hip_atomic_store(a.cnt + tA, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (last & 2u) __hip_atomic_store(a.cnt + tB, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (c.S > 1 && A < B) {
      // K in chunks: the range holds whole tiles of one chunk.  Arrive at each of
      // their output tiles (one thread per tile); the last of the S chunks to
      // arrive adds the S partial results in chunk order and writes y.
      __builtin_amdgcn_s_waitcnt(0);              // this thread's partial stores are complete
      __syncthreads();
      const int cc = tA / c.treal, r0 = tA - cc * c.treal, count = tB - tA + 1;
      if (tid < count) {
        const uint32_t old = __hip_atomic_fetch_add(a.cnt + r0 + tid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_chunk_last[tid] = old == (uint32_t)(c.S - 1) ? 1 : 0;
      }
      __syncthreads();
      const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, (uint32_t)(c.T * nwn * NT * RT * 1024));
      constexpr int FB = RT == 1 ? 8 : (RT == 2 ? 4 : 2);
      for (int pi = w; pi < count * nwn; pi += NW) {
        const int i = pi / nwn, wn = pi - i * nwn;
        if (!s_chunk_last[i]) continue;
        const int tr = r0 + i;
        f32x4 sum[NT][RT];
        for (int u = 0; u < NT; ++u)
          for (int rt = 0; rt < RT; ++rt) sum[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int q0 = 0; q0 < c.S; q0 += FB) {
          f32x4 v[FB][NT][RT];
          for (int k = 0; k < FB; ++k) {
            const int vt = (q0 + k) * c.treal + tr;
            for (int u = 0; u < NT; ++u)
              for (int rt = 0; rt < RT; ++rt)
                v[k][u][rt] = bload<f32x4, SC1>(
                    pr, q0 + k < c.S ? (uint32_t)(((((vt * nwn + wn) * NT + u) * RT + rt) * 64 + lane) * 16) : OOB);
          }
          for (int k = 0; k < FB; ++k)
            if (q0 + k < c.S)
              for (int u = 0; u < NT; ++u)
                for (int rt = 0; rt < RT; ++rt) sum[u][rt] += v[k][u][rt];
        }
        write_y(d, tr, wn, sum);
      }
      __syncthreads();
      if (tid < count && s_chunk_last[tid])
        __hip_atomic_store(a.cnt + r0 + tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();                              // pieces and activations may be reused
  };

  // ---- prologue: the first activation batch, then the weight ring (the load
  // cursor starts RING steps ahead) ---------------------------------------------
  Cursor L, C;
  enter(C, 0);
  GemmDesc D = get_desc(0);
  x_load(D, C.jb, C.A % C.KB, (int)x_slots<uint32_t>(C.A, C.B, C.KB), tid >> 5);
  L = C;
  // The ring's first loads go out before the activations are staged, so that
  // they land meanwhile; with sub-block sums (MSUM) they go out after: the
  // compiler then keeps the ring slots in fixed registers through the step
  // loop, where across the longer staging code it copies them on every pass
  // (which waits for every load in flight).
  WStage<NT> W[RING];
  auto ring_fill = [&]() __attribute__((always_inline)) {
    for (int s = 0; s < RING; ++s) {
      load_w(W[s], L);
      next(L);
    }
  };
  if constexpr (!MSUM) ring_fill();
  int xs = 0;                                     // activation slot of C's step
  int ja = 0;                                     // first block of the current segment
  int a_w = 0;                                    // first step of this wave's sub-range

  // one step at ring position s; true at the end of this wave's sub-range
  auto step = [&](auto S) __attribute__((always_inline)) -> bool {
    constexpr int s = decltype(S)::value;
    if constexpr (VALU)
      compute_valu(W[s], xs);
    else
      compute(W[s], xs);
    // keep the refill after the step's last use of the slot, so that the load
    // writes the slot's own registers (a load hoisted above would need other
    // registers and a copy, which waits for every load in flight)
    __builtin_amdgcn_sched_barrier(0);
    load_w(W[s], L);                              // the slot takes the step RING ahead
    next(L);
    const bool tile_end = C.j == C.KB - 1;
    const bool sub_end = C.it + 1 == C.it1;
    if (tile_end || sub_end) {
      if constexpr (VALU) vacc_to_acc();
      finish_segment(C, D, ja, a_w);
      zero_acc();
      ja = 0;
    }
    if (sub_end) return true;
    C.it = uni(C.it + 1);
    C.j = uni(C.j + 1);
    if (C.j == C.KB) { C.j = 0; next_tile(C); }
    xs = uni(xs + 1);
    if (xs == C.KB) xs = 0;
    return false;
  };

  // One range per workgroup and GEMM (the host sizes V = P).
  // (the first activation batch is already in flight)
  auto start_range = [&]() __attribute__((always_inline)) {
    x_convert_rest(D, C.jb, C.A % C.KB, (int)x_slots<uint32_t>(C.A, C.B, C.KB));
    __syncthreads();
    xs = uni((C.it - C.A) % C.KB);
    ja = C.j;
    a_w = C.it;
    zero_acc();
  };
  // the unrolled step loop (ring slots 0 .. RING-1); true from STEP ends it
  auto run_ring = [&](auto STEP) __attribute__((always_inline)) {
    for (;;) {
      if (STEP(std::integral_constant<int, 0>{})) break;
      if (STEP(std::integral_constant<int, 1>{})) break;
      if (STEP(std::integral_constant<int, 2>{})) break;
      if (STEP(std::integral_constant<int, 3>{})) break;
      if constexpr (RING > 4) {
        if (STEP(std::integral_constant<int, 4 % RING>{})) break;
        if (STEP(std::integral_constant<int, 5 % RING>{})) break;
      }
      if constexpr (RING > 6) {
        if (STEP(std::integral_constant<int, 6 % RING>{})) break;
        if (STEP(std::integral_constant<int, 7 % RING>{})) break;
      }
    }
  };
  start_range();
  if constexpr (MSUM) ring_fill();
  if (C.it < C.it1) {
    run_ring([&](auto S) __attribute__((always_inline)) { return step(S); });
  }
  close_range(C, D);
}

// ---------------------------------------------------------------------------
// dequantised weights from the packed layout, fp32 row-major N x K:
// w = fma(d sc, q, -dmin m), d sc and dmin m exact in fp32, one rounding.
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ packed, float* __restrict__ w, int64_t N, int64_t KB,
               int64_t NS, int64_t hdr_off) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= NS * KB * 64) return;
  int lane = (int)(tid & 63);
  int64_t pair = tid >> 6;
  int64_t ns = pair / KB, j = pair % KB;
  int g = lane >> 4, nl = lane & 15;
  int64_t n = ns * TILE_N + nl;
  if (n >= N) return;
  const uint8_t* qp = packed + quant_chunk_off(ns, j, KB) + lane * 16;
  u32x4 q0 = *reinterpret_cast<const u32x4*>(qp);
  u32x4 q1 = *reinterpret_cast<const u32x4*>(qp + 1024);
  u32x4 h = *reinterpret_cast<const u32x4*>(packed + hdr_off + header_chunk_off(ns, j, KB) + nl * 16);
  uint32_t F = header_group(h.y, h.z, h.w, g);
  float d = (float)bitcast<_Float16>((uint16_t)(h.x & 0xFFFFu));
  float dmin = (float)bitcast<_Float16>((uint16_t)(h.x >> 16));
  float A[2] = {d * (float)grp_sc(F, 0), d * (float)grp_sc(F, 1)};
  float B[2] = {dmin * (float)grp_m(F, 0), dmin * (float)grp_m(F, 1)};
  float* row = w + n * (KB * SB_W) + j * SB_W;
  for (int t = 0; t < 8; ++t) {
    uint32_t wd = (t < 4) ? q0[t] : q1[t - 4];
    for (int p = 0; p < 8; ++p) {
      int hb = p >> 2;
      float q = (float)((wd >> (4 * p)) & 15u);
      row[slot_k(g, t, p)] = __builtin_fmaf(A[hb], q, -B[hb]);
    }
  }
}

// ---------------------------------------------------------------------------
// A plain read of n16 16-byte words: thread t of the grid reads words t,
// t + stride, ..., four loads in flight (nontemporal hint), and folds them into
// a value that is stored only if it equals a constant no real buffer is likely
// to give (the loads must not be dropped).
__global__ void __launch_bounds__(512) read_probe_kernel(const u32x4* __restrict__ p, uint64_t n16,
                                                         u32x4* __restrict__ sink) {
  constexpr int U = 4;
  const uint64_t tid = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint64_t i = tid; i < n16; i += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t k = i + (uint64_t)u * stride;
      v[u] = k < n16 ? __builtin_nontemporal_load(p + k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[tid & 1023] = acc;
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, void* sink, int cus, hipStream_t st) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)cus), dim3(512), 0, st, reinterpret_cast<const u32x4*>(buf),
                     bytes / 16, reinterpret_cast<u32x4*>(sink));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// per-row argmax, lowest index among equal maxima; NaN never wins.  One
// workgroup per row; the row is read as 16-byte vectors (after a scalar head up
// to 16-byte alignment), four independent loads in flight per thread, so one
// workgroup streams its row at close to a CU's load bandwidth.  Which thread
// sees which element does not matter: (value, lowest index) is the same maximum
// in any order.
__global__ void __launch_bounds__(1024)
argmax_kernel(const float* __restrict__ y, int64_t N, int32_t* __restrict__ idx) {
  constexpr int NT = 1024, U = 4;
  __shared__ float sv[NT / 64];
  __shared__ int64_t si[NT / 64];
  const int64_t r = blockIdx.x;
  const float* row = y + r * N;
  const int tid = threadIdx.x;
  float bv = -__builtin_inff();
  int64_t bi = N;                      // N = "none yet"
  auto take = [&](float v, int64_t n) {
    if (v > bv || (v == bv && n < bi)) { bv = v; bi = n; }
  };
  const int64_t mis = (int64_t)((16u - ((uintptr_t)row & 15u)) & 15u) / 4;
  const int64_t head = mis < N ? mis : N;
  if (tid < head) take(row[tid], tid);
  const int64_t nvec = (N - head) / 4;
  const float4* vrow = reinterpret_cast<const float4*>(row + head);
  for (int64_t i0 = 0; i0 < nvec; i0 += (int64_t)NT * U) {
    float4 v[U];
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT + tid;
      v[u] = i < nvec ? vrow[i] : make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                              __builtin_nanf(""));
    }
    for (int u = 0; u < U; ++u) {
      const int64_t n = head + 4 * (i0 + (int64_t)u * NT + tid);
      take(v[u].x, n);
      take(v[u].y, n + 1);
      take(v[u].z, n + 2);
      take(v[u].w, n + 3);
    }
  }
  for (int64_t n = head + 4 * nvec + tid; n < N; n += NT) take(row[n], n);
  // wave, then workgroup: keep the larger value, the lower index on ties; "none"
  // (index N) loses to anything
  auto merge = [&](float ov, int64_t oi) {
    if (oi != N && (bi == N || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
  };
  for (int off = 32; off > 0; off >>= 1) merge(__shfl_xor(bv, off), __shfl_xor(bi, off));
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid < 64) {
    bv = tid < NT / 64 ? sv[tid] : -__builtin_inff();
    bi = tid < NT / 64 ? si[tid] : N;
    for (int off = 32; off > 0; off >>= 1) merge(__shfl_xor(bv, off), __shfl_xor(bi, off));
    if (tid == 0) idx[r] = (int32_t)(bi == N ? 0 : bi);
  }
}

// ---------------------------------------------------------------------------
// Greedy verification of draft tokens.  Agent a owns rows a (D + 1) .. a (D + 1)
// + D of the pass: its current token and its D drafts (OpenJet multi-agent
// serving page, section on moving the weights only once: the drafts are checked
// in the same round).  Row i's argmax p_i is the choice for the position after
// row i's input, so draft i (row i + 1's input) stands iff it equals p_i; the
// agent emits p_0 and p_{i+1} for each draft accepted in order, up to the first
// rejection.  One thread per agent; argmax rows read through `load`.
template <class Load>
__device__ __forceinline__ void verify_agent(int a, int D, Load load, const int32_t* __restrict__ drafts,
                                             int32_t* __restrict__ tokens, int32_t* __restrict__ n_new) {
  const int base = a * (D + 1);
  int n = 1;
  tokens[base] = load(base);
  bool open = true;
  for (int i = 0; i < D; ++i) {
    open = open && load(base + i) == drafts[a * D + i];
    tokens[base + i + 1] = open ? load(base + i + 1) : -1;
    n += open ? 1 : 0;
  }
  n_new[a] = n;
}

__global__ void __launch_bounds__(64)
verify_kernel(const int32_t* __restrict__ idx, int A, int D, const int32_t* __restrict__ drafts,
              int32_t* __restrict__ tokens, int32_t* __restrict__ n_new) {
  const int a = threadIdx.x;
  if (a < A) verify_agent(a, D, [&](int r) { return idx[r]; }, drafts, tokens, n_new);
}

// Row argmax over column chunks, with a workspace (the same result as
// argmax_kernel: the largest value, lowest index among equal maxima, NaN never
// wins).  Grid (C, R): workgroup (c, r) takes columns [c chunk, (c + 1) chunk) of
// row r, publishes its (value, index) in part[r C + c] and arrives at cnt[r];
// the last of row r's C arrivals adds the partials in chunk order, writes idx[r]
// and arrives at cnt[R]; the last row to finish runs the draft verification when
// drafts are given.  Every arrival counter it uses is back at zero when the
// kernel ends.
__global__ void __launch_bounds__(256)
argmax_split_kernel(const float* __restrict__ y, int R, int64_t N, int64_t chunk, int C,
                    unsigned long long* __restrict__ part, uint32_t* __restrict__ cnt, int32_t* __restrict__ idx,
                    const int32_t* __restrict__ drafts, int D, int32_t* __restrict__ tokens,
                    int32_t* __restrict__ n_new) {
  constexpr int NT = 256, U = 4;
  constexpr uint32_t NONE = 0xFFFFFFFFu;
  __shared__ float sv[NT / 64];
  __shared__ int64_t si[NT / 64];
  __shared__ uint32_t s_last;
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  const int64_t n0 = (int64_t)c * chunk, n1 = n0 + chunk < N ? n0 + chunk : N;
  const float* row = y + (int64_t)r * N;
  float bv = -__builtin_inff();
  int64_t bi = N;                                 // N = "none yet"
  auto take = [&](float v, int64_t n) {
    if (v > bv || (v == bv && n < bi)) { bv = v; bi = n; }
  };
  // scalar head up to 16-byte alignment, 16-byte vectors, scalar tail
  const int64_t mis = (int64_t)((16u - ((uintptr_t)(row + n0) & 15u)) & 15u) / 4;
  const int64_t h1 = n0 + mis < n1 ? n0 + mis : n1;
  if (n0 + tid < h1) take(row[n0 + tid], n0 + tid);
  const int64_t nvec = (n1 - h1) / 4;
  const float4* vrow = reinterpret_cast<const float4*>(row + h1);
  for (int64_t i0 = 0; i0 < nvec; i0 += (int64_t)NT * U) {
    float4 v[U];
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * NT + tid;
      v[u] = i < nvec ? vrow[i] : make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                              __builtin_nanf(""));
    }
    for (int u = 0; u < U; ++u) {
      const int64_t n = h1 + 4 * (i0 + (int64_t)u * NT + tid);
      take(v[u].x, n);
      take(v[u].y, n + 1);
      take(v[u].z, n + 2);
      take(v[u].w, n + 3);
    }
  }
  for (int64_t n = h1 + 4 * nvec + tid; n < n1; n += NT) take(row[n], n);
  auto merge = [&](float ov, int64_t oi) {
    if (oi != N && (bi == N || ov > bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
  };
  for (int off = 32; off > 0; off >>= 1) merge(__shfl_xor(bv, off), __shfl_xor(bi, off));
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < NT / 64; ++k) merge(sv[k], si[k]);
    const unsigned long long key =
        ((unsigned long long)__builtin_bit_cast(uint32_t, bv) << 32) | (bi == N ? NONE : (uint32_t)bi);
    __hip_atomic_store(part + (int64_t)r * C + c, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = __hip_atomic_fetch_add(cnt + r, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(C - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // the row's last arrival: every thread takes some chunks' partials, then the
  // workgroup reduces them (the maximum with the lowest index does not depend
  // on the order in which partials meet)
  bv = -__builtin_inff();
  bi = N;
  for (int k = tid; k < C; k += NT) {
    const unsigned long long key = __hip_atomic_load(part + (int64_t)r * C + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t ki = (uint32_t)key;
    if (ki != NONE) merge(__builtin_bit_cast(float, (uint32_t)(key >> 32)), (int64_t)ki);
  }
  for (int off = 32; off > 0; off >>= 1) merge(__shfl_xor(bv, off), __shfl_xor(bi, off));
  __syncthreads();                                // the first reduction's LDS reads are done
  if ((tid & 63) == 0) { sv[tid >> 6] = bv; si[tid >> 6] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < NT / 64; ++k) merge(sv[k], si[k]);
    __hip_atomic_store(idx + r, (int32_t)(bi == N ? 0 : bi), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(cnt + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = __hip_atomic_fetch_add(cnt + R, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(R - 1);
  }
  __syncthreads();
  if (!s_last) return;
  // the last row: draft verification, one thread per agent, argmax rows staged in LDS
  __shared__ int32_t s_idx[MAX_ROWS];
  if (tid < R) s_idx[tid] = __hip_atomic_load(idx + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) __hip_atomic_store(cnt + R, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (tokens && tid < R / (D + 1)) verify_agent(tid, D, [&](int q) { return s_idx[q]; }, drafts, tokens, n_new);
}

// ---------------------------------------------------------------------------
// launch wrappers

static inline unsigned blocks_for(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

hipError_t launch_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K, hipStream_t st) {
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  int64_t total = NS * KB * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st, canon, packed, N, KB, NS);
  return hipGetLastError();
}

#define QG_STREAM_VARIANTS(X) X(1, 1, 8) X(2, 1, 8) X(3, 1, 8) X(4, 1, 8)

template <int RT, int NT, int NW>
static hipError_t launch_stream_t(const StreamArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)a.P), block(NW * 64);
  if constexpr (RT == 1 && NT == 1 && NW == 8) {
    if (a.valu) {
      if (!a.msum || a.R < 1 || a.R > VROWS) return hipErrorInvalidValue;
      switch (a.R) {
        case 1: hipLaunchKernelGGL((stream_kernel<1, 1, 8, true, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((stream_kernel<1, 1, 8, true, 2>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((stream_kernel<1, 1, 8, true, 3>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((stream_kernel<1, 1, 8, true, 4>), grid, block, 0, st, a); break;
      }
      return hipGetLastError();
    }
  }
  if (a.valu) return hipErrorInvalidValue;
  if (a.msum)
    hipLaunchKernelGGL((stream_kernel<RT, NT, NW, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((stream_kernel<RT, NT, NW, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs& a, hipStream_t st) {
#define QG_CASE(rt, nt, nw) \
  if (a.RT == rt && a.NT == nt && a.NW == nw) return launch_stream_t<rt, nt, nw>(a, st);
  QG_STREAM_VARIANTS(QG_CASE)
#undef QG_CASE
  return hipErrorInvalidValue;
}

bool stream_variant_exists(int RT, int NT, int NW) {
#define QG_CASE(rt, nt, nw) \
  if (RT == rt && NT == nt && NW == nw) return true;
  QG_STREAM_VARIANTS(QG_CASE)
#undef QG_CASE
  return false;
}

// resident workgroups per CU of a variant (both min-term forms have the same LDS footprint)
int stream_occupancy(int RT, int NT, int NW) {
  int blocks = 0;
#define QG_CASE(rt, nt, nw) \
  if (RT == rt && NT == nt && NW == nw) { \
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, stream_kernel<rt, nt, nw, true>, nw * 64, 0) != \
        hipSuccess) \
      return 0; \
    return blocks; \
  }
  QG_STREAM_VARIANTS(QG_CASE)
#undef QG_CASE
  return 0;
}

hipError_t launch_dequant(const uint8_t* packed, float* w, int64_t N, int64_t K, hipStream_t st) {
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  int64_t total = NS * KB * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st, packed, w, N, KB, NS,
                     quant_region_bytes(N, K));
  return hipGetLastError();
}

hipError_t launch_argmax(const float* y, int R, int64_t N, int32_t* idx, hipStream_t st) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)R), dim3(1024), 0, st, y, N, idx);
  return hipGetLastError();
}

hipError_t launch_argmax_split(const float* y, int R, int64_t N, int32_t* idx, void* ws, const int32_t* drafts,
                               int D, int32_t* tokens, int32_t* n_new, hipStream_t st) {
  if (R == 0) return hipSuccess;
  const int C = argmax_chunks(N);
  const int64_t chunk = (N + C - 1) / C;
  unsigned long long* part = reinterpret_cast<unsigned long long*>(ws);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(part + (int64_t)R * C);
  hipLaunchKernelGGL(argmax_split_kernel, dim3((unsigned)C, (unsigned)R), dim3(256), 0, st, y, R, N, chunk, C, part,
                     cnt, idx, drafts, D, tokens, n_new);
  return hipGetLastError();
}

hipError_t launch_verify(const int32_t* idx, int R, const int32_t* drafts, int D, int32_t* tokens, int32_t* n_new,
                         hipStream_t st) {
  if (R == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_kernel, dim3(1), dim3(64), 0, st, idx, R / (D + 1), D, drafts, tokens, n_new);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fixed device scratch of the allocation-free entry point (qgemm_run_static):
// per-tile arrival counters, then partial output tiles.  Every GPU the library
// runs on holds its own copy for the life of the process.  In host code the
// array's name is not a device address: its address on the current device
// comes from hipGetSymbolAddress, taken once per device and kept.
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch_address(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// n 32-bit words set to zero (a kernel rather than a memset node, so that a
// captured graph replays it reliably)
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace qg
