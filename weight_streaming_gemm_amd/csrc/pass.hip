// pass.hip — the whole weight pass (a sequence of GEMMs) in one persistent launch,
// for up to 48 activation rows in one to three 16-row tiles.
//
// The pages' decode step streams every quantised weight once and applies it to
// all stacked rows (OpenJet multi-agent serving page, section on moving the
// weights only once), with one persistent megakernel for the whole step (the
// section on going from one session to four agents).  Here one cooperative
// launch runs all GEMMs of the pass in order; GEMM g + 1 computes only after
// every workgroup has finished GEMM g (each projection's input depends on the
// previous output), but its weights are already in flight: the weight stream
// does not stop at GEMM boundaries.
//
// Roles.  A workgroup (one per compute unit) has 8 compute waves and 4 helper
// waves.  A compute wave streams its weight steps through a register ring of
// RING steps that runs straight across GEMM boundaries, multiplies them on the
// matrix cores against activations in LDS, and hands each finished partial
// tile ("piece", RT 16 x 16 tiles) to LDS.  Compute waves issue only loads, so
// waiting for a step's weights never waits for a store.  The helper waves copy
// each GEMM's activations into LDS (all 12 waves then convert them in place),
// add the pieces of each unit in wave order, store y (or a chunk's partial
// tile), run the K-chunk sums, and arrive at and wait on the device-wide barrier
// between GEMMs.  Every wave passes two workgroup barriers per GEMM: the raw
// activations have landed, and they are converted.
//
// Work (pass_sched.h): a GEMM is cut along K into S chunks of kbc blocks; chunk c
// goes to a contiguous set of workgroups, which share its sub-tiles as runs of
// whole units (a unit = one 16-output sub-tile over one chunk).  With S > 1 the
// chunks' partial tiles of a sub-tile are added in chunk order, at one row tile
// by the last chunk to arrive and from two on by one designated workgroup; every
// sum has a fixed order, so results are bitwise repeatable.
//
// Per step (16 outputs x 256 weights of one block) the arithmetic is the
// streaming kernel's: B = sc q exact in binary16, 8 v_mfma_f32_16x16x32_f16 per
// row tile against the activations; the min term from 8 more products with the
// mins, or (MSUM) from the sub-block sums staged as two binary16 parts in one
// v_mfma_f32_16x16x16_f16 per tile; then acc += d ds - dmin ms in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "layout.h"
#include "operand.h"
#include "pass_sched.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t OOB = 0x80000000u;          // beyond every buffer (sizes < 2^31)
constexpr uint32_t SPIN_LIMIT = 1u << 21;      // polls of a device-wide wait before giving up
constexpr uint32_t LDS_SPIN_LIMIT = 1u << 24;  // polls of a wait on another wave of the workgroup
constexpr int SC1 = 16;                        // cache policy: coherent across the device
// s_waitcnt with lgkmcnt(0) only (vmcnt and expcnt at their maxima): LDS done,
// loads in flight untouched
constexpr int WAIT_LGKM0 = 0xC07F;
// s_waitcnt with vmcnt(0) only (lgkmcnt and expcnt at their maxima)
constexpr int WAIT_VM0 = 0x0F70;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
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
__device__ __forceinline__ void bstore1_sc1(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, SC1);
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}
// the sum of four bf16 values (two dwords) in fp32, with two dot products against ones
__device__ __forceinline__ float sum4_bf16(uint32_t d0, uint32_t d1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3F803F80u);
  const float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d0), one, 0.0f, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, d1), one, s, false);
}
// The min term's fp32 sub-block sums as matrix-core A operands: X_s 2^-8 (in
// binary16's range for |x| <= 65504: 32 x 65504 / 256 < 8192) in two binary16
// parts, hi = f16(X_s 2^-8) and lo = f16(X_s 2^-8 - hi) (the difference is exact
// in fp32), so that one v_mfma_f32_16x16x16_f16 against the mins (exact in
// binary16) adds m_s (hi + lo) over the 8 sub-blocks; the 2^8 goes back into
// -dmin (exact).  hi + lo holds X_s 2^-8 to 22 bits, or to 2^-25 absolute where
// lo is subnormal.
constexpr float SUM_SCALE = 1.0f / 256.0f, SUM_SCALE_INV = 256.0f;
__device__ __forceinline__ f16x4 sum_parts(float s0, float s1) {
  const float a0 = s0 * SUM_SCALE, a1 = s1 * SUM_SCALE;
  const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
  return f16x4{h0, h1, (_Float16)(a0 - (float)h0), (_Float16)(a1 - (float)h1)};
}
// B of that product for lane group g: (m_2g, m_2g+1) against both parts
__device__ __forceinline__ f16x4 min_parts_b(const WConst& c) { return f16x4{c.m[0], c.m[1], c.m[0], c.m[1]}; }
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t lds_load(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// GEMM g's descriptor, read through the scalar unit (wave-uniform by construction)
__device__ __forceinline__ PassGemm get_gemm(const PassGemm* __restrict__ t, int g) {
  typedef const PassGemm __attribute__((address_space(4)))* cptr;
  const cptr src = (cptr)(t + g);
  PassGemm d;
  d.qbase = uniform_ptr(src->qbase);
  d.hbase = uniform_ptr(src->hbase);
  d.qbytes = (uint32_t)uni((int)src->qbytes);
  d.hbytes = (uint32_t)uni((int)src->hbytes);
  d.x = uniform_ptr(src->x);
  d.y = uniform_ptr(src->y);
  d.N = uni(src->N);
  d.NS = uni(src->NS);
  d.KB = uni(src->KB);
  d.S = uni(src->S);
  d.kbc = uni(src->kbc);
  d.rot = uni(src->rot);
  d.masks = uniform_ptr(src->masks);
  return d;
}
__device__ __forceinline__ PassWave get_wave(const PassWave* __restrict__ t, int idx) {
  typedef const PassWave __attribute__((address_space(4)))* cptr;
  const cptr src = (cptr)(t + idx);
  PassWave v;
  v.count = uni(src->count);
  v.step0 = uni(src->step0);
  v.jj0 = uni(src->jj0);
  v.next = uni(src->next);
  v.xblk = 0;
  return v;
}

__device__ __forceinline__ int xblk_of(const PassWave* __restrict__ t, int idx) {
  typedef const PassWave __attribute__((address_space(4)))* cptr;
  return uni(((cptr)(t + idx))->xblk);
}

// RT 16 x 16 tiles of one lane (a piece, a sum, a partial result)
template <int RT>
struct Tiles {
  f32x4 v[RT];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) v[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void add(const Tiles& o) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) v[rt] += o.v[rt];
  }
};

// f(0), f(1), ..., f(n - 1) with compile-time indices (ring slots stay in registers)
template <class F, int... I>
__device__ __forceinline__ void for_each_slot(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// where a compute wave stands in the sequence (all wave-uniform)
struct Span {
  int g;                           // GEMM index; >= G past the end of the sequence
  int KB, kbc;                     // blocks of a row, blocks of a chunk
  int left;                        // steps of this GEMM left, the current one included
  int step, jj;                    // packed step (sub-tile * KB + block), block within the chunk
  int k;                           // pieces written in this GEMM (compute cursor)
  __amdgpu_buffer_rsrc_t qr, hr;   // quant and header regions
};

}  // namespace

// RT row tiles of 16 rows (R <= 16 RT): every weight step feeds RT products
// per activation operand; pieces and partial tiles hold RT 16 x 16 tiles
template <int RING, bool MSUM, int RT>
__global__ void __launch_bounds__(PASS_THREADS, 1)
pass_kernel(PassArgs a) {
  static_assert(RING >= 2 && RING <= 12, "ring of 2 to 12 steps");
  static_assert(RT >= 1 && RT <= PASS_MAX_RT, "one to PASS_MAX_RT row tiles");
  __shared__ __attribute__((aligned(16))) uint8_t xlds[pass_x_area(RT)];
  constexpr int PC = pass_pieces(RT);           // piece slots per compute wave
  __shared__ f32x4 pieces[PASS_NC * PC * RT * 64];
  __shared__ uint32_t s_go;                     // GEMM whose activations the helpers may stage
  __shared__ uint32_t s_written[PASS_NC];       // pieces each compute wave has written in this GEMM
  __shared__ uint32_t s_consumed[PASS_NC][PASS_PIECES];  // times each piece slot has been added
  __shared__ uint32_t s_done;                   // helpers through with their units (all GEMMs so far)
  __shared__ uint32_t s_last;                   // last workgroup out of the launch
  __shared__ uint32_t s_release;                // this workgroup's arrival completed the barrier

  const int tid = threadIdx.x, lane = tid & 63, wv = uni(tid >> 6), g4 = lane >> 4, nl = lane & 15;
  const int p = blockIdx.x, P = a.P, R = a.R, G = a.G;
  const PassGemm* __restrict__ gemms = a.gemms;
  const int XS = PASS_X_ROW * pass_x_rows(R), SB = pass_x_block_bytes(R);
  constexpr int GL = (16 / RT) * RT;            // partial tiles loaded together by a helper

  // ---- the conversion of the raw bf16 rows into the blocks' images, in place.
  // Rows go in pairs, 32 lanes (gg, t) per row: x[r, 64 gg + 4 t + {0..3}] and
  // the same 32 further on make operand (gg, t).  Raw pair q lies at 1056 q, the
  // place of its own operands (row 2 q + h at 1056 q + 512 h raw, 1056 q + 528 h
  // converted), so a pair is read and written over by one wave and by nothing
  // else (its reads come first: a wave's LDS accesses run in program order).
  // With a block for every wave, wave v takes the blocks v mod (PASS_NC +
  // PASS_NH); with fewer, the pairs of all blocks are dealt to all waves: the
  // units (block, pair) u = v, v + PASS_NC + PASS_NH, ... go to wave v.
  auto convert_share = [&](int xblk, int v) __attribute__((always_inline)) {
    constexpr int NW = PASS_NC + PASS_NH;
    const int RP = (R + 1) >> 1, units = xblk * RP;
    const int half = lane >> 5, sub = lane & 31, gg = sub >> 3, t = sub & 7;
    const int lin = half * 512 + (64 * gg + 4 * t) * 2, lout = half * PASS_X_ROW + sub * 16;
    auto sums = [&](uint8_t* slot, u32x2 lo, u32x2 hi, int r) __attribute__((always_inline)) {
      if constexpr (MSUM) {
        // sub-block sums: the 8 lanes t of lane group gg add their run sums as
        // ((s0 + s1) + (s2 + s3)) + ((s4 + s5) + (s6 + s7))
        float s0 = sum4_bf16(lo.x, lo.y), s1 = sum4_bf16(hi.x, hi.y);
        s0 += dpp_f32<0xB1>(s0); s1 += dpp_f32<0xB1>(s1);    // lane ^ 1
        s0 += dpp_f32<0x4E>(s0); s1 += dpp_f32<0x4E>(s1);    // lane ^ 2
        s0 += dpp_f32<0x104>(s0); s1 += dpp_f32<0x104>(s1);  // lane + 4 (for lane t = 0)
        if (r < R && t == 0) *reinterpret_cast<f16x4*>(slot + XS + (gg * R + r) * 8) = sum_parts(s0, s1);
      }
    };
    // pairs q0 of block b0 and q1 of block b1 (when two), both read before either is written
    auto convert2 = [&](int b0, int q0, int b1, int q1, bool two) __attribute__((always_inline)) {
      uint8_t* const s0 = xlds + b0 * SB + q0 * 1056;
      uint8_t* const s1 = xlds + b1 * SB + q1 * 1056;
      const u32x2 lo0 = *reinterpret_cast<const u32x2*>(s0 + lin);
      const u32x2 hi0 = *reinterpret_cast<const u32x2*>(s0 + lin + 64);
      u32x2 lo1 = lo0, hi1 = hi0;
      if (two) {
        lo1 = *reinterpret_cast<const u32x2*>(s1 + lin);
        hi1 = *reinterpret_cast<const u32x2*>(s1 + lin + 64);
      }
      *reinterpret_cast<f16x8*>(s0 + lout) = build_a(lo0.x, lo0.y, hi0.x, hi0.y);
      sums(xlds + b0 * SB, lo0, hi0, 2 * q0 + half);
      if (two) {
        *reinterpret_cast<f16x8*>(s1 + lout) = build_a(lo1.x, lo1.y, hi1.x, hi1.y);
        sums(xlds + b1 * SB, lo1, hi1, 2 * q1 + half);
      }
    };
    if (xblk >= NW) {
      // enough blocks for every wave: whole blocks, b = v mod NW
      for (int bb = v; bb < xblk; bb += NW)
        for (int q = 0; q < RP; q += 2) convert2(bb, q, bb, q + 1, q + 1 < RP);
      return;
    }
    // fewer: the units (block, pair) u = v, v + NW, ...
    int b0 = 0, q0 = v;
    while (q0 >= RP) {
      q0 -= RP;
      ++b0;
    }
    auto step = [&](int& bb, int& qq) __attribute__((always_inline)) {
      qq += NW;
      while (qq >= RP) {
        qq -= RP;
        ++bb;
      }
    };
    for (int u = v; u < units; u += 2 * NW) {
      int b1 = b0, q1 = q0;
      step(b1, q1);
      convert2(b0, q0, b1, q1, u + NW < units);
      b0 = b1;
      q0 = q1;
      step(b0, q0);
    }
  };

  if (wv < PASS_NC) {
    // ======================= compute wave ======================================
    const int w = wv;
    // this lane's A operands of row tile rt (step t at + 16 t) and sub-block sums
    // inside a slot; rows >= R reuse row R - 1 (never stored)
    int xoff[RT], soff[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int xr = 16 * rt + nl < R ? 16 * rt + nl : R - 1;
      xoff[rt] = xr * PASS_X_ROW + g4 * 128;
      soff[rt] = XS + (g4 * R + xr) * 8;
    }
    const PassWave* __restrict__ waves = a.waves;
    // the wave's share of GEMM g, or of the first later GEMM with steps for it
    auto enter = [&](Span& s, int g) __attribute__((always_inline)) {
      PassWave v = g < G ? get_wave(waves, (g * P + p) * PASS_NC + w) : PassWave{0, 0, 0, G, 0};
      if (v.count == 0 && v.next < G) {
        g = v.next;
        v = get_wave(waves, (g * P + p) * PASS_NC + w);
      }
      if (v.count == 0) g = G;
      s.g = g;
      s.left = v.count;
      s.step = v.step0;
      s.jj = v.jj0;
      s.k = 0;
      if (g < G) {
        const PassGemm d = get_gemm(gemms, g);
        s.KB = d.KB;
        s.kbc = d.kbc;
        s.qr = make_rsrc(d.qbase, d.qbytes);
        s.hr = make_rsrc(d.hbase, d.hbytes);
      } else {
        s.KB = 1;
        s.kbc = 1;
        s.qr = make_rsrc(nullptr, 0);
        s.hr = make_rsrc(nullptr, 0);
      }
    };
    // the next step of a cursor; at the end of its share, the next GEMM's
    auto advance = [&](Span& s) __attribute__((always_inline)) {
      s.left = uni(s.left - 1);
      if (s.left > 0) {
        s.jj = uni(s.jj + 1);
        s.step = uni(s.step + 1);
        if (s.jj == s.kbc) {
          s.jj = 0;
          s.step = uni(s.step + s.KB - s.kbc);
        }
      } else {
        enter(s, s.g + 1);
      }
    };
    typedef struct { u32x4 qa, qb, hd; } Stage;
    // the lane's offsets are fixed (lane 16 B into a quant half, output nl's 16 B of a
    // header chunk); the step's offset is wave-uniform and goes in the scalar
    // offset, so a refill needs no address registers and lands in the slot's own.
    // Past the end of the sequence the resources have no records: the loads
    // return zeros without touching memory.
    const int qlane = lane * 16, hlane = nl * 16;
    auto load_w = [&](Stage& st, const Span& s) __attribute__((always_inline)) {
      st.qa = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s.qr, qlane, s.step * CHUNK_Q, 2));
      st.qb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s.qr, qlane + 1024, s.step * CHUNK_Q, 2));
      st.hd = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(s.hr, hlane, s.step * CHUNK_H, 2));
    };
    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const Stage& st, int slot) __attribute__((always_inline)) {
      if constexpr (RT == 1) {
        const WConst cst = header_consts(st.hd.x, st.hd.y, st.hd.z, st.hd.w, g4);
        // d and -dmin as fp32 values of their own right away: folded into the final
        // multiply-adds as binary16 operands, they would keep the header's registers
        // alive past the slot's refill
        float dd = cst.d, dm = cst.nmin;
        asm volatile("" : "+v"(dd), "+v"(dm));
        f32x4 ds = {0.f, 0.f, 0.f, 0.f}, ms = {0.f, 0.f, 0.f, 0.f};
        const int base = slot * SB;
        if constexpr (MSUM) {
          for (int t = 0; t < 8; ++t) {
            const f16x8 xa = *reinterpret_cast<const f16x8*>(xlds + base + xoff[0] + t * 16);
            const uint32_t wd = (t < 4) ? st.qa[t] : st.qb[t - 4];
            ds = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, build_b(wd, cst), ds, 0, 0, 0);
          }
          const f16x4 xs = *reinterpret_cast<const f16x4*>(xlds + base + soff[0]);
          ms = __builtin_amdgcn_mfma_f32_16x16x16f16(xs, min_parts_b(cst), ms, 0, 0, 0);
          dm *= SUM_SCALE_INV;
      } else {
          const f16x8 bm = build_m_full(cst);
          for (int t = 0; t < 8; ++t) {
            const f16x8 xa = *reinterpret_cast<const f16x8*>(xlds + base + xoff[0] + t * 16);
            const uint32_t wd = (t < 4) ? st.qa[t] : st.qb[t - 4];
            ds = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, build_b(wd, cst), ds, 0, 0, 0);
            ms = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, bm, ms, 0, 0, 0);
          }
        }
        for (int i = 0; i < 4; ++i) {
          acc[0][i] = __builtin_fmaf(dd, ds[i], acc[0][i]);
          acc[0][i] = __builtin_fmaf(dm, ms[i], acc[0][i]);
        }
      } else {
        // RT row tiles: the same B operand for every tile
        const WConst cst = header_consts(st.hd.x, st.hd.y, st.hd.z, st.hd.w, g4);
        // d and -dmin as fp32 values of their own right away: folded into the final
        // multiply-adds as binary16 operands, they would keep the header's registers
        // alive past the slot's refill
        float dd = cst.d, dm = cst.nmin;
        asm volatile("" : "+v"(dd), "+v"(dm));
        f32x4 ds[RT], ms[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) ds[rt] = ms[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int base = slot * SB;
        static_assert(MSUM, "several row tiles take the min term from the sub-block sums");
        for (int t = 0; t < 8; ++t) {
          f16x8 xa[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) xa[rt] = *reinterpret_cast<const f16x8*>(xlds + base + xoff[rt] + t * 16);
          const uint32_t wd = (t < 4) ? st.qa[t] : st.qb[t - 4];
          const f16x8 b = build_b(wd, cst);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) ds[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rt], b, ds[rt], 0, 0, 0);
        }
        const f16x4 bm4 = min_parts_b(cst);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const f16x4 xs = *reinterpret_cast<const f16x4*>(xlds + base + soff[rt]);
          ms[rt] = __builtin_amdgcn_mfma_f32_16x16x16f16(xs, bm4, ms[rt], 0, 0, 0);
        }
        dm *= SUM_SCALE_INV;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          for (int i = 0; i < 4; ++i) {
            acc[rt][i] = __builtin_fmaf(dd, ds[rt][i], acc[rt][i]);
            acc[rt][i] = __builtin_fmaf(dm, ms[rt][i], acc[rt][i]);
          }
      }
    };
    // piece k of this wave's sub-range (one per unit it touches) into slot k mod
    // PC, once a helper has taken piece k - PC from it (the slot's k / PC earlier
    // pieces added)
    auto put_piece = [&](Span& s) __attribute__((always_inline)) {
      const uint32_t k = (uint32_t)s.k;
      s.k = uni(s.k + 1);
      if (k >= PC) {
        uint32_t n = 0;
        while (lds_load(&s_consumed[w][k % PC]) < k / PC) {
          if (++n > LDS_SPIN_LIMIT) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      asm volatile("" ::: "memory");             // the slot is free before it is written
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) pieces[((w * PC + (int)(k % PC)) * RT + rt) * 64 + lane] = acc[rt];
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);    // the piece is in LDS before it is announced
      asm volatile("" ::: "memory");
      if (lane == 0) lds_store(&s_written[w], k + 1);
    };

    // the wave's part in the staging of GEMM g: once the helpers' copies of the
    // raw activations have landed, convert its share of the blocks; the GEMM's
    // steps start after every wave's share is done
    auto stage_gemm = [&](int g) __attribute__((always_inline)) {
      const int xblk = uni(xblk_of(waves, (g * P + p) * PASS_NC + w));
      __builtin_amdgcn_s_barrier();
      convert_share(xblk, w);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      __builtin_amdgcn_s_barrier();
    };
    int passed = 0;                              // GEMMs staged so far
    Span L, C;
    enter(C, 0);
    L = C;
    Stage W[RING];
    // the ring's first RING steps (unrolled: the slots must stay in registers)
    auto fill = [&](auto SL) __attribute__((always_inline)) {
      load_w(W[decltype(SL)::value], L);
      advance(L);
    };
    for_each_slot(fill, std::make_integer_sequence<int, RING>{});
    // one step at ring slot s; true at the end of the sequence
    auto step = [&](auto SL) __attribute__((always_inline)) -> bool {
      constexpr int s = decltype(SL)::value;
      compute(W[s], C.jj);
      // the refill goes after the slot's last use, into the slot's own registers
      __builtin_amdgcn_sched_barrier(0);
      load_w(W[s], L);
      advance(L);
      if (C.g < G && (C.jj == C.kbc - 1 || C.left == 1)) {      // the step ends a unit or the share
        put_piece(C);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      advance(C);
      while (passed <= C.g && C.g < G) {         // the next step's GEMM: stage it first
        stage_gemm(passed);
        passed = uni(passed + 1);
      }
      return C.g >= G;
    };
    while (passed <= C.g && C.g < G) {
      stage_gemm(passed);
      passed = uni(passed + 1);
    }
    if (C.g < G)
    for (;;) {
      for_each_slot(step, std::make_integer_sequence<int, RING>{});
      if (C.g >= G) break;
    }
    while (passed < G) {                         // GEMMs past this wave's last step
      stage_gemm(passed);
      passed = uni(passed + 1);
    }
    return;
  }

  // ========================= helper waves ========================================
  const int h = wv - PASS_NC;                    // 0 .. PASS_NH - 1
  uint32_t* const bar = a.bar;
  const int groups = P < 8 ? P : 8;
  const int grp = p % 8, members = (P - grp + 7) / 8;
  bool dead = false;                             // a device-wide wait gave up: no more waiting

  if (h == 0) {
    if (lane < PASS_NC * PASS_PIECES) (&s_consumed[0][0])[lane] = 0u;
    if (lane < PASS_NC) s_written[lane] = 0u;
    if (lane == 0) {
      s_go = 0u;
      s_done = 0u;
    }
  }

  // ---- the activations of GEMM g for this workgroup's chunk: block c kbc + b of x
  // goes to slot b, and helper h copies the blocks b = h mod PASS_NH: row pair
  // q of the block (2 x 512 bytes of bf16) to slot + 1056 q, one load that
  // writes LDS directly (lane l's 16 bytes land at the load's base + 16 l), all
  // of the helper's loads in flight together.  All waves then convert the
  // pairs in place (convert_share).
  auto stage_raw = [&](const PassGemm& d, int c) __attribute__((always_inline)) {
    const int K = d.KB * SB_W;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(d.x, (uint32_t)(R * K * 2));
    const int RP = (R + 1) >> 1, half = lane >> 5;
    for (int b = h; b < d.kbc; b += PASS_NH) {
      const uint32_t blk = (uint32_t)((c * d.kbc + b) * SB_W * 2) + (uint32_t)(lane & 31) * 16u;
      for (int pr = 0; pr < RP; ++pr) {
        const int r = 2 * pr + half;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void*)(xlds + b * SB + pr * 1056), 16,
            r < R ? (uint32_t)(r * K * 2) + blk : OOB, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);        // the raw rows are in LDS
    asm volatile("" ::: "memory");
  };

  // ---- device-wide barrier after GEMM g (generation g + 1): arrive at the
  // group counter of workgroups p mod 8; the group's last arrival arrives at the
  // global counter, and the last arrival there writes the generation to every
  // group's release word, which the group's workgroups wait on (32 waiters per
  // word rather than all on one).  Every helper's stores of GEMM g are complete
  // by then.
  auto grid_arrive = [&](int g) __attribute__((always_inline)) {
    const uint32_t gen = (uint32_t)g + 1;
    if (lane == 0) {
      uint32_t last = 0;
      const uint32_t old = __hip_atomic_fetch_add(bar + 32 + 32 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == gen * (uint32_t)members) {
        const uint32_t all = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = all + 1 == gen * (uint32_t)groups ? 1u : 0u;
      }
      s_release = last;
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    if (lds_load(&s_release) && lane < groups)
      __hip_atomic_store(bar + PASS_RELEASE_WORD + 32 * lane, gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto grid_wait = [&](int g) __attribute__((always_inline)) {
    if (lane == 0 && !dead) {
      const uint32_t target = (uint32_t)g + 1;
      uint32_t n = 0;
      while (__hip_atomic_load(bar + PASS_RELEASE_WORD + 32 * grp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
             target) {
        if (++n > SPIN_LIMIT) {
          __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          dead = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
  };

  // ---- GEMM g with gated input, chunk c: wait only for the workgroups that hold
  // the previous GEMM's outputs the chunk reads.  Each of them, once through the
  // previous GEMM, adds one to the counter of every chunk of GEMM g that reads
  // its outputs; the chunk's counter reaching the target in the table means all
  // have (targets add up over the launch's gated GEMMs)
  auto gated_wait = [&](const PassGemm& d, int c) __attribute__((always_inline)) {
    if (lane != 0 || dead) return;
    const uint32_t target = (uint32_t)d.masks[PASS_MASK_WORDS * c + 4];
    uint32_t n = 0;
    while (__hip_atomic_load(bar + PASS_DEP_WORD + PASS_DEP_STRIDE * c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           target) {
      if (++n > SPIN_LIMIT) {
        __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dead = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  };
  // ... and the producer's side, after its stores of the previous GEMM are
  // complete: lane c' for chunk c' of the next GEMM dn
  auto gated_signal = [&](const PassGemm& dn) __attribute__((always_inline)) {
    if (lane < dn.S) {
      const uint64_t w = dn.masks[PASS_MASK_WORDS * lane + (p >> 6)];
      if ((w >> (p & 63)) & 1u)
        __hip_atomic_fetch_add(bar + PASS_DEP_WORD + PASS_DEP_STRIDE * lane, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // ---- the units of GEMM g at one row tile.  A unit inside one compute wave's sub-range has
  // one piece; helper h takes those of waves h and h + PASS_NH as they are
  // written, and the units those two waves begin and later waves finish, adding
  // their pieces in wave order.  The last wave's piece of such a unit is its
  // first, written early: it is taken (and its slot handed back) as soon as it
  // is written, so that no wave waits long for a free piece slot.  Then y (one
  // chunk) or the chunk's partial tile; after its last unit the chunk sums of
  // those of its sub-tiles whose last chunk this workgroup was.
  auto finish_one = [&](const PassGemm& d, int g, int c, int ns0, int ns1) __attribute__((always_inline)) {
    const int units = ns1 - ns0, n = units * d.kbc, kbc = d.kbc;
    // y goes out device-coherent: the next GEMM may run on any die
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(d.y, (uint32_t)(R * d.N * 4));
    const uint32_t part_tile = (uint32_t)d.NS * 1024u;                 // bytes of one chunk's partials
    // GEMMs of even and odd index use separate halves of the partials and their
    // counters: with gated inputs a workgroup may start GEMM g + 1 while others
    // still finish GEMM g
    const uint32_t half = (uint32_t)(g & 1);
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part + half * (a.part_bytes / 8), a.part_bytes / 2);
    uint32_t* const cnt = a.cnt + half * a.cnt_half;
    // piece j of wave w, once written; its slot is handed back
    auto take = [&](int w, int j) __attribute__((always_inline)) -> f32x4 {
      uint32_t spins = 0;
      while (lds_load(&s_written[w]) <= (uint32_t)j) {
        if (++spins > LDS_SPIN_LIMIT) break;
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");             // the piece is read after its announcement
      const f32x4 v = pieces[(w * PASS_PIECES + j % PASS_PIECES) * 64 + lane];
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);    // and before its slot is handed back
      asm volatile("" ::: "memory");
      if (lane == 0) lds_store(&s_consumed[w][j % PASS_PIECES], (uint32_t)(j / PASS_PIECES) + 1u);
      return v;
    };
    auto put = [&](int u, const f32x4& sum) __attribute__((always_inline)) {
      const int ns = ns0 + u;
      if (d.S == 1) {
        const int nn = ns * TILE_N + nl;
        if (nn < d.N)
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            if (r < R) bstore1_sc1(sum[i], yr, (uint32_t)((r * d.N + nn) * 4));
          }
      } else {
        bstore_sc1(sum, pr, (uint32_t)c * part_tile + (uint32_t)ns * 1024u + lane * 16);
      }
    };
    // waves h and h + PASS_NH: sub-range [a, b), units [f, l] touched (piece
    // u - f of unit u), internal units [u, e), the unit it begins that later
    // waves finish (ul, or -1) and the last of those waves (wl)
    int wv2[2], a2[2], f2[2], u2[2], e2[2], ul2[2], wl2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int w = h + i * PASS_NH;
      const int aw = pass_wave_first(w, PASS_NC, n), bw = pass_wave_first(w + 1, PASS_NC, n);
      wv2[i] = w;
      a2[i] = aw;
      f2[i] = aw / kbc;
      u2[i] = (aw + kbc - 1) / kbc;
      e2[i] = aw < bw ? bw / kbc : u2[i];
      const int ul = (bw - 1) / kbc;
      const bool shared = aw < bw && ul * kbc >= aw && (ul + 1) * kbc > bw;
      ul2[i] = shared ? ul : -1;
      wl2[i] = shared ? pass_step_owner((ul + 1) * kbc - 1, PASS_NC, n) : w;
    }
    f32x4 hv[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    bool have[2] = {ul2[0] < 0, ul2[1] < 0};
    uint32_t spins = 0;
    for (;;) {
      bool moved = false, pending = false;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (u2[i] < e2[i]) {
          const int j = u2[i] - f2[i];
          if (lds_load(&s_written[wv2[i]]) > (uint32_t)j) {
            f32x4 sum = {0.f, 0.f, 0.f, 0.f};
            sum += take(wv2[i], j);
            put(u2[i], sum);
            u2[i] = uni(u2[i] + 1);
            moved = true;
          }
          pending = pending || u2[i] < e2[i];
        }
        if (!have[i]) {                          // the last wave's (first) piece of the shared unit
          if (lds_load(&s_written[wl2[i]]) > 0u) {
            hv[i] = take(wl2[i], 0);
            have[i] = true;
            moved = true;
          } else {
            pending = true;
          }
        }
      }
      if (!pending) break;
      if (!moved) {
        if (++spins > LDS_SPIN_LIMIT) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // the shared units, their pieces in wave order (the last wave's taken above)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ul = ul2[i];
      if (ul < 0) continue;
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
      sum += take(wv2[i], ul - f2[i]);
      for (int ww = wv2[i] + 1; ww < wl2[i]; ++ww) {
        if (pass_wave_first(ww, PASS_NC, n) == pass_wave_first(ww + 1, PASS_NC, n)) continue;   // no piece
        sum += take(ww, 0);                      // a middle wave's only piece
      }
      sum += hv[i];
      put(ul, sum);
    }
    if (d.S == 1 || units == 0) return;
    // every partial tile of this helper is stored; arrive at each of its units'
    // sub-tile counters (one lane per unit: the units whose first step lies in
    // wave h or h + PASS_NH); the last of the S chunks to arrive adds the S
    // partial tiles in chunk order and writes y.  A round takes as many of those
    // sub-tiles as 16 loads hold (8 of 2 chunks, 4 of up to 4, 2 of up to 8),
    // all loads in flight together; sub-tile indices stay in vector registers.
    auto gather = [&](auto PSC, uint64_t& mask, int ub) __attribute__((always_inline)) {
      constexpr int PS = decltype(PSC)::value, NB = 16 / PS;
      int nsj[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        nsj[j] = -1;
        if (mask) {
          nsj[j] = ns0 + ub + __builtin_ctzll(mask);
          mask &= mask - 1;
        }
        asm volatile("" : "+v"(nsj[j]));
      }
      f32x4 v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int j = k / PS, cc = k % PS;
        v[k] = bload<f32x4, SC1>(pr, nsj[j] >= 0 && cc < d.S ? (uint32_t)cc * part_tile + (uint32_t)nsj[j] * 1024u + lane * 16 : OOB);
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (nsj[j] < 0) continue;
        f32x4 sum = v[j * PS];
#pragma unroll
        for (int cc = 1; cc < PS; ++cc)
          if (cc < d.S) sum += v[j * PS + cc];
        const int nn = nsj[j] * TILE_N + nl;
        if (nn < d.N)
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g4 + i;
            if (r < R) bstore1_sc1(sum[i], yr, (uint32_t)((r * d.N + nn) * 4));
          }
        if (lane == 0) __hip_atomic_store(cnt + nsj[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    __builtin_amdgcn_s_waitcnt(0);
    for (int ub = 0; ub < units; ub += 64) {
      bool last = false;
      const int u = ub + lane;
      if (u < units && pass_step_owner(u * kbc, PASS_NC, n) % PASS_NH == h) {
        const uint32_t old = __hip_atomic_fetch_add(cnt + ns0 + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (uint32_t)(d.S - 1);
      }
      uint64_t mask = __builtin_amdgcn_ballot_w64(last);
      while (mask) {
        if (d.S <= 2)
          gather(std::integral_constant<int, 2>{}, mask, ub);
        else if (d.S <= 4)
          gather(std::integral_constant<int, 4>{}, mask, ub);
        else if (d.S <= 8)
          gather(std::integral_constant<int, 8>{}, mask, ub);
        else
          gather(std::integral_constant<int, 16>{}, mask, ub);
      }
    }
  };

  // ---- the units of GEMM g.  A unit inside one compute wave's sub-range has
  // one piece; helper h takes those of waves h and h + PASS_NH as they are
  // written, and the units those two waves begin and later waves finish, adding
  // their pieces in wave order.  The last wave's piece of such a unit is its
  // first, written early: it is taken (and its slot handed back) as soon as it
  // is written, so that no wave waits long for a free piece slot.  Then y (one
  // chunk) or the chunk's partial tile; after its last unit the chunk sums of
  // those of its sub-tiles whose last chunk this workgroup was.
  auto finish_tiles = [&](const PassGemm& d, int g, int c, int ns0, int ns1) __attribute__((always_inline)) {
    const int units = ns1 - ns0, n = units * d.kbc, kbc = d.kbc;
    // y goes out device-coherent: the next GEMM may run on any die
    const __amdgpu_buffer_rsrc_t yr = make_rsrc(d.y, (uint32_t)(R * d.N * 4));
    // chunk c's partial result of sub-tile ns, row tile rt: at ((ns S + c) RT + rt) KiB, so that a
    // sub-tile's S RT partial tiles lie together, in the order they are added
    const uint32_t sub_tile = RT * 1024u;
    // GEMMs of even and odd index use separate halves of the partials and their
    // counters: with gated inputs a workgroup may start GEMM g + 1 while others
    // still finish GEMM g
    const uint32_t half = (uint32_t)(g & 1);
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part + half * (a.part_bytes / 8), a.part_bytes / 2);
    uint32_t* const cnt = a.cnt + half * a.cnt_half;
    // piece j of wave w, once written; its slot is handed back
    auto take = [&](int w, int j) __attribute__((always_inline)) -> Tiles<RT> {
      uint32_t spins = 0;
      while (lds_load(&s_written[w]) <= (uint32_t)j) {
        if (++spins > LDS_SPIN_LIMIT) break;
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");             // the piece is read after its announcement
      Tiles<RT> v;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) v.v[rt] = pieces[((w * PC + j % PC) * RT + rt) * 64 + lane];
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);    // and before its slot is handed back
      asm volatile("" ::: "memory");
      if (lane == 0) lds_store(&s_consumed[w][j % PC], (uint32_t)(j / PC) + 1u);
      return v;
    };
    // y of sub-tile ns: lane (g4, nl) holds rows 16 rt + 4 g4 + i of output 16 ns + nl
    auto store_y = [&](int ns, const Tiles<RT>& sum) __attribute__((always_inline)) {
      const int nn = ns * TILE_N + nl;
      if (nn < d.N)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * g4 + i;
            if (r < R) bstore1_sc1(sum.v[rt][i], yr, (uint32_t)((r * d.N + nn) * 4));
          }
    };
    auto put = [&](int u, const Tiles<RT>& sum) __attribute__((always_inline)) {
      const int ns = ns0 + u;
      if (d.S == 1) {
        store_y(ns, sum);
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          bstore_sc1(sum.v[rt], pr, (uint32_t)(ns * d.S + c) * sub_tile + rt * 1024u + lane * 16);
      }
    };
    // waves h and h + PASS_NH: sub-range [a, b), units [f, l] touched (piece
    // u - f of unit u), internal units [u, e), the unit it begins that later
    // waves finish (ul, or -1) and the last of those waves (wl)
    int wv2[2], a2[2], f2[2], u2[2], e2[2], ul2[2], wl2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int w = h + i * PASS_NH;
      const int aw = pass_wave_first(w, PASS_NC, n), bw = pass_wave_first(w + 1, PASS_NC, n);
      wv2[i] = w;
      a2[i] = aw;
      f2[i] = aw / kbc;
      u2[i] = (aw + kbc - 1) / kbc;
      e2[i] = aw < bw ? bw / kbc : u2[i];
      const int ul = (bw - 1) / kbc;
      const bool shared = aw < bw && ul * kbc >= aw && (ul + 1) * kbc > bw;
      ul2[i] = shared ? ul : -1;
      wl2[i] = shared ? pass_step_owner((ul + 1) * kbc - 1, PASS_NC, n) : w;
    }
    Tiles<RT> hv[2];
    hv[0].zero();
    hv[1].zero();
    bool have[2] = {ul2[0] < 0, ul2[1] < 0};
    uint32_t spins = 0;
    for (;;) {
      bool moved = false, pending = false;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (u2[i] < e2[i]) {
          const int j = u2[i] - f2[i];
          if (lds_load(&s_written[wv2[i]]) > (uint32_t)j) {
            Tiles<RT> sum;
            sum.zero();
            sum.add(take(wv2[i], j));
            put(u2[i], sum);
            u2[i] = uni(u2[i] + 1);
            moved = true;
          }
          pending = pending || u2[i] < e2[i];
        }
        if (!have[i]) {                          // the last wave's (first) piece of the shared unit
          if (lds_load(&s_written[wl2[i]]) > 0u) {
            hv[i] = take(wl2[i], 0);
            have[i] = true;
            moved = true;
          } else {
            pending = true;
          }
        }
      }
      if (!pending) break;
      if (!moved) {
        if (++spins > LDS_SPIN_LIMIT) break;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // the shared units, their pieces in wave order (the last wave's taken above)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ul = ul2[i];
      if (ul < 0) continue;
      Tiles<RT> sum;
      sum.zero();
      sum.add(take(wv2[i], ul - f2[i]));
      for (int ww = wv2[i] + 1; ww < wl2[i]; ++ww) {
        if (pass_wave_first(ww, PASS_NC, n) == pass_wave_first(ww + 1, PASS_NC, n)) continue;   // no piece
        sum.add(take(ww, 0));                    // a middle wave's only piece
      }
      sum.add(hv[i]);
      put(ul, sum);
    }
    if (d.S == 1 || units == 0) return;
    // every partial tile of this helper is stored; arrive at each of its units'
    // sub-tile counters (one lane per unit: the units whose first step lies in
    // wave h or h + PASS_NH).  Then the sub-tiles this workgroup adds up: of
    // its units, those with ns mod S = c (so every sub-tile has one such
    // workgroup, and the work is spread evenly rather than left to whichever
    // chunk arrives last): once all S chunks have arrived, the S RT partial
    // tiles (item k = c RT + rt) added per row tile in chunk order, GL loads in
    // flight together.  The counters of all pending sub-tiles are read at once
    // and a round takes the ready sub-tiles that fit: at two row tiles 16 loads
    // (4 sub-tiles of 2 chunks, 2 of 3 or 4), at three 24 (2 sub-tiles of up
    // to 4 chunks); a sub-tile of more items takes rounds of its own.
    // Addresses and sub-tile indices stay in vector registers (no scalar
    // registers tied up across the kernel).
    __builtin_amdgcn_s_waitcnt(0);
    for (int ub = 0; ub < units; ub += 64) {
      const int u = ub + lane;
      if (u < units && pass_step_owner(u * kbc, PASS_NC, n) % PASS_NH == h)
        __hip_atomic_fetch_add(cnt + ns0 + u, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    constexpr int GLN = RT == 3 ? 8 * RT : GL;   // partial tiles in flight per round
    const int per = d.S * RT;
    // one round over up to GLN / PS of the ready sub-tiles in rdy, sub-tile j's items
    // at slots j PS + i (PS >= per, or PS = GLN with rounds of GLN items of one)
    auto gather = [&](auto PSC, uint64_t& rdy, int ub) __attribute__((always_inline)) {
      constexpr int PS = decltype(PSC)::value, NB = GLN / PS;
      int nsj[NB];
      uint32_t off[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        nsj[j] = -1;
        if (rdy) {
          nsj[j] = ns0 + ub + __builtin_ctzll(rdy);
          rdy &= rdy - 1;
        }
        asm volatile("" : "+v"(nsj[j]));        // in a vector register: no scalar registers held
      }
      Tiles<RT> sj[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) sj[j].zero();
      for (int k0 = 0; k0 < per; k0 += GLN) {    // several rounds only for one sub-tile of more than GLN items
#pragma unroll
        for (int j = 0; j < NB; ++j) off[j] = nsj[j] < 0 ? OOB : (uint32_t)(nsj[j] * per + k0) * 1024u + lane * 16;
        f32x4 v[GLN];
#pragma unroll
        for (int k = 0; k < GLN; ++k)            // slots past a sub-tile's items load what follows, unused
          v[k] = bload<f32x4, SC1>(pr, off[k / PS] + (uint32_t)(k % PS) * 1024u);
#pragma unroll
        for (int k = 0; k < GLN; ++k) {
          const int j = k / PS, i = k % PS, rt = i % RT;   // item k0 + i: chunk (k0 + i) / RT, row tile rt
          if (k0 + i < per) sj[j].v[rt] = k0 + i < RT ? v[k] : sj[j].v[rt] + v[k];
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (nsj[j] < 0) continue;
        store_y(nsj[j], sj[j]);
        if (lane == 0) __hip_atomic_store(cnt + nsj[j], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    for (int ub = 0; ub < units; ub += 64) {
      const int u = ub + lane;
      const bool mine = u < units && pass_step_owner(u * kbc, PASS_NC, n) % PASS_NH == h && (ns0 + u) % d.S == c;
      uint64_t pend = __builtin_amdgcn_ballot_w64(mine);
      uint32_t spins = 0;
      while (pend) {
        // the counters of all pending sub-tiles in one read; the complete ones are added up
        bool ready = dead;
        if (!dead && ((pend >> lane) & 1u))
          ready = __hip_atomic_load(cnt + ns0 + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)d.S;
        uint64_t rdy = __builtin_amdgcn_ballot_w64(ready) & pend;
        if (!rdy) {
          if (++spins > SPIN_LIMIT) {
            if (lane == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            dead = true;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        pend &= ~rdy;
        asm volatile("" ::: "memory");           // the partial tiles are read after the arrivals
        while (rdy) {
          if constexpr (RT == 2) {               // several sub-tiles per round where their items fit
            if (per <= 2 * RT)
              gather(std::integral_constant<int, 2 * RT>{}, rdy, ub);
            else if (per <= 4 * RT)
              gather(std::integral_constant<int, 4 * RT>{}, rdy, ub);
            else
              gather(std::integral_constant<int, GLN>{}, rdy, ub);
          } else {
            if (per <= GLN / 2)
              gather(std::integral_constant<int, GLN / 2>{}, rdy, ub);
            else
              gather(std::integral_constant<int, GLN>{}, rdy, ub);
          }
        }
      }
    }
  };

  for (int g = 0; g < G; ++g) {
    const PassGemm d = get_gemm(gemms, g);
    int c, ns0, ns1;
    pass_units(p, d.S, P, d.NS, d.rot, &c, &ns0, &ns1);
    c = uni(c); ns0 = uni(ns0); ns1 = uni(ns1);
    if (g > 0) {
      if (h == 0) {
        if (d.masks)
          gated_wait(d, c);
        else
          grid_wait(g - 1);
        if (lane < PASS_NC * PASS_PIECES) lds_store(&s_consumed[0][0] + lane, 0u);
        if (lane < PASS_NC) lds_store(&s_written[lane], 0u);
        __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
        if (lane == 0) lds_store(&s_go, (uint32_t)g);
      } else {
        uint32_t n = 0;
        while (lds_load(&s_go) < (uint32_t)g) {
          if (++n > LDS_SPIN_LIMIT) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    if (ns1 > ns0) stage_raw(d, c);
    __builtin_amdgcn_s_barrier();                // the raw activations of GEMM g are in LDS
    convert_share(ns1 > ns0 ? d.kbc : 0, PASS_NC + h);
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    __builtin_amdgcn_s_barrier();                // and converted
    if constexpr (RT == 1)
      finish_one(d, g, c, ns0, ns1);
    else
      finish_tiles(d, g, c, ns0, ns1);
    __builtin_amdgcn_s_waitcnt(0);               // this helper's stores of GEMM g are complete
    asm volatile("" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&s_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (h == 0 && g + 1 < G) {
      uint32_t n = 0;
      while (lds_load(&s_done) < (uint32_t)(PASS_NH * (g + 1))) {
        if (++n > LDS_SPIN_LIMIT) break;
        __builtin_amdgcn_s_sleep(1);
      }
      const PassGemm dn = get_gemm(gemms, g + 1);
      if (dn.masks) gated_signal(dn);
      grid_arrive(g);
    }
  }

  // the last workgroup out re-arms the barrier counters for the next launch
  if (h == 0) {
    if (lane == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(bar + 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)P - 1 ? 1u : 0u;
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    if (lds_load(&s_last)) {
      if (lane < 18) {                           // the global, exit and 8 group counters, 8 release words
        const int i = lane == 0 ? 0
                      : lane == 1 ? 16
                      : lane < 10 ? 32 + 32 * (lane - 2)
                                  : PASS_RELEASE_WORD + 32 * (lane - 10);
        __hip_atomic_store(bar + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (lane < PASS_MAX_CHUNKS)                // the gated-input counters
        __hip_atomic_store(bar + PASS_DEP_WORD + PASS_DEP_STRIDE * lane, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int RT>
const void* pass_kernel_for(bool msum) {
  constexpr int RING = pass_ring(RT);
  if constexpr (RT > 1) {
    // several row tiles take the sub-block sums whatever msum says: the
    // products with the mins grow with the row tiles (8 per tile and step)
    (void)msum;
    return reinterpret_cast<const void*>(&pass_kernel<RING, true, RT>);
  } else {
    return msum ? reinterpret_cast<const void*>(&pass_kernel<RING, true, RT>)
                : reinterpret_cast<const void*>(&pass_kernel<RING, false, RT>);
  }
}

hipError_t launch_pass(const PassArgs& a, bool msum, hipStream_t st) {
  const int RT = pass_row_tiles(a.R);
  if (RT < 1 || RT > PASS_MAX_RT) return hipErrorInvalidValue;
  PassArgs args = a;
  void* params[] = {&args};
  const void* k = RT == 1 ? pass_kernel_for<1>(msum) : RT == 2 ? pass_kernel_for<2>(msum) : pass_kernel_for<3>(msum);
  return hipLaunchCooperativeKernel(k, dim3((unsigned)a.P), dim3(PASS_THREADS), params, 0, st);
}

int pass_occupancy() {
  int lo = 1 << 30;
  for (int RT = 1; RT <= PASS_MAX_RT; ++RT)
    for (int m = 0; m < 2; ++m) {
      const void* k = RT == 1 ? pass_kernel_for<1>(m) : RT == 2 ? pass_kernel_for<2>(m) : pass_kernel_for<3>(m);
      int b = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, k, PASS_THREADS, 0) != hipSuccess) return 0;
      lo = b < lo ? b : lo;
    }
  return lo;
}

}  // namespace qg
