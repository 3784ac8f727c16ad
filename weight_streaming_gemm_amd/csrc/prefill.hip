// prefill.hip — the same fused dequantise-and-multiply for many rows: a prompt
// chunk (tens to thousands of rows) together with the agents' decode rows.
//
// The OpenJet page's claim that a long prompt need not stall decode (section on
// what the design buys: another agent's 20K-token prefill running while the
// others decode) needs the prompt's rows to go through the same weight pass.
// With hundreds of rows a weight is used hundreds of times, so the product is
// bound by the matrix cores, not by the weight stream: this kernel tiles rows
// as well as outputs, and every weight read serves a 128-row tile.
//
//   y[r, n] = sum_k w[n, k] x[r, k],  w[n, k] = d sc_s q_k - dmin m_s
//
// is computed per 256-weight block exactly as in the streaming kernel:
// ds = sum_k (sc_s q_k) x[r, k] on the fp16 matrix cores (exact integer B
// operands, fp32 sums) and ms = sum_s m_s X_s from the fp32 sub-block sums X_s
// written as two binary16 parts of X_s / 256 (one v_mfma_f32_16x16x16_f16 per
// tile against the mins, as in the pass kernel), then acc += d ds - 256 dmin ms.
//
// Work: one workgroup per (128-row tile, output tile of 32 WN), over the whole
// of K (no split unless the grid is small, so every output is written once, in
// a fixed order).  2 x WN waves (WN = 4 or 6: two or three per SIMD): two along
// the rows, WN along the outputs; a wave owns 64 rows (4 row tiles of 16) x 32
// outputs (2 sub-tiles of 16): 8 accumulator tiles.  A first kernel converts x
// once into the LDS image of every (128-row tile, block): binary16 operands in
// the matrix-core lane layout plus the 8 sub-block sums per row (72 KiB).  The
// main kernel copies each block's image straight into LDS with buffer loads
// that write LDS directly (no registers, no vector instructions),
// double-buffered: the next block's activations and weights are in flight
// while the current block is multiplied.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "operand.h"
#include "prefill_plan.h"
#include "qgemm_internal.h"

namespace qg {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// The min term's sub-block sums as matrix-core A operands: X_s / 256 (in
// binary16's range for |x| <= 65504) in two binary16 parts, hi = f16(X_s / 256)
// and lo = f16(X_s / 256 - hi) (the difference exact in fp32): lane group g holds
// (hi_2g, hi_2g+1, lo_2g, lo_2g+1) of its row, and B = (m_2g, m_2g+1, m_2g,
// m_2g+1) of its output, so one 16 x 16 x 16 product adds m_s (hi + lo) over the
// 8 sub-blocks; the 256 goes back into -dmin (exact).
__device__ __forceinline__ f16x4 sum_parts(float s0, float s1) {
  const float a0 = s0 * (1.0f / 256.0f), a1 = s1 * (1.0f / 256.0f);
  const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
  return f16x4{h0, h1, (_Float16)(a0 - (float)h0), (_Float16)(a1 - (float)h1)};
}
__device__ __forceinline__ f16x4 min_parts_b(const WConst& c) { return f16x4{c.m[0], c.m[1], c.m[0], c.m[1]}; }



__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}

// s plus the eight bf16 values of a 16-byte load, each widened exactly to fp32
// (a bf16 is the high half of a binary32), added in order.  (A chain of bf16
// dot products against ones over the four dwords of one vector was compiled to
// four reads of the first dword on gfx950, so plain adds are used.)
__device__ __forceinline__ float sum8_bf16(u32x4 v, float s) {
  for (int i = 0; i < 4; ++i) {
    s += __builtin_bit_cast(float, v[i] << 16);
    s += __builtin_bit_cast(float, v[i] & 0xFFFF0000u);
  }
  return s;
}

}  // namespace

// grid (row tiles of 64 WM, output tiles of 32 WN, K chunks); WM x WN waves:
// WM along the rows, WN side by side along the outputs
template <int WM, int WN, int RTW>
__global__ void __launch_bounds__(64 * WM * WN, RTW == 2 ? 2 : 1)
prefill_kernel(const uint8_t* __restrict__ packed, uint32_t quant_bytes, uint32_t hdr_bytes,
               const uint8_t* __restrict__ ximg, uint32_t img_bytes, float* __restrict__ y, int R, int N, int NS,
               int KB, int kc, int64_t slice) {
  constexpr int PF_WN = WN, PF_WAVES = WM * WN, PF_RT = RTW, MT = WM * PF_RT;
  constexpr int PF_BUF = pf_buf(MT), NCH = PF_BUF / PF_CHUNK;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * PF_BUF];
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, nl = lane & 15;
  const int wm = w % WM, wn = w / WM;                // the wave's place in the WM x WN grid
  const int m0 = blockIdx.x * (MT * 16);             // first row of the workgroup
  const int ns0 = (blockIdx.y * PF_WN + wn) * PF_U;  // first sub-tile of the wave
  // K in gridDim.z chunks of kc blocks: chunk z covers blocks jb .. je - 1 and
  // writes its partial sums to slice z (R x N, `slice` floats apart) of y; with
  // one chunk, y itself
  const int jb = blockIdx.z * kc, je = jb + kc < KB ? jb + kc : KB;
  y += (int64_t)blockIdx.z * slice;

  const __amdgpu_buffer_rsrc_t qr = rsrc(packed, quant_bytes);
  const __amdgpu_buffer_rsrc_t hr = rsrc(packed + quant_bytes, hdr_bytes);
  constexpr uint32_t OOB = 0x80000000u;

  // ---- weights of block j for the wave's sub-tiles (past N: no traffic, zeros) ----
  struct WB { u32x4 qa[PF_U], qb[PF_U], hd[PF_U]; };
  auto load_w = [&](WB& b, int j) __attribute__((always_inline)) {
    for (int u = 0; u < PF_U; ++u) {
      const int ns = ns0 + u;
      const bool ok = ns < NS;
      const uint32_t qo = ok ? (uint32_t)(ns * KB + j) * CHUNK_Q + lane * 16 : OOB;
      const uint32_t ho = ok ? (uint32_t)(ns * KB + j) * CHUNK_H + nl * 16 : OOB;
      b.qa[u] = load16<2>(qr, qo);
      b.qb[u] = load16<2>(qr, qo + 1024);
      b.hd[u] = load16<2>(hr, ho);
    }
  };

  // ---- activations of block j: its 72 one-KiB chunks of the image, 18 per wave,
  // copied into LDS buffer `buf` by buffer loads that write LDS (lane l's 16
  // bytes land at the chunk's base + 16 l) ----
  const __amdgpu_buffer_rsrc_t ir = rsrc(ximg, img_bytes);
  auto stage_x = [&](int j, int buf) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)pf_chunk_off(blockIdx.x, j, KB, MT, 0);
    for (int c = w; c < NCH; c += PF_WAVES) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ir, (__attribute__((address_space(3))) void*)(lds + buf * PF_BUF + c * PF_CHUNK), 16,
          base + (uint32_t)(c * PF_CHUNK + lane * 16), 0, 0, 0);
    }
  };

  f32x4 acc[PF_RT][PF_U];
  for (int rt = 0; rt < PF_RT; ++rt)
    for (int u = 0; u < PF_U; ++u) acc[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- one block: ds on the matrix cores over its 8 steps, then the min term ----
  auto compute = [&](const WB& b, int buf) __attribute__((always_inline)) {
    const uint8_t* const X = lds + buf * PF_BUF;
    WConst c[PF_U];
    for (int u = 0; u < PF_U; ++u) c[u] = header_consts(b.hd[u].x, b.hd[u].y, b.hd[u].z, b.hd[u].w, g4);
    f32x4 ds[PF_RT][PF_U];
    for (int rt = 0; rt < PF_RT; ++rt)
      for (int u = 0; u < PF_U; ++u) ds[rt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < 8; ++t) {
      f16x8 a[PF_RT];
      for (int rt = 0; rt < PF_RT; ++rt)
        a[rt] = *reinterpret_cast<const f16x8*>(X + pf_operand_chunk(wm * PF_RT + rt, t) * PF_CHUNK + lane * 16);
      for (int u = 0; u < PF_U; ++u) {
        const uint32_t wd = t < 4 ? b.qa[u][t] : b.qb[u][t - 4];
        const f16x8 bo = build_b(wd, c[u]);
        for (int rt = 0; rt < PF_RT; ++rt)
          ds[rt][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[rt], bo, ds[rt][u], 0, 0, 0);
      }
    }
    f16x4 bm[PF_U];
    float nmin[PF_U];
    for (int u = 0; u < PF_U; ++u) {
      bm[u] = min_parts_b(c[u]);
      nmin[u] = c[u].nmin * 256.0f;
    }
    for (int rt = 0; rt < PF_RT; ++rt) {
      const f16x4 sx = *reinterpret_cast<const f16x4*>(X + pf_sum_chunk(MT, wm * PF_RT + rt) * PF_CHUNK + lane * 16);
      for (int u = 0; u < PF_U; ++u) {
        const f32x4 ms = __builtin_amdgcn_mfma_f32_16x16x16f16(sx, bm[u], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        for (int i = 0; i < 4; ++i) {
          acc[rt][u][i] = __builtin_fmaf(c[u].d, ds[rt][u][i], acc[rt][u][i]);
          acc[rt][u][i] = __builtin_fmaf(nmin[u], ms[i], acc[rt][u][i]);
        }
      }
    }
  };

  // ---- the K loop, two blocks per pass so that the register buffers alternate
  // without copies; block j + 1's loads are in flight during block j ----
  WB wa, wb;
  stage_x(jb, 0);
  load_w(wa, jb);
  __syncthreads();
  for (int j = jb; j < je; j += 2) {
    const bool more1 = j + 1 < je, more2 = j + 2 < je;
    if (more1) { stage_x(j + 1, 1); load_w(wb, j + 1); }
    compute(wa, 0);
    __syncthreads();
    if (!more1) break;
    if (more2) { stage_x(j + 2, 0); load_w(wa, j + 2); }
    compute(wb, 1);
    __syncthreads();
  }

  // ---- outputs: lane (g, nl) of tile (rt, u) holds rows 4 g .. 4 g + 3 of output nl ----
  typedef float __attribute__((address_space(1))) global_float;
  global_float* const yg = (global_float*)y;
  for (int u = 0; u < PF_U; ++u) {
    const int n = (ns0 + u) * TILE_N + nl;
    if (n >= N) continue;
    for (int rt = 0; rt < PF_RT; ++rt)
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + (wm * PF_RT + rt) * 16 + 4 * g4 + i;
        if (row < R) yg[(int64_t)row * N + n] = acc[rt][u][i];
      }
  }
}

// The LDS image of x for workgroups of MT row tiles: for row tile group m and
// block j, at (m KB + j) * 9 MT KiB, chunk (row tile rt, step t) at 1 KiB (8 rt + t)
// holds lane 16 g + r's binary16 A operand of row 16 (MT m + rt) + r (k = 256 j +
// 64 g + 32 (e & 1) + 4 t + (e >> 1) for element e), and chunk 8 MT + rt the
// sub-block sums of those rows (lane 16 g + r: the two binary16 parts of X_2g /
// 256 and X_2g+1 / 256, then 8 zero bytes).  Rows past R are zeros.  One thread per
// (m, j, rt, lane): it reads the row's 64 values of sub-blocks 2g, 2g + 1 (one
// 128-byte line) and writes 8 operands and one sum entry.
__global__ void __launch_bounds__(256)
prefill_image_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ img, int R, int KB, int MT, int64_t total) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  const int lane = (int)(id & 63), g = lane >> 4, r = lane & 15;
  const int64_t q = id >> 6;                       // (m KB + j) * MT + rt
  const int rt = (int)(q % MT);
  const int64_t mj = q / MT;
  const int64_t m = mj / KB, j = mj - m * KB;
  const int64_t row = m * (MT * 16) + rt * 16 + r;
  u32x4 v[8];
  if (row < R) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + row * (int64_t)KB * SB_W + j * SB_W + 64 * g);
    for (int c = 0; c < 8; ++c) v[c] = src[c];
  } else {
    for (int c = 0; c < 8; ++c) v[c] = u32x4{0u, 0u, 0u, 0u};
  }
  uint8_t* const dst = img + pf_chunk_off(m, j, KB, MT, 0);
  // v[c] holds k = 64 g + 8 c .. 8 c + 7: c < 4 sub-block 2g, c >= 4 sub-block 2g + 1
  for (int t = 0; t < 8; ++t) {
    const u32x4 lo = v[t >> 1], hi = v[4 + (t >> 1)];
    const int o = (t & 1) * 2;                     // dwords of k = 4 t .. 4 t + 3 within the 8-value load
    *reinterpret_cast<f16x8*>(dst + pf_operand_chunk(rt, t) * PF_CHUNK + lane * 16) =
        build_a(lo[o], lo[o + 1], hi[o], hi[o + 1]);
  }
  float s0 = 0.f, s1 = 0.f;
  for (int c = 0; c < 4; ++c) s0 = sum8_bf16(v[c], s0);
  for (int c = 4; c < 8; ++c) s1 = sum8_bf16(v[c], s1);
  const f16x4 parts = sum_parts(s0, s1);
  *reinterpret_cast<u32x4*>(dst + pf_sum_chunk(MT, rt) * PF_CHUNK + lane * 16) =
      u32x4{__builtin_bit_cast(uint32_t, f16x2{parts[0], parts[1]}), __builtin_bit_cast(uint32_t, f16x2{parts[2], parts[3]}), 0u, 0u};
}

// y[i] = sum over chunks z = 0 .. S-1 of part[z * slice + i], in chunk order;
// up to 16 chunks' loads are issued before the adds (the planner makes at most
// KB / 8 chunks, and more than 16 only for K > 32768)
__global__ void __launch_bounds__(256)
prefill_reduce_kernel(const float* __restrict__ part, float* __restrict__ y, int64_t count, int64_t slice, int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float s = 0.f;
  for (int z0 = 0; z0 < S; z0 += 16) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = z0 + k < S ? part[(z0 + k) * slice + i] : 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (z0 + k < S) s = (z0 + k == 0) ? v[k] : s + v[k];
  }
  y[i] = s;
}

hipError_t launch_prefill(const uint8_t* packed, int64_t N, int64_t K, const void* x, float* y, int R,
                          const PrefillPlan& p, void* ws, hipStream_t st) {
  const int64_t NS = padded_n(N) / TILE_N, KB = K / SB_W;
  const uint32_t qb = (uint32_t)quant_region_bytes(N, K);
  const uint32_t hb = (uint32_t)(packed_bytes(N, K) - quant_region_bytes(N, K));
  uint8_t* const img = reinterpret_cast<uint8_t*>(ws);
  const int MT = p.wm * p.rtw;
  const int64_t total = p.mt * KB * MT * 64;
  hipLaunchKernelGGL(prefill_image_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const uint16_t*>(x), img, R, (int)KB, MT, total);
  const dim3 grid((unsigned)p.mt, (unsigned)p.nt, (unsigned)p.S);
  float* out = p.S > 1 ? reinterpret_cast<float*>(img + p.img_bytes) : y;
  const int64_t slice = p.S > 1 ? p.slice : 0;
#define QG_PF_LAUNCH(WM_, WN_, RT_)                                                                          \
  hipLaunchKernelGGL((prefill_kernel<WM_, WN_, RT_>), grid, dim3(64 * WM_ * WN_), 0, st, packed, qb, hb, img,    \
                     (uint32_t)p.img_bytes, out, R, (int)N, (int)NS, (int)KB, (int)p.kc, slice)
  if (p.wm == 2 && p.wn == 6)
    QG_PF_LAUNCH(2, 6, 4);
  else if (p.wm == 1 && p.wn == 8 && p.rtw == 2)
    QG_PF_LAUNCH(1, 8, 2);
  else if (p.wm == 1 && p.wn == 8)
    QG_PF_LAUNCH(1, 8, 4);
  else
    QG_PF_LAUNCH(2, 4, 4);
#undef QG_PF_LAUNCH
  if (p.S > 1) {
    const int64_t count = (int64_t)R * N;
    hipLaunchKernelGGL(prefill_reduce_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, st, out, y, count,
                       p.slice, (int)p.S);
  }
  return hipGetLastError();
}

}  // namespace qg
