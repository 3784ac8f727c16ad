// qgemm_kernels.hip — gfx950 kernels of the weight-streaming Q4_K-style GEMM.
//
// The method (OpenJet multi-agent serving page, section on moving the weights
// only once): the quantised weights are streamed from HBM once per decode step
// and every weight that arrives is applied to all R stacked activation rows, so
// a step costs one weight read whatever R is.  Here that is
//
//   y[r, n] = sum_k w[n, k] x[r, k],  w[n, k] = d sc_s q_k - dmin m_s
//
// computed as, per 256-weight block (d, dmin, sc_s, m_s of output n):
//
//   y[r, n] += d * sum_k (sc_s q_k) x[r, k]  -  sum_s (dmin m_s) X_s[r]
//
// where X_s[r] is the sum of x[r, k] over sub-block s.  sc_s q_k is an integer
// <= 945, exact in binary16, so the first sum runs on the fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulate) with exact products; dmin m_s is
// exact in fp32 and the second sum runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).  x enters the fp16 matrix core as binary16, which
// holds every bf16 value of magnitude in [2^-17, 65504] exactly.
//
// Layouts: layout.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
#include "operand.h"
#include "stream_sched.h"
#include "qgemm_internal.h"

namespace qg {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
// bf16 activations -> matrix-core operand layout + sub-block sums.
// One thread per (row tile, block, lane): 64 contiguous x values of its row.
__global__ void __launch_bounds__(256)
xprep_kernel(const uint16_t* __restrict__ x, f16x8* __restrict__ xq, f32x2* __restrict__ xs,
             int R, int64_t K, int64_t KB, int RT) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)RT * KB * 64;
  if (tid >= total) return;
  int lane = (int)(tid & 63);
  int64_t rj = tid >> 6;               // rt * KB + j
  int rt = (int)(rj / KB);
  int64_t j = rj % KB;
  int g = lane >> 4, rr = lane & 15;
  int r = rt * 16 + rr;
  float vals[64];
  if (r < R) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)r * K + j * SB_W + 64 * g);
    for (int i = 0; i < 8; ++i) {
      u32x4 v = src[i];
      for (int b = 0; b < 4; ++b) {
        vals[8 * i + 2 * b] = bitcast<float>(v[b] << 16);
        vals[8 * i + 2 * b + 1] = bitcast<float>(v[b] & 0xFFFF0000u);
      }
    }
  } else {
    for (int i = 0; i < 64; ++i) vals[i] = 0.0f;
  }
  // vals[32 hbit + c] = x[r, 256 j + 64 g + 32 hbit + c]
  for (int t = 0; t < 8; ++t) {
    f16x8 o;
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)vals[32 * (e & 1) + 4 * t + (e >> 1)];
    xq[(rj * 8 + t) * 64 + lane] = o;
  }
  float s0 = 0.0f, s1 = 0.0f;
  for (int c = 0; c < 32; ++c) s0 += vals[c];
  for (int c = 0; c < 32; ++c) s1 += vals[32 + c];
  xs[rj * 64 + lane] = f32x2{s0, s1};
}

// ---------------------------------------------------------------------------
// Matrix-core streaming GEMM (stream-K over the whole matrix).
//
// Work: a tile is 4 waves x NT sub-tiles x 16 outputs; tile t needs KB block
// steps.  The T*KB (tile, block) steps are cut into P equal contiguous ranges,
// one per workgroup, so every CU gets the same number of bytes to stream
// whatever the shape.  A range that starts or ends inside a tile leaves a
// partial result; the last workgroup to finish a tile sums its partials in
// workgroup order (fixed: results are deterministic) with no waiting.
//
// Per block step each wave reads, for each of its NT sub-tiles, one 2 KiB
// quant chunk and its outputs' 16-byte headers (raw buffer loads, streaming
// hint), three steps deep in a register ring; the x operands of the step are
// shared by the four waves through a two-slot LDS ring.  Loads past the end of
// a range address beyond the buffer's size and return zeros without memory
// traffic, so the tail needs no branches.
constexpr int NWAVE = 4;
constexpr uint32_t OOB = 0x80000000u;   // beyond every buffer (sizes < 2^31)

// aux 2 = streaming (non-temporal) hint for data read once; 0 for shared data
template <class T, int AUX>
__device__ __forceinline__ T bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX));
}

template <int NT>
struct WStage {
  u32x4 qa[NT], qb[NT], hd[NT];
};

template <int RT, int NT>
__global__ void __launch_bounds__(256)
stream_kernel(StreamArgs a) {
  __shared__ u32x4 xl[2][RT][8 * 64];
  __shared__ u32x4 xsl[2][RT][32];
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, nl = lane & 15;
  const int64_t p = blockIdx.x;
  const int64_t I = a.I;
  const int64_t it0 = range_first(p, a.P, I), it1 = range_first(p + 1, a.P, I);
  const int KB = a.KB;

  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc((void*)a.packed, 0, (int)a.quant_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.packed + a.hdr_off), 0, (int)a.hdr_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, (int)(RT * KB * 8192), 0x00020000);
  const __amdgpu_buffer_rsrc_t xsr = __builtin_amdgcn_make_buffer_rsrc((void*)a.xs, 0, (int)(RT * KB * 512), 0x00020000);

  // (tile, block) of the current step and the two steps ahead
  int64_t t_c = it0 / KB;
  int j_c = (int)(it0 - t_c * KB);
  const int j_first = j_c;

  auto load_w = [&](WStage<NT>& st, int64_t it, int64_t t, int j) {
    for (int u = 0; u < NT; ++u) {
      int64_t ns = (t * NWAVE + w) * NT + u;
      bool ok = it < it1 && ns < a.NS;
      uint32_t qo = ok ? (uint32_t)((ns * KB + j) * CHUNK_Q) + lane * 16 : OOB;
      uint32_t ho = ok ? (uint32_t)((ns * KB + j) * CHUNK_H) + nl * 16 : OOB;
      st.qa[u] = bload<u32x4, 2>(qr, qo);
      st.qb[u] = bload<u32x4, 2>(qr, qo + 1024);
      st.hd[u] = bload<u32x4, 2>(hr, ho);
    }
  };
  u32x4 xv[RT][2], xsv_g[RT];
  auto load_x = [&](int64_t it, int j) {
    bool ok = it < it1;
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t base = (uint32_t)((rt * KB + j) * 8192);
      xv[rt][0] = bload<u32x4, 0>(xr, ok ? base + tid * 16 : OOB);
      xv[rt][1] = bload<u32x4, 0>(xr, ok ? base + 4096 + tid * 16 : OOB);
      xsv_g[rt] = bload<u32x4, 0>(xsr, (ok && tid < 32) ? (uint32_t)((rt * KB + j) * 512) + tid * 16 : OOB);
    }
  };
  auto store_x = [&](int slot) {
    for (int rt = 0; rt < RT; ++rt) {
      xl[slot][rt][tid] = xv[rt][0];
      xl[slot][rt][256 + tid] = xv[rt][1];
      if (tid < 32) xsl[slot][rt][tid] = xsv_g[rt];
    }
  };

  f32x4 acc[NT][RT], macc[NT][RT];
  auto zero_acc = [&]() {
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt) {
        acc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        macc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  zero_acc();

  auto advance = [](int64_t& t, int& j, int KB_) {
    if (++j == KB_) { j = 0; ++t; }
  };

  // prologue: x of step it0 into slot 0; weights of it0, it0+1; x of it0+1 in flight
  int64_t t_n1 = t_c, t_n2;
  int j_n1 = j_c, j_n2;
  advance(t_n1, j_n1, KB);
  t_n2 = t_n1; j_n2 = j_n1;
  advance(t_n2, j_n2, KB);
  load_x(it0, j_c);
  store_x(0);
  WStage<NT> W0, W1, W2;
  load_w(W0, it0, t_c, j_c);
  load_w(W1, it0 + 1, t_n1, j_n1);
  load_x(it0 + 1, j_n1);
  __syncthreads();

  int64_t it = it0;
  int slot = 0;

  auto finish_segment = [&](int64_t t, int ja) {
    // segment [ja, j_c] of tile t is complete
    const bool full = (ja == 0) && (j_c == KB - 1);
    if (full) {
      for (int u = 0; u < NT; ++u) {
        int64_t n = ((t * NWAVE + w) * NT + u) * TILE_N + nl;
        if (n >= a.N) continue;
        for (int rt = 0; rt < RT; ++rt)
          for (int i = 0; i < 4; ++i) {
            int r = rt * 16 + 4 * g + i;
            if (r < a.R) a.y[(int64_t)r * a.N + n] = acc[u][rt][i] + macc[u][rt][i];
          }
      }
      return;
    }
    const int64_t pslot = partial_slot(p, t, KB, a.P, I);
    float* dst = a.part + (pslot * NWAVE + w) * (NT * RT * 256);
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt)
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(dst + ((u * RT + rt) * 4 + i) * 64 + lane, acc[u][rt][i] + macc[u][rt][i],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // workgroups that hold a piece of tile t: those containing steps tKB .. tKB+KB-1
    const int64_t q_lo = tile_first_owner(t, KB, a.P, I);
    const int64_t q_hi = tile_last_owner(t, KB, a.P, I);
    if (tid == 0) {
      uint32_t prev = __hip_atomic_fetch_add(a.cnt + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (uint32_t)(q_hi - q_lo)) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last) return;
    f32x4 sum[NT][RT];
    for (int u = 0; u < NT; ++u)
      for (int rt = 0; rt < RT; ++rt) sum[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t q = q_lo; q <= q_hi; ++q) {
      const int64_t qslot = partial_slot(q, t, KB, a.P, I);
      const float* src = a.part + (qslot * NWAVE + w) * (NT * RT * 256);
      for (int u = 0; u < NT; ++u)
        for (int rt = 0; rt < RT; ++rt)
          for (int i = 0; i < 4; ++i)
            sum[u][rt][i] += __hip_atomic_load(src + ((u * RT + rt) * 4 + i) * 64 + lane, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int u = 0; u < NT; ++u) {
      int64_t n = ((t * NWAVE + w) * NT + u) * TILE_N + nl;
      if (n >= a.N) continue;
      for (int rt = 0; rt < RT; ++rt)
        for (int i = 0; i < 4; ++i) {
          int r = rt * 16 + 4 * g + i;
          if (r < a.R) a.y[(int64_t)r * a.N + n] = sum[u][rt][i];
        }
    }
    if (tid == 0) __hip_atomic_store(a.cnt + t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  auto compute = [&](const WStage<NT>& st) {
    f16x8 xa[RT][8];
    f32x2 xs2[RT];
    for (int rt = 0; rt < RT; ++rt) {
      for (int t = 0; t < 8; ++t) xa[rt][t] = __builtin_bit_cast(f16x8, xl[slot][rt][t * 64 + lane]);
      xs2[rt] = reinterpret_cast<const f32x2*>(&xsl[slot][rt][0])[lane];
    }
    for (int u = 0; u < NT; ++u) {
      WConst c = header_consts(st.hd[u], g);
      f32x4 dsum[RT];
      for (int rt = 0; rt < RT; ++rt) dsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < 8; ++t) {
        uint32_t wd = (t < 4) ? st.qa[u][t] : st.qb[u][t - 4];
        f16x8 b = build_b(wd, c);
        for (int rt = 0; rt < RT; ++rt)
          dsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rt][t], b, dsum[rt], 0, 0, 0);
      }
      for (int rt = 0; rt < RT; ++rt) {
        acc[u][rt] += c.d * dsum[rt];
        macc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs2[rt][0], c.bm0, macc[u][rt], 0, 0, 0);
        macc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs2[rt][1], c.bm1, macc[u][rt], 0, 0, 0);
      }
    }
  };

  int ja = j_first;   // first block of the current segment
  // one step: prefetch weights two steps ahead into `ahead`, compute `cur`,
  // stage the next step's x into the other LDS slot, then close the segment if
  // the step ends a tile or the range
  auto step = [&](WStage<NT>& cur, WStage<NT>& ahead) -> bool {
    load_w(ahead, it + 2, t_n2, j_n2);
    compute(cur);
    store_x(slot ^ 1);
    int64_t t_n3 = t_n2;
    int j_n3 = j_n2;
    advance(t_n3, j_n3, KB);
    load_x(it + 2, j_n2);
    __syncthreads();
    const bool last = (it + 1 == it1);
    if (j_c == KB - 1 || last) {
      finish_segment(t_c, ja);
      zero_acc();
      ja = 0;
    }
    ++it;
    slot ^= 1;
    t_c = t_n1; j_c = j_n1;
    t_n1 = t_n2; j_n1 = j_n2;
    t_n2 = t_n3; j_n2 = j_n3;
    return !last;
  };

  while (it < it1) {
    if (!step(W0, W2)) break;
    if (!step(W1, W0)) break;
    if (!step(W2, W1)) break;
  }
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
// per-row argmax, lowest index among equal maxima; NaN never wins
__global__ void __launch_bounds__(1024)
argmax_kernel(const float* __restrict__ y, int64_t N, int32_t* __restrict__ idx) {
  __shared__ float sv[1024];
  __shared__ int64_t si[1024];
  const int64_t r = blockIdx.x;
  const float* row = y + r * N;
  float bv = -__builtin_inff();
  int64_t bi = N;                      // N = "none yet"
  for (int64_t n = threadIdx.x; n < N; n += blockDim.x) {
    float v = row[n];
    if (v > bv || (bi == N && v == bv)) { bv = v; bi = n; }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int st = blockDim.x / 2; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) {
      float ov = sv[threadIdx.x + st];
      int64_t oi = si[threadIdx.x + st];
      float mv = sv[threadIdx.x];
      int64_t mi = si[threadIdx.x];
      bool take = (oi != N) && (mi == N || ov > mv || (ov == mv && oi < mi));
      if (take) { sv[threadIdx.x] = ov; si[threadIdx.x] = oi; }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) idx[r] = (int32_t)(si[0] == N ? 0 : si[0]);
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

hipError_t launch_xprep(const uint16_t* x, void* xq, void* xs, int R, int64_t K, int RT, hipStream_t st) {
  int64_t KB = K / SB_W;
  int64_t total = (int64_t)RT * KB * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(xprep_kernel, dim3(blocks_for(total, 256)), dim3(256), 0, st, x,
                     reinterpret_cast<f16x8*>(xq), reinterpret_cast<f32x2*>(xs), R, K, KB, RT);
  return hipGetLastError();
}

template <int RT, int NT>
static hipError_t launch_stream_t(const StreamArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((stream_kernel<RT, NT>), dim3((unsigned)a.P), dim3(256), 0, st, a);
  return hipGetLastError();
}

#define QG_STREAM_VARIANTS(X) X(1, 1) X(1, 2) X(1, 4) X(2, 1) X(2, 2) X(3, 1) X(4, 1)

hipError_t launch_stream(const StreamArgs& a, hipStream_t st) {
#define QG_CASE(rt, nt) \
  if (a.RT == rt && a.NT == nt) return launch_stream_t<rt, nt>(a, st);
  QG_STREAM_VARIANTS(QG_CASE)
#undef QG_CASE
  return hipErrorInvalidValue;
}

int stream_occupancy(int RT, int NT) {
  int blocks = 0;
#define QG_CASE(rt, nt) \
  if (RT == rt && NT == nt) { \
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, stream_kernel<rt, nt>, 256, 0) != hipSuccess) return 0; \
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

}  // namespace qg
