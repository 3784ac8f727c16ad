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
// Matrix-core GEMM.  A wave owns NT consecutive sub-tiles (16 outputs each)
// over the block range of one K split, and all RT row tiles (16 rows each).
// Per block it loads x operands once (shared by its sub-tiles) and for every
// sub-tile one 2 KiB quant chunk and the 16-byte header of its output.
template <int RT, int NT>
__global__ void __launch_bounds__(256)
mfma_kernel(const uint8_t* __restrict__ packed, const f16x8* __restrict__ xq,
            const f32x2* __restrict__ xs, float* __restrict__ out, int64_t N, int64_t KB,
            int64_t NS, int R, int S, int64_t kbs, int64_t hdr_off) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t NG = (NS + NT - 1) / NT;
  const int64_t s = gw / NG;
  if (s >= S) return;
  const int64_t ng = gw - s * NG;
  const int64_t ns0 = ng * NT;
  const int64_t j0 = s * kbs;
  const int64_t j1 = (j0 + kbs < KB) ? j0 + kbs : KB;
  const int g = lane >> 4, nl = lane & 15;

  const uint8_t* qbase = packed + lane * 16;
  const uint8_t* hbase = packed + hdr_off + nl * 16;

  f32x4 acc[NT][RT], macc[NT][RT];
  for (int u = 0; u < NT; ++u)
    for (int rt = 0; rt < RT; ++rt) {
      acc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      macc[u][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  bool valid[NT];
  for (int u = 0; u < NT; ++u) valid[u] = (ns0 + u) < NS;

  u32x4 qa[NT], qb[NT], hd[NT];
  f16x8 xa[RT][8];
  f32x2 xsv[RT];

  auto load = [&](int64_t j, u32x4* qa_, u32x4* qb_, u32x4* hd_, f16x8 (*xa_)[8], f32x2* xs_) {
    for (int u = 0; u < NT; ++u) {
      int64_t ns = valid[u] ? ns0 + u : ns0;
      const uint8_t* qp = qbase + quant_chunk_off(ns, j, KB);
      qa_[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp));
      qb_[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qp + 1024));
      hd_[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(hbase + header_chunk_off(ns, j, KB)));
    }
    for (int rt = 0; rt < RT; ++rt) {
      const f16x8* xp = xq + ((rt * KB + j) * 8) * 64 + lane;
      for (int t = 0; t < 8; ++t) xa_[rt][t] = xp[t * 64];
      xs_[rt] = xs[(rt * KB + j) * 64 + lane];
    }
  };

  if (j0 < j1) load(j0, qa, qb, hd, xa, xsv);
  for (int64_t j = j0; j < j1; ++j) {
    u32x4 nqa[NT], nqb[NT], nhd[NT];
    f16x8 nxa[RT][8];
    f32x2 nxs[RT];
    const bool more = (j + 1 < j1);
    if (more) load(j + 1, nqa, nqb, nhd, nxa, nxs);
    for (int u = 0; u < NT; ++u) {
      WConst c = header_consts(hd[u], g);
      f32x4 dsum[RT];
      for (int rt = 0; rt < RT; ++rt) dsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < 8; ++t) {
        uint32_t w = (t < 4) ? qa[u][t] : qb[u][t - 4];
        f16x8 b = build_b(w, c);
        for (int rt = 0; rt < RT; ++rt)
          dsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[rt][t], b, dsum[rt], 0, 0, 0);
      }
      for (int rt = 0; rt < RT; ++rt) {
        acc[u][rt] += c.d * dsum[rt];
        macc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsv[rt][0], c.bm0, macc[u][rt], 0, 0, 0);
        macc[u][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xsv[rt][1], c.bm1, macc[u][rt], 0, 0, 0);
      }
    }
    if (more) {
      for (int u = 0; u < NT; ++u) { qa[u] = nqa[u]; qb[u] = nqb[u]; hd[u] = nhd[u]; }
      for (int rt = 0; rt < RT; ++rt) {
        for (int t = 0; t < 8; ++t) xa[rt][t] = nxa[rt][t];
        xsv[rt] = nxs[rt];
      }
    }
  }

  // lane (g, nl) holds rows 16 rt + 4 g + i, output 16 ns + nl
  float* dst = out + s * (int64_t)R * N;
  for (int u = 0; u < NT; ++u) {
    if (!valid[u]) continue;
    int64_t n = (ns0 + u) * TILE_N + nl;
    if (n >= N) continue;
    for (int rt = 0; rt < RT; ++rt)
      for (int i = 0; i < 4; ++i) {
        int r = rt * 16 + 4 * g + i;
        if (r < R) dst[(int64_t)r * N + n] = acc[u][rt][i] + macc[u][rt][i];
      }
  }
}

// y[r, n] = sum over splits s = 0, 1, ..., S-1 of part[s, r, n] (fixed order)
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, float* __restrict__ y, int64_t RN, int S) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= RN) return;
  float v = part[i];
  for (int s = 1; s < S; ++s) v += part[(int64_t)s * RN + i];
  y[i] = v;
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
static hipError_t launch_mfma_t(const MfmaArgs& a, hipStream_t st) {
  int64_t NG = (a.NS + NT - 1) / NT;
  int64_t waves = NG * a.S;
  hipLaunchKernelGGL((mfma_kernel<RT, NT>), dim3(blocks_for(waves, 4)), dim3(256), 0, st, a.packed,
                     reinterpret_cast<const f16x8*>(a.xq), reinterpret_cast<const f32x2*>(a.xs), a.out,
                     a.N, a.KB, a.NS, a.R, a.S, a.kbs, a.hdr_off);
  return hipGetLastError();
}

hipError_t launch_mfma(const MfmaArgs& a, hipStream_t st) {
  switch (a.RT * 16 + a.NT) {
    case 1 * 16 + 1: return launch_mfma_t<1, 1>(a, st);
    case 1 * 16 + 2: return launch_mfma_t<1, 2>(a, st);
    case 1 * 16 + 4: return launch_mfma_t<1, 4>(a, st);
    case 2 * 16 + 1: return launch_mfma_t<2, 1>(a, st);
    case 2 * 16 + 2: return launch_mfma_t<2, 2>(a, st);
    case 3 * 16 + 1: return launch_mfma_t<3, 1>(a, st);
    case 3 * 16 + 2: return launch_mfma_t<3, 2>(a, st);
    case 4 * 16 + 1: return launch_mfma_t<4, 1>(a, st);
    case 4 * 16 + 2: return launch_mfma_t<4, 2>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_reduce(const float* part, float* y, int64_t RN, int S, hipStream_t st) {
  if (RN == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks_for(RN, 256)), dim3(256), 0, st, part, y, RN, S);
  return hipGetLastError();
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
