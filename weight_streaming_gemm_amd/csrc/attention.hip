// attention.hip — gfx950 decode attention of the agents' step rows over their
// own KV caches (split over the sequence, then one combine pass).
//
// OpenJet multi-agent serving page, section on moving the weights only once:
// the stacked rows share every weight read, but each agent reads its own KV
// cache, and attention grows with the number of agents.  An agent's step has
// `rows` query rows (its current token and its drafts) at positions L, L + 1,
// ... of its sequence; their keys and values are already in its cache.  Row i
// sees positions 0 .. L + i.  Query head hq reads key/value head hq / 8
// (groups of 8 query heads); head size 128; scores q.k / sqrt(128).
//
// Split kernel: workgroup (s, h, a) takes positions [s split, (s + 1) split) of
// agent a's cache for key/value head h, for all rows x 8 query heads of the
// group at once (at most 32 query vectors: the columns of two 16 x 16
// matrix-core tiles).  Each of its 4 waves takes every 4th tile of 32 positions:
//   S^T = K Q^T     bf16 matrix-core products, fp32 (exact products); a lane
//                   holds 8 scores of one query vector
//   online softmax  fp32, base-2 exponent with log2(e) / sqrt(128) folded in;
//                   a vector's maximum and sum over its 4 lanes
//   O^T += V^T P^T  P as a binary16 head + tail pair (P in [0, 1]: the pair
//                   holds it to about 2^-22) straight from the softmax's
//                   registers, V converted bf16 -> binary16 (exact), two fp16
//                   matrix-core products, fp32 accumulation
// V reaches its operand layout through a small LDS area per wave (transposed,
// its positions placed in the k slots where the lanes hold P).  The waves'
// (max, sum, O) are merged in LDS and written as the split's partial result (O
// not yet divided by the sum).  Combine kernel: per (agent, row, query head), the
// splits' partials rescaled to the common maximum and divided by the sum.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"
#include "attention.h"

namespace qg {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t w32x4 __attribute__((ext_vector_type(4)));

constexpr int AD = ATTN_HEAD_DIM;       // 128
constexpr int GRP = ATTN_GROUP;         // 8 query heads per key/value head
constexpr int TK = 32;                  // positions per wave step
constexpr int NWAVE = 4;
constexpr uint32_t AOOB = 0x80000000u;  // beyond every buffer: the load returns zeros

// per-wave LDS: V^T [128 dims][32 positions] as binary16, rows padded to 80 bytes
constexpr int PSTRIDE = 80, VBYTES = AD * PSTRIDE;
constexpr int WAVE_LDS = VBYTES;
// merge area: per wave (max, sum) of 32 rows and O [32][128] fp32
constexpr int MERGE_LDS = NWAVE * (32 * 2 * 4 + 32 * AD * 4);
constexpr int ATTN_LDS = (NWAVE * WAVE_LDS > MERGE_LDS) ? NWAVE * WAVE_LDS : MERGE_LDS;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes >= 0x80000000ull ? 0x80000000u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ w32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(w32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// v of the lane that the data-parallel-primitive control CTRL picks within the
// lane's row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float row_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// maximum and sum over the 16 lanes of a row, the same in every lane: lanes
// paired as lane ^ 1, lane ^ 2 (quad permutations), then the other quad of the
// half row and the other half of the row (mirrors).  The sum is associated as
// ((q0 + q1) + (q2 + q3)) over the four quads' sums in every lane.
// (scores are never NaN: the maximum needs no NaN rule)
__device__ __forceinline__ float row16_max(float v) {
  v = __builtin_fmaxf(v, row_dpp<0xB1>(v));           // quad_perm [1, 0, 3, 2]
  v = __builtin_fmaxf(v, row_dpp<0x4E>(v));           // quad_perm [2, 3, 0, 1]
  v = __builtin_fmaxf(v, row_dpp<0x141>(v));          // row_half_mirror
  v = __builtin_fmaxf(v, row_dpp<0x140>(v));          // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row_dpp<0xB1>(v);
  v += row_dpp<0x4E>(v);
  v += row_dpp<0x141>(v);
  v += row_dpp<0x140>(v);
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

}  // namespace

__global__ void __launch_bounds__(NWAVE * 64)
attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[ATTN_LDS];
  const int s = blockIdx.x, h = blockIdx.y, ag = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, nl = lane & 15;
  const int rows = a.rows, nq = rows * GRP;                 // query vectors of the group
  const int L0 = a.lengths[ag];
  const int L = L0 < 0 ? 0 : (L0 > a.max_len ? a.max_len : L0);
  const int total = L + rows;                               // positions the last row sees
  const int SPLIT = a.split;                                // positions per workgroup
  const int p_begin = s * SPLIT;
  if (p_begin >= total) return;                             // the combine reads only splits below total
  const int p_end = p_begin + SPLIT < total ? p_begin + SPLIT : total;
  const int Hq = a.Hkv * GRP;
  const uint64_t cache_bytes = (uint64_t)a.A * a.cap * a.Hkv * AD * 2;
  const __amdgpu_buffer_rsrc_t kr = rsrc(a.k, cache_bytes), vr = rsrc(a.v, cache_bytes);
  const __amdgpu_buffer_rsrc_t qr = rsrc(a.q, (uint64_t)a.A * rows * Hq * AD * 2);

  // B operands of Q: row tile rt, k-step c: query vector 16 rt + nl (row i =
  // vector / 8, head h * 8 + vector % 8), dims 32 c + 8 g .. + 7
  b16x8 qa[2][4];
  for (int rt = 0; rt < 2; ++rt) {
    const int qv = 16 * rt + nl;
    const uint32_t base = qv < nq ? (uint32_t)((((ag * rows + qv / GRP) * Hq + h * GRP + qv % GRP) * AD) * 2) : AOOB;
    for (int c = 0; c < 4; ++c)
      qa[rt][c] = __builtin_bit_cast(b16x8, load16(qr, base == AOOB ? AOOB : base + (32 * c + 8 * g) * 2));
  }

  // softmax state of query vector 16 rt + nl (the same in the 4 lane groups)
  const float NEG = -__builtin_inff();
  float mrow[2], lrow[2];
  f32x4 o[2][8];                                            // O[16 rt + nl][16 dt + 4 g + i]
  for (int rt = 0; rt < 2; ++rt) { mrow[rt] = NEG; lrow[rt] = 0.f; }
  for (int rt = 0; rt < 2; ++rt)
    for (int dt = 0; dt < 8; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* vbuf = lds + w * WAVE_LDS;                        // V^T of the wave's step
  // byte offset of (position p, head h, dim d) in a cache
  // (head-major: a head's positions are contiguous, a step's K or V one 8 KB run)
  auto coff = [&](int p, int d) { return (uint32_t)((((uint64_t)ag * a.Hkv + h) * a.cap + p) * AD + d) * 2; };

  // loads of one 32-position step: K as A operands (position 16 kt + nl, dims
  // 32 c + 8 g .. + 7); V as 512 chunks of 16 bytes, lane (dc, m) taking
  // positions 2m and 2m + 1 of dim chunks 4 it + dc.  The next step's loads go
  // out as soon as this step's K (after S) and V (after its LDS copy) are used.
  const int vm = lane & 15, vdc = lane >> 4;
  b16x8 kb[2][4];
  w32x4 vc[8];
  auto load_k = [&](int t0) __attribute__((always_inline)) {
    for (int kt = 0; kt < 2; ++kt) {
      const int p = t0 + 16 * kt + nl;
      for (int c = 0; c < 4; ++c)
        kb[kt][c] = __builtin_bit_cast(b16x8, load16(kr, p < p_end ? coff(p, 32 * c + 8 * g) : AOOB));
    }
  };
  auto load_v = [&](int t0) __attribute__((always_inline)) {
    for (int it = 0; it < 4; ++it)
      for (int e = 0; e < 2; ++e) {
        const int pp = t0 + 2 * vm + e;
        vc[2 * it + e] = load16(vr, pp < p_end ? coff(pp, 8 * (4 * it + vdc)) : AOOB);
      }
  };
  load_k(p_begin + TK * w);
  load_v(p_begin + TK * w);
  for (int t0 = p_begin + TK * w; t0 < p_end; t0 += TK * NWAVE) {
    const int tn = t0 + TK * NWAVE;                         // the next step (loads return zeros past p_end)
    // S^T = K Q^T; lane (g, nl) holds S[16 rt + nl][16 kt + 4 g + i]: the lane's
    // query vector is its column, the same in all the products below
    f32x4 sc[2][2];
    for (int rt = 0; rt < 2; ++rt)
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kt][c], qa[rt][c], acc, 0, 0, 0);
        sc[rt][kt] = acc;
      }
    load_k(tn);
    // mask, scale, online softmax: a vector's 32 scores sit 8 per lane in the 4
    // lanes nl, nl + 16, nl + 32, nl + 48
    h16x8 pb[2], pl[2];                                     // P^T as B operands: head and tail
    for (int rt = 0; rt < 2; ++rt) {
      const int qv = 16 * rt + nl;
      const int last = L + qv / GRP;                        // vector qv's row sees positions <= last
      float x[2][4];
      float mx = NEG;
      for (int kt = 0; kt < 2; ++kt)
        for (int i = 0; i < 4; ++i) {
          const int p = t0 + 16 * kt + 4 * g + i;
          x[kt][i] = (qv < nq && p < p_end && p <= last) ? sc[rt][kt][i] * a.scale_log2 : NEG;
          mx = __builtin_fmaxf(mx, x[kt][i]);
        }
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
      mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = __builtin_fmaxf(mrow[rt], mx);
      // a vector with no visible position yet keeps alpha = 1 and P = 0
      const bool live = mnew != NEG;
      const float alpha = live ? __builtin_amdgcn_exp2f(mrow[rt] - mnew) : 1.f;
      float sum = 0.f;
      for (int kt = 0; kt < 2; ++kt)
        for (int i = 0; i < 4; ++i) {
          // k slot 8 g + 4 kt + i of the product holds position 16 kt + 4 g + i
          const float pv = live ? __builtin_amdgcn_exp2f(x[kt][i] - mnew) : 0.f;
          sum += pv;
          const _Float16 hi = (_Float16)pv;
          pb[rt][4 * kt + i] = hi;
          pl[rt][4 * kt + i] = (_Float16)(pv - (float)hi);
        }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      mrow[rt] = mnew;
      lrow[rt] = lrow[rt] * alpha + sum;
      for (int dt = 0; dt < 8; ++dt) o[rt][dt] *= alpha;
    }
    // V^T (bf16 -> binary16) with its positions in the k slots of P^T: one 4-byte
    // write per dim holds positions 2m and 2m + 1
    __asm__ volatile("" ::: "memory");
    const int pos = 2 * vm;
    const int slot = pos < 16 ? 8 * (pos >> 2) + (pos & 3) : 8 * ((pos - 16) >> 2) + 4 + (pos & 3);
    for (int it = 0; it < 4; ++it) {
      const w32x4 a0 = vc[2 * it], a1 = vc[2 * it + 1];
      const uint32_t w0[4] = {a0.x, a0.y, a0.z, a0.w}, w1[4] = {a1.x, a1.y, a1.z, a1.w};
      const int d0 = 8 * (4 * it + vdc);
      for (int j = 0; j < 8; ++j) {
        const float f0 = (j & 1) ? bf16_hi(w0[j >> 1]) : bf16_lo(w0[j >> 1]);
        const float f1 = (j & 1) ? bf16_hi(w1[j >> 1]) : bf16_lo(w1[j >> 1]);
        typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<h16x2*>(vbuf + (d0 + j) * PSTRIDE + slot * 2) = h16x2{(_Float16)f0, (_Float16)f1};
      }
    }
    load_v(tn);
    __asm__ volatile("" ::: "memory");       // one wave's LDS accesses run in order
    // O^T += V^T P^T (P as head + tail)
    for (int dt = 0; dt < 8; ++dt) {
      const h16x8 va = *reinterpret_cast<const h16x8*>(vbuf + (16 * dt + nl) * PSTRIDE + 16 * g);
      for (int rt = 0; rt < 2; ++rt) {
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[rt], o[rt][dt], 0, 0, 0);
        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pl[rt], o[rt][dt], 0, 0, 0);
      }
    }
    __asm__ volatile("" ::: "memory");       // the next step's LDS writes come after these reads
  }

  // merge the 4 waves: (max, sum) per row, O rescaled to the common max
  __syncthreads();                                          // the per-wave areas become the merge area
  float* mlw = reinterpret_cast<float*>(lds);               // [wave][32 rows][2]
  float* ow = mlw + NWAVE * 32 * 2;                         // [wave][32 rows][128]
  for (int rt = 0; rt < 2; ++rt) {
    const int qv = 16 * rt + nl;
    if (g == 0) {
      mlw[(w * 32 + qv) * 2] = mrow[rt];
      mlw[(w * 32 + qv) * 2 + 1] = lrow[rt];
    }
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(ow + (w * 32 + qv) * AD + 16 * dt + 4 * g) = o[rt][dt];
  }
  __syncthreads();
  const size_t item = ((size_t)ag * a.Hkv + h) * a.nsplit + s;
  for (int e = tid; e < nq * AD; e += NWAVE * 64) {
    const int qv = e / AD, d = e % AD;
    float m = NEG;
    for (int ww = 0; ww < NWAVE; ++ww) m = mlw[(ww * 32 + qv) * 2] > m ? mlw[(ww * 32 + qv) * 2] : m;
    float acc = 0.f, l = 0.f;
    if (m != NEG)
      for (int ww = 0; ww < NWAVE; ++ww) {
        const float f = __builtin_amdgcn_exp2f(mlw[(ww * 32 + qv) * 2] - m);
        acc += f * ow[(ww * 32 + qv) * AD + d];
        l += f * mlw[(ww * 32 + qv) * 2 + 1];
      }
    a.part_o[(item * 32 + qv) * AD + d] = acc;
    if (d == 0) {
      a.part_ml[(item * 32 + qv) * 2] = m;
      a.part_ml[(item * 32 + qv) * 2 + 1] = l;
    }
  }
}

// out[a][i][hq][d]: the splits of (agent, key/value head) rescaled to the common
// maximum, summed in split order, divided by the summed weights.  The splits are
// read 16 at a time with all their loads in flight together (the partials come
// from other dies' caches: each round trip is long); the running maximum moves
// from one group of 16 to the next, and with at most 16 splits there is one
// group, so every split is scaled by the overall maximum directly.
__global__ void __launch_bounds__(AD)
attn_combine_kernel(AttnArgs a, float* __restrict__ out) {
  constexpr int CH = 16;
  constexpr float NEG_INF = -__builtin_inff();
  const int hq = blockIdx.x, i = blockIdx.y, ag = blockIdx.z, d = threadIdx.x;
  const int h = hq / GRP, qv = i * GRP + hq % GRP, Hq = a.Hkv * GRP;
  const int L0 = a.lengths[ag];
  const int total = (L0 < 0 ? 0 : (L0 > a.max_len ? a.max_len : L0)) + a.rows;
  const int ns = (total + a.split - 1) / a.split;           // <= nsplit (sized for max_len)
  const size_t item0 = ((size_t)ag * a.Hkv + h) * a.nsplit;
  float m = NEG_INF, acc = 0.f, l = 0.f;
  for (int s0 = 0; s0 < ns; s0 += CH) {
    float mv[CH], lv[CH], ov[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      // past the last split, the last split's address (loaded and not used): the
      // loads carry no branches and issue back to back
      const bool ok = s0 + u < ns;
      const size_t it = (item0 + (ok ? s0 + u : ns - 1)) * 32 + qv;
      const float mu = a.part_ml[it * 2], lu = a.part_ml[it * 2 + 1], ou = a.part_o[it * AD + d];
      mv[u] = ok ? mu : NEG_INF;
      lv[u] = ok ? lu : 0.f;
      ov[u] = ok ? ou : 0.f;
    }
    float mc = m;
#pragma unroll
    for (int u = 0; u < CH; ++u) mc = mv[u] > mc ? mv[u] : mc;
    if (mc == NEG_INF) continue;                              // no position of these splits is visible
    if (m != NEG_INF) {                                       // earlier groups to the new maximum
      const float sc = __builtin_amdgcn_exp2f(m - mc);
      acc *= sc;
      l *= sc;
    }
    m = mc;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if (mv[u] == NEG_INF) continue;
      const float f = __builtin_amdgcn_exp2f(mv[u] - m);
      acc += f * ov[u];
      l += f * lv[u];
    }
  }
  out[(((size_t)ag * a.rows + i) * Hq + hq) * AD + d] = acc / l;
}

hipError_t launch_attention(const AttnArgs& a, float* out, hipStream_t st) {
  if (a.A == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_split_kernel, dim3((unsigned)a.nsplit, (unsigned)a.Hkv, (unsigned)a.A), dim3(NWAVE * 64),
                     0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(a.Hkv * GRP), (unsigned)a.rows, (unsigned)a.A), dim3(AD), 0,
                     st, a, out);
  return hipGetLastError();
}

}  // namespace qg

// ---- C ABI (include/qgemm.h) ------------------------------------------------
namespace {
bool attn_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

using namespace qg;

extern "C" {

int qgemm_attention_workspace_size(int agents, int rows, int kv_heads, int max_len, size_t* bytes) {
  if (!bytes) return QGEMM_EINVAL;
  if (agents < 0 || kv_heads < 1 || max_len < 0 || rows < 1 || rows > ATTN_MAX_ROWS) return QGEMM_ESHAPE;
  *bytes = attn_ws_bytes(agents, kv_heads, rows, max_len);
  return QGEMM_OK;
}

int qgemm_decode_attention(const void* q_bf16, const void* k_cache, const void* v_cache, const int32_t* lengths,
                           int agents, int rows, int q_heads, int kv_heads, int head_dim, int cap, int max_len,
                           float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (agents < 0 || kv_heads < 1 || rows < 1 || rows > ATTN_MAX_ROWS || head_dim != ATTN_HEAD_DIM ||
      q_heads != ATTN_GROUP * kv_heads || max_len < 0 || cap < max_len + rows)
    return QGEMM_ESHAPE;
  // every offset into q, the caches and the workspace must fit the kernels' 32-bit buffer offsets
  const uint64_t cache_bytes = (uint64_t)agents * cap * kv_heads * ATTN_HEAD_DIM * 2;
  const uint64_t q_bytes = (uint64_t)agents * rows * q_heads * ATTN_HEAD_DIM * 2;
  if (cache_bytes >= (uint64_t(1) << 31) || q_bytes >= (uint64_t(1) << 31)) return QGEMM_ESHAPE;
  if (agents == 0) return QGEMM_OK;
  if (!q_bf16 || !k_cache || !v_cache || !lengths || !out || !workspace) return QGEMM_EINVAL;
  if (workspace_bytes < attn_ws_bytes(agents, kv_heads, rows, max_len)) return QGEMM_EINVAL;
  if (!attn_aligned16(q_bf16) || !attn_aligned16(k_cache) || !attn_aligned16(v_cache) || !attn_aligned16(out) || !attn_aligned16(workspace))
    return QGEMM_EALIGN;
  AttnArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q_bf16);
  a.k = reinterpret_cast<const uint16_t*>(k_cache);
  a.v = reinterpret_cast<const uint16_t*>(v_cache);
  a.lengths = lengths;
  a.A = agents;
  a.rows = rows;
  a.Hkv = kv_heads;
  a.cap = cap;
  a.max_len = max_len;
  a.split = attn_split_len(agents, kv_heads, max_len, rows);
  a.nsplit = attn_splits(agents, kv_heads, max_len, rows);
  a.part_o = reinterpret_cast<float*>(workspace);
  a.part_ml = a.part_o + (size_t)agents * kv_heads * a.nsplit * 32 * ATTN_HEAD_DIM;
  a.scale_log2 = (float)(1.4426950408889634 / 11.313708498984761);   // log2(e) / sqrt(128)
  return launch_attention(a, out, reinterpret_cast<hipStream_t>(stream)) == hipSuccess ? QGEMM_OK : QGEMM_EHIP;
}

}  // extern "C"
