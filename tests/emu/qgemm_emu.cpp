// qgemm_emu.cpp — CPU emulation of the gfx950 kernels' data flow, lane by lane.
//
// Test infrastructure: it compiles the library's own layout.h / operand.h /
// stream_sched.h (the code the kernels run) for the host and replays the pack,
// the streaming kernel (activation staging into the operand layout, the
// matrix-core steps with the documented lane layout of
// v_mfma_f32_16x16x32_f16, the stream-K schedule with partial tiles and
// last-arriver sums, several GEMMs sharing one workspace) and the
// dequantisation kernel thread by thread.  It lets the CPU suite check every
// index mapping against the fp64 oracle before any GPU run.  The matrix-core
// lane layout assumed here is itself checked on the GPU by a probe test.
#include <stdint.h>
#include <string.h>
#include <vector>

#include "../../weight_streaming_gemm_amd/csrc/layout.h"
#include "../../weight_streaming_gemm_amd/csrc/operand.h"
#include "../../weight_streaming_gemm_amd/csrc/stream_sched.h"
#include "../../weight_streaming_gemm_amd/csrc/prefill_plan.h"
#include "../../weight_streaming_gemm_amd/csrc/pass_sched.h"
#include <algorithm>
#include <cmath>
#include <random>

using namespace qg;

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

// D = A x B + C on a 16 x 16 tile with K = 32 (fp16 in, fp32 out); per lane:
// a[l][e] = A[l % 16][8 (l / 16) + e], b[l][e] = B[8 (l / 16) + e][l % 16],
// d[l][v] = D[4 (l / 16) + v][l % 16]
void mfma_16x16x32(const f16x8* a, const f16x8* b, f32x4* c) {
  float A[16][32], B[32][16];
  for (int l = 0; l < 64; ++l)
    for (int e = 0; e < 8; ++e) {
      A[l % 16][8 * (l / 16) + e] = (float)a[l][e];
      B[8 * (l / 16) + e][l % 16] = (float)b[l][e];
    }
  f32x4 out[64];
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < 4; ++v) {
      int i = 4 * (l / 16) + v, j = l % 16;
      double s = c[l][v];
      for (int k = 0; k < 32; ++k) s += (double)A[i][k] * (double)B[k][j];
      out[l][v] = (float)s;
    }
  for (int l = 0; l < 64; ++l) c[l] = out[l];
}

// D = A x B + C on a 16 x 16 tile with K = 4 (fp32 in, fp32 out); per lane:
// a[l] = A[l % 16][l / 16], b[l] = B[l / 16][l % 16], d[l][v] = D[4 (l / 16) + v][l % 16]
void mfma_16x16x4_f32(const float* a, const float* b, f32x4* c) {
  f32x4 out[64];
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * (l / 16) + v, j = l % 16;
      double s = c[l][v];
      for (int k = 0; k < 4; ++k) s += (double)a[16 * k + i] * (double)b[16 * k + j];
      out[l][v] = (float)s;
    }
  for (int l = 0; l < 64; ++l) c[l] = out[l];
}

// the min term of a block from fp32 sub-block sums: xs[l] = (X_2g, X_2g+1) of
// lane l's row, the mins of lane l's output from c[l]; two products of depth 4
void min_term_f32(const float (*xs)[2], const WConst* c, f32x4* ms) {
  for (int h = 0; h < 2; ++h) {
    float a[64], b[64];
    for (int l = 0; l < 64; ++l) {
      a[l] = xs[l][h];
      b[l] = min_operand(c[l], h);
    }
    mfma_16x16x4_f32(a, b, ms);
  }
}

// The pass kernel's form of the same min term: X_s / 256 in two binary16 parts
// (hi = f16(X_s / 256), lo = f16(X_s / 256 - hi)), lane group g's A holding
// (hi_2g, hi_2g+1, lo_2g, lo_2g+1) of its row and B (m_2g, m_2g+1, m_2g, m_2g+1)
// of its output, in one 16 x 16 x 16 product; the caller scales -dmin by 256.
void min_term_parts(const float (*xs)[2], const WConst* c, f32x4* ms) {
  float A[16][16], B[16][16];
  for (int l = 0; l < 64; ++l) {
    float part[4];
    for (int h = 0; h < 2; ++h) {
      const float a = xs[l][h] * (1.0f / 256.0f);
      const _Float16 hi = (_Float16)a;
      part[h] = (float)hi;
      part[2 + h] = (float)(_Float16)(a - (float)hi);
    }
    for (int e = 0; e < 4; ++e) {
      A[l % 16][4 * (l / 16) + e] = part[e];
      B[4 * (l / 16) + e][l % 16] = (float)c[l].m[e & 1];
    }
  }
  f32x4 out[64];
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < 4; ++v) {
      const int i = 4 * (l / 16) + v, j = l % 16;
      double s = ms[l][v];
      for (int k = 0; k < 16; ++k) s += (double)A[i][k] * (double)B[k][j];
      out[l][v] = (float)s;
    }
  for (int l = 0; l < 64; ++l) ms[l] = out[l];
}

void pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K) {
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  for (int64_t ns = 0; ns < NS; ++ns)
    for (int64_t j = 0; j < KB; ++j)
      for (int lane = 0; lane < 64; ++lane) {
        int g = lane >> 4, nl = lane & 15;
        int64_t n = ns * TILE_N + nl;
        uint8_t blk[SB_CANON];
        if (n < N) memcpy(blk, canon + (n * KB + j) * SB_CANON, SB_CANON);
        else memset(blk, 0, SB_CANON);
        uint8_t* qdst = packed + quant_chunk_off(ns, j, KB) + lane * 16;
        for (int h = 0; h < 2; ++h)
          for (int u = 0; u < 4; ++u) {
            uint32_t w = pack_quant_dword(blk, g, 4 * h + u);
            memcpy(qdst + h * 1024 + 4 * u, &w, 4);
          }
        if (g == 0) {
          uint32_t hd[4];
          pack_header(blk, hd);
          memcpy(packed + quant_region_bytes(N, K) + header_chunk_off(ns, j, KB) + nl * 16, hd, 16);
        }
      }
}


// ---- the row-tiled kernel (prefill.hip): plan, activation image, product ----

// the image as prefill_image_kernel lays it out: per (row tile group m, block j,
// row tile rt, lane 16 g + r) the row's 64 values of sub-blocks 2g, 2g + 1 as 8
// A operands and the two sums (bf16 widened to fp32, added in k order; kept here
// in fp32, and split into the kernel's two binary16 parts by min_term_parts)
void prefill_image(const uint16_t* x, int R, int64_t KB, int MT, int64_t mt, std::vector<uint8_t>& img) {
  img.assign((size_t)mt * KB * pf_buf(MT), 0);
  for (int64_t m = 0; m < mt; ++m)
    for (int64_t j = 0; j < KB; ++j)
      for (int rt = 0; rt < MT; ++rt)
        for (int lane = 0; lane < 64; ++lane) {
          const int g = lane >> 4, r = lane & 15;
          const int64_t row = m * MT * 16 + rt * 16 + r;
          uint32_t v[32];                       // 64 bf16 values as 32 dwords
          for (int i = 0; i < 32; ++i) {
            uint32_t d = 0;
            if (row < R) memcpy(&d, x + row * KB * SB_W + j * SB_W + 64 * g + 2 * i, 4);
            v[i] = d;
          }
          for (int t = 0; t < 8; ++t) {
            const int lo = 2 * t, hi = 16 + 2 * t;   // dwords of k = 4 t .. 4 t + 3 and 32 further on
            const f16x8 op = build_a(v[lo], v[lo + 1], v[hi], v[hi + 1]);
            memcpy(img.data() + pf_chunk_off(m, j, KB, MT, pf_operand_chunk(rt, t)) + lane * 16, &op, 16);
          }
          float s0 = 0.f, s1 = 0.f;
          for (int i = 0; i < 16; ++i) {
            s0 += bitcast<float>(v[i] << 16);
            s0 += bitcast<float>(v[i] & 0xFFFF0000u);
          }
          for (int i = 16; i < 32; ++i) {
            s1 += bitcast<float>(v[i] << 16);
            s1 += bitcast<float>(v[i] & 0xFFFF0000u);
          }
          const float sv[4] = {s0, s1, 0.f, 0.f};
          memcpy(img.data() + pf_chunk_off(m, j, KB, MT, pf_sum_chunk(MT, rt)) + lane * 16, sv, 16);
        }
}

int64_t x_slot_of_emu(int64_t j, int64_t j0, int64_t KB) { return (j - j0 + KB) % KB; }

// Activation staging of one range: the kernel's x_load / x_store, slot b <-
// block (j0 + b) mod KB for b < nslots; slot layout [b][t][gg][r < R] of
// 16-byte A operands, and per (b, gg, r) the fp32 sums of sub-blocks 2 gg and
// 2 gg + 1.
struct Sum2 { float v[2]; };
void convert_x(const uint16_t* x, int R, int64_t K, int64_t jbase, int64_t kbv, int64_t j0, int64_t nslots,
               std::vector<f16x8>& slots, std::vector<Sum2>& sums) {
  const int64_t KB = kbv;   // blocks of the step order's tile (a chunk's with K in chunks)
  slots.assign((size_t)nslots * 8 * 4 * R, f16x8{});
  sums.assign((size_t)nslots * 4 * R, Sum2{});
  for (int64_t b = 0; b < nslots; ++b)
    for (int r = 0; r < R; ++r)
      for (int gg = 0; gg < 4; ++gg)
        for (int t = 0; t < 8; ++t) {
          int64_t j = j0 + b;
          if (j >= KB) j -= KB;
          j += jbase;
          const uint16_t* lo = x + (int64_t)r * K + j * SB_W + 64 * gg + 4 * t;
          const uint32_t d0 = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
          const uint32_t d1 = (uint32_t)lo[2] | ((uint32_t)lo[3] << 16);
          const uint32_t d2 = (uint32_t)lo[32] | ((uint32_t)lo[33] << 16);
          const uint32_t d3 = (uint32_t)lo[34] | ((uint32_t)lo[35] << 16);
          slots[(size_t)((b * 8 + t) * 4 + gg) * R + r] = build_a(d0, d1, d2, d3);
        }
  // sub-block sums: thread t adds its four bf16 values of each run (the kernel
  // uses two bf16 dot products with ones, which may round differently), then the
  // eight threads' partial sums are added in the kernel's tree order
  for (int64_t b = 0; b < nslots; ++b)
    for (int r = 0; r < R; ++r)
      for (int gg = 0; gg < 4; ++gg) {
        int64_t j = j0 + b;
        if (j >= KB) j -= KB;
        j += jbase;
        float p0[8], p1[8];
        for (int t = 0; t < 8; ++t) {
          const uint16_t* lo = x + (int64_t)r * K + j * SB_W + 64 * gg + 4 * t;
          auto f = [](uint16_t v) { return bitcast<float>((uint32_t)v << 16); };
          p0[t] = ((f(lo[0]) + f(lo[1])) + f(lo[2])) + f(lo[3]);
          p1[t] = ((f(lo[32]) + f(lo[33])) + f(lo[34])) + f(lo[35]);
        }
        sums[(size_t)(b * 4 + gg) * R + r] = Sum2{{tree8(p0), tree8(p1)}};
      }
}

// the A operand of lane (row tile rt, lane) at step t from slot b; rows >= R
// of a row tile read row R - 1 (their products are never stored)
f16x8 a_operand(const std::vector<f16x8>& slots, int R, int64_t b, int rt, int t, int lane) {
  int r = rt * 16 + (lane & 15);
  const int gg = lane >> 4;
  if (r >= R) r = R - 1;
  return slots[(size_t)((b * 8 + t) * 4 + gg) * R + r];
}
// the sub-block sums of lane (row tile rt, lane)'s row from slot b
Sum2 s_operand(const std::vector<Sum2>& sums, int R, int64_t b, int rt, int lane) {
  int r = rt * 16 + (lane & 15);
  const int gg = lane >> 4;
  if (r >= R) r = R - 1;
  return sums[(size_t)(b * 4 + gg) * R + r];
}

// One step of a wave at sub-tiles ns0 .. ns0 + NT - 1, block j (activation
// slot b): the kernel's compute() for its NT sub-tiles and all 64 lanes,
// accumulating into acc[NT][RT][64].
void wave_step(const uint8_t* packed, int64_t hdr_off, int64_t ns0, int NT, int64_t NS, int64_t j, int64_t KB,
               const std::vector<f16x8>& slots, const std::vector<Sum2>& sums, int R, int64_t b, int RT,
               int msum, f32x4* acc) {
  for (int u = 0; u < NT; ++u) {
    const int64_t ns = ns0 + u;
    WConst c[64];
    f16x8 bm[64];
    uint32_t qd[64][8];
    for (int lane = 0; lane < 64; ++lane) {
      uint32_t h[4] = {0, 0, 0, 0};
      if (ns < NS) {
        const uint8_t* qp = packed + lane * 16 + quant_chunk_off(ns, j, KB);
        memcpy(qd[lane], qp, 16);
        memcpy(qd[lane] + 4, qp + 1024, 16);
        memcpy(h, packed + hdr_off + (lane & 15) * 16 + header_chunk_off(ns, j, KB), 16);
      } else {
        memset(qd[lane], 0, sizeof(qd[lane]));   // loads past the end return zeros
      }
      c[lane] = header_consts(h[0], h[1], h[2], h[3], lane >> 4);
      bm[lane] = build_m_full(c[lane]);
    }
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 ds[64], ms[64];
      for (int l = 0; l < 64; ++l) ds[l] = ms[l] = f32x4{0, 0, 0, 0};
      if (msum) {
        float sv[64][2];
        for (int lane = 0; lane < 64; ++lane) {
          const Sum2 sp = s_operand(sums, R, b, rt, lane);
          sv[lane][0] = sp.v[0];
          sv[lane][1] = sp.v[1];
        }
        if (msum == 2)
          min_term_parts(sv, c, ms);
        else
          min_term_f32(sv, c, ms);
      }
      for (int tt = 0; tt < 8; ++tt) {
        f16x8 av[64], bb[64];
        for (int lane = 0; lane < 64; ++lane) {
          av[lane] = a_operand(slots, R, b, rt, tt, lane);
          bb[lane] = build_b(qd[lane][tt], c[lane]);
        }
        mfma_16x16x32(av, bb, ds);
        if (!msum) mfma_16x16x32(av, bm, ms);
      }
      f32x4* ac = acc + (size_t)(u * RT + rt) * 64;
      for (int lane = 0; lane < 64; ++lane)
        for (int i = 0; i < 4; ++i) {
          float v = ac[lane][i];
          v = std::fma(c[lane].d, ds[lane][i], v);
          v = std::fma(msum == 2 ? c[lane].nmin * 256.0f : c[lane].nmin, ms[lane][i], v);
          ac[lane][i] = v;
        }
    }
  }
}

struct EmuGemm {
  std::vector<uint8_t> packed;
  const uint16_t* x;
  float* y;
  int64_t N, K, KB, NS, T, I, V, hdr_off;
  int64_t S, KBv, Treal;   // K in S chunks of KBv blocks; T = S Treal virtual tiles
  int nwn, aligned, msum;
};

}  // namespace

extern "C" {

// Emulated launch of the streaming kernel over G GEMMs (shapes N[g] x K[g],
// canonical weights canon[g], bf16 x[g], outputs y[g]): NW waves per
// workgroup in an nwn[g] x (NW / nwn[g]) grid, tiles of nwn[g] * NT
// sub-tiles, V[g] ranges per GEMM (one per workgroup).  GEMM by GEMM (the
// launch's barrier); ranges in a seeded random order (the arrival order at
// tiles shared between ranges); waves of a range one after another (the
// pieces of a tile shared by waves meet in "LDS" and are added in sub-range
// order after the range); one partial-slot workspace and one set of tile
// counters shared by all GEMMs.  Returns 0, -1 on a bad plan, -2 if a tile
// counter is left armed, -3 on an inconsistent activation slot.
int emu_stream_seq(int G, const uint8_t* const* canon, const int64_t* Ns, const int64_t* Ks,
                   const uint16_t* const* xs, float* const* ys, int R, int NT, int NW, const int* nwns,
                   const int64_t* Vs, const int* aligned, const int* msums, const int* chunks,
                   uint64_t order_seed) {
  const int RT = (R + 15) / 16;
  std::vector<EmuGemm> gs((size_t)G);
  int64_t Tmax = 0, Vslots = 0;
  for (int g = 0; g < G; ++g) {
    EmuGemm& e = gs[(size_t)g];
    e.N = Ns[g]; e.K = Ks[g]; e.KB = e.K / SB_W; e.NS = padded_n(e.N) / TILE_N;
    e.nwn = nwns[g];
    e.aligned = aligned[g];
    e.msum = msums[g];
    if (e.nwn < 1 || NW % e.nwn) return -1;
    e.Treal = (e.NS + (int64_t)e.nwn * NT - 1) / ((int64_t)e.nwn * NT);
    e.S = chunks[g];
    if (e.S < 1 || e.KB % e.S) return -1;
    e.KBv = e.KB / e.S;
    e.T = e.S * e.Treal;
    e.I = e.T * e.KBv;
    e.V = Vs[g];
    if (e.V > (e.aligned ? e.T : e.I) || e.V < 1) return -1;
    // K in chunks: ranges of whole tiles of one chunk each
    if (e.S > 1 && (!e.aligned || e.V % e.S || e.nwn != 1)) return -1;
    e.packed.resize((size_t)packed_bytes(e.N, e.K));
    pack(canon[g], e.packed.data(), e.N, e.K);
    e.hdr_off = quant_region_bytes(e.N, e.K);
    e.x = xs[g];
    e.y = ys[g];
    Tmax = std::max(Tmax, e.Treal);
    Vslots = std::max(Vslots, std::max(2 * e.V * e.nwn, e.T * e.nwn));
  }
  const size_t tile_f4 = (size_t)NT * RT * 64;            // f32x4 per wave piece (one column of a tile)
  std::vector<f32x4> part((size_t)Vslots * tile_f4, f32x4{NAN, NAN, NAN, NAN});
  std::vector<uint32_t> cnt((size_t)Tmax, 0);
  std::vector<f16x8> xslots;
  std::vector<Sum2> xsums;
  std::mt19937_64 rng(order_seed);
  for (int g = 0; g < G; ++g) {
    EmuGemm& e = gs[(size_t)g];
    const int64_t KB = e.KBv;   // blocks per tile of the step order
    const int nwn = e.nwn, nwk = NW / e.nwn;
    for (int64_t i = 0; i < (int64_t)R * e.N; ++i) e.y[i] = std::nanf("");
    // column wn of tile t: sub-tiles (t nwn + wn) NT + u
    auto write_y = [&](int64_t t, int wn, const f32x4* v) {
      for (int u = 0; u < NT; ++u)
        for (int rt = 0; rt < RT; ++rt)
          for (int lane = 0; lane < 64; ++lane)
            for (int i = 0; i < 4; ++i) {
              const int64_t n = ((t * nwn + wn) * NT + u) * TILE_N + (lane & 15);
              const int r = rt * 16 + 4 * (lane >> 4) + i;
              if (n < e.N && r < R) e.y[(int64_t)r * e.N + n] = v[(size_t)(u * RT + rt) * 64 + lane][i];
            }
    };
    // a full tile's result: y, or with K in chunks the chunk's partial (slot vt)
    auto tile_result = [&](int64_t vt, int wn, const f32x4* v) {
      if (e.S == 1) {
        write_y(vt, wn, v);
      } else {
        std::copy(v, v + tile_f4, part.begin() + (size_t)(vt * nwn + wn) * tile_f4);
      }
    };
    std::vector<int64_t> order((size_t)e.V);
    for (int64_t v = 0; v < e.V; ++v) order[(size_t)v] = v;
    std::shuffle(order.begin(), order.end(), rng);
    for (int64_t v : order) {
      // equal step ranges, or ranges of whole tiles
      const int64_t A = e.aligned ? KB * range_first(v, e.V, e.T) : range_first(v, e.V, e.I);
      const int64_t B = e.aligned ? KB * range_first(v + 1, e.V, e.T) : range_first(v + 1, e.V, e.I);
      const int64_t L = B - A;
      const int64_t j0 = A % KB;
      const int64_t jbase = (A / KB / e.Treal) * KB;          // the range's chunk
      convert_x(e.x, R, e.K, jbase, KB, j0, x_slots(A, B, KB), xslots, xsums);
      // pieces[wk][slot][wn][tile_f4]
      auto piece = [&](int64_t wk, int sl, int wn) { return (size_t)((wk * 2 + sl) * nwn + wn) * tile_f4; };
      std::vector<f32x4> pieces((size_t)NW * 2 * tile_f4, f32x4{NAN, NAN, NAN, NAN});
      for (int w = 0; w < NW; ++w) {
        const int wn = w % nwn, wk = w / nwn;
        const int64_t a_w = A + range_first<int64_t>(wk, nwk, L), b_w = A + range_first<int64_t>(wk + 1, nwk, L);
        std::vector<f32x4> acc(tile_f4, f32x4{0, 0, 0, 0});
        int64_t ja = a_w % KB;
        for (int64_t it = a_w; it < b_w; ++it) {
          const int64_t t = it / KB, j = it % KB;
          const int64_t b = (it - A) % KB;
          if (b != x_slot_of_emu(j, j0, KB)) return -3;
          const int64_t tr = t % e.Treal, jr = (t / e.Treal) * KB + j;   // output tile, block
          if ((t / e.Treal) * KB != jbase) return -3;
          wave_step(e.packed.data(), e.hdr_off, (tr * nwn + wn) * NT, NT, e.NS, jr, e.KB, xslots, xsums, R, b, RT,
                    e.msum != 0 ? 2 : 0, acc.data());
          const bool sub_end = it + 1 == b_w;
          if (j != KB - 1 && !sub_end) continue;
          if (ja == 0 && j == KB - 1) {
            tile_result(t, wn, acc.data());
          } else {
            const int sl = (a_w > t * KB) ? 0 : 1;
            std::copy(acc.begin(), acc.end(), pieces.begin() + piece(wk, sl, wn));
          }
          std::fill(acc.begin(), acc.end(), f32x4{0, 0, 0, 0});
          ja = 0;
        }
      }
      // after the range: tiles shared by waves, then tiles shared with other ranges
      const int64_t tA = A / KB, tB = (B - 1) / KB;
      const bool cross_a = tA * KB < A, cross_b = (tB + 1) * KB > B;
      for (int64_t t = tA; t <= tB; ++t)
        for (int wn = 0; wn < nwn; ++wn) {
          const int64_t s0 = std::max(A, t * KB) - A, s1 = std::min(B, (t + 1) * KB) - A;
          const int64_t k_lo = range_owner<int64_t>(s0, nwk, L), k_hi = range_owner<int64_t>(s1 - 1, nwk, L);
          const bool crossing = (t == tA && cross_a) || (t == tB && cross_b);
          if (k_lo == k_hi && !crossing) continue;
          std::vector<f32x4> sum(tile_f4, f32x4{0, 0, 0, 0});
          for (int64_t kk = k_lo; kk <= k_hi; ++kk) {
            const int64_t a_k = A + range_first<int64_t>(kk, nwk, L), b_k = A + range_first<int64_t>(kk + 1, nwk, L);
            if (a_k == b_k) continue;
            const int sl = (a_k > t * KB) ? 0 : 1;
            for (size_t k = 0; k < tile_f4; ++k) sum[k] += pieces[piece(kk, sl, wn) + k];
          }
          if (!crossing) {
            tile_result(t, wn, sum.data());
          } else {
            const int64_t gsl = partial_slot(v, t, KB, e.V, e.I);
            std::copy(sum.begin(), sum.end(), part.begin() + (size_t)(gsl * nwn + wn) * tile_f4);
          }
        }
      auto arrive = [&](int64_t t) {
        const int64_t q_lo = tile_first_owner(t, KB, e.V, e.I), q_hi = tile_last_owner(t, KB, e.V, e.I);
        const uint32_t prev = cnt[(size_t)t]++;
        if (prev != (uint32_t)(q_hi - q_lo)) return;
        for (int wn = 0; wn < nwn; ++wn) {
          std::vector<f32x4> sum(tile_f4, f32x4{0, 0, 0, 0});
          for (int64_t q = q_lo; q <= q_hi; ++q) {
            const int64_t qs = partial_slot(q, t, KB, e.V, e.I);
            for (size_t k = 0; k < tile_f4; ++k) sum[k] += part[(size_t)(qs * nwn + wn) * tile_f4 + k];
          }
          write_y(t, wn, sum.data());
        }
        cnt[(size_t)t] = 0;
      };
      if (cross_a) arrive(tA);
      if (cross_b && !(cross_a && tB == tA)) arrive(tB);
      if (e.S > 1 && A < B) {
        // K in chunks: arrive at the range's output tiles; the last of the S
        // chunks adds the partials in chunk order
        for (int64_t t = tA; t <= tB; ++t) {
          const int64_t tr = t % e.Treal;
          if (++cnt[(size_t)tr] != (uint32_t)e.S) continue;
          for (int wn = 0; wn < nwn; ++wn) {
            std::vector<f32x4> sum(tile_f4, f32x4{0, 0, 0, 0});
            for (int64_t c = 0; c < e.S; ++c)
              for (size_t k = 0; k < tile_f4; ++k) sum[k] += part[(size_t)((c * e.Treal + tr) * nwn + wn) * tile_f4 + k];
            write_y(tr, wn, sum.data());
          }
          cnt[(size_t)tr] = 0;
        }
      }
    }
    for (int64_t t = 0; t < Tmax; ++t)
      if (cnt[(size_t)t] != 0) return -2;   // a counter was left armed
  }
  return 0;
}

int emu_stream(const uint8_t* canon, int64_t N, int64_t K, const uint16_t* x, int R, int NT, int NW, int nwn,
               int64_t V, int aligned, int msum, int chunks, uint64_t order_seed, float* y) {
  return emu_stream_seq(1, &canon, &N, &K, &x, &y, R, NT, NW, &nwn, &V, &aligned, &msum, &chunks, order_seed);
}

int emu_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K) {
  pack(canon, packed, N, K);
  return 0;
}

// Emulated dequantisation kernel (from the packed layout).
int emu_dequant(const uint8_t* canon, int64_t N, int64_t K, float* w) {
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  std::vector<uint8_t> packed((size_t)packed_bytes(N, K));
  pack(canon, packed.data(), N, K);
  int64_t hdr_off = quant_region_bytes(N, K);
  for (int64_t ns = 0; ns < NS; ++ns)
    for (int64_t j = 0; j < KB; ++j)
      for (int lane = 0; lane < 64; ++lane) {
        int g = lane >> 4, nl = lane & 15;
        int64_t n = ns * TILE_N + nl;
        if (n >= N) continue;
        uint32_t q[8], h[4];
        const uint8_t* qp = packed.data() + quant_chunk_off(ns, j, KB) + lane * 16;
        memcpy(q, qp, 16);
        memcpy(q + 4, qp + 1024, 16);
        memcpy(h, packed.data() + hdr_off + header_chunk_off(ns, j, KB) + nl * 16, 16);
        uint32_t F = header_group(h[1], h[2], h[3], g);
        float d = (float)bitcast<_Float16>((uint16_t)(h[0] & 0xFFFFu));
        float dmin = (float)bitcast<_Float16>((uint16_t)(h[0] >> 16));
        float A[2] = {d * (float)grp_sc(F, 0), d * (float)grp_sc(F, 1)};
        float B[2] = {dmin * (float)grp_m(F, 0), dmin * (float)grp_m(F, 1)};
        for (int t = 0; t < 8; ++t)
          for (int p = 0; p < 8; ++p) {
            int hb = p >> 2;
            float qq = (float)((q[t] >> (4 * p)) & 15u);
            w[n * K + j * SB_W + slot_k(g, t, p)] = std::fma(A[hb], qq, -B[hb]);
          }
      }
  return 0;
}


// The row-tiled kernel's plan (wm, wn, mt, nt, S, kc, img_bytes, ws_bytes, rtw).
int emu_prefill_plan(int64_t N, int64_t K, int R, int cus, int64_t* out) {
  const PrefillPlan p = prefill_plan(N, K, R, cus);
  const int64_t v[9] = {p.wm, p.wn, p.mt, p.nt, p.S, p.kc, (int64_t)p.img_bytes, (int64_t)p.ws_bytes, p.rtw};
  memcpy(out, v, sizeof(v));
  return 0;
}

// Replay of the row-tiled path: the plan, the image, every workgroup's waves
// (row tiles wm RTW .., sub-tiles (tile WN + wn) PF_U ..) over its K chunk with
// the matrix-core products emulated, the per-block d / dmin update, and with K
// chunks the partial slices added in chunk order.  y: R x N fp32.
int emu_prefill(const uint8_t* canon, int64_t N, int64_t K, const uint16_t* x, int R, int cus, float* y) {
  const PrefillPlan p = prefill_plan(N, K, R, cus);
  const int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  const int RTW = p.rtw, MT = p.wm * RTW;
  std::vector<uint8_t> packed((size_t)packed_bytes(N, K));
  pack(canon, packed.data(), N, K);
  const int64_t hdr_off = quant_region_bytes(N, K);
  std::vector<uint8_t> img;
  prefill_image(x, R, KB, MT, p.mt, img);
  std::vector<float> part((size_t)p.S * p.slice, 0.f);
  for (int64_t z = 0; z < p.S; ++z)
    for (int64_t m = 0; m < p.mt; ++m)
      for (int64_t nt = 0; nt < p.nt; ++nt)
        for (int wm = 0; wm < p.wm; ++wm)
          for (int wn = 0; wn < p.wn; ++wn) {
            const int64_t jb = z * p.kc, je = std::min<int64_t>(jb + p.kc, KB);
            f32x4 acc[4][PF_U][64] = {};
            for (int64_t j = jb; j < je; ++j) {
              WConst c[PF_U][64];
              uint32_t q[PF_U][64][8];
              for (int u = 0; u < PF_U; ++u) {
                const int64_t ns = (nt * p.wn + wn) * PF_U + u;
                for (int lane = 0; lane < 64; ++lane) {
                  const int g = lane >> 4, nl = lane & 15;
                  uint32_t h[4] = {0, 0, 0, 0};
                  for (int t = 0; t < 8; ++t) q[u][lane][t] = 0;
                  if (ns < NS) {
                    const uint8_t* qp = packed.data() + quant_chunk_off(ns, j, KB) + lane * 16;
                    memcpy(q[u][lane], qp, 16);
                    memcpy(q[u][lane] + 4, qp + 1024, 16);
                    memcpy(h, packed.data() + hdr_off + header_chunk_off(ns, j, KB) + nl * 16, 16);
                  }
                  c[u][lane] = header_consts(h[0], h[1], h[2], h[3], g);
                }
              }
              f32x4 ds[4][PF_U][64] = {};
              for (int t = 0; t < 8; ++t)
                for (int rt = 0; rt < RTW; ++rt) {
                  f16x8 a[64];
                  memcpy(a, img.data() + pf_chunk_off(m, j, KB, MT, pf_operand_chunk(wm * RTW + rt, t)), 1024);
                  for (int u = 0; u < PF_U; ++u) {
                    f16x8 b[64];
                    for (int lane = 0; lane < 64; ++lane) b[lane] = build_b(q[u][lane][t], c[u][lane]);
                    mfma_16x16x32(a, b, ds[rt][u]);
                  }
                }
              for (int rt = 0; rt < RTW; ++rt) {
                float sx4[64][4], sx[64][2];
                memcpy(sx4, img.data() + pf_chunk_off(m, j, KB, MT, pf_sum_chunk(MT, wm * RTW + rt)), 1024);
                for (int lane = 0; lane < 64; ++lane) {
                  sx[lane][0] = sx4[lane][0];
                  sx[lane][1] = sx4[lane][1];
                }
                for (int u = 0; u < PF_U; ++u) {
                  f32x4 ms[64] = {};
                  min_term_parts(sx, c[u], ms);       // the kernel's two binary16 parts of X_s / 256
                  for (int lane = 0; lane < 64; ++lane)
                    for (int i = 0; i < 4; ++i) {
                      acc[rt][u][lane][i] = std::fma(c[u][lane].d, ds[rt][u][lane][i], acc[rt][u][lane][i]);
                      acc[rt][u][lane][i] = std::fma(c[u][lane].nmin * 256.0f, ms[lane][i], acc[rt][u][lane][i]);
                    }
                }
              }
            }
            for (int rt = 0; rt < RTW; ++rt)
              for (int u = 0; u < PF_U; ++u)
                for (int lane = 0; lane < 64; ++lane) {
                  const int64_t n = ((nt * p.wn + wn) * PF_U + u) * TILE_N + (lane & 15);
                  if (n >= N) continue;
                  for (int i = 0; i < 4; ++i) {
                    const int64_t row = m * MT * 16 + (wm * RTW + rt) * 16 + 4 * (lane >> 4) + i;
                    if (row < R) part[(size_t)(z * p.slice + row * N + n)] = acc[rt][u][lane][i];
                  }
                }
          }
  for (int64_t i = 0; i < (int64_t)R * N; ++i) {
    float s = part[(size_t)i];
    for (int64_t z = 1; z < p.S; ++z) s += part[(size_t)(z * p.slice + i)];
    y[i] = s;
  }
  return 0;
}

// ---- the persistent pass kernel (pass.hip) -----------------------------------

// Every compute wave's cursor over its share, as the kernel walks it: count
// steps from packed step step0 at chunk block jj0, +1 per step and KB - kbc more
// at a chunk's end.  counts[g][ns * KB + j] += 1 for every step taken.
// the pass kernel's deal: workgroup p's chunk and units [ns0, ns1) (out[0..2])
void emu_pass_units(int p, int S, int P, int NS, int rot, int* out) { pass_units(p, S, P, NS, rot, out, out + 1, out + 2); }

// the workgroups a gated chunk waits for (pass_sched.h), 4 words
void emu_pass_gated_mask(int c, int kbc, int half, int P, int NSp, int Sp, int rot_p, uint64_t* w) {
  pass_gated_mask(c, kbc, half, P, NSp, Sp, rot_p, w);
}

// LDS bytes of one block's activations in the pass kernel
int emu_pass_block_bytes(int R) { return pass_x_block_bytes(R); }

// the pass kernel's split of a workgroup's n steps over NC compute waves (pass_sched.h)
int emu_pass_wave_first(int w, int NC, int n) { return pass_wave_first(w, NC, n); }
int emu_pass_step_owner(int i, int NC, int n) { return pass_step_owner(i, NC, n); }

int emu_pass_coverage(int G, const int64_t* Ns, const int64_t* Ks, int R, int P, int NC, int x_area, int max_chunks,
                      int32_t* counts, int32_t* chunks_out) {
  int64_t off = 0;
  for (int g = 0; g < G; ++g) {
    const int KB = (int)(Ks[g] / SB_W), NS = (int)(padded_n(Ns[g]) / TILE_N);
    const int S = pass_chunks(KB, R, P, x_area, max_chunks);
    chunks_out[g] = S;
    const int kbc = S ? KB / S : 1, rot = (int)((g * 37) % P);
    for (int p = 0; p < P && S > 0; ++p)
      for (int w = 0; w < NC; ++w) {
        int count, step, jj;
        pass_wave_share(p, w, NC, P, NS, KB, S, kbc, rot, &count, &step, &jj);
        for (int i = 0; i < count; ++i) {
          if (step < 0 || step >= NS * KB) return -2;
          counts[off + step] += 1;
          if (++jj == kbc) {
            jj = 0;
            step += KB - kbc + 1;
          } else {
            step += 1;
          }
        }
      }
    off += (int64_t)NS * KB;
  }
  return 0;
}

// Replay of the pass: per GEMM, every workgroup's compute waves walk their shares
// with the streaming kernel's step arithmetic against the chunk's staged
// activations and leave a piece at each unit end; helper 0 adds each unit's
// pieces in wave order (waves from pass_step_owner, piece index from
// pass_wave_first) and writes y, or with K chunks the chunk's partial tile; the
// partial tiles of a sub-tile are added in chunk order.
int emu_pass(int G, const uint8_t* const* canons, const int64_t* Ns, const int64_t* Ks, const uint16_t* const* xs,
             float* const* ys, int R, int P, int NC, int x_area, int max_chunks, int msum) {
  typedef std::vector<f32x4> Tile;   // RT row tiles x 64 lanes
  const int RT = (R + 15) / 16;
  for (int g = 0; g < G; ++g) {
    const int64_t N = Ns[g], K = Ks[g];
    const int KB = (int)(K / SB_W), NS = (int)(padded_n(N) / TILE_N);
    const int S = pass_chunks(KB, R, P, x_area, max_chunks);
    if (S == 0) return -1;
    const int kbc = KB / S, rot = (int)((g * 37) % P);
    std::vector<uint8_t> packed((size_t)packed_bytes(N, K));
    pack(canons[g], packed.data(), N, K);
    const int64_t hdr_off = quant_region_bytes(N, K);
    std::vector<Tile> partial((size_t)S * NS, Tile((size_t)RT * 64, f32x4{0, 0, 0, 0}));
    auto store_y = [&](int ns, const Tile& t) {
      for (int rt = 0; rt < RT; ++rt)
        for (int lane = 0; lane < 64; ++lane) {
          const int64_t n = (int64_t)ns * TILE_N + (lane & 15);
          if (n >= N) continue;
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * (lane >> 4) + i;
            if (r < R) ys[g][(int64_t)r * N + n] = t[(size_t)rt * 64 + lane][i];
          }
        }
    };
    for (int p = 0; p < P; ++p) {
      int c, ns0, ns1;
      pass_units(p, S, P, NS, rot, &c, &ns0, &ns1);
      if (ns1 == ns0) continue;
      std::vector<f16x8> slots;
      std::vector<Sum2> sums;
      convert_x(xs[g], R, K, (int64_t)c * kbc, kbc, 0, kbc, slots, sums);
      std::vector<std::vector<Tile>> pieces(NC);
      for (int w = 0; w < NC; ++w) {
        int count, step, jj;
        pass_wave_share(p, w, NC, P, NS, KB, S, kbc, rot, &count, &step, &jj);
        Tile acc((size_t)RT * 64, f32x4{0, 0, 0, 0});
        for (int left = count; left > 0; --left) {
          const int ns = step / KB, j = step % KB;
          wave_step(packed.data(), hdr_off, ns, 1, NS, j, KB, slots, sums, R, jj, RT, msum != 0 || RT > 1 ? 2 : 0, acc.data());
          if (jj == kbc - 1 || left == 1) {
            pieces[w].push_back(acc);
            acc.assign((size_t)RT * 64, f32x4{0, 0, 0, 0});
          }
          if (++jj == kbc) {
            jj = 0;
            step += KB - kbc + 1;
          } else {
            step += 1;
          }
        }
      }
      const int units = ns1 - ns0, n = units * kbc;
      for (int u = 0; u < units; ++u) {
        const int w_lo = pass_step_owner(u * kbc, NC, n), w_hi = pass_step_owner((u + 1) * kbc - 1, NC, n);
        Tile sum((size_t)RT * 64, f32x4{0, 0, 0, 0});
        for (int w = w_lo; w <= w_hi; ++w) {
          const int a_w = pass_wave_first(w, NC, n);
          if (a_w == pass_wave_first(w + 1, NC, n)) continue;   // an empty share leaves no piece
          const int k = u - a_w / kbc;
          if (k < 0 || k >= (int)pieces[w].size()) return -3;
          for (size_t l = 0; l < sum.size(); ++l) sum[l] += pieces[w][k][l];
        }
        if (S == 1)
          store_y(ns0 + u, sum);
        else
          partial[(size_t)c * NS + ns0 + u] = sum;
      }
    }
    if (S > 1)
      for (int ns = 0; ns < NS; ++ns) {
        Tile sum = partial[ns];
        for (int cc = 1; cc < S; ++cc)
          for (size_t l = 0; l < sum.size(); ++l) sum[l] += partial[(size_t)cc * NS + ns][l];
        store_y(ns, sum);
      }
  }
  return 0;
}

}  // extern "C"
