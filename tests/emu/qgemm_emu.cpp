// qgemm_emu.cpp — CPU emulation of the gfx950 kernels' data flow, lane by lane.
//
// Test infrastructure: it compiles the library's own layout.h / operand.h
// (the code the kernels run) for the host and replays the pack, activation
// staging, matrix-core GEMM (with the documented lane layouts of
// v_mfma_f32_16x16x32_f16 and v_mfma_f32_16x16x4_f32), split-K reduction and
// dequantisation kernels thread by thread.  It lets the CPU suite check every
// index mapping against the fp64 oracle before any GPU run.  The matrix-core
// lane layout assumed here is itself checked on the GPU by a probe test.
#include <stdint.h>
#include <string.h>
#include <vector>

#include "../../weight_streaming_gemm_amd/csrc/layout.h"
#include "../../weight_streaming_gemm_amd/csrc/operand.h"
#include "../../weight_streaming_gemm_amd/csrc/stream_sched.h"
#include <algorithm>
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

// K = 4 fp32 variant: a[l] = A[l % 16][l / 16], b[l] = B[l / 16][l % 16]
void mfma_16x16x4(const float* a, const float* b, f32x4* c) {
  f32x4 out[64];
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < 4; ++v) {
      int i = 4 * (l / 16) + v, j = l % 16;
      double s = c[l][v];
      for (int k = 0; k < 4; ++k) s += (double)a[i + 16 * k] * (double)b[j + 16 * k];
      out[l][v] = (float)s;
    }
  for (int l = 0; l < 64; ++l) c[l] = out[l];
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

float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void xprep(const uint16_t* x, f16x8* xq, float* xs, int R, int64_t K, int RT) {
  int64_t KB = K / SB_W;
  for (int64_t rj = 0; rj < RT * KB; ++rj)
    for (int lane = 0; lane < 64; ++lane) {
      int rt = (int)(rj / KB);
      int64_t j = rj % KB;
      int g = lane >> 4, r = rt * 16 + (lane & 15);
      float vals[64];
      for (int c = 0; c < 64; ++c) vals[c] = (r < R) ? bf16f(x[(int64_t)r * K + j * SB_W + 64 * g + c]) : 0.f;
      for (int t = 0; t < 8; ++t) {
        f16x8 o;
        for (int e = 0; e < 8; ++e) o[e] = (_Float16)vals[32 * (e & 1) + 4 * t + (e >> 1)];
        xq[(rj * 8 + t) * 64 + lane] = o;
      }
      float s0 = 0.f, s1 = 0.f;
      for (int c = 0; c < 32; ++c) s0 += vals[c];
      for (int c = 0; c < 32; ++c) s1 += vals[32 + c];
      xs[(rj * 64 + lane) * 2] = s0;
      xs[(rj * 64 + lane) * 2 + 1] = s1;
    }
}

// one block step of one 16-output sub-tile, all 64 lanes, into acc/macc[RT][64]
void wave_step(const uint8_t* packed, int64_t hdr_off, int64_t ns, int64_t j, int64_t KB, const f16x8* xq,
               const float* xs, int RT, f32x4* acc, f32x4* macc) {
  WConst c[64];
  uint32_t qd[64][8];
  for (int lane = 0; lane < 64; ++lane) {
    const uint8_t* qp = packed + lane * 16 + quant_chunk_off(ns, j, KB);
    memcpy(qd[lane], qp, 16);
    memcpy(qd[lane] + 4, qp + 1024, 16);
    uint32_t h[4];
    memcpy(h, packed + hdr_off + (lane & 15) * 16 + header_chunk_off(ns, j, KB), 16);
    c[lane] = header_consts(h[0], h[1], h[2], h[3], lane >> 4);
  }
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 dsum[64];
    for (int l = 0; l < 64; ++l) dsum[l] = f32x4{0, 0, 0, 0};
    for (int t = 0; t < 8; ++t) {
      f16x8 a[64], b[64];
      for (int lane = 0; lane < 64; ++lane) {
        a[lane] = xq[((rt * KB + j) * 8 + t) * 64 + lane];
        b[lane] = build_b(qd[lane][t], c[lane]);
      }
      mfma_16x16x32(a, b, dsum);
    }
    float xa0[64], xa1[64], b0[64], b1[64];
    for (int lane = 0; lane < 64; ++lane) {
      acc[rt * 64 + lane] += c[lane].d * dsum[lane];
      xa0[lane] = xs[((rt * KB + j) * 64 + lane) * 2];
      xa1[lane] = xs[((rt * KB + j) * 64 + lane) * 2 + 1];
      b0[lane] = c[lane].bm0;
      b1[lane] = c[lane].bm1;
    }
    mfma_16x16x4(xa0, b0, &macc[rt * 64]);
    mfma_16x16x4(xa1, b1, &macc[rt * 64]);
  }
}

}  // namespace

extern "C" {

// Emulated stream-K run: P workgroups of 4 waves x NT sub-tiles, executed one
// after another in a seeded random order (the arrival order at shared tiles).
int emu_stream(const uint8_t* canon, int64_t N, int64_t K, const uint16_t* x, int R, int NT, int64_t P,
               uint64_t order_seed, float* y) {
  const int NW = 4;
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  int RT = (R + 15) / 16;
  int64_t T = (NS + NW * NT - 1) / (NW * NT), I = T * KB;
  if (P > I || P < 1) return -1;
  std::vector<uint8_t> packed((size_t)packed_bytes(N, K));
  pack(canon, packed.data(), N, K);
  int64_t hdr_off = quant_region_bytes(N, K);
  std::vector<f16x8> xq((size_t)RT * KB * 8 * 64);
  std::vector<float> xs((size_t)RT * KB * 64 * 2);
  xprep(x, xq.data(), xs.data(), R, K, RT);
  const size_t slot_floats = (size_t)NW * NT * RT * 256;
  std::vector<float> part((size_t)2 * P * slot_floats, std::nanf(""));
  std::vector<uint32_t> cnt((size_t)T, 0);
  std::vector<int64_t> order((size_t)P);
  for (int64_t p = 0; p < P; ++p) order[(size_t)p] = p;
  std::mt19937_64 rng(order_seed);
  std::shuffle(order.begin(), order.end(), rng);
  for (int i = 0; i < R * N; ++i) y[i] = std::nanf("");
  for (int64_t p : order) {
    int64_t it0 = range_first(p, P, I), it1 = range_first(p + 1, P, I);
    std::vector<f32x4> acc((size_t)NW * NT * RT * 64), macc(acc.size());
    auto zero = [&]() { for (auto& v : acc) v = f32x4{0, 0, 0, 0}; for (auto& v : macc) v = f32x4{0, 0, 0, 0}; };
    zero();
    int64_t ja = it0 % KB;
    for (int64_t it = it0; it < it1; ++it) {
      int64_t t = it / KB, j = it % KB;
      for (int w = 0; w < NW; ++w)
        for (int u = 0; u < NT; ++u) {
          int64_t ns = (t * NW + w) * NT + u;
          if (ns >= NS) continue;
          size_t base = (size_t)((w * NT + u) * RT) * 64;
          wave_step(packed.data(), hdr_off, ns, j, KB, xq.data(), xs.data(), RT, &acc[base], &macc[base]);
        }
      bool last = it + 1 == it1;
      if (j != KB - 1 && !last) continue;
      bool full = ja == 0 && j == KB - 1;
      auto out_index = [&](int w, int u, int rt, int lane, int i, int64_t* o) {
        int64_t n = ((t * NW + w) * NT + u) * TILE_N + (lane & 15);
        int r = rt * 16 + 4 * (lane >> 4) + i;
        if (n >= N || r >= R) return false;
        *o = (int64_t)r * N + n;
        return true;
      };
      if (full) {
        for (int w = 0; w < NW; ++w) for (int u = 0; u < NT; ++u) for (int rt = 0; rt < RT; ++rt)
          for (int lane = 0; lane < 64; ++lane) for (int i = 0; i < 4; ++i) {
            int64_t o;
            size_t a = (size_t)((w * NT + u) * RT + rt) * 64 + lane;
            if (out_index(w, u, rt, lane, i, &o)) y[o] = acc[a][i] + macc[a][i];
          }
      } else {
        int64_t ps = partial_slot(p, t, KB, P, I);
        for (int w = 0; w < NW; ++w) for (int u = 0; u < NT; ++u) for (int rt = 0; rt < RT; ++rt)
          for (int lane = 0; lane < 64; ++lane) for (int i = 0; i < 4; ++i) {
            size_t a = (size_t)((w * NT + u) * RT + rt) * 64 + lane;
            part[(size_t)(ps * NW + w) * NT * RT * 256 + ((u * RT + rt) * 4 + i) * 64 + lane] = acc[a][i] + macc[a][i];
          }
        int64_t q_lo = tile_first_owner(t, KB, P, I), q_hi = tile_last_owner(t, KB, P, I);
        uint32_t prev = cnt[(size_t)t]++;
        if (prev == (uint32_t)(q_hi - q_lo)) {
          for (int w = 0; w < NW; ++w) for (int u = 0; u < NT; ++u) for (int rt = 0; rt < RT; ++rt)
            for (int lane = 0; lane < 64; ++lane) for (int i = 0; i < 4; ++i) {
              float v = 0.f;
              for (int64_t q = q_lo; q <= q_hi; ++q) {
                int64_t qs = partial_slot(q, t, KB, P, I);
                v += part[(size_t)(qs * NW + w) * NT * RT * 256 + ((u * RT + rt) * 4 + i) * 64 + lane];
              }
              int64_t o;
              if (out_index(w, u, rt, lane, i, &o)) y[o] = v;
            }
          cnt[(size_t)t] = 0;
        }
      }
      zero();
      ja = 0;
    }
  }
  for (int64_t t = 0; t < T; ++t)
    if (cnt[(size_t)t] != 0) return -2;   // a counter was left armed
  return 0;
}

int emu_packed_size(int64_t N, int64_t K, int64_t* bytes) {
  *bytes = packed_bytes(N, K);
  return 0;
}

int emu_pack(const uint8_t* canon, uint8_t* packed, int64_t N, int64_t K) {
  pack(canon, packed, N, K);
  return 0;
}

// Emulated matrix-core run with NT sub-tiles per wave and S K-splits; writes y.
int emu_gemm(const uint8_t* canon, int64_t N, int64_t K, const uint16_t* x, int R, int NT, int S, float* y) {
  int64_t KB = K / SB_W, NS = padded_n(N) / TILE_N;
  int RT = (R + 15) / 16;
  std::vector<uint8_t> packed((size_t)packed_bytes(N, K));
  pack(canon, packed.data(), N, K);
  std::vector<f16x8> xq((size_t)RT * KB * 8 * 64);
  std::vector<float> xs((size_t)RT * KB * 64 * 2);
  xprep(x, xq.data(), xs.data(), R, K, RT);
  int64_t kbs = (KB + S - 1) / S;
  S = (int)((KB + kbs - 1) / kbs);
  std::vector<float> part((size_t)S * R * N, 0.f);
  int64_t hdr_off = quant_region_bytes(N, K);
  int64_t NG = (NS + NT - 1) / NT;
  for (int64_t s = 0; s < S; ++s)
    for (int64_t ng = 0; ng < NG; ++ng)
      for (int u = 0; u < NT; ++u) {
        int64_t ns = ng * NT + u;
        if (ns >= NS) continue;
        std::vector<f32x4> acc((size_t)RT * 64, f32x4{0, 0, 0, 0}), macc((size_t)RT * 64, f32x4{0, 0, 0, 0});
        int64_t j1 = (s * kbs + kbs < KB) ? s * kbs + kbs : KB;
        for (int64_t j = s * kbs; j < j1; ++j) {
          WConst c[64];
          uint32_t qd[64][8];
          for (int lane = 0; lane < 64; ++lane) {
            const uint8_t* qp = packed.data() + lane * 16 + quant_chunk_off(ns, j, KB);
            memcpy(qd[lane], qp, 16);
            memcpy(qd[lane] + 4, qp + 1024, 16);
            uint32_t h[4];
            memcpy(h, packed.data() + hdr_off + (lane & 15) * 16 + header_chunk_off(ns, j, KB), 16);
            c[lane] = header_consts(h[0], h[1], h[2], h[3], lane >> 4);
          }
          for (int rt = 0; rt < RT; ++rt) {
            std::vector<f32x4> dsum(64, f32x4{0, 0, 0, 0});
            for (int t = 0; t < 8; ++t) {
              f16x8 a[64], b[64];
              for (int lane = 0; lane < 64; ++lane) {
                a[lane] = xq[((rt * KB + j) * 8 + t) * 64 + lane];
                b[lane] = build_b(qd[lane][t], c[lane]);
              }
              mfma_16x16x32(a, b, dsum.data());
            }
            float xa0[64], xa1[64], b0[64], b1[64];
            for (int lane = 0; lane < 64; ++lane) {
              acc[rt * 64 + lane] += c[lane].d * dsum[lane];
              xa0[lane] = xs[((rt * KB + j) * 64 + lane) * 2];
              xa1[lane] = xs[((rt * KB + j) * 64 + lane) * 2 + 1];
              b0[lane] = c[lane].bm0;
              b1[lane] = c[lane].bm1;
            }
            mfma_16x16x4(xa0, b0, &macc[rt * 64]);
            mfma_16x16x4(xa1, b1, &macc[rt * 64]);
          }
        }
        for (int lane = 0; lane < 64; ++lane) {
          int64_t n = ns * TILE_N + (lane & 15);
          if (n >= N) continue;
          for (int rt = 0; rt < RT; ++rt)
            for (int i = 0; i < 4; ++i) {
              int r = rt * 16 + 4 * (lane >> 4) + i;
              if (r < R) part[((size_t)s * R + r) * N + n] = acc[rt * 64 + lane][i] + macc[rt * 64 + lane][i];
            }
        }
      }
  for (int64_t i = 0; i < (int64_t)R * N; ++i) {
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[(size_t)s * R * N + i];
    y[i] = v;
  }
  return S;
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
            w[n * K + j * SB_W + slot_k(g, t, p)] = __builtin_fmaf(A[hb], qq, -B[hb]);
          }
      }
  return 0;
}

}  // extern "C"
