// layout.h — the GPU-side packed layout of Q4_K-style weights and the
// activation operand layout, as pure index/bit functions usable on host and
// device.  Nothing here does arithmetic of the GEMM; it only moves bits.
//
// Canonical super-block (input, 144 B): d (binary16) | dmin (binary16) |
// 12-byte LE stream of sixteen 6-bit fields (sc_s at bits 6s, m_s at 48+6s) |
// 128 quant bytes (byte i = q[2i] | q[2i+1] << 4).  Block (n, j) covers
// W[n, 256j .. 256j+255] and sits at 144 * (n*KB + j), KB = K/256.
//
// Packed layout.  N is padded to Np = 16 * NS.  Sub-tile ns covers outputs
// n = 16 ns .. 16 ns + 15.  A 64-lane wave works on one (ns, j) pair at a time:
// lane l = 16 g + nl handles output n = 16 ns + nl and the 64 weights of
// sub-blocks 2g and 2g+1 of block j.
//
//   quants:  chunk (ns, j) of 2048 B at (ns*KB + j) * 2048.  Inside: half h
//            (0, 1) at 1024 h, lane l at 16 l, dword u at 4 u.  Dword u of half
//            h serves matrix-core step t = 4h + u and holds eight nibbles; the
//            nibble at bit position 4p is
//              p = v     (v = 0..3): k = 256 j + 64 g + 4 t + v       (sub-block 2g)
//              p = 4 + v (v = 0..3): k = 256 j + 64 g + 32 + 4 t + v  (sub-block 2g+1)
//   headers: after all quant chunks; chunk (ns, j) of 256 B at (ns*KB + j)*256,
//            output nl at 16 nl:
//              dword 0 = d | dmin << 16 (binary16 bits)
//              bytes 4..15 = four 24-bit groups, group g at bytes 4+3g .. 6+3g:
//                F_g = sc_{2g} | sc_{2g+1} << 6 | m_{2g} << 12 | m_{2g+1} << 18
//
// Size: NS * KB * (2048 + 256) = Np * KB * 144 bytes, i.e. the canonical size
// of the padded matrix (padding rows are all-zero blocks).
//
// Activation operands (staged by the streaming kernel into LDS, see there): for
// row r, step t and lane group g, the binary16 A operand element e = 2v + hbit
// holds x[r, 256 j + 64 g + 32 hbit + 4 t + v] (operand_k below).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define QG_HD __host__ __device__ inline
#else
#define QG_HD static inline
#endif

namespace qg {

constexpr int SB_W = 256;          // weights per super-block
constexpr int SB_CANON = 144;      // canonical bytes per super-block
constexpr int CHUNK_Q = 2048;      // packed quant bytes per (sub-tile, block)
constexpr int CHUNK_H = 256;       // packed header bytes per (sub-tile, block)
constexpr int TILE_N = 16;         // outputs per sub-tile

QG_HD int64_t padded_n(int64_t N) { return (N + TILE_N - 1) / TILE_N * TILE_N; }
QG_HD int64_t packed_bytes(int64_t N, int64_t K) { return padded_n(N) * (K / SB_W) * SB_CANON; }
QG_HD int64_t quant_region_bytes(int64_t N, int64_t K) {
  return padded_n(N) / TILE_N * (K / SB_W) * CHUNK_Q;
}
QG_HD int64_t quant_chunk_off(int64_t ns, int64_t j, int64_t KB) { return (ns * KB + j) * CHUNK_Q; }
QG_HD int64_t header_chunk_off(int64_t ns, int64_t j, int64_t KB) { return (ns * KB + j) * CHUNK_H; }

// k (within the block, 0..255) of nibble position p (0..7) of step t for lane group g
QG_HD int slot_k(int g, int t, int p) {
  return 64 * g + 32 * (p >> 2) + 4 * t + (p & 3);
}
// k of operand element e (0..7) of step t for lane group g: e = 2v + hbit
QG_HD int operand_k(int g, int t, int e) {
  return 64 * g + 32 * (e & 1) + 4 * t + (e >> 1);
}

// canonical accessors
QG_HD uint32_t canon_field6(const uint8_t* sb, int f) {
  // f in 0..15; 6 bits at stream bit 6f of bytes 4..15
  uint32_t bit = 6u * (uint32_t)f;
  uint32_t byte = 4u + bit / 8u, sh = bit % 8u;
  uint32_t v = (uint32_t)sb[byte] | ((uint32_t)sb[byte + 1] << 8);  // byte+1 <= 16: inside the block
  return (v >> sh) & 63u;
}
QG_HD uint32_t canon_nibble(const uint8_t* sb, int k) {
  uint32_t b = sb[16 + (k >> 1)];
  return (k & 1) ? (b >> 4) : (b & 15u);
}

// the packed quant dword for lane group g, step t, from a canonical block
QG_HD uint32_t pack_quant_dword(const uint8_t* sb, int g, int t) {
  uint32_t w = 0;
  for (int p = 0; p < 8; ++p) w |= canon_nibble(sb, slot_k(g, t, p)) << (4 * p);
  return w;
}

// the packed 16-byte header (as four dwords) from a canonical block
QG_HD void pack_header(const uint8_t* sb, uint32_t out[4]) {
  out[0] = (uint32_t)sb[0] | ((uint32_t)sb[1] << 8) | ((uint32_t)sb[2] << 16) | ((uint32_t)sb[3] << 24);
  uint8_t bytes[12];
  for (int g = 0; g < 4; ++g) {
    uint32_t F = canon_field6(sb, 2 * g) | (canon_field6(sb, 2 * g + 1) << 6) |
                 (canon_field6(sb, 8 + 2 * g) << 12) | (canon_field6(sb, 8 + 2 * g + 1) << 18);
    bytes[3 * g] = (uint8_t)(F & 0xFF);
    bytes[3 * g + 1] = (uint8_t)((F >> 8) & 0xFF);
    bytes[3 * g + 2] = (uint8_t)((F >> 16) & 0xFF);
  }
  for (int i = 0; i < 3; ++i)
    out[1 + i] = (uint32_t)bytes[4 * i] | ((uint32_t)bytes[4 * i + 1] << 8) |
                 ((uint32_t)bytes[4 * i + 2] << 16) | ((uint32_t)bytes[4 * i + 3] << 24);
}

// 24-bit group field F_g from the packed header dwords h1, h2, h3
// Group g starts at bit 24g of the 96-bit field: in dword 1 + (24g)/32 at bit
// (24g) mod 32.  Selects without branches (g is fixed per lane).
QG_HD uint32_t header_group(uint32_t h1, uint32_t h2, uint32_t h3, int g) {
  uint32_t lo = (g == 3) ? h3 : ((g == 2) ? h2 : h1);
  uint32_t hi = (g >= 2) ? h3 : h2;
  uint32_t sh = (uint32_t)(24 * g) & 31u;
  uint64_t v = ((uint64_t)hi << 32) | lo;
  return (uint32_t)(v >> sh) & 0xFFFFFFu;
}
QG_HD uint32_t grp_sc(uint32_t F, int hbit) { return (F >> (6 * hbit)) & 63u; }
QG_HD uint32_t grp_m(uint32_t F, int hbit) { return (F >> (12 + 6 * hbit)) & 63u; }

}  // namespace qg
