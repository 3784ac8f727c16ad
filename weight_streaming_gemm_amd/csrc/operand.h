// operand.h — per-lane decoding of the packed header and of packed quant
// dwords into matrix-core operands.  Host and device compile the same code so
// the operand arithmetic can be exercised on the CPU.
//
// For lane group g (sub-blocks 2g, 2g+1 of a block) the B operand element e of
// step t is sc_{2g + (e & 1)} * q_k for k = operand_k(g, t, e) (layout.h): an
// integer <= 63 * 15 = 945, exact in binary16.  The min term is either a
// product of the activation operands with the mins (build_m_full), or a product
// of the sub-block sums of x with the mins (min_operand, and the kernels' own
// two-part staging of the sums).
#pragma once
#include <stdint.h>

#include "layout.h"

namespace qg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <class T, class F>
QG_HD T bitcast(F v) { return __builtin_bit_cast(T, v); }

// fused multiply-add on binary16 pairs (one rounding)
QG_HD f16x2 fma2(f16x2 a, f16x2 b, f16x2 c) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_elementwise_fma(a, b, c);
#else
  // products and sums of binary16 values are exact in double; one rounding
  f16x2 r;
  r[0] = (_Float16)((double)a[0] * (double)b[0] + (double)c[0]);
  r[1] = (_Float16)((double)a[1] * (double)b[1] + (double)c[1]);
  return r;
#endif
}

// per-(output, block, lane-group) constants decoded from the packed header
struct WConst {
  f16x2 sc;     // (sc_{2g}, sc_{2g+1})              binary16, exact
  f16x2 sc16;   // (sc_{2g}/16, sc_{2g+1}/16)        exact
  f16x2 b1;     // (-1024 sc_{2g}, -1024 sc_{2g+1})  exact
  f16x2 b16;    // (-64 sc_{2g}, -64 sc_{2g+1})      exact
  f16x2 m;      // (m_{2g}, m_{2g+1})                exact
  float d;      // d
  float nmin;   // -dmin
};

QG_HD WConst header_consts(uint32_t h0, uint32_t h1, uint32_t h2, uint32_t h3, int g) {
  WConst c;
  uint32_t F = header_group(h1, h2, h3, g);
  uint32_t scpair = (F & 63u) | (((F >> 6) & 63u) << 16);
  // binary16 with 1024 + sc (the integer sits in the mantissa), minus 1024: exact
  f16x2 sc = bitcast<f16x2>(scpair | 0x64006400u) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
  c.sc = sc;
  c.sc16 = sc * f16x2{(_Float16)0.0625f, (_Float16)0.0625f};
  c.b1 = sc * f16x2{(_Float16)-1024.0f, (_Float16)-1024.0f};
  c.b16 = sc * f16x2{(_Float16)-64.0f, (_Float16)-64.0f};
  uint32_t mpair = ((F >> 12) & 63u) | (((F >> 18) & 63u) << 16);
  c.m = bitcast<f16x2>(mpair | 0x64006400u) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
  c.d = (float)bitcast<_Float16>((uint16_t)(h0 & 0xFFFFu));
  c.nmin = -(float)bitcast<_Float16>((uint16_t)(h0 >> 16));
  return c;
}

// (a & mask) | c in one instruction.  The compiler would otherwise split it in
// two: the three-operand form takes no literal and at most one scalar operand,
// so the constant c is passed in a vector register.
QG_HD uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(c));
  return r;
#else
  return (a & mask) | c;
#endif
}

// Eight weights of one packed dword as the B operand, each equal to sc * q.
// Nibble positions (0,4) and (2,6) become 1024 + q in the binary16 mantissa,
// positions (1,5) and (3,7) become 1024 + 16 q; one fused multiply-add per
// pair removes the offset: (1024 + q) sc - 1024 sc = sc q and
// (1024 + 16 q) (sc/16) - 64 sc = sc q, both exact.
QG_HD f16x8 build_b(uint32_t w, const WConst& c) {
  const uint32_t magic = 0x64006400u;
  uint32_t w8 = w >> 8;
  f16x2 p0 = bitcast<f16x2>(and_or(w, 0x000F000Fu, magic));
  f16x2 p1 = bitcast<f16x2>(and_or(w, 0x00F000F0u, magic));
  f16x2 p2 = bitcast<f16x2>(and_or(w8, 0x000F000Fu, magic));
  f16x2 p3 = bitcast<f16x2>(and_or(w8, 0x00F000F0u, magic));
  f16x2 o0 = fma2(p0, c.sc, c.b1);
  f16x2 o1 = fma2(p1, c.sc16, c.b16);
  f16x2 o2 = fma2(p2, c.sc, c.b1);
  f16x2 o3 = fma2(p3, c.sc16, c.b16);
  return f16x8{o0[0], o0[1], o1[0], o1[1], o2[0], o2[1], o3[0], o3[1]};
}

// The min term of a block, sum over k of m_sub(k) x_k, is sum over s of m_s X_s
// with X_s the sum of x over sub-block s.  The sums are formed in fp32 (a bf16 sum
// of 32 values reaches 32 * 65504, far beyond binary16's range); the matrix-core
// kernels stage them as two binary16 parts of X_s / 256 for one fp16 product per
// tile, and the vector-unit variant multiplies them in fp32 by the mins below
// (lane group g: m_2g for h = 0, m_2g+1 for h = 1).
QG_HD float min_operand(const WConst& c, int h) { return (float)c.m[h]; }
// Without the sums, the min term is the product of each step's activation
// operand with B = (m_2g, m_2g+1) in every pair (eight products per block).
QG_HD f16x8 build_m_full(const WConst& c) {
  return f16x8{c.m[0], c.m[1], c.m[0], c.m[1], c.m[0], c.m[1], c.m[0], c.m[1]};
}

// the sum of the 8 per-step partial sums of a sub-block, in a fixed tree order
QG_HD float tree8(const float p[8]) {
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// Eight activations of one matrix-core A operand from two runs of four bf16
// values, lo = x[k0 .. k0+3] and hi = x[k0+32 .. k0+35] (two dwords each, low
// half first): element 2v + h is run h's value v, converted to binary16 with
// round-to-nearest-even (exact for |x| in [2^-17, 65504]).
QG_HD f16x8 build_a(uint32_t lo0, uint32_t lo1, uint32_t hi0, uint32_t hi1) {
  const float a0 = bitcast<float>(lo0 << 16), a1 = bitcast<float>(lo0 & 0xFFFF0000u);
  const float a2 = bitcast<float>(lo1 << 16), a3 = bitcast<float>(lo1 & 0xFFFF0000u);
  const float b0 = bitcast<float>(hi0 << 16), b1 = bitcast<float>(hi0 & 0xFFFF0000u);
  const float b2 = bitcast<float>(hi1 << 16), b3 = bitcast<float>(hi1 & 0xFFFF0000u);
  return f16x8{(_Float16)a0, (_Float16)b0, (_Float16)a1, (_Float16)b1,
               (_Float16)a2, (_Float16)b2, (_Float16)a3, (_Float16)b3};
}

}  // namespace qg
