// float64 sine and cosine of a rotary angle, for 0 <= x < 2^31.
//
// The rotary angle is position * inv_freq with position < 2^31 and
// inv_freq <= 1, so a three-part Cody-Waite reduction by pi/2 is exact
// enough over the whole range (W. J. Cody and W. Waite, "Software Manual for
// the Elementary Functions", 1980: subtract k*(P1 + P2 + P3) with the leading
// parts short enough that k*P1 and k*P2 are exact products).  Here
// P1 and P2 carry 21 significant bits of pi/2 each (k < 2^31 has at most 31
// bits, so k*P1 and k*P2 fit in 52 bits), P3 the next 53 bits; what is left
// of pi/2 after them is below 1e-31, i.e. below 2^-71 after multiplying by k.
// The reduced argument r lies in [-pi/4, pi/4] (up to rounding of k) and is
// accurate to a few units of 2^-54 in absolute terms.  sin r and cos r are
// the Taylor series through r^19 and r^20 (first omitted terms below 1e-21
// on |r| <= 0.8), evaluated by Horner's rule with fused multiply-adds after
// a first step of a multiply and an add; the coefficients are 1/n! rounded
// to float64.  The constants were derived from
// pi and n! directly (mpmath at 400 bits).
//
// Exact at x = 0: sin 0 = 0 and cos 0 = 1, so position 0 is the identity.
// Usable from device code and from a host C or C++ compiler (for CPU checks).

#ifndef ROPE_SINCOS_H
#define ROPE_SINCOS_H

#include <math.h>

#if defined(__HIPCC__)
#define ROPE_HD __host__ __device__ __forceinline__
#else
#define ROPE_HD static inline
#endif

// a * b + c for a constant c.  On the GPU c is taken from scalar registers
// by a three-operand FMA: the compiler's own choice, the two-operand form,
// needs c in the destination and so copies every constant into vector
// registers first (two moves per coefficient).  A plain fma on the host.
ROPE_HD double rope_fma_k(double a, double b, double c) {
#if defined(__HIP_DEVICE_COMPILE__)
  double d;
  __asm__("v_fma_f64 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "s"(c));
  return d;
#else
  return fma(a, b, c);
#endif
}

// a * k + c for constants k and c, rounded twice (a multiply, then an add):
// the first Horner step of a series.  As one FMA it would need one of its two
// constants in a vector register (an instruction reads at most one scalar
// register), which the compiler then keeps live across a whole loop of
// tables.  The highest-order term it rounds is below 2^-60 of the result.
ROPE_HD double rope_mul_add_k(double a, double k, double c) {
#if defined(__clang__)
#pragma clang fp contract(off)
#endif
  const double t = a * k;
  return t + c;
}

ROPE_HD void rope_sincos(double x, double* s_out, double* c_out) {
  const double kTwoOverPi = 0x1.45f306dc9c883p-1;
  const double kP1 = 0x1.921fb00000000p+0;   // pi/2, leading 21 bits
  const double kP2 = 0x1.5110b00000000p-22;  // next 21 bits
  const double kP3 = 0x1.18469898cc517p-44;  // next 53 bits
  const double k = rint(x * kTwoOverPi);
  double r = fma(-k, kP1, x);  // exact
  r = fma(-k, kP2, r);         // exact product, one rounding
  r = fma(-k, kP3, r);
  const double z = r * r;
  // sin r = r (1 - z/3! + z^2/5! - ... - z^9/19!)
  double ps = rope_mul_add_k(z, -0x1.2f49b46814157p-57,  // -1/19!
                             0x1.952c77030ad4ap-49);  // +1/17!
  ps = rope_fma_k(ps, z, -0x1.ae7f3e733b81fp-41);        // -1/15!
  ps = rope_fma_k(ps, z, 0x1.6124613a86d09p-33);         // +1/13!
  ps = rope_fma_k(ps, z, -0x1.ae64567f544e4p-26);        // -1/11!
  ps = rope_fma_k(ps, z, 0x1.71de3a556c734p-19);         // +1/9!
  ps = rope_fma_k(ps, z, -0x1.a01a01a01a01ap-13);        // -1/7!
  ps = rope_fma_k(ps, z, 0x1.1111111111111p-7);          // +1/5!
  ps = rope_fma_k(ps, z, -0x1.5555555555555p-3);         // -1/3!
  const double sr = fma(ps * z, r, r);
  // cos r = 1 - z/2! + z^2/4! - ... + z^10/20!
  double pc = rope_mul_add_k(z, 0x1.e542ba4020225p-62,   // +1/20!
                             -0x1.6827863b97d97p-53);  // -1/18!
  pc = rope_fma_k(pc, z, 0x1.ae7f3e733b81fp-45);         // +1/16!
  pc = rope_fma_k(pc, z, -0x1.93974a8c07c9dp-37);        // -1/14!
  pc = rope_fma_k(pc, z, 0x1.1eed8eff8d898p-29);         // +1/12!
  pc = rope_fma_k(pc, z, -0x1.27e4fb7789f5cp-22);        // -1/10!
  pc = rope_fma_k(pc, z, 0x1.a01a01a01a01ap-16);         // +1/8!
  pc = rope_fma_k(pc, z, -0x1.6c16c16c16c17p-10);        // -1/6!
  pc = rope_fma_k(pc, z, 0x1.5555555555555p-5);          // +1/4!
  pc = rope_fma_k(pc, z, -0.5);                          // -1/2!
  const double cr = fma(pc, z, 1.0);
  // x = k pi/2 + r: rotate (cos r, sin r) by the quadrant k mod 4
  const int q = (int)((long long)k & 3);
  const double s = (q & 1) ? cr : sr;
  const double c = (q & 1) ? sr : cr;
  *s_out = (q & 2) ? -s : s;
  *c_out = ((q + 1) & 2) ? -c : c;
}

#undef ROPE_HD

#endif  // ROPE_SINCOS_H
