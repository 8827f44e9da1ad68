// Device helpers shared by the kernel files of the fact-store library.
// Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fsd {

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, 64);
    return v;
}

// The two bf16 halves of a 32-bit word, as exact fp32 values.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round an fp64 value to the nearest bf16, ties to even, without double
// rounding: narrow to fp32 with round-to-odd (Boldo & Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE Trans. Computers 2008: an intermediate format with >= 2 more bits,
// rounded to odd, makes the final round-to-nearest correct), then round the
// fp32 bits to 16 bits to nearest-even.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double y) {
    const float f = static_cast<float>(y);
    uint32_t u = __float_as_uint(f);
    const double back = static_cast<double>(f);
    if (back != y) {
        if (fabs(back) > fabs(y)) u -= 1u;   // rounded away from zero: step back
        u |= 1u;                             // sticky bit: round-to-odd
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// sin and cos of a RoPE angle x = p * w, for 0 <= x < 2^31 (p an int32
// position, w <= 1), each within about 1.5 ulp, branch-free.
//   Reduction (Cody & Waite, "Software Manual for the Elementary Functions",
//   1980): n = nearest integer to x * 2/pi, r = x - n * pi/2 with pi/2 split
//   into three doubles P1 + P2 + P3 (P1 = pi/2 rounded, P2 and P3 the next
//   two roundings of the remainder; pi taken to 400 bits).  In this range
//   x - n*P1 is exact in one FMA (a multiple of 2^-52 below 1 in magnitude),
//   and so is the next step when r is small, so r keeps its relative
//   accuracy even next to a multiple of pi/2; the omitted remainder of pi/2
//   is below 2^-163.
//   Kernels on |r| <= pi/4: the Taylor series of sin to r^17 and of cos to
//   r^18 (coefficients 1/n! rounded to double); the first omitted terms are
//   below 1e-19 and 1e-20.  The quadrant n mod 4 then picks the signs.
__device__ __forceinline__ void sincos_angle(double x, double* s, double* c) {
    const double n = rint(x * 0x1.45f306dc9c883p-1);          // 2/pi
    double r = fma(-n, 0x1.921fb54442d18p+0, x);
    r = fma(-n, 0x1.1a62633145c07p-54, r);
    r = fma(-n, -0x1.f1976b7ed8fbcp-110, r);
    const double z = r * r;
    // sin(r) = r + r^3 * ps(z): ps = -1/3! + z/5! - z^2/7! + ... + z^7/17!
    double ps = 0x1.952c77030ad4ap-49;                         //  1/17!
    ps = fma(ps, z, -0x1.ae7f3e733b81fp-41);                   // -1/15!
    ps = fma(ps, z, 0x1.6124613a86d09p-33);                    //  1/13!
    ps = fma(ps, z, -0x1.ae64567f544e4p-26);                   // -1/11!
    ps = fma(ps, z, 0x1.71de3a556c734p-19);                    //  1/9!
    ps = fma(ps, z, -0x1.a01a01a01a01ap-13);                   // -1/7!
    ps = fma(ps, z, 0x1.1111111111111p-7);                     //  1/5!
    ps = fma(ps, z, -0x1.5555555555555p-3);                    // -1/3!
    // cos(r) = 1 + z * pc(z): pc = -1/2! + z/4! - z^2/6! + ... - z^8/18!
    double pc = -0x1.6827863b97d97p-53;                        // -1/18!
    pc = fma(pc, z, 0x1.ae7f3e733b81fp-45);                    //  1/16!
    pc = fma(pc, z, -0x1.93974a8c07c9dp-37);                   // -1/14!
    pc = fma(pc, z, 0x1.1eed8eff8d898p-29);                    //  1/12!
    pc = fma(pc, z, -0x1.27e4fb7789f5cp-22);                   // -1/10!
    pc = fma(pc, z, 0x1.a01a01a01a01ap-16);                    //  1/8!
    pc = fma(pc, z, -0x1.6c16c16c16c17p-10);                   // -1/6!
    pc = fma(pc, z, 0x1.5555555555555p-5);                     //  1/4!
    pc = fma(pc, z, -0.5);                                     // -1/2!
    const double sr = fma(r * z, ps, r);
    const double cr = fma(z, pc, 1.0);
    // x = r + n * pi/2: quadrant 0 (s, c) = (sr, cr), 1 (cr, -sr),
    // 2 (-sr, -cr), 3 (-cr, sr)
    const int q = static_cast<int>(n) & 3;
    const double a = (q & 1) ? cr : sr;
    const double b = (q & 1) ? sr : cr;
    *s = (q & 2) ? -a : a;
    *c = ((q + 1) & 2) ? -b : b;
}

}  // namespace fsd
