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

}  // namespace fsd
