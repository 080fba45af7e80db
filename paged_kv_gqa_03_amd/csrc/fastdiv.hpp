// fastdiv.hpp -- exact unsigned 32-bit division by a runtime divisor.
//
// Page and block lookups divide a token or slot index by the page size, a
// runtime value, inside the kernels' address math.  The divisor's constant
// is computed once on the host:  c = ceil(2^64 / d)  (d >= 2), and then
//     floor(n / d) = floor(n * c / 2^64)   for every n < 2^32,
// the "direct computation" result of Lemire, Kaser and Kurz, "Faster
// remainder by direct computation" (Software: Practice and Experience, 2019):
// with F = 64 >= 32 + ceil(log2 d) fractional bits the rounded-up reciprocal
// is exact over all 32-bit numerators.  d = 1 would need c = 2^64 and is
// handled by a select.  The product's bits 64..95 come from two 32 x 32 -> 64
// multiplies.
//
// Plain C++ with no HIP dependence: the functions are constexpr, which HIP
// compiles for both host and device, so the same code is checked
// exhaustively on the CPU by the test suite.
#pragma once
#include <stdint.h>

namespace pa {

struct DivU32 {
    uint64_t c;   // ceil(2^64 / d) for d >= 2, unused for d = 1
    uint32_t d;   // the divisor (>= 1)
};

constexpr DivU32 make_divu32(uint32_t d) {
    return DivU32{d > 1 ? ~0ull / d + 1 : 0ull, d};
}

// floor(n / f.d), exact for every 32-bit n.
constexpr uint32_t divu32(uint32_t n, DivU32 f) {
    const uint64_t lo = (uint64_t)n * (uint32_t)f.c;            // n * c_lo
    const uint64_t hi = (uint64_t)n * (uint32_t)(f.c >> 32);    // n * c_hi
    const uint32_t q = (uint32_t)((hi + (lo >> 32)) >> 32);     // bits 64..95 of n * c
    return f.d == 1 ? n : q;
}

}  // namespace pa
