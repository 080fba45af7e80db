// Exhaustive host check of the kernels' exact division (fastdiv.hpp):
// divu32(n, make_divu32(d)) == n / d for every 32-bit n and the divisors
// given on the command line, then for random (n, d) pairs.  The expected
// quotient is tracked incrementally (no division in the inner loop).
// Prints "ok" and exits 0, or prints the first mismatch and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fastdiv.hpp"

static int check_divisor(uint32_t d) {
    const pa::DivU32 f = pa::make_divu32(d);
    const int64_t chunks = 256;
    const uint64_t span = (1ull << 32) / chunks;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int64_t c = 0; c < chunks; ++c) {
        const uint64_t n0 = (uint64_t)c * span, n1 = n0 + span;
        uint64_t q = n0 / d, r = n0 % d;
        for (uint64_t n = n0; n < n1; ++n) {
            if (pa::divu32((uint32_t)n, f) != (uint32_t)q) {
                bad = 1;
                break;
            }
            if (++r == d) {
                r = 0;
                ++q;
            }
        }
    }
    if (bad) {
        for (uint64_t n = 0; n < (1ull << 32); ++n)
            if (pa::divu32((uint32_t)n, f) != (uint32_t)(n / d)) {
                printf("mismatch: n=%llu d=%u got %u want %llu\n", (unsigned long long)n, d,
                       pa::divu32((uint32_t)n, f), (unsigned long long)(n / d));
                break;
            }
    }
    return bad;
}

int main(int argc, char **argv) {
    for (int i = 1; i < argc; ++i) {
        const uint32_t d = (uint32_t)strtoul(argv[i], nullptr, 10);
        if (d == 0 || check_divisor(d)) {
            if (d == 0) printf("bad divisor argument %s\n", argv[i]);
            return 1;
        }
    }
    // Random pairs: a 64-bit LCG (Knuth's MMIX constants), divisors spread
    // over every bit length.
    uint64_t x = 0x9E3779B97F4A7C15ull;
    for (int i = 0; i < 20000000; ++i) {
        x = x * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t n = (uint32_t)(x >> 32);
        x = x * 6364136223846793005ull + 1442695040888963407ull;
        const uint32_t bits = 1 + (uint32_t)((x >> 59) & 31);
        uint32_t d = (uint32_t)(x >> 16) & (uint32_t)((1ull << bits) - 1);
        if (d == 0) d = 1;
        if (pa::divu32(n, pa::make_divu32(d)) != n / d) {
            printf("mismatch: n=%u d=%u got %u want %u\n", n, d, pa::divu32(n, pa::make_divu32(d)), n / d);
            return 1;
        }
    }
    printf("ok\n");
    return 0;
}
