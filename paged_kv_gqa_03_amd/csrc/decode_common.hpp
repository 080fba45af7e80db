// decode_common.hpp -- pieces shared by the decode kernels (VALU and MFMA):
// 16-byte K/V loads and the balanced partition's scan of the row lengths.
#pragma once
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

__device__ __forceinline__ void load16(const uint16_t *ptr, uint32_t (&dst)[4]) {
    const uint4 t = *reinterpret_cast<const uint4 *>(ptr);
    dst[0] = t.x; dst[1] = t.y; dst[2] = t.z; dst[3] = t.w;
}

// K and V bytes are read exactly once per call: non-temporal loads keep them
// from displacing other lines in L2 / MALL (about 10% more HBM throughput on
// the serving batches than plain loads).
__device__ __forceinline__ void load16_stream(const uint16_t *ptr, uint32_t (&dst)[4]) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
    dst[0] = t.x; dst[1] = t.y; dst[2] = t.z; dst[3] = t.w;
}

__device__ __forceinline__ int row_len(const DecodeParams &p, int r) {
    return p.kv_lens ? p.kv_lens[r / p.ngrp] : p.kv_len_const;
}

// Row totals of the balanced partition: lane i sums rows [i*rpl, (i+1)*rpl);
// `base` is the exclusive prefix of those sums across lanes.  The host keeps
// the whole line below 2^31 tokens.
struct RowScan {
    int base, sum, total, rpl;
};

__device__ __forceinline__ RowScan scan_rows(const DecodeParams &p) {
    const int lane = threadIdx.x & 63;
    RowScan s;
    s.rpl = (p.R + 63) / 64;
    int sum = 0;
    const int r0 = lane * s.rpl, r1 = min(p.R, r0 + s.rpl);
    for (int r = r0; r < r1; ++r) sum += row_len(p, r);
    int inc = sum;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const int o = __shfl_up(inc, k);
        if (lane >= k) inc += o;
    }
    s.sum = sum;
    s.base = inc - sum;
    s.total = __builtin_amdgcn_readfirstlane(__shfl(inc, 63));
    return s;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// This slice's first row: the first row that ends after position a (found
// from the lane whose rows hold a, then a walk), and the line position P
// where it starts.  Wave-uniform results.
__device__ __forceinline__ void first_row(const DecodeParams &p, const RowScan &rs, int a, int &r, int &P) {
    const uint64_t hit = __ballot(rs.base + rs.sum > a && rs.sum > 0);
    const int l0 = uniform(__ffsll((unsigned long long)hit) - 1);
    r = l0 * rs.rpl;
    P = uniform(__shfl(rs.base, l0));
    for (int n0 = uniform(row_len(p, r)); P + n0 <= a; n0 = uniform(row_len(p, r))) {
        P += n0;
        ++r;
    }
}

}  // namespace pa
