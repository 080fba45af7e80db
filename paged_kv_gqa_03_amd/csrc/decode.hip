// decode.hip -- split-KV GQA decode and the log-sum-exp combine for gfx950.
//
// Method (AstrAI csrc commit history, the split-KV decode commit): the KV
// range of every (sequence, KV head) is cut into splits; each split keeps a
// running max, a sum of exponentials and an unnormalised weighted-V
// accumulator, and a combine kernel merges the splits.  When one split per
// sequence already fills the device the kernel writes the normalised output
// directly (same commit).  The KV source is either a paged pool read through
// the block table with a lookup per token (the commit that replaced the
// per-tile page lookup by a per-element one) or contiguous strides.
//
// Work decomposition on gfx950: a one-wave workgroup owns one split of one
// sequence for HW adjacent KV heads (HW in {1, 2, 4, 8}), so the dispatcher
// refills a compute unit as soon as any split finishes, whatever the ragged
// lengths of its neighbours.  Units are ordered split-major, so the last
// splits of long sequences run last and the tail is at most one split long.
// The wave carries all G = Hq/Hkv query heads of each
// of its KV heads, so K/V bytes are read once for the whole group (cf. the
// GQA head-packing commit in the doc's history).
//
// Lane layout: lane l = 8*grp + jj, with lane group grp = tg*HW + hw: hw
// picks the KV head, tg one of TG = 8/HW token streams, jj one of 8 chunk
// lanes.  A tile is 2*TG tokens; per tile a lane holds tokens tg and tg+TG
// and, for each, the 16-byte chunks jj, jj+8, ... of its head's K and V rows
// (D/64 chunks).  HW is chosen from the layout so that one load instruction
// reads memory that is contiguous: with the KV heads of a token adjacent
// ([pages, slot, head, dim] pools, blhd) HW = 8 and a tile is 2 tokens of
// whole 2 KB rows (a 16-token page is one 32 KB stream); with a head's
// tokens adjacent ([pages, head, slot, dim], bhld) HW = 1 and a tile is 16
// tokens of one head (4 KB contiguous).
//   scores  v_dot2_f32_bf16 of q and K chunks, summed over the 8 chunk lanes
//           with three DPP adds (quad_perm x2, row_half_mirror);
//   softmax each lane group keeps its own running state; the reference max
//           is only raised when a score exceeds it by more than 2^8 (base 2),
//           so rescaling of the accumulator is rare, and every exp2
//           argument stays <= 8;
//   P.V     the two tokens' V rows are interleaved into bf16 pairs and
//           accumulated with v_dot2 against the pair of bf16 weights, so
//           each V element costs G/2 dot2 plus half a permute.
// The TG token streams of a head are merged once per split (xor shuffles),
// then the wave writes either the normalised bf16 output (single split,
// direct mode) or the fp32 partial (m, l, o).
// Loads run two tiles ahead of the math (three register stages).  The
// split's block-table slice is copied into LDS once per wave before the loop,
// so page lookups inside the loop are LDS reads (lgkmcnt) and never sit in
// the in-order vmcnt queue between K/V loads.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

constexpr float kRescaleTh = 8.0f;  // log2 units

template <int NCH>
struct KVRegs {
    uint32_t ka[NCH][4], kb[NCH][4], va[NCH][4], vb[NCH][4];
};

// Per-lane page id and slot of the tile's two tokens (paged source only).
struct TokAddr {
    int pa, sa, pb, sb;
};

__device__ __forceinline__ void load16(const uint16_t *ptr, uint32_t (&dst)[4]) {
    const uint4 t = *reinterpret_cast<const uint4 *>(ptr);
    dst[0] = t.x; dst[1] = t.y; dst[2] = t.z; dst[3] = t.w;
}

template <int D, int G, int HW, bool PAGED>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeParams p) {
    constexpr int NCH = D / 64;
    constexpr int TG = 8 / HW;          // token streams per head
    constexpr int TILE = 2 * TG;        // tokens per tile
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x;
    const int ngrp = p.Hkv / HW;
    const int hgrp = u % ngrp;
    const int bsx = u / ngrp;
    const int b = bsx % p.B;
    const int s = bsx / p.B;
    const int n = p.kv_lens ? p.kv_lens[b] : p.kv_len_const;
    const int j0 = s * p.chunk;
    const int j1 = min(n, j0 + p.chunk);
    if (j0 >= j1 && s > 0) return;  // past the end of this sequence: no partial
    const int grp = lane >> 3, jj = lane & 7;
    const int hw = grp % HW, tg = grp / HW;
    const int g = hgrp * HW + hw;       // this lane's KV head
    const int last = j1 - 1;

    // Query slices of the G heads of this KV head, chunks jj + 8c.
    uint32_t qv[G][NCH][4];
    {
        const uint16_t *qb = p.q + b * p.q_sb + (int64_t)(g * G) * p.q_sh + jj * 8;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int c = 0; c < NCH; ++c) load16(qb + h * p.q_sh + c * 64, qv[h][c]);
    }

    float o[G][NCH][8];
    float mref[G], lsum[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mref[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h][c][e] = 0.f;
    }

    const int ntiles = (j1 - j0 + TILE - 1) / TILE;
    // Block-table slice of this split: page indices first_pg .. (j1-1)/ps.
    __shared__ int32_t pages[kDecodeMaxSplitPages];
    int first_pg = 0;
    if constexpr (PAGED) {
        if (ntiles > 0) {
            const int32_t *bt_row = p.bt + b * p.bt_sb;
            first_pg = (int)udiv_magic((uint32_t)j0, p.ps_magic);
            const int npg = (int)udiv_magic((uint32_t)last, p.ps_magic) - first_pg + 1;
            for (int i = lane; i < npg; i += 64) pages[i] = bt_row[first_pg + i];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
    // Base pointers of this (sequence, KV head) and this lane's chunk.  The
    // host guarantees every per-token offset below fits 32 bits except the
    // page term, which is a single 32x32->64 multiply-add.
    const uint16_t *kbase = p.k + jj * 8 + (PAGED ? g * p.s_head : b * p.k_sb + g * p.k_sh);
    const uint16_t *vbase = p.v + jj * 8 + (PAGED ? g * p.s_head : b * p.v_sb + g * p.v_sh);
    const uint32_t s_page = (uint32_t)p.s_page, s_slot = (uint32_t)p.s_slot;
    const uint32_t k_sl = (uint32_t)p.k_sl, v_sl = (uint32_t)p.v_sl;

    // Page ids (from the LDS slice) and slots of the lane's two tokens of tile t.
    auto lookup = [&](int t) {
        TokAddr a;
        const int ja = min(j0 + t * TILE + tg, last);
        const int jb = min(j0 + t * TILE + tg + TG, last);
        if constexpr (PAGED) {
            const uint32_t ia = udiv_magic((uint32_t)ja, p.ps_magic);
            const uint32_t ib = udiv_magic((uint32_t)jb, p.ps_magic);
            a.pa = pages[ia - first_pg];
            a.pb = pages[ib - first_pg];
            a.sa = ja - (int)(ia * p.ps);
            a.sb = jb - (int)(ib * p.ps);
        } else {
            a.pa = 0; a.pb = 0; a.sa = ja; a.sb = jb;
        }
        return a;
    };
    // Issue the 16-byte K/V loads of one tile.
    auto issue = [&](const TokAddr &a, KVRegs<NCH> &r) {
        uint64_t oka, okb, ova, ovb;
        if constexpr (PAGED) {
            oka = ova = (uint64_t)(uint32_t)a.pa * s_page + (uint32_t)a.sa * s_slot;
            okb = ovb = (uint64_t)(uint32_t)a.pb * s_page + (uint32_t)a.sb * s_slot;
        } else {
            oka = (uint32_t)a.sa * k_sl;
            okb = (uint32_t)a.sb * k_sl;
            ova = (uint32_t)a.sa * v_sl;
            ovb = (uint32_t)a.sb * v_sl;
        }
        const uint16_t *kA = kbase + oka, *kB = kbase + okb;
        const uint16_t *vA = vbase + ova, *vB = vbase + ovb;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            load16(kA + c * 64, r.ka[c]);
            load16(kB + c * 64, r.kb[c]);
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            load16(vA + c * 64, r.va[c]);
            load16(vB + c * 64, r.vb[c]);
        }
    };
    // Math of tile t on registers r.
    auto compute = [&](int t, const KVRegs<NCH> &r) {
        const int ja = j0 + t * TILE + tg;
        const bool oka = ja < j1, okb = ja + TG < j1;
        float xa[G], xb[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float sa = 0.f, sb = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    sa = dot2(r.ka[c][w], qv[h][c][w], sa);
                    sb = dot2(r.kb[c][w], qv[h][c][w], sb);
                }
            sa = sum8(sa);
            sb = sum8(sb);
            xa[h] = oka ? sa * p.sl2 : -INFINITY;
            xb[h] = okb ? sb * p.sl2 : -INFINITY;
        }
        bool need = false;
        float mt[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mt[h] = fmaxf(xa[h], xb[h]);
            need |= mt[h] > mref[h] + kRescaleTh;
        }
        if (need) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (mt[h] > mref[h] + kRescaleTh) {
                    const float alpha = exp2_fast(mref[h] - mt[h]);
                    lsum[h] *= alpha;
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[h][c][e] *= alpha;
                    mref[h] = mt[h];
                }
            }
        }
        uint32_t pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mu = fmaxf(mref[h], -3.0e38f);
            pp[h] = pack_bf16(exp2_fast(xa[h] - mu), exp2_fast(xb[h] - mu));
            lsum[h] += bf16_lo(pp[h]) + bf16_hi(pp[h]);
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t A = r.va[c][w], Bv = r.vb[c][w];
                const uint32_t lo = (A & 0xffffu) | (Bv << 16);
                const uint32_t hi = (A >> 16) | (Bv & 0xffff0000u);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    o[h][c][2 * w] = dot2(lo, pp[h], o[h][c][2 * w]);
                    o[h][c][2 * w + 1] = dot2(hi, pp[h], o[h][c][2 * w + 1]);
                }
            }
    };

    // The page lookup of a tile sits right before its loads: page ids are
    // never carried across iterations.  Past the last tile the loads repeat
    // the last tile (always in bounds, never used).
    // Three register stages: while tile t is computed, tiles t+1 and t+2 are
    // in flight.  The loop has a single exit at the bottom, so the compiler's
    // wait-count pass keeps both tiles outstanding across the back edge.
    if (ntiles > 0) {
        const int tl = ntiles - 1;
        KVRegs<NCH> r0, r1, r2;
        issue(lookup(0), r0);
        issue(lookup(min(1, tl)), r1);
        int t = 0;
        for (; t + 2 < ntiles; t += 3) {
            issue(lookup(t + 2), r2);
            compute(t, r0);
            issue(lookup(min(t + 3, tl)), r0);
            compute(t + 1, r1);
            issue(lookup(min(t + 4, tl)), r1);
            compute(t + 2, r2);
        }
        if (t < ntiles) compute(t, r0);
        if (t + 1 < ntiles) compute(t + 1, r1);
    }

    // Merge the TG token streams of each head (lanes equal in hw and jj,
    // i.e. lane ids differing in the bits above 8*HW).
    if constexpr (TG > 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float M = mref[h];
#pragma unroll
            for (int m = 8 * HW; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
            const float f = (mref[h] == -INFINITY) ? 0.f : exp2_fast(mref[h] - M);
            float l = lsum[h] * f;
#pragma unroll
            for (int m = 8 * HW; m < 64; m <<= 1) l += __shfl_xor(l, m);
            lsum[h] = l;
            mref[h] = M;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = o[h][c][e] * f;
#pragma unroll
                    for (int m = 8 * HW; m < 64; m <<= 1) x += __shfl_xor(x, m);
                    o[h][c][e] = x;
                }
        }
    }

    // After the merge every token stream holds the head's totals; stream tg
    // writes the query heads h with h % TG == tg.
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (h % TG != tg) continue;
        const int hq = g * G + h;
        if (p.direct) {
            const float inv = lsum[h] > 0.f ? 1.f / lsum[h] : 0.f;
            uint16_t *dst = p.o + b * p.o_sb + hq * p.o_sh + jj * 8;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                uint4 w;
                w.x = pack_bf16(o[h][c][0] * inv, o[h][c][1] * inv);
                w.y = pack_bf16(o[h][c][2] * inv, o[h][c][3] * inv);
                w.z = pack_bf16(o[h][c][4] * inv, o[h][c][5] * inv);
                w.w = pack_bf16(o[h][c][6] * inv, o[h][c][7] * inv);
                *reinterpret_cast<uint4 *>(dst + c * 64) = w;
            }
        } else {
            const size_t row = ((size_t)s * p.B + b) * p.Hq + hq;
            float *dst = p.o_part + row * D + jj * 8;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                *reinterpret_cast<float4 *>(dst + c * 64) =
                    make_float4(o[h][c][0], o[h][c][1], o[h][c][2], o[h][c][3]);
                *reinterpret_cast<float4 *>(dst + c * 64 + 4) =
                    make_float4(o[h][c][4], o[h][c][5], o[h][c][6], o[h][c][7]);
            }
            if (jj == 0)
                *reinterpret_cast<float2 *>(p.ml_part + row * 2) = make_float2(mref[h] * kLn2, lsum[h]);
        }
    }
}

// One wave per output row: M = max_s m_s, w_s = exp(m_s - M),
// out = sum_s w_s o_s / sum_s w_s l_s.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
    constexpr int NC = D / 64;
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + wave_id();
    if (r >= p.R) return;
    int S = p.S;
    if (p.chunk > 0) {
        const int seq = r / p.rows_per_seq;
        const int n = p.kv_lens ? p.kv_lens[seq] : p.kv_len_const;
        S = min(S, max(1, (n + p.chunk - 1) / p.chunk));
    }
    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, p.ml_part[((size_t)s * p.R + r) * 2]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k));
    float acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.f;
    float L = 0.f;
    if (M != -INFINITY) {
        // Eight splits per step, all loads issued before the math.
        constexpr int U = 8;
        const size_t rstride = (size_t)p.R;
        for (int s0 = 0; s0 < S; s0 += U) {
            float2 ml[U];
            float ov[U][NC];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int sk = min(s0 + k, S - 1);
                ml[k] = *reinterpret_cast<const float2 *>(p.ml_part + ((size_t)sk * rstride + r) * 2);
                const float *op = p.o_part + ((size_t)sk * rstride + r) * D + lane * NC;
#pragma unroll
                for (int c = 0; c < NC; ++c) ov[k][c] = op[c];
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const bool use = (s0 + k < S) && ml[k].x != -INFINITY;
                const float w = use ? exp2_fast((ml[k].x - M) * kLog2e) : 0.f;
                L = fmaf(w, use ? ml[k].y : 0.f, L);
#pragma unroll
                for (int c = 0; c < NC; ++c) acc[c] = fmaf(w, use ? ov[k][c] : 0.f, acc[c]);
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (p.out_f32) {
#pragma unroll
        for (int c = 0; c < NC; ++c) p.out_f32[(size_t)r * D + lane * NC + c] = acc[c] * inv;
    }
    if (p.out_bf16) {
        uint16_t *dst = p.out_bf16 + (int64_t)(r / p.rows_per_seq) * p.o_sb +
                        (int64_t)(r % p.rows_per_seq) * p.o_sh + lane * NC;
        if constexpr (NC == 2) {
            *reinterpret_cast<uint32_t *>(dst) = pack_bf16(acc[0] * inv, acc[1] * inv);
        } else {
            const uint32_t w = pack_bf16(acc[0] * inv, 0.f);
            dst[0] = (uint16_t)(w & 0xffffu);
        }
    }
    if (p.lse && lane == 0) p.lse[r] = (L > 0.f) ? M + __logf(L) : -INFINITY;
}

template <int D, int G, int HW, bool PAGED>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<D, G, HW, PAGED>), dim3(p.units), dim3(64), 0, stream, p);
    return hipGetLastError();
}

template <int D, int HW, bool PAGED>
hipError_t launch_decode_g(const DecodeParams &p, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_decode_t<D, 1, HW, PAGED>(p, stream);
        case 2: return launch_decode_t<D, 2, HW, PAGED>(p, stream);
        case 4: return launch_decode_t<D, 4, HW, PAGED>(p, stream);
        case 8: return launch_decode_t<D, 8, HW, PAGED>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool PAGED>
hipError_t launch_decode_hw(const DecodeParams &p, int G, hipStream_t stream) {
    switch (p.HW) {
        case 1: return launch_decode_g<D, 1, PAGED>(p, G, stream);
        case 2: return launch_decode_g<D, 2, PAGED>(p, G, stream);
        case 4: return launch_decode_g<D, 4, PAGED>(p, G, stream);
        case 8: return launch_decode_g<D, 8, PAGED>(p, G, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int D, int G, bool paged, hipStream_t stream) {
    if (p.units <= 0) return hipSuccess;
    if (D == 64) return paged ? launch_decode_hw<64, true>(p, G, stream) : launch_decode_hw<64, false>(p, G, stream);
    if (D == 128) return paged ? launch_decode_hw<128, true>(p, G, stream) : launch_decode_hw<128, false>(p, G, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_combine(const CombineParams &p, int D, hipStream_t stream) {
    if (p.R <= 0) return hipSuccess;
    const int blocks = (p.R + 3) / 4;
    if (D == 64) hipLaunchKernelGGL((combine_kernel<64>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 128) hipLaunchKernelGGL((combine_kernel<128>), dim3(blocks), dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
