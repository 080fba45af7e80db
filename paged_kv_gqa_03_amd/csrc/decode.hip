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
// Work decomposition on gfx950: one wave64 per (sequence b, KV head g,
// split s); a workgroup holds four independent waves that never synchronise
// with each other (each owns a private LDS slice for its page ids).  The wave carries all G = Hq/Hkv query heads of its
// KV head, so K/V bytes are read once for the whole group (cf. the GQA head
// packing commit in the doc's history).
//
// Lane layout: a tile is 16 tokens.  Lane l owns token group tok = l/8 and
// chunk lane jj = l%8; per tile it holds tokens tok and tok+8 and, for each,
// the 16-byte chunks jj, jj+8, ... of the K and V rows (D/64 chunks).  One
// load instruction therefore reads 8 rows x 128 contiguous bytes.
//   scores  v_dot2_f32_bf16 of q and K chunks, summed over the 8 lanes of a
//           token with three DPP adds (quad_perm x2, row_half_mirror);
//   softmax each token group keeps its own running state; the reference
//           max is only raised when a score exceeds it by more than 2^8
//           (base 2), so rescaling of the accumulator is rare, and every
//           exp2 argument stays <= 8;
//   P.V     the two tokens' V rows are interleaved into bf16 pairs and
//           accumulated with v_dot2 against the pair of bf16 weights, so
//           each V element costs G/2 dot2 plus half a permute.
// The eight token groups are merged once per split (xor shuffles), then the
// wave writes either the normalised bf16 output (single split, direct mode)
// or the fp32 partial (m, l, o).
// Loads run one tile ahead of the math (double-buffered registers).  The
// split's block-table slice is copied into LDS once per wave before the loop,
// so page lookups inside the loop are LDS reads (lgkmcnt) and never sit in
// the in-order vmcnt queue between K/V loads.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

constexpr int kTile = 16;
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

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeParams p) {
    constexpr int NCH = D / 64;
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * 4 + wave_id();
    if (u >= p.units) return;
    const int g = u % p.Hkv;
    const int bsx = u / p.Hkv;
    const int b = bsx % p.B;
    const int s = bsx / p.B;
    const int n = p.kv_lens ? p.kv_lens[b] : p.kv_len_const;
    const int j0 = s * p.chunk;
    const int j1 = min(n, j0 + p.chunk);
    if (j0 >= j1 && s > 0) return;  // past the end of this sequence: no partial
    const int tok = lane >> 3, jj = lane & 7;
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

    const int ntiles = (j1 - j0 + kTile - 1) / kTile;
    // Block-table slice of this split: page indices first_pg .. (j1-1)/ps.
    __shared__ int32_t s_pages[4][kDecodeMaxSplitPages];
    int32_t *pages = s_pages[wave_id()];
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
    const int64_t head_off_k = PAGED ? g * p.s_head : b * p.k_sb + g * p.k_sh;
    const int64_t head_off_v = PAGED ? g * p.s_head : b * p.v_sb + g * p.v_sh;

    // Page ids (from the LDS slice) and slots of the lane's two tokens of tile t.
    auto lookup = [&](int t) {
        TokAddr a;
        const int ja = min(j0 + t * kTile + tok, last);
        const int jb = min(j0 + t * kTile + tok + 8, last);
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
        int64_t oka, okb, ova, ovb;
        if constexpr (PAGED) {
            oka = ova = (int64_t)a.pa * p.s_page + (int64_t)a.sa * p.s_slot + head_off_k;
            okb = ovb = (int64_t)a.pb * p.s_page + (int64_t)a.sb * p.s_slot + head_off_k;
        } else {
            oka = head_off_k + (int64_t)a.sa * p.k_sl;
            okb = head_off_k + (int64_t)a.sb * p.k_sl;
            ova = head_off_v + (int64_t)a.sa * p.v_sl;
            ovb = head_off_v + (int64_t)a.sb * p.v_sl;
        }
        const uint16_t *kA = p.k + oka + jj * 8, *kB = p.k + okb + jj * 8;
        const uint16_t *vA = p.v + ova + jj * 8, *vB = p.v + ovb + jj * 8;
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
        const int ja = j0 + t * kTile + tok;
        const bool oka = ja < j1, okb = ja + 8 < j1;
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
    // The loop has a single exit at the bottom so the compiler's wait-count
    // pass keeps exactly one tile of loads in flight across the back edge.
    if (ntiles > 0) {
        const int tl = ntiles - 1;
        KVRegs<NCH> r0, r1;
        issue(lookup(0), r0);
        int t = 0;
        for (; t + 1 < ntiles; t += 2) {
            issue(lookup(t + 1), r1);
            compute(t, r0);
            issue(lookup(min(t + 2, tl)), r0);
            compute(t + 1, r1);
        }
        if (t < ntiles) compute(t, r0);
    }

    // Merge the eight token groups (lanes with equal jj).
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = mref[h];
        M = fmaxf(M, __shfl_xor(M, 8));
        M = fmaxf(M, __shfl_xor(M, 16));
        M = fmaxf(M, __shfl_xor(M, 32));
        const float f = (mref[h] == -INFINITY) ? 0.f : exp2_fast(mref[h] - M);
        float l = lsum[h] * f;
        l += __shfl_xor(l, 8);
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        lsum[h] = l;
        mref[h] = M;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = o[h][c][e] * f;
                x += __shfl_xor(x, 8);
                x += __shfl_xor(x, 16);
                x += __shfl_xor(x, 32);
                o[h][c][e] = x;
            }
    }

    // Token group `tok` writes head tok of the group.
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if (tok != h) continue;
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
        for (int s = 0; s < S; ++s) {
            const float2 ml = *reinterpret_cast<const float2 *>(p.ml_part + ((size_t)s * p.R + r) * 2);
            const float w = (ml.x == -INFINITY) ? 0.f : exp2_fast((ml.x - M) * kLog2e);
            L += w * ml.y;
            const float *op = p.o_part + ((size_t)s * p.R + r) * D + lane * NC;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c] = fmaf(w, op[c], acc[c]);
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

template <int D, int G, bool PAGED>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t stream) {
    const int blocks = (p.units + 3) / 4;
    hipLaunchKernelGGL((decode_split_kernel<D, G, PAGED>), dim3(blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t launch_decode_g(const DecodeParams &p, int G, hipStream_t stream) {
    switch (G) {
        case 1: return launch_decode_t<D, 1, PAGED>(p, stream);
        case 2: return launch_decode_t<D, 2, PAGED>(p, stream);
        case 4: return launch_decode_t<D, 4, PAGED>(p, stream);
        case 8: return launch_decode_t<D, 8, PAGED>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int D, int G, bool paged, hipStream_t stream) {
    if (p.units <= 0) return hipSuccess;
    if (D == 64) return paged ? launch_decode_g<64, true>(p, G, stream) : launch_decode_g<64, false>(p, G, stream);
    if (D == 128) return paged ? launch_decode_g<128, true>(p, G, stream) : launch_decode_g<128, false>(p, G, stream);
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
