// decode.hip -- split-KV GQA decode and the log-sum-exp combine for gfx950.
//
// Method (AstrAI csrc commit history, the split-KV decode commit): the KV
// range of every (sequence, KV head) is cut into pieces; each piece keeps a
// running max, a sum of exponentials and an unnormalised weighted-V
// accumulator, and a combine kernel merges the pieces.  A sequence that one
// piece covers entirely is written directly, normalised (same commit's
// single-pass direct write).  The KV source is either a paged pool read
// through the block table with a lookup per token (the commit that replaced
// the per-tile page lookup by a per-element one) or contiguous strides.
//
// Balanced partition.  The rows r = (sequence b, group of HW adjacent KV
// heads) are laid end to end, row r holding kv_lens[b] tokens; the whole
// line of T tokens is cut into W equal slices and wave w takes tokens
// [w*T/W, (w+1)*T/W).  Every wave therefore streams the same number of
// bytes whatever the spread of lengths, and the planner keeps W near three
// waves per compute unit (long, contiguous streams).  A wave finds its
// slice with a wave-wide scan of kv_lens (no extra launch) and writes one
// partial per row it touches at slot r + w: moving along the line, every
// wave or row boundary increments w or r, so r + w names each piece
// uniquely and a row's pieces occupy consecutive slots.
//
// Lane layout: lane l = JJ*grp + jj, with lane group grp = tg*HW + hw: hw
// picks the KV head of the row, tg one of TG = (64/JJ)/HW token streams, jj
// one of JJ chunk lanes (JJ = 8 for D = 64 and 128, 4 for D = 32, 16 for
// D = 256).  A tile is 2*TG tokens; per tile a lane holds tokens tg and
// tg+TG and, for each, the 16-byte chunks jj, jj+JJ, ... of its head's K and
// V rows (NCH = D/(8*JJ) chunks: 1, or 2 at D = 128 and 256).  HW is chosen
// from the layout so that one load instruction reads memory that is
// contiguous: with the KV heads of a token adjacent ([pages, slot, head,
// dim] pools, blhd) HW = min(8, 64/JJ) and at D = 128 a tile is two tokens
// of whole 2 KB rows (a 16-token page is one 32 KB stream); with a head's
// tokens adjacent ([pages, head, slot, dim], bhld) HW = 1 and at D = 128 a
// tile is 16 tokens of one head (4 KB contiguous).
//   scores  v_dot2_f32_bf16 of q and K chunks, summed over the JJ chunk
//           lanes with DPP adds (quad_perm x2, row_half_mirror, row_mirror);
//   softmax each lane group keeps its own running state; the reference max
//           is only raised when a score exceeds it by more than 2^8 (base 2),
//           so rescaling of the accumulator is rare, and every exp2
//           argument stays <= 8;
//   P.V     the two tokens' V rows are interleaved into bf16 pairs and
//           accumulated with v_dot2 against the pair of bf16 weights, so
//           each V element costs G/2 dot2 plus half a permute.
// Loads run two tiles ahead of the math (three register stages).  The
// piece's block-table slice is copied into LDS before its tile loop, so page
// lookups inside the loop are LDS reads (lgkmcnt) and never sit in the
// in-order vmcnt queue between K/V loads; pieces longer than the slice run
// as consecutive sub-pieces.
#include "decode_common.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

constexpr float kRescaleTh = 8.0f;  // log2 units

template <int NCH>
struct KVRegs {
    uint32_t ka[NCH][4], kb[NCH][4], va[NCH][4], vb[NCH][4];
};

// Page id and slot of the lane's two tokens of a tile (slot = position for
// a contiguous source).
struct TokAddr {
    int pa, sa, pb, sb;
};

// Chunk lanes per head row and 16-byte chunks per lane at head dim D.
template <int D>
constexpr int chunk_lanes() { return D == 32 ? 4 : (D == 256 ? 16 : 8); }

// Sum over aligned groups of JJ lanes (4, 8 or 16), result in every lane.
template <int JJ>
__device__ __forceinline__ float sum_lanes(float x) {
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    if constexpr (JJ >= 8) x += dpp_mov<kDppHalfMirror>(x);
    if constexpr (JJ >= 16) x += dpp_mov<kDppMirror>(x);
    return x;
}

// Per-lane state of one wave handed to the others of its workgroup: for each
// query head, the reference, the sum and the NCH x 8 accumulators, stored
// field-major so a wave's 64 lanes touch consecutive words.
template <int G, int NCH>
constexpr int xch_fields() { return G * (2 + 8 * NCH); }

template <int D, int G, int HW, bool PAGED, int NW>
__global__ __launch_bounds__(64 * NW, (G >= 8 ? 1 : 2)) void decode_split_kernel(const DecodeParams p) {
    constexpr int JJ = chunk_lanes<D>();
    constexpr int NCH = D / (8 * JJ);   // 16-byte chunks per lane and row
    constexpr int CS = 8 * JJ;          // elements between a lane's chunks
    constexpr int TG = 64 / JJ / HW;    // token streams per head
    static_assert(TG >= 1, "a wave holds at most 64 / JJ KV heads");
    constexpr int TILE = 2 * TG;        // tokens per tile
    constexpr int HWG = HW * G;         // query heads per row
    constexpr int NT = 64 * NW;         // threads of the workgroup
    const int lane = threadIdx.x & 63;
    // Wave of the workgroup: the NW waves take alternate tiles of every
    // piece of the slice and merge their states through LDS at its end.
    const int wv = NW > 1 ? wave_id() : 0;
    const int w = blockIdx.x;
    const int grp = lane / JJ, jj = lane % JJ;
    const int hw = grp % HW, tg = grp / HW;

    // This wave's slice [a, e) of the line of all rows (wave-uniform values,
    // kept in scalar registers).
    const RowScan rs = scan_rows(p);
    const int T = rs.total;
    const int a = uniform((int)((int64_t)w * T / p.W)), e = uniform((int)((int64_t)(w + 1) * T / p.W));
    if (a >= T) return;   // an empty slice at the end of the line
    // First row that ends after a: the lane whose rows hold it, then a walk.
    const uint64_t hit = __ballot(rs.base + rs.sum > a && rs.sum > 0);
    const int l0 = uniform(__ffsll((unsigned long long)hit) - 1);
    int r = l0 * rs.rpl;
    int P = uniform(__shfl(rs.base, l0));
    for (int n0 = uniform(row_len(p, r)); P + n0 <= a; n0 = uniform(row_len(p, r))) {
        P += n0;
        ++r;
    }
    if (a >= e) {
        // Empty slices exist only when W exceeds the keys of all rows.  One
        // whose position lies strictly inside row r sits inside that row's
        // run of slots r + w, which the combine merges whole: mark the slot
        // empty (m = -inf, l = 0; the combine then ignores its o).
        if (P < a && wv == 0)
            for (int i = lane; i < HWG; i += 64)
                *reinterpret_cast<float2 *>(p.ml_part + ((int64_t)(r + w) * HWG + i) * 2) =
                    make_float2(-INFINITY, 0.f);
        return;
    }

    __shared__ int32_t pages[kDecodeMaxSplitPages];
    __shared__ float xch[NW > 1 ? NW * xch_fields<G, NCH>() * 64 : 1];
    const uint32_t s_page = (uint32_t)p.s_page, s_slot = (uint32_t)p.s_slot;
    const uint32_t k_sl = (uint32_t)p.k_sl, v_sl = (uint32_t)p.v_sl;

    for (; P < e && r < p.R; ++r) {
        const int n = uniform(row_len(p, r));
        const int lo = max(a, P) - P, hi = min(e, P + n) - P;
        P += n;
        if (lo >= hi) continue;
        // The waves holding the row's first and last keys record themselves,
        // so the combine finds the row's pieces (slots r + first .. r + last)
        // without scanning the lengths.
        if (p.ranges && lane == 0 && wv == 0) {
            if (lo == 0) p.ranges[2 * (int64_t)r] = w;
            if (hi == n) p.ranges[2 * (int64_t)r + 1] = w;
        }
        const int b = r / p.ngrp, hgrp = r % p.ngrp;
        // A row is (sequence, group of HW KV heads), or with several passes
        // (sequence, KV head, pass): pass j covers query heads j*G .. j*G+G-1
        // of the KV head's G_all.
        const int g = (hgrp / p.passes) * HW + hw;   // this lane's KV head
        const int h0 = g * p.G_all + (hgrp % p.passes) * G;   // first query head of the pass

        // Query slices of the G heads of this pass, chunks jj + JJ*c.
        uint32_t qv[G][NCH][4];
        {
            const uint16_t *qb = p.q + b * p.q_sb + (int64_t)h0 * p.q_sh + jj * 8;
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int c = 0; c < NCH; ++c) load16(qb + h * p.q_sh + c * CS, qv[h][c]);
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
                for (int x = 0; x < 8; ++x) o[h][c][x] = 0.f;
        }
        // Base pointers of this (sequence, KV head) and this lane's chunk.
        // The host guarantees every per-token offset below fits 32 bits
        // except the page term, a single 32x32->64 multiply-add.
        const uint16_t *kbase = p.k + jj * 8 + (PAGED ? g * p.s_head : b * p.k_sb + g * p.k_sh);
        const uint16_t *vbase = p.v + jj * 8 + (PAGED ? g * p.s_head : b * p.v_sb + g * p.v_sh);

        // Sub-pieces small enough for the LDS page slice.
        for (int j0 = lo; j0 < hi; j0 += p.max_sub) {
            const int j1 = min(hi, j0 + p.max_sub);
            const int last = j1 - 1;
            const int ntiles = (j1 - j0 + TILE - 1) / TILE;
            int first_pg = 0;
            if constexpr (PAGED) {
                const int32_t *bt_row = p.bt + b * p.bt_sb;
                first_pg = (int)divu32((uint32_t)j0, p.ps_div);
                const int npg = (int)divu32((uint32_t)last, p.ps_div) - first_pg + 1;
                if constexpr (NW > 1) {
                    __syncthreads();   // earlier readers of the slice are done
                    for (int i = threadIdx.x; i < npg; i += NT) pages[i] = bt_row[first_pg + i];
                    __syncthreads();
                } else {
                    __builtin_amdgcn_wave_barrier();   // earlier readers of the slice are done
                    for (int i = lane; i < npg; i += 64) pages[i] = bt_row[first_pg + i];
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
            }

            // This wave's tiles of the sub-piece: wv, wv + NW, wv + 2 NW, ...;
            // k below counts them.
            const int ntw = ntiles > wv ? (ntiles - wv + NW - 1) / NW : 0;
            auto lookup = [&](int k) {
                TokAddr ad;
                const int t = wv + NW * k;
                const int ja = min(j0 + t * TILE + tg, last);
                const int jb = min(j0 + t * TILE + tg + TG, last);
                if constexpr (PAGED) {
                    const uint32_t ia = divu32((uint32_t)ja, p.ps_div);
                    const uint32_t ib = divu32((uint32_t)jb, p.ps_div);
                    ad.pa = pages[ia - first_pg];
                    ad.pb = pages[ib - first_pg];
                    ad.sa = ja - (int)(ia * p.ps);
                    ad.sb = jb - (int)(ib * p.ps);
                } else {
                    ad.pa = 0; ad.pb = 0; ad.sa = ja; ad.sb = jb;
                }
                return ad;
            };
            auto issue = [&](const TokAddr &ad, KVRegs<NCH> &rg) {
                uint64_t oka, okb, ova, ovb;
                if constexpr (PAGED) {
                    oka = ova = (uint64_t)(uint32_t)ad.pa * s_page + (uint32_t)ad.sa * s_slot;
                    okb = ovb = (uint64_t)(uint32_t)ad.pb * s_page + (uint32_t)ad.sb * s_slot;
                } else {
                    oka = (uint32_t)ad.sa * k_sl;
                    okb = (uint32_t)ad.sb * k_sl;
                    ova = (uint32_t)ad.sa * v_sl;
                    ovb = (uint32_t)ad.sb * v_sl;
                }
                const uint16_t *kA = kbase + oka, *kB = kbase + okb;
                const uint16_t *vA = vbase + ova, *vB = vbase + ovb;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    load16_stream(kA + c * CS, rg.ka[c]);
                    load16_stream(kB + c * CS, rg.kb[c]);
                }
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    load16_stream(vA + c * CS, rg.va[c]);
                    load16_stream(vB + c * CS, rg.vb[c]);
                }
            };
            auto compute = [&](int k, const KVRegs<NCH> &rg) {
                const int ja = j0 + (wv + NW * k) * TILE + tg;
                const bool oka = ja < j1, okb = ja + TG < j1;
                float xa[G], xb[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    float sa = 0.f, sb = 0.f;
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            sa = dot2(rg.ka[c][q], qv[h][c][q], sa);
                            sb = dot2(rg.kb[c][q], qv[h][c][q], sb);
                        }
                    sa = sum_lanes<JJ>(sa);
                    sb = sum_lanes<JJ>(sb);
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
                                for (int x = 0; x < 8; ++x) o[h][c][x] *= alpha;
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
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t A = rg.va[c][q], Bv = rg.vb[c][q];
                        const uint32_t lo2 = (A & 0xffffu) | (Bv << 16);
                        const uint32_t hi2 = (A >> 16) | (Bv & 0xffff0000u);
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            o[h][c][2 * q] = dot2(lo2, pp[h], o[h][c][2 * q]);
                            o[h][c][2 * q + 1] = dot2(hi2, pp[h], o[h][c][2 * q + 1]);
                        }
                    }
            };

            // Three register stages: while tile t is computed, tiles t+1 and
            // t+2 are in flight.  The loop has a single exit at the bottom,
            // so the compiler's wait-count pass keeps both tiles outstanding
            // across the back edge.  Page lookups sit right before their
            // loads and are never carried across iterations; past the last
            // tile the loads repeat the last tile (in bounds, never used).
            if (ntw > 0) {
                const int tl = ntw - 1;
                KVRegs<NCH> r0, r1, r2;
                issue(lookup(0), r0);
                issue(lookup(min(1, tl)), r1);
                int t = 0;
                for (; t + 2 < ntw; t += 3) {
                    issue(lookup(t + 2), r2);
                    compute(t, r0);
                    issue(lookup(min(t + 3, tl)), r0);
                    compute(t + 1, r1);
                    issue(lookup(min(t + 4, tl)), r1);
                    compute(t + 2, r2);
                }
                if (t < ntw) compute(t, r0);
                if (t + 1 < ntw) compute(t + 1, r1);
            }
        }

        // Merge the TG token streams of each head (lanes equal in hw and jj,
        // i.e. lane ids differing in the bits above JJ*HW).
        if constexpr (TG > 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float M = mref[h];
#pragma unroll
                for (int m = JJ * HW; m < 64; m <<= 1) M = fmaxf(M, __shfl_xor(M, m));
                const float f = (mref[h] == -INFINITY) ? 0.f : exp2_fast(mref[h] - M);
                float l = lsum[h] * f;
#pragma unroll
                for (int m = JJ * HW; m < 64; m <<= 1) l += __shfl_xor(l, m);
                lsum[h] = l;
                mref[h] = M;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        float v = o[h][c][x] * f;
#pragma unroll
                        for (int m = JJ * HW; m < 64; m <<= 1) v += __shfl_xor(v, m);
                        o[h][c][x] = v;
                    }
            }
        }

        // Merge the NW waves' states of the piece: every wave leaves its
        // (reference, sum, accumulators) in LDS, then wave wv merges the
        // query heads h with h % NW == wv from all of them.
        if constexpr (NW > 1) {
            constexpr int F = 2 + 8 * NCH;
            __syncthreads();   // the previous piece's readers are done with xch
            float *mine = xch + wv * (G * F * 64);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                mine[(h * F + 0) * 64 + lane] = mref[h];
                mine[(h * F + 1) * 64 + lane] = lsum[h];
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int x = 0; x < 8; ++x) mine[(h * F + 2 + 8 * c + x) * 64 + lane] = o[h][c][x];
            }
            __syncthreads();
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (h % NW != wv) continue;
                float M = -INFINITY;
#pragma unroll
                for (int v = 0; v < NW; ++v) M = fmaxf(M, xch[(v * G * F + h * F) * 64 + lane]);
                float l = 0.f;
#pragma unroll
                for (int c = 0; c < NCH; ++c)
#pragma unroll
                    for (int x = 0; x < 8; ++x) o[h][c][x] = 0.f;
#pragma unroll
                for (int v = 0; v < NW; ++v) {
                    const float *src = xch + (v * G * F + h * F) * 64 + lane;
                    const float mv = src[0];
                    const float f = mv == -INFINITY ? 0.f : exp2_fast(mv - M);
                    l += f * src[64];
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
#pragma unroll
                        for (int x = 0; x < 8; ++x) o[h][c][x] += f * src[(2 + 8 * c + x) * 64];
                }
                mref[h] = M;
                lsum[h] = l;
            }
        }

        // Every token stream now holds the head's totals; stream tg of wave
        // wv writes the query heads h with h % NW == wv and (h / NW) % TG ==
        // tg.  A piece covering the whole row is the row's only piece:
        // written normalised when direct writes are on.
        const bool direct = p.direct && lo == 0 && hi == n;
        const int64_t slot = (int64_t)r + w;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (h % NW != wv || (h / NW) % TG != tg) continue;
            const int hq = h0 + h;
            if (direct) {
                const float inv = lsum[h] > 0.f ? 1.f / lsum[h] : 0.f;
                uint16_t *dst = p.o + b * p.o_sb + hq * p.o_sh + jj * 8;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    uint4 v;
                    v.x = pack_bf16(o[h][c][0] * inv, o[h][c][1] * inv);
                    v.y = pack_bf16(o[h][c][2] * inv, o[h][c][3] * inv);
                    v.z = pack_bf16(o[h][c][4] * inv, o[h][c][5] * inv);
                    v.w = pack_bf16(o[h][c][6] * inv, o[h][c][7] * inv);
                    *reinterpret_cast<uint4 *>(dst + c * CS) = v;
                }
            } else {
                const int64_t prow = slot * HWG + hw * G + h;
                float *dst = p.o_part + prow * D + jj * 8;
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    *reinterpret_cast<float4 *>(dst + c * CS) =
                        make_float4(o[h][c][0], o[h][c][1], o[h][c][2], o[h][c][3]);
                    *reinterpret_cast<float4 *>(dst + c * CS + 4) =
                        make_float4(o[h][c][4], o[h][c][5], o[h][c][6], o[h][c][7]);
                }
                if (jj == 0)
                    *reinterpret_cast<float2 *>(p.ml_part + prow * 2) = make_float2(partial_m(mref[h], lsum[h]), lsum[h]);
            }
        }
    }
}

// Floats of a head row each combine lane holds, and the lanes that hold
// some (D / epl; all 64 except at D = 32).
template <int D>
constexpr int combine_epl() { return D >= 64 ? D / 64 : 1; }

// Log-sum-exp merge of S partials at rows first + s*stride:
// M = max_s m_s, w_s = exp(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s.
// Lanes past the row (D = 32) read its last elements and are not stored.
template <int D>
__device__ __forceinline__ void merge_partials(const float *o_part, const float *ml_part, int64_t first,
                                               int64_t stride, int S, int lane,
                                               float (&acc)[combine_epl<D>()], float &L, float &M) {
    constexpr int NC = combine_epl<D>();
    const int ln = min(lane, D / NC - 1);
    constexpr int U = 8;
    M = -INFINITY;
    L = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.f;
    // Rows of more than 2U pieces: the maximum first, from one round of
    // loads spread over the lanes (which also brings every (m, l) into the
    // caches), then the sums.  Shorter rows: rounds of U pieces, every lane
    // loading all (m, l) and its share of o, the running maximum rescaling
    // what was summed before it.  (Measured on the B = 32 and B = 128 serving
    // batches, whose rows have about 24 and 6-12 pieces.)
    if (S > 2 * U) {
        for (int s = lane; s < S; s += 64) M = fmaxf(M, ml_part[(first + s * stride) * 2]);
#pragma unroll
        for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k));
        if (M == -INFINITY) return;
    }
    for (int s0 = 0; s0 < S; s0 += U) {
        float2 ml[U];
        float ov[U][NC];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t row = first + (int64_t)min(s0 + k, S - 1) * stride;
            ml[k] = *reinterpret_cast<const float2 *>(ml_part + row * 2);
            const float *op = o_part + row * D + ln * NC;
#pragma unroll
            for (int c = 0; c < NC; ++c) ov[k][c] = op[c];
        }
        float mc = M;
#pragma unroll
        for (int k = 0; k < U; ++k) mc = (s0 + k < S) ? fmaxf(mc, ml[k].x) : mc;
        if (mc == -INFINITY) continue;   // nothing but empty pieces so far
        if (mc > M) {
            const float f = M == -INFINITY ? 0.f : exp2_fast((M - mc) * kLog2e);
            L *= f;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c] *= f;
            M = mc;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const bool use = (s0 + k < S) && ml[k].x != -INFINITY;
            const float wgt = use ? exp2_fast((ml[k].x - M) * kLog2e) : 0.f;
            L = fmaf(wgt, use ? ml[k].y : 0.f, L);
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c] = fmaf(wgt, use ? ov[k][c] : 0.f, acc[c]);
        }
    }
}

// The lane's NC floats of a row, scaled by inv, as bf16 (32-bit stores).
template <int NC>
__device__ __forceinline__ void store_row_bf16(uint16_t *dst, const float (&acc)[NC], float inv) {
    if constexpr (NC == 1) {
        dst[0] = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
    } else {
#pragma unroll
        for (int c = 0; c < NC; c += 2)
            *reinterpret_cast<uint32_t *>(dst + c) = pack_bf16(acc[c] * inv, acc[c + 1] * inv);
    }
}

// Combine of the balanced decode partition: one wave per (sequence, query
// head), four to a workgroup.  A row's pieces are the slots r + w for the
// waves w that hold its first and last token.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const DecodeCombineParams p) {
    constexpr int NC = combine_epl<D>();
    const int lane = threadIdx.x & 63;
    const bool holds = lane < D / NC;
    const int item = blockIdx.x * 4 + wave_id();
    if (item >= p.B * p.Hq) return;
    const int b = item / p.Hq, hq = item - b * p.Hq;
    const int hwg = p.Hq / p.ngrp;                 // query heads per row
    const int r = b * p.ngrp + hq / hwg;           // this head's row
    // The length and the row's slice range are loaded together (the range
    // is read even for an empty row; the split kernel leaves it unwritten
    // then, and it is not used).
    int2 rg = make_int2(0, 0);
    if (p.W > 1) rg = *reinterpret_cast<const int2 *>(p.ranges + 2 * (int64_t)r);
    const int n = p.kv_lens ? p.kv_lens[b] : p.kv_len_const;
    uint16_t *dst = p.o + (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + lane * NC;
    if (n == 0) {   // no keys: the row is zero
        float zero[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) zero[c] = 0.f;
        if (holds) store_row_bf16<NC>(dst, zero, 0.f);
        return;
    }
    // The waves that held the row's first and last keys (recorded by the
    // split kernel); with a single slice the row was written directly.
    if (p.W == 1 && p.direct_single) return;
    const int w0 = rg.x, w1 = rg.y;
    if (w0 == w1 && p.direct_single) return;   // written directly by the split kernel
    float acc[NC], L, M;
    merge_partials<D>(p.o_part, p.ml_part, ((int64_t)r + w0) * hwg + hq % hwg, hwg, w1 - w0 + 1, lane, acc, L, M);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (holds) store_row_bf16<NC>(dst, acc, inv);
}

// Generic combine: every row r merges partials s = 0..S-1 at rows s*R + r.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(const CombineParams p) {
    constexpr int NC = combine_epl<D>();
    const int lane = threadIdx.x & 63;
    const bool holds = lane < D / NC;
    const int r = blockIdx.x * 4 + wave_id();
    if (r >= p.R) return;
    float acc[NC], L, M;
    merge_partials<D>(p.o_part, p.ml_part, r, p.R, p.S, lane, acc, L, M);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (p.out_f32 && holds) {
#pragma unroll
        for (int c = 0; c < NC; ++c) p.out_f32[(size_t)r * D + lane * NC + c] = acc[c] * inv;
    }
    if (p.out_bf16 && holds) store_row_bf16<NC>(p.out_bf16 + (size_t)r * D + lane * NC, acc, inv);
    if (p.lse && lane == 0) p.lse[r] = (L > 0.f) ? M + __logf(L) : -INFINITY;
}

template <int D, int G, int HW, bool PAGED>
hipError_t launch_decode_t(const DecodeParams &p, hipStream_t stream) {
    if (p.NW == 4) {
        if constexpr (G <= 4) {
            hipLaunchKernelGGL((decode_split_kernel<D, G, HW, PAGED, 4>), dim3(p.W), dim3(256), 0, stream, p);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((decode_split_kernel<D, G, HW, PAGED, 1>), dim3(p.W), dim3(64), 0, stream, p);
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
        case 8:
            if constexpr (64 / chunk_lanes<D>() >= 8) return launch_decode_g<D, 8, PAGED>(p, G, stream);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int D, int G, bool paged, hipStream_t stream) {
    if (p.W <= 0 || p.R <= 0) return hipSuccess;
    if (D == 32) return paged ? launch_decode_hw<32, true>(p, G, stream) : launch_decode_hw<32, false>(p, G, stream);
    if (D == 64) return paged ? launch_decode_hw<64, true>(p, G, stream) : launch_decode_hw<64, false>(p, G, stream);
    if (D == 128) return paged ? launch_decode_hw<128, true>(p, G, stream) : launch_decode_hw<128, false>(p, G, stream);
    if (D == 256) return paged ? launch_decode_hw<256, true>(p, G, stream) : launch_decode_hw<256, false>(p, G, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeCombineParams &p, int D, hipStream_t stream) {
    const int rows = p.B * p.Hq;
    if (rows <= 0) return hipSuccess;
    const int blocks = (rows + 3) / 4;
    if (D == 32) hipLaunchKernelGGL((decode_combine_kernel<32>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 64) hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 128) hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 256) hipLaunchKernelGGL((decode_combine_kernel<256>), dim3(blocks), dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_combine(const CombineParams &p, int D, hipStream_t stream) {
    if (p.R <= 0) return hipSuccess;
    const int blocks = (p.R + 3) / 4;
    if (D == 32) hipLaunchKernelGGL((combine_kernel<32>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 64) hipLaunchKernelGGL((combine_kernel<64>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 128) hipLaunchKernelGGL((combine_kernel<128>), dim3(blocks), dim3(256), 0, stream, p);
    else if (D == 256) hipLaunchKernelGGL((combine_kernel<256>), dim3(blocks), dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace pa
