// decode_mfma.hip -- split-KV GQA decode with the query heads of a KV head on
// bf16 MFMA rows (group sizes other than 1, 2 and 4; head dims 64 and 128).
//
// Same method and partition as decode.hip (AstrAI csrc commit history: the
// split-KV decode with (o, m, l) partials and its log-sum-exp combine; the
// per-element page lookup): rows r = (sequence, group of HG adjacent KV
// heads, pass) are laid end to end and W slices of the line are one
// four-wave workgroup each.  Wave wv takes KV head wv % HG of the row; with
// HG = 4 each wave streams its head's keys of the piece alone, with HG = 2
// or 1 the waves of a head take alternate 32-key tiles and merge their
// states through LDS at the piece's end.  The waves of a workgroup read the
// same tokens of HG heads together, which HBM serves measurably faster than
// one head's keys alone.  A piece is written directly (normalised) when it
// is its row's only one, else as an fp32 partial at slot r + w.
//
// With Gm query heads sharing a KV head (Gm up to 32: NB = 1 or 2 blocks of
// 16 MFMA rows) a row holds Gm heads, so each key is read once for all of
// them (the VALU kernel would hold 8 x D/8 accumulators per lane per head).
// Per 32-key tile a wave computes, with v_mfma_f32_16x16x32_bf16,
//   S^T (32 keys x 16 heads) = K (32 x D) . Q^T (D x 16)        2 D/32 MFMA
//   O^T (D x 16 heads)     += V^T (D x 32) . P^T (32 x 16)      D/16 MFMA
// per row block.  K comes straight from HBM in the A-operand layout (lane l:
// key l % 16 of a 16-key block, 8 dims at 8 (l / 16) of a 32-dim step).  V
// is loaded as 4 keys x 8 dims per lane and transposed in registers into a
// wave-private LDS tile V^T, whose key order puts keys 4g..4g+3 and
// 16+4g..16+4g+3 at slots 8g..8g+7: exactly the eight S^T values lane
// group g holds, so P^T feeds the second MFMA from registers.  In the
// transposed form lane l always holds query head l % 16 of a block, so the
// softmax statistics are per-lane scalars reduced over the four lane groups
// with two row swaps.  Scores are scaled after the dot product (csrc commit
// that moved the scale after Q.K^T); the reference is raised lazily (by more
// than 2^8, base 2), as in decode.hip.  Two register stages: while one tile
// is staged and computed the next one's K and V are in flight.
#include "decode_common.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int BKM = 32;              // keys per tile
constexpr int NWM = 4;               // waves per workgroup (slice)
constexpr float kRaise = 8.0f;       // lazy reference raise threshold, log2 units
constexpr int VTLD = BKM + 8;        // V^T row stride in LDS (elements): 80 bytes

// Maximum over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48), in every lane, with two VALU row swaps.
__device__ __forceinline__ float max_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// First V^T slot of staging group kg (keys 4kg .. 4kg+3 of the tile).
__device__ __forceinline__ int vslot(int kg) { return kg < 4 ? 8 * kg : 8 * (kg - 4) + 4; }

// Loads of one tile held by a lane.
template <int D>
struct MTile {
    static constexpr int NS = D / 32;                 // 32-dim steps
    static constexpr int VG = (BKM / 4) * (D / 8) / 64;   // V groups (4 keys x 8 dims) per lane
    uint4 k[2][NS];
    uint4 v[VG][4];
};

__device__ __forceinline__ uint4 ld16_nt(const uint16_t *ptr) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// 4 keys x 8 dims (one uint4 per key) -> V^T rows 8c .. 8c+7, slots base .. base+3.
__device__ __forceinline__ void stage_group(uint16_t *vt, int c, int base, const uint4 (&v)[4]) {
    const uint32_t k0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
    const uint32_t k1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
    const uint32_t k2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
    const uint32_t k3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // v_perm selectors: bytes 0-3 from the second operand, 4-7 from the
        // first; 0x05040100 = (b.lo16, a.lo16), 0x07060302 = (b.hi16, a.hi16).
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(k1[e], k0[e], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(k3[e], k2[e], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(k1[e], k0[e], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(k3[e], k2[e], 0x07060302u);
        *reinterpret_cast<uint2 *>(&vt[(8 * c + 2 * e) * VTLD + base]) = lo;
        *reinterpret_cast<uint2 *>(&vt[(8 * c + 2 * e + 1) * VTLD + base]) = hi;
    }
}

// KV modes: contiguous K/V; paged, V read key by key; paged with a page size
// that is a multiple of 4, V read as groups of 4 keys that share a page.  The
// mode is fixed per launch so the tile loop has no branch on it.
enum { kContig = 0, kPagedKeys = 1, kPagedQuads = 2 };

// HG KV heads per row and workgroup: wave wv takes head wv % HG of the row
// and tiles wv / HG, + NWT, ... of each piece (NWT = 4 / HG waves per head,
// merged through LDS when more than one).
template <int D, int NB, int MODE, int HG>
__global__ __launch_bounds__(256, NB == 1 ? 2 : 1) void decode_mfma_kernel(const DecodeParams p) {
    constexpr bool PAGED = MODE != kContig;
    constexpr int NWT = NWM / HG;
    constexpr int NS = D / 32;    // depth steps of S^T
    constexpr int NM = D / 16;    // 16-dim blocks of O^T
    constexpr int VCH = D / 8;    // 16-byte chunks of a key row
    constexpr int VG = MTile<D>::VG;
    static_assert(VG >= 1 && (BKM / 4) * VCH == 64 * VG, "V staging covers the tile");
    constexpr int F = 2 + 4 * NM;                              // merge floats per lane and block
    constexpr int VT_ELEMS = D * VTLD;                         // one wave's V^T tile
    constexpr int XCH_FLOATS = NWT > 1 ? NWM * NB * F * 64 : 0;
    constexpr int LDS_BYTES = (NWM * VT_ELEMS * 2 > XCH_FLOATS * 4) ? NWM * VT_ELEMS * 2 : XCH_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) unsigned char lds[LDS_BYTES];
    __shared__ int32_t pages[kDecodeMaxSplitPages];

    const int lane = threadIdx.x & 63;
    const int wv = wave_id();
    const int w = blockIdx.x;
    const int g16 = lane & 15, lg = lane >> 4;   // MFMA row / column within a block, lane group
    const int hw = wv % HG, wt = wv / HG;        // this wave's head in the row, tile phase
    const int Gm = p.G_all / p.passes;           // query heads per KV head and row
    const int HPR = HG * Gm;                     // query heads per row
    uint16_t *vt = reinterpret_cast<uint16_t *>(lds) + wv * VT_ELEMS;
    float *xch = reinterpret_cast<float *>(lds);

    const RowScan rs = scan_rows(p);
    const int T = rs.total;
    const int a = uniform((int)((int64_t)w * T / p.W)), e = uniform((int)((int64_t)(w + 1) * T / p.W));
    if (a >= T) return;
    int r, P;
    first_row(p, rs, a, r, P);
    if (a >= e) {
        // An empty slice strictly inside row r holds a slot of the row's run:
        // marked empty (m = -inf, l = 0) so the combine ignores it.
        if (P < a)
            for (int i = threadIdx.x; i < HPR; i += 64 * NWM)
                *reinterpret_cast<float2 *>(p.ml_part + ((int64_t)(r + w) * HPR + i) * 2) = make_float2(-INFINITY, 0.f);
        return;
    }
    const float sl2 = p.sl2;

    for (; P < e && r < p.R; ++r) {
        const int n = uniform(row_len(p, r));
        const int lo = max(a, P) - P, hi = min(e, P + n) - P;
        P += n;
        if (lo >= hi) continue;
        if (p.ranges && threadIdx.x == 0) {
            if (lo == 0) p.ranges[2 * (int64_t)r] = w;
            if (hi == n) p.ranges[2 * (int64_t)r + 1] = w;
        }
        const int b = r / p.ngrp, hgrp = r % p.ngrp;
        const int g = (hgrp / p.passes) * HG + hw;               // this wave's KV head
        const int h0 = g * p.G_all + (hgrp % p.passes) * Gm;     // its first query head in the row

        // Q^T operands: head h0 + 16 nb + lane % 16 (zero past Gm), dims 32 s + 8 lg.
        bf16x8_t qf[NB][NS];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int hl = 16 * nb + g16;
            const uint16_t *qr = p.q + b * p.q_sb + (int64_t)(h0 + min(hl, Gm - 1)) * p.q_sh + 8 * lg;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                uint4 v = *reinterpret_cast<const uint4 *>(qr + 32 * s);
                if (hl >= Gm) v = make_uint4(0u, 0u, 0u, 0u);
                qf[nb][s] = as_bf16x8(v);
            }
        }
        f32x4_t oacc[NB][NM];
        float mref[NB], lsum[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            mref[nb] = -INFINITY;
            lsum[nb] = 0.f;
#pragma unroll
            for (int m = 0; m < NM; ++m) oacc[nb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        const uint16_t *kbase = p.k + (PAGED ? g * p.s_head : b * p.k_sb + g * p.k_sh);
        const uint16_t *vbase = p.v + (PAGED ? g * p.s_head : b * p.v_sb + g * p.v_sh);
        const uint32_t s_page = (uint32_t)p.s_page, s_slot = (uint32_t)p.s_slot;
        const uint32_t k_sl = (uint32_t)p.k_sl, v_sl = (uint32_t)p.v_sl;

        for (int j0 = lo; j0 < hi; j0 += p.max_sub) {
            const int j1 = min(hi, j0 + p.max_sub);
            const int last = j1 - 1;
            // Tiles start at jb: j0 rounded down to a multiple of 4 for V
            // groups of 4 keys (the up to 3 keys below j0 are in j0's page,
            // loaded and masked), else j0.
            const int jb = MODE == kPagedQuads ? (j0 & ~3) : j0;
            const int ntiles = (j1 - jb + BKM - 1) / BKM;
            int first_pg = 0;
            // Every wave is done with the previous sub-piece's page slice and
            // the previous row's merge area before this one's V^T staging
            // (the V^T tiles and the merge area share LDS).
            __syncthreads();
            if constexpr (PAGED) {
                const int32_t *bt_row = p.bt + b * p.bt_sb;
                first_pg = (int)divu32((uint32_t)j0, p.ps_div);
                const int npg = (int)divu32((uint32_t)last, p.ps_div) - first_pg + 1;
                for (int i = threadIdx.x; i < npg; i += 64 * NWM) pages[i] = bt_row[first_pg + i];
                __syncthreads();
            }
            // Element offsets of key j (clamped to the sub-piece) in K and V.
            auto koff = [&](int j) -> uint64_t {
                j = min(j, last);
                if constexpr (PAGED) {
                    const uint32_t pi = divu32((uint32_t)j, p.ps_div);
                    const uint32_t page = (uint32_t)pages[pi - first_pg];
                    return (uint64_t)page * s_page + ((uint32_t)j - pi * p.ps) * s_slot;
                } else {
                    return (uint64_t)(uint32_t)j * k_sl;
                }
            };
            auto voff = [&](int j) -> uint64_t {
                if constexpr (PAGED) return koff(j);
                else return (uint64_t)(uint32_t)min(j, last) * v_sl;
            };
            // This wave's tiles: wv, wv + NWM, ...; k counts them.
            const int ntw = ntiles > wt ? (ntiles - wt + NWT - 1) / NWT : 0;
            // The phases below are kept in program order (sched_barrier):
            // hoisting a tile's loads above the previous compute would hold
            // three tiles in registers.
            auto issue = [&](int k, MTile<D> &t) {
                __builtin_amdgcn_sched_barrier(0);
                const int base = jb + (wt + NWT * k) * BKM;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint16_t *kr = kbase + koff(base + 16 * kb + g16) + 8 * lg;
#pragma unroll
                    for (int s = 0; s < NS; ++s) t.k[kb][s] = ld16_nt(kr + 32 * s);
                }
#pragma unroll
                for (int gi = 0; gi < VG; ++gi) {
                    const int q = lane + 64 * gi, kg = q / VCH, c = q % VCH;
                    if constexpr (MODE == kPagedQuads) {
                        // the group's four keys start on a multiple of 4 and
                        // the page size is one: they share a page
                        const int j = base + 4 * kg;
                        const int jr = last - j;   // keys past the end repeat the last one
                        const uint64_t o0 = voff(j);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            t.v[gi][i] = ld16_nt(vbase + o0 + (uint32_t)min(i, max(jr, 0)) * s_slot + 8 * c);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) t.v[gi][i] = ld16_nt(vbase + voff(base + 4 * kg + i) + 8 * c);
                    }
                }
            };
            auto stage = [&](const MTile<D> &t) {
                __builtin_amdgcn_sched_barrier(0);
                // the previous tile's V^T reads come before these writes
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int gi = 0; gi < VG; ++gi) {
                    const int q = lane + 64 * gi, kg = q / VCH, c = q % VCH;
                    stage_group(vt, c, vslot(kg), t.v[gi]);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            };
            auto compute = [&](int k, const MTile<D> &t) {
                __builtin_amdgcn_sched_barrier(0);
                const int tbase = jb + (wt + NWT * k) * BKM;
                // S^T blocks: keys 16 kb + 4 lg + i, head 16 nb + g16.
                f32x4_t st[NB][2];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) st[nb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < NS; ++s)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) st[nb][kb] = mfma16(as_bf16x8(t.k[kb][s]), qf[nb][s], st[nb][kb]);
                // key 16 kb + i of the lane is admitted iff skip <= it < room
                const int room = j1 - (tbase + 4 * lg), skip = j0 - (tbase + 4 * lg);
                uint32_t pw[NB][4];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float x[2][4];
                    float mt = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bool in = 16 * kb + i < room && (MODE != kPagedQuads || 16 * kb + i >= skip);
                            x[kb][i] = in ? st[nb][kb][i] * sl2 : -INFINITY;
                            mt = fmaxf(mt, x[kb][i]);
                        }
                    mt = max_over_rows(mt);
                    if (mt > mref[nb] + kRaise) {
                        const float alpha = exp2_fast(mref[nb] - mt);   // 0 from -inf
                        lsum[nb] *= alpha;
#pragma unroll
                        for (int m = 0; m < NM; ++m) oacc[nb][m] *= alpha;
                        mref[nb] = mt;
                    }
                    const float mu = fmaxf(mref[nb], -3.0e38f);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; i += 2) {
                            const uint32_t pk = pack_bf16(exp2_fast(x[kb][i] - mu), exp2_fast(x[kb][i + 1] - mu));
                            pw[nb][2 * kb + i / 2] = pk;
                            lsum[nb] += bf16_lo(pk) + bf16_hi(pk);
                        }
                }
                // O^T += V^T . P^T
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const bf16x8_t va =
                        as_bf16x8(*reinterpret_cast<const uint4 *>(&vt[(16 * m + g16) * VTLD + 8 * lg]));
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        oacc[nb][m] = mfma16(va, as_bf16x8(make_uint4(pw[nb][0], pw[nb][1], pw[nb][2], pw[nb][3])),
                                             oacc[nb][m]);
                }
            };

            // Two tiles in flight at every wait: tile k + 1 is issued before
            // tile k is staged, tile k + 2 as soon as tile k is computed.
            // Every issue in the loop is unconditional: a load issued under
            // a condition would make the compiler wait for all of them.
            // Past the end every key is clamped to the piece's last one, so
            // such a tile reads one key row (never used).
            if (ntw > 0) {
                MTile<D> ra, rb;
                issue(0, ra);
                int k = 0;
                for (; k + 1 < ntw; k += 2) {
                    issue(k + 1, rb);
                    stage(ra);
                    compute(k, ra);
                    issue(k + 2, ra);
                    stage(rb);
                    compute(k + 1, rb);
                }
                if (k < ntw) {
                    stage(ra);
                    compute(k, ra);
                }
            }
        }

        // Sums over the four lane groups (each holds 8 of every 32 keys).
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) lsum[nb] = sum_over_rows(lsum[nb]);

        // With several waves on a head, merge their states: each leaves
        // (reference, sum, O^T) in LDS, then wave wv merges the 16-dim blocks
        // m with m % NWT == wt over the waves hw, hw + HG, ...
        if constexpr (NWT > 1) {
            __syncthreads();   // every wave is done with its V^T tile
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float *mine = xch + ((wv * NB + nb) * F) * 64 + lane;
                mine[0] = mref[nb];
                mine[64] = lsum[nb];
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mine[(2 + 4 * m + i) * 64] = oacc[nb][m][i];
            }
            __syncthreads();
        }
        const bool direct = p.direct && lo == 0 && hi == n;
        const int64_t slot = (int64_t)r + w;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int hl = 16 * nb + g16;   // this lane's query head of the wave's KV head
            float M, L;
            float fv[NWT];
            if constexpr (NWT > 1) {
                M = -INFINITY;
#pragma unroll
                for (int t = 0; t < NWT; ++t) M = fmaxf(M, xch[(((hw + HG * t) * NB + nb) * F) * 64 + lane]);
                L = 0.f;
#pragma unroll
                for (int t = 0; t < NWT; ++t) {
                    const int v = hw + HG * t;
                    const float mv = xch[((v * NB + nb) * F) * 64 + lane];
                    fv[t] = mv == -INFINITY ? 0.f : exp2_fast(mv - M);
                    L += fv[t] * xch[((v * NB + nb) * F + 1) * 64 + lane];
                }
            } else {
                M = mref[nb];
                L = lsum[nb];
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;
            const int64_t prow = slot * HPR + hw * Gm + hl;   // partial row of this head
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m % NWT != wt) continue;
                float ov[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (NWT > 1) {
                        float acc = 0.f;
#pragma unroll
                        for (int t = 0; t < NWT; ++t)
                            acc += fv[t] * xch[(((hw + HG * t) * NB + nb) * F + 2 + 4 * m + i) * 64 + lane];
                        ov[i] = acc;
                    } else {
                        ov[i] = oacc[nb][m][i];
                    }
                }
                if (hl >= Gm) continue;
                const int d0 = 16 * m + 4 * lg;
                if (direct) {
                    uint2 v;
                    v.x = pack_bf16(ov[0] * inv, ov[1] * inv);
                    v.y = pack_bf16(ov[2] * inv, ov[3] * inv);
                    *reinterpret_cast<uint2 *>(p.o + b * p.o_sb + (int64_t)(h0 + hl) * p.o_sh + d0) = v;
                } else {
                    *reinterpret_cast<float4 *>(p.o_part + prow * D + d0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
                }
            }
            if (!direct && hl < Gm && wt == 0 && lg == 0)
                *reinterpret_cast<float2 *>(p.ml_part + prow * 2) = make_float2(partial_m(M, L), L);
        }
    }
}

template <int D, int MODE, int HG>
hipError_t launch_mfma_hg(const DecodeParams &p, hipStream_t stream) {
    if (p.NB == 1) hipLaunchKernelGGL((decode_mfma_kernel<D, 1, MODE, HG>), dim3(p.W), dim3(64 * NWM), 0, stream, p);
    else if (p.NB == 2) hipLaunchKernelGGL((decode_mfma_kernel<D, 2, MODE, HG>), dim3(p.W), dim3(64 * NWM), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_mfma_d(const DecodeParams &p, hipStream_t stream) {
    if (p.HW == 1) return launch_mfma_hg<D, MODE, 1>(p, stream);
    if (p.HW == 2) return launch_mfma_hg<D, MODE, 2>(p, stream);
    if (p.HW == 4) return launch_mfma_hg<D, MODE, 4>(p, stream);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_mfma_mode(const DecodeParams &p, bool paged, hipStream_t stream) {
    if (!paged) return launch_mfma_d<D, kContig>(p, stream);
    if ((p.ps & 3u) == 0) return launch_mfma_d<D, kPagedQuads>(p, stream);
    return launch_mfma_d<D, kPagedKeys>(p, stream);
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams &p, int D, bool paged, hipStream_t stream) {
    if (p.W <= 0 || p.R <= 0) return hipSuccess;
    if (D == 64) return launch_mfma_mode<64>(p, paged, stream);
    if (D == 128) return launch_mfma_mode<128>(p, paged, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
