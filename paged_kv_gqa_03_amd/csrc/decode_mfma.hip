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
// is copied from HBM straight into a wave-private LDS tile of natural key
// rows (global_load_lds) and read back transposed (ds_read_b64_tr_b16) as
// V^T operands holding keys 4g..4g+3 and 16+4g..16+4g+3: exactly the eight
// S^T values lane group g holds, so P^T feeds the second MFMA from
// registers.  In the
// transposed form lane l always holds query head l % 16 of a block, so the
// softmax statistics are per-lane scalars reduced over the four lane groups
// with two row swaps.  Scores are scaled after the dot product (csrc commit
// that moved the scale after Q.K^T); the reference is raised lazily (by more
// than 2^8, base 2), as in decode.hip.  Two stages: while one tile is
// computed the next one's K (registers) and V (the other LDS tile) are in
// flight.
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

// K of one tile held by a lane (A-operand layout, see above).
template <int D>
struct MTile {
    static constexpr int NS = D / 32;                 // 32-dim steps
    uint4 k[2][NS];
};

__device__ __forceinline__ uint4 ld16_nt(const uint16_t *ptr) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
    return make_uint4(t.x, t.y, t.z, t.w);
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// 16 bytes a lane from global memory straight into LDS (global_load_lds,
// non-temporal): lane l's bytes land at dst + 16 l (dst is wave-uniform).
__device__ __forceinline__ void copy16_to_lds(const uint16_t *src, uint16_t *dst) {
    __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 16, 0, 2);
}

// A V tile in LDS holds the tile's 32 keys in natural order, one D-dim row
// per key, its 16-byte chunks permuted by an XOR with an even value that
// depends on the key (so the 16 rows a transposed operand read takes fall
// on different banks; the same chunk pair stays adjacent).  Physical chunk
// of chunk c of row `key`:
template <int D>
__device__ __forceinline__ int vchunk(int key, int c) {
    constexpr int NCH = D / 8, RPB = 256 / (2 * D);   // chunks per row, rows per 256-byte bank line
    return c ^ (2 * ((key / RPB) % (NCH / 2)));
}

// s_waitcnt operand that waits for at most n vector memory operations
// (expcnt and lgkmcnt left at their maximum).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait until at most N vector memory operations are in flight.  The s_nop
// after it matters: with global_load_lds copies in flight the compiler asks
// for vmcnt(0) before any use of a register loaded earlier, and it folds
// that demand into a wait that directly precedes the use.  Behind the s_nop
// this wait is counted first, the older loads are retired by it, and the
// compiler adds nothing.
template <int N>
__device__ __forceinline__ void wait_tiles() {
    __builtin_amdgcn_s_waitcnt(vm_wait(N));
    asm volatile("s_nop 0");
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
    constexpr int KPI = 64 / VCH; // keys per V load instruction (1 KB)
    constexpr int NVL = BKM / KPI;           // V load instructions per tile
    constexpr int NLD = 2 * NS + NVL;        // vector memory instructions per tile
    constexpr int F = 2 + 4 * NM;                              // merge floats per lane and block
    constexpr int VB_ELEMS = BKM * D;                          // one V tile
    constexpr int XCH_FLOATS = NWT > 1 ? NWM * NB * F * 64 : 0;
    constexpr int T0_ELEMS = (NWM * VB_ELEMS > 2 * XCH_FLOATS) ? NWM * VB_ELEMS : 2 * XCH_FLOATS;
    // The waves' first and second V tiles sit in two separate arrays (the
    // first also holds the merge area): the compiler then knows that reads
    // of one tile do not depend on copies still landing in the other and
    // waits only for the tile it reads.
    __shared__ __attribute__((aligned(16))) uint16_t vt0[T0_ELEMS];
    __shared__ __attribute__((aligned(16))) uint16_t vt1[NWM * VB_ELEMS];
    __shared__ int32_t pages[kDecodeMaxSplitPages];

    const int lane = threadIdx.x & 63;
    const int wv = wave_id();
    const int w = blockIdx.x;
    const int g16 = lane & 15, lg = lane >> 4;   // MFMA row / column within a block, lane group
    const int hw = wv % HG, wt = wv / HG;        // this wave's head in the row, tile phase
    const int Gm = p.G_all / p.passes;           // query heads per KV head and row
    const int HPR = HG * Gm;                     // query heads per row
    float *xch = reinterpret_cast<float *>(vt0);

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
            // issue: K into registers (A-operand layout), V straight into the
            // LDS tile `vb` (global_load_lds, 16 bytes a lane, 1 KB of LDS a
            // instruction: KPI keys of natural rows, chunks swizzled).
            auto issue = [&](int k, MTile<D> &t, uint16_t *vb) {
                __builtin_amdgcn_sched_barrier(0);
                const int base = jb + (wt + NWT * k) * BKM;
                // Every page lookup of the tile first, then its loads.
                uint64_t ko[2], vo[NVL];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) ko[kb] = koff(base + 16 * kb + g16);
                const int kl = lane / VCH, pc = lane % VCH;   // key in the instruction, physical chunk
#pragma unroll
                for (int n = 0; n < NVL; ++n) {
                    const int tk = KPI * n + kl;              // key of the tile
                    const int c = vchunk<D>(tk, pc);          // the chunk this lane carries
                    if constexpr (MODE == kPagedQuads) {
                        // the key's group of four starts on a multiple of 4
                        // and the page size is one: they share a page
                        const int jq = base + (tk & ~3);
                        vo[n] = voff(jq) + (uint32_t)min(tk & 3, max(last - jq, 0)) * s_slot + 8 * c;
                    } else {
                        vo[n] = voff(base + tk) + 8 * c;
                    }
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const uint16_t *kr = kbase + ko[kb] + 8 * lg;
#pragma unroll
                    for (int s = 0; s < NS; ++s) t.k[kb][s] = ld16_nt(kr + 32 * s);
                }
#pragma unroll
                for (int n = 0; n < NVL; ++n)
                    copy16_to_lds(vbase + vo[n], vb + KPI * n * D);
            };
            auto compute = [&](int k, const MTile<D> &t, const uint16_t *vb) {
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
                // V^T operands of O^T += V^T . P^T, read now so that their
                // latency hides under the softmax.  Lane: dim 16 m + g16,
                // keys 4 lg .. +3 and 16 + 4 lg .. +3 (the order of the lane
                // group's eight S^T values), from two transposed reads:
                // within a 16-lane group, lane i receives element i % 4 of the
                // 8-byte segments that lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12
                // address, so lane j addresses dims 16 m + 4 (j % 4) .. +3 of
                // key 4 lg + j / 4 (then 16 + 4 lg + j / 4).
                bf16x8_t va[NM];
                const int ka = 4 * lg + (g16 >> 2), kbk = 16 + 4 * lg + (g16 >> 2);
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const int c = 2 * m + ((g16 & 3) >> 1), e = 4 * (g16 & 1);
                    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_t *)(vb + ka * D + 8 * vchunk<D>(ka, c) + e));
                    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4i16_t *)(vb + kbk * D + 8 * vchunk<D>(kbk, c) + e));
                    va[m] = __builtin_bit_cast(
                        bf16x8_t, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                             __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
                }
                __builtin_amdgcn_sched_barrier(0);
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
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        oacc[nb][m] = mfma16(va[m], as_bf16x8(make_uint4(pw[nb][0], pw[nb][1], pw[nb][2], pw[nb][3])),
                                             oacc[nb][m]);
            };

            // Two tiles in flight at every wait: tile k + 1 is issued before
            // tile k is computed, tile k + 2 right after.  The V tiles arrive
            // in LDS outside the compiler's view, so the wait for tile k
            // (vmcnt: only tile k + 1's NLD instructions still in flight) is
            // explicit.  Every issue in the loop is unconditional: a load
            // issued under a condition would make the compiler wait for all
            // of them.  Past the end every key is clamped to the piece's last
            // one, so such a tile reads one key row (never used); nothing is
            // left in flight when the loop ends (the LDS is reused next).
            if (ntw > 0) {
                MTile<D> ra, rb;
                uint16_t *va_t = vt0 + wv * VB_ELEMS, *vb_t = vt1 + wv * VB_ELEMS;
                issue(0, ra, va_t);
                int k = 0;
                for (; k + 1 < ntw; k += 2) {
                    issue(k + 1, rb, vb_t);
                    wait_tiles<NLD>();
                    compute(k, ra, va_t);
                    issue(k + 2, ra, va_t);
                    wait_tiles<NLD>();
                    compute(k + 1, rb, vb_t);
                }
                __builtin_amdgcn_s_waitcnt(vm_wait(0));
                if (k < ntw) compute(k, ra, va_t);
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
        // Merge inputs of this wave (the waves of its head: references, sums
        // and its 16-dim blocks m = wt, wt + NWT, ...), read from LDS all
        // together before any of the math, so the reads do not wait one by
        // one.
        constexpr int MPW = NWT > 1 ? NM / NWT : 1;   // 16-dim blocks a wave merges
        float xm[NB][NWT], xl[NB][NWT], xo[NB][MPW][4][NWT];
        if constexpr (NWT > 1) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int t = 0; t < NWT; ++t) {
                    const float *src = xch + (((hw + HG * t) * NB + nb) * F) * 64 + lane;
                    xm[nb][t] = src[0];
                    xl[nb][t] = src[64];
#pragma unroll
                    for (int mm = 0; mm < MPW; ++mm)
#pragma unroll
                        for (int i = 0; i < 4; ++i) xo[nb][mm][i][t] = src[(2 + 4 * (wt + NWT * mm) + i) * 64];
                }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int hl = 16 * nb + g16;   // this lane's query head of the wave's KV head
            float M, L;
            float fv[NWT];
            if constexpr (NWT > 1) {
                M = -INFINITY;
#pragma unroll
                for (int t = 0; t < NWT; ++t) M = fmaxf(M, xm[nb][t]);
                L = 0.f;
#pragma unroll
                for (int t = 0; t < NWT; ++t) {
                    fv[t] = xm[nb][t] == -INFINITY ? 0.f : exp2_fast(xm[nb][t] - M);
                    L += fv[t] * xl[nb][t];
                }
            } else {
                M = mref[nb];
                L = lsum[nb];
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;
            const int64_t prow = slot * HPR + hw * Gm + hl;   // partial row of this head
#pragma unroll
            for (int mm = 0; mm < (NWT > 1 ? MPW : NM); ++mm) {
                const int m = NWT > 1 ? wt + NWT * mm : mm;
                float ov[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (NWT > 1) {
                        float acc = 0.f;
#pragma unroll
                        for (int t = 0; t < NWT; ++t) acc += fv[t] * xo[nb][mm][i][t];
                        ov[i] = acc;
                    } else {
                        ov[i] = oacc[nb][mm][i];
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
