// prefill.hip -- ragged paged GQA prefill on bf16 MFMA for gfx950.
//
// Method (AstrAI "CUDA Kernels" doc, sections "Q Scheduling and KV
// Addressing" and the Overview entry for attn_paged_prefill; csrc commits on
// the unified causal_offset, coexisting causal + mask, and 2-D / 3-D masks):
// packed queries of a ragged batch are cut into fixed-height tiles listed by
// a work map (tile -> sequence, tile index inside it), each tile attends its
// sequence's keys through the block table, with causality j <= c_b + i and
// an optional keep-mask, using an online softmax over KV tiles.
//
// Work decomposition: one workgroup per (work-map tile, KV head, head
// group), which packs HP query heads that share the KV head (the largest
// power of two dividing G, at most 8; all G heads for G in {1, 2, 4, 8}),
// so every K/V tile is read once for the whole group (csrc commit on GQA
// head packing: up to one head per warp of a block, K/V streamed once per
// block).  A wave holds two 16-row MFMA blocks: for HP <= 4, 32 rows of one
// head (a tile then has 128 / HP rows); for HP = 8, the same 16 rows of two
// heads (16-row tiles).  A workgroup is one team of four waves, or two teams
// that take alternate KV tiles of the same rows and merge at the end (the
// host picks two only for grids of at most one workgroup per two CUs).  At
// D = 256 a wave holds one 16-row block and a workgroup one team.
// Split KV (for short query runs over long contexts, where tiles x KV heads
// would not fill the device): kv_splits workgroups share a tile's keys in
// equal runs of 64-key tiles, each writes an unnormalised fp32 partial
// (o, m, l) per row and head, and a combine merges them by log-sum-exp.
//
// Per KV tile of 64 keys the workgroup stages K and V in LDS.  At D = 128
// both are copied from HBM straight into LDS as natural key rows
// (global_load_lds) and V^T operands are read back transposed
// (ds_read_b64_tr_b16); otherwise K is stored row-major and V transposed
// (d-major, keys permuted) from registers.  Each wave then runs, with
// v_mfma_f32_16x16x32_bf16, per row block
//   S^T (64 keys x 16 rows) = K (64 x 128) . Q^T (128 x 16)     16 MFMA
//   O^T (128 x 16)        += V^T (128 x 64) . P^T (64 x 16)     16 MFMA
// and every K or V^T operand read from LDS feeds both row blocks.  In this
// transposed form lane l always holds query row l % 16 of a block: its
// scores are 16 keys of that row (keys 4*(l/16) + i of each 16-key block), so
// the row max / sum need only two cross-lane steps, the softmax rescale of O
// is a per-lane scalar, and P^T feeds the second MFMA straight from
// registers (V^T is stored with the matching key order).  Scores are scaled
// in fp32 after the dot product (csrc commit that moved the scale after
// Q.K^T).  Keys past the causal frontier of the tile are never loaded.
//
// Pipeline (per team): two LDS buffers.  Register staging: while a tile is
// computed from one buffer, the team's next tile (loaded a whole iteration
// earlier) is stored into the other, and the one after is loaded.  LDS
// copies: while a tile is computed from one buffer, the next one lands in
// the other.  One barrier per tile.  Page ids come from a slice of the
// block table staged in LDS, so no global load sits between a tile's
// address math and its K/V loads, and the keep-mask words of a tile travel
// with its stage.  Inside a tile the LDS operand reads run ahead of the
// MFMAs: K two depth steps ahead, V^T two stages of two 16-dim blocks ahead,
// its first two stages read before the exponentials, so no MFMA waits on a
// read issued just before it.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;           // keys per KV tile
// Row strides in LDS (elements): K rows D + 16 (288 B at D = 128), V^T
// rows BK + 16 (160 B).  Measured on gfx950 with SQ_LDS_BANK_CONFLICT: at
// D + 8 / BK + 8 the 16-byte operand reads of both tiles conflicted (45% of
// the LDS-active cycles were conflict cycles); with 16 elements of padding
// the reads are conflict-free and only the V^T staging stores conflict
// (14%), 3-5% less time per prefill call.
template <int D>
constexpr int kld() { return D + 16; }
constexpr int VLD = BK + 16;     // V^T row stride in LDS (elements): 160 B
constexpr int kPages = 512;      // block-table entries staged in LDS at a time

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Maximum over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48), in every lane: two row swaps in the vector ALU (v_permlane16_swap,
// v_permlane32_swap) rather than LDS permutes, which would queue behind the
// MFMA operand reads.  Either output order gives the same maximum.
__device__ __forceinline__ float max_over_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Position of key k (0..63) inside the transposed V tile: within each group
// of 32 keys, key 16h + 4q + i sits at 8q + 4h + i, so the eight keys that
// lane group q contributes to one P^T operand are contiguous.
__device__ __forceinline__ int v_phys(int k) {
    const int k32 = k & 31;
    return (k & ~31) + 8 * ((k32 & 15) >> 2) + 4 * (k32 >> 4) + (k32 & 3);
}

// LDS-copy staging (D = 128): a K or V tile is 64 natural key rows of
// 256 B copied from HBM straight into LDS (global_load_lds, 16 bytes a lane,
// four key rows an instruction), with the 16-byte chunks of each row
// XOR-swizzled: K chunk c of key k sits at
// c ^ (k & 15), so the 16 rows an S^T operand read takes (one chunk each)
// fall on 16 different 16-byte bank groups; V chunk c at c ^ 2 (k & 7), so
// the four keys x four 8-byte pieces of a transposed read spread likewise.
// V^T operands come back with ds_read_b64_tr_b16: within a 16-lane group,
// lane i receives element i % 4 of the 8-byte pieces that lanes i/4,
// i/4 + 4, i/4 + 8, i/4 + 12 address.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ int kchunk_swz(int key, int c) { return c ^ (key & 15); }
__device__ __forceinline__ int vchunk_swz(int key, int c) { return c ^ (2 * (key & 7)); }

// 16 bytes a lane from global memory into LDS at dst + 8 * lane (dst is
// wave-uniform); non-temporal when nothing else reads the keys.
__device__ __forceinline__ void copy16_to_lds(const uint16_t *src, uint16_t *dst, bool nt) {
    if (nt) __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 16, 0, 2);
    else __builtin_amdgcn_global_load_lds(src, (lds_void_t *)dst, 16, 0, 0);
}

// V^T operand of the LDS-copy tile at buf + v0 (64 key rows of 128 dims):
// dims 16 m + g16 (g16 = lane % 16) of keys 32 s2 + 4 lq .. +3 and 32 s2 +
// 16 + 4 lq .. +3, the key order of the lane group's P^T values.  Each
// address is one index off the LDS array itself: the compiler attaches the
// array's alias scope only to accesses a few address steps from it, and a
// read without it waits for every LDS copy in flight.
__device__ __forceinline__ bf16x8_t vt_operand(const uint16_t *buf, int v0, int m, int s2, int lane) {
    const int g16 = lane & 15, lq = lane >> 4;
    const int ka = 32 * s2 + 4 * lq + (g16 >> 2), kb = ka + 16;
    const int c = 2 * m + ((g16 & 3) >> 1), e = 4 * (g16 & 1);
    const v4i16_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(buf + (v0 + ka * 128 + 8 * vchunk_swz(ka, c) + e)));
    const v4i16_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(buf + (v0 + kb * 128 + 8 * vchunk_swz(kb, c) + e)));
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    return as_bf16x8(make_uint4(l.x, l.y, h.x, h.y));
}

// s_waitcnt operand: every vector memory operation of the wave complete
// (expcnt and lgkmcnt left at their maximum).
constexpr int kWaitVmem0 = (7 << 4) | (15 << 8);

// Per-thread share of one KV tile in flight: four K chunks, four V chunks.
struct Stage {
    uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

struct StageCtx {
    int cc;                         // this thread's 16-byte chunk of a K/V row
    bool stream;                    // no other workgroup reads these keys: non-temporal loads
    int first_pg, c1;               // page slice start; keys of this chunk end at c1
    const int32_t *pages;           // LDS page slice
    const uint16_t *kbase, *vbase;
};

__device__ __forceinline__ uint64_t key_off(const PrefillParams &p, const StageCtx &sc, int key) {
    const int kc = min(key, sc.c1 - 1);   // keys past the chunk end repeat its last key
    const uint32_t pi = divu32((uint32_t)kc, p.ps_div);
    const int page = sc.pages[pi - sc.first_pg];
    const uint32_t slot = (uint32_t)kc - pi * p.ps;
    return (uint64_t)(uint32_t)page * (uint32_t)p.s_page + slot * (uint32_t)p.s_slot;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *ptr) { return *reinterpret_cast<const uint4 *>(ptr); }
__device__ __forceinline__ uint4 ld16_nt(const uint16_t *ptr) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ptr));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// A share of tile kt: keys 4kg .. 4kg+3, chunk cc, of K and of V (the
// sources share strides, so the four offsets serve both).  Paged: when the
// page size is a multiple of 4 the four keys sit in one page, one lookup
// then slot steps.  Keys past the chunk end repeat its last key.
template <bool PAGED>
__device__ __forceinline__ void load_stage(const PrefillParams &p, const StageCtx &sc, int kg, int kt, Stage &r) {
    const int k0 = min(kt * BK + 4 * kg, sc.c1 - 1);
    uint64_t off[4];
    if constexpr (!PAGED) {   // contiguous source: key j at j * s_slot from the sequence's base
        const int rmax = sc.c1 - 1 - k0;
#pragma unroll
        for (int i = 0; i < 4; ++i) off[i] = (uint64_t)(k0 + min(i, rmax)) * (uint64_t)p.s_slot;
    } else if ((p.ps & 3u) == 0) {
        const int rmax = sc.c1 - 1 - k0;
        off[0] = key_off(p, sc, k0);
#pragma unroll
        for (int i = 1; i < 4; ++i) off[i] = off[0] + (uint32_t)min(i, rmax) * (uint32_t)p.s_slot;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) off[i] = key_off(p, sc, k0 + i);
    }
    if (sc.stream) {
        r.k0 = ld16_nt(sc.kbase + off[0]);
        r.k1 = ld16_nt(sc.kbase + off[1]);
        r.k2 = ld16_nt(sc.kbase + off[2]);
        r.k3 = ld16_nt(sc.kbase + off[3]);
        r.v0 = ld16_nt(sc.vbase + off[0]);
        r.v1 = ld16_nt(sc.vbase + off[1]);
        r.v2 = ld16_nt(sc.vbase + off[2]);
        r.v3 = ld16_nt(sc.vbase + off[3]);
    } else {
        r.k0 = ld16(sc.kbase + off[0]);
        r.k1 = ld16(sc.kbase + off[1]);
        r.k2 = ld16(sc.kbase + off[2]);
        r.k3 = ld16(sc.kbase + off[3]);
        r.v0 = ld16(sc.vbase + off[0]);
        r.v1 = ld16(sc.vbase + off[1]);
        r.v2 = ld16(sc.vbase + off[2]);
        r.v3 = ld16(sc.vbase + off[3]);
    }
}

// Keep-mask of one tile, staged like K and V: thread t loads bytes
// 8(t & 7) .. +8 of mask rows (t >> 3) + 32 q (q < NQ) of the tile's 64 keys,
// and stores them as 8 bits, so LDS holds 64 bits per mask row.  A 3-D mask
// has one row per query row of the work-map tile, a 2-D mask one row.
// With one mask row per thread (NQ = 1) loading only issues loads, and the
// bytes are assembled when the stage is stored (a tile's compute later), so
// no wait for them sits between the tile's K/V loads and the next compute.
// With several rows per thread the three raw words per row would cost too
// many registers across the compute, so the bytes are assembled at once.
template <int MASK, int NQ>
struct MaskStage {
    static constexpr bool kDefer = NQ == 1;
    uint32_t w[NQ][kDefer ? 3 : 2];   // deferred: the aligned dwords holding the eight bytes;
                                      // else the eight bytes, zero past the row's end
    uint32_t meta[NQ];                // deferred: bits 0-3 bytes that exist, bits 4-5 the
                                      // offset of the first byte in w[q][0]
};

struct MaskCtx {
    const uint8_t *base;   // mask row of the tile's first query row (2-D: the sequence's row)
    int64_t m_sq;
    int rows;              // mask rows that exist (3-D: query rows of the tile)
};

// Bytes [j, j + 8) of mask row `row`; bytes at or past key n count as 0, and
// rows past `rows` as all 0.  Mask rows may start at any byte.  Every load
// reads an aligned dword that holds at least one byte of the row below key
// n, so no read can cross into another page.  Deferred (one row per
// thread), the loads are unconditional (a dword past byte n - 1 is replaced
// by the one holding it, a row past `rows` by the last row), which keeps the
// compiler from waiting on them.
template <int MASK, int NQ>
__device__ __forceinline__ void load_mask(const MaskCtx &mc, int tid, int n, int kt, MaskStage<MASK, NQ> &m) {
    const int j = kt * BK + 8 * (tid & 7);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = (tid >> 3) + 32 * q;
        if constexpr (MaskStage<MASK, NQ>::kDefer) {
            const uint8_t *rp = mc.base + (int64_t)min(row, mc.rows - 1) * mc.m_sq;
            // Offsets from rp (kept as offsets so the loads stay global
            // ones): the aligned dword holding byte j, and the one holding
            // byte n - 1.
            const uint32_t sh = (uint32_t)reinterpret_cast<uintptr_t>(rp + j) & 3u;
            const int o0 = j - (int)sh;
            const int ol = (n - 1) - (int)((uint32_t)reinterpret_cast<uintptr_t>(rp + (n - 1)) & 3u);
#pragma unroll
            for (int k = 0; k < 3; ++k) m.w[q][k] = *reinterpret_cast<const uint32_t *>(rp + min(o0 + 4 * k, ol));
            m.meta[q] = (uint32_t)(row < mc.rows ? max(0, min(8, n - j)) : 0) | (sh << 4);
        } else {
            // Several rows per thread: the two or three dwords (or, at the
            // row's end, the bytes below n) are read and joined at once.
            m.w[q][0] = m.w[q][1] = 0u;
            if (row < mc.rows) {
                const uint8_t *mp = mc.base + row * mc.m_sq + j;
                if (j + 8 <= n) {
                    const uint32_t sh = (uint32_t)reinterpret_cast<uintptr_t>(mp) & 3u;
                    const uint32_t *wp = reinterpret_cast<const uint32_t *>(mp - sh);
                    const uint32_t w0 = wp[0], w1 = wp[1];
                    const uint32_t w2 = sh ? wp[2] : 0u;
                    m.w[q][0] = __builtin_amdgcn_alignbyte(w1, w0, sh);
                    m.w[q][1] = __builtin_amdgcn_alignbyte(w2, w1, sh);
                } else {
                    for (int i = 0; i < 8 && j + i < n; ++i) m.w[q][i >> 2] |= (uint32_t)mp[i] << (8 * (i & 3));
                }
            }
        }
    }
}

// Four mask bytes -> four bits (bit i set iff byte i is nonzero).
__device__ __forceinline__ uint32_t nz_bits4(uint32_t w) {
    w |= w >> 4;
    w |= w >> 2;
    w |= w >> 1;
    return ((w & 0x01010101u) * 0x01020408u) >> 24;
}

template <int MASK, int NQ, int ROWS>
__device__ __forceinline__ void store_mask(const MaskStage<MASK, NQ> &m, int tid, uint8_t *bits) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int row = (tid >> 3) + 32 * q;
        if (row < ROWS) {
            if constexpr (MaskStage<MASK, NQ>::kDefer) {
                const uint32_t sh = m.meta[q] >> 4, keep = m.meta[q] & 15u;
                const uint32_t lo = __builtin_amdgcn_alignbyte(m.w[q][1], m.w[q][0], sh);
                const uint32_t hi = __builtin_amdgcn_alignbyte(m.w[q][2], m.w[q][1], sh);
                const uint32_t b = nz_bits4(lo) | (nz_bits4(hi) << 4);
                bits[row * 8 + (tid & 7)] = (uint8_t)(b & ((1u << keep) - 1u));
            } else {
                bits[row * 8 + (tid & 7)] = (uint8_t)(nz_bits4(m.w[q][0]) | (nz_bits4(m.w[q][1]) << 4));
            }
        }
    }
}

// Column of V^T row d where the 8-key group `grp` is stored: groups are
// XOR-swizzled by the row's 16-row block, which spreads the staging stores
// (16 lanes writing rows 8 apart) over the banks, while an operand read
// (one 16-row block, whole 8-key groups) stays a contiguous 16 bytes.
__device__ __forceinline__ int v_col(int d, int grp) { return 8 * (grp ^ ((d >> 4) & 7)); }

// One 32-bit column pair of the 4 x 8 V block: dims (2j, 2j+1) of 4 keys
// at permuted position ph (a multiple of 4).
__device__ __forceinline__ void store_v_pair(uint16_t *v_lds, int d, int ph, uint32_t a, uint32_t b, uint32_t c,
                                             uint32_t e) {
    // v_perm selectors: bytes 0-3 pick from the second operand, 4-7 from
    // the first; 0x05040100 = (b.lo16, a.lo16), 0x07060302 = (b.hi16, a.hi16).
    uint2 lo, hi;
    lo.x = __builtin_amdgcn_perm(b, a, 0x05040100u);
    lo.y = __builtin_amdgcn_perm(e, c, 0x05040100u);
    hi.x = __builtin_amdgcn_perm(b, a, 0x07060302u);
    hi.y = __builtin_amdgcn_perm(e, c, 0x07060302u);
    const int col = v_col(d, ph >> 3) + (ph & 7);   // d and d + 1 share a 16-row block
    *reinterpret_cast<uint2 *>(&v_lds[d * VLD + col]) = lo;
    *reinterpret_cast<uint2 *>(&v_lds[(d + 1) * VLD + col]) = hi;
}

template <int D>
__device__ __forceinline__ void store_stage(const StageCtx &sc, int kg, const Stage &r, uint16_t *k_lds,
                                            uint16_t *v_lds) {
    constexpr int KLD = kld<D>();
    *reinterpret_cast<uint4 *>(&k_lds[(4 * kg + 0) * KLD + sc.cc * 8]) = r.k0;
    *reinterpret_cast<uint4 *>(&k_lds[(4 * kg + 1) * KLD + sc.cc * 8]) = r.k1;
    *reinterpret_cast<uint4 *>(&k_lds[(4 * kg + 2) * KLD + sc.cc * 8]) = r.k2;
    *reinterpret_cast<uint4 *>(&k_lds[(4 * kg + 3) * KLD + sc.cc * 8]) = r.k3;
    // 4 keys x 8 dims -> 8 dims x 4 keys
    const int ph = v_phys(4 * kg), d0 = sc.cc * 8;
    store_v_pair(v_lds, d0 + 0, ph, r.v0.x, r.v1.x, r.v2.x, r.v3.x);
    store_v_pair(v_lds, d0 + 2, ph, r.v0.y, r.v1.y, r.v2.y, r.v3.y);
    store_v_pair(v_lds, d0 + 4, ph, r.v0.z, r.v1.z, r.v2.z, r.v3.z);
    store_v_pair(v_lds, d0 + 6, ph, r.v0.w, r.v1.w, r.v2.w, r.v3.w);
}

// Head dims up to 128: two 16-row blocks per wave, and one or two teams of
// four waves (two teams halve each workgroup's serial walk over the keys;
// one team uses half the LDS, so two independent workgroups share a CU and
// their waves' MFMA and softmax phases drift apart and overlap).  D = 256:
// one team, one 16-row block per wave (O^T alone takes 64 registers per
// block, and one K + V^T stage is 74 KB of LDS).
template <int D, int HP, int MASK, bool PAGED, int TEAMS>
__global__ __launch_bounds__(256 * TEAMS, D <= 128 ? 2 : 1) void prefill_kernel(const PrefillParams p) {
    static_assert(TEAMS == 1 || D <= 128, "two teams only up to D = 128");
    constexpr int RB = D <= 128 ? 2 : 1;          // 16-row blocks per wave
    constexpr int NT = 256 * TEAMS;               // threads
    static_assert(RB == 2 || HP <= 4, "one block per wave packs at most four heads");
    constexpr int R = RB == 2 ? (HP <= 4 ? 128 / HP : 16) : 64 / HP;   // rows per work-map tile
    constexpr int KLD = kld<D>();
    constexpr int NS = D / 32;    // 32-deep steps of Q.K^T
    constexpr int NM = D / 16;    // 16-row blocks of O^T
    constexpr int CPR = D / 8;    // 16-byte chunks per K/V row
    constexpr int XCH = D / 2 + 4;                            // floats per lane handed from team 1 to team 0
    // D = 128 stages by LDS copies into natural key rows; other head dims
    // through registers into padded K rows and a V^T tile.
    constexpr bool kDma = D == 128;
    constexpr int SBUF = kDma ? 2 * BK * D : BK * KLD + D * VLD;   // one K tile + one V (or V^T) tile
    static_assert(TEAMS == 1 || kDma || 4 * XCH * 64 * 4 <= 4 * SBUF * 2, "team exchange must fit the stage buffers");
    static_assert(TEAMS == 1 || !kDma || 2 * XCH * 64 * 4 <= TEAMS * SBUF * 2, "team exchange must fit the copy buffers");
    __shared__ __attribute__((aligned(16))) uint16_t stage_lds[kDma ? 8 : TEAMS * 2 * SBUF];   // [team][buffer]
    // LDS-copy buffers [team], one array per buffer: the compiler then knows
    // that reads of one do not wait on copies still landing in the other.
    __shared__ __attribute__((aligned(16))) uint16_t dma0[kDma ? TEAMS * SBUF : 8];
    __shared__ __attribute__((aligned(16))) uint16_t dma1[kDma ? TEAMS * SBUF : 8];
    __shared__ int32_t pages[kPages];
    constexpr int MROWS = MASK == 3 ? R : 1;                  // mask rows per tile
    constexpr int NQ = MASK == 3 && R > 32 ? R / 32 : 1;      // mask rows per thread
    __shared__ __attribute__((aligned(8))) uint8_t mbits[TEAMS][2][MROWS * 8];

    // With two teams of four waves, they take alternate KV tiles of the same
    // query rows and heads; team 1 hands its state to team 0 at the end.
    const int tid = threadIdx.x, lane = tid & 63;
    // team and wave are wave-uniform: taken through readfirstlane so that
    // what derives from them (heads, row offsets) sits in scalar registers.
    const int ttid = tid & 255;
    const int team = TEAMS == 2 ? __builtin_amdgcn_readfirstlane(tid >> 8) : 0;
    const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    // Tiles in reverse work-map order (a sequence's last, longest tiles
    // first), the head groups of a tile next to each other.
    // With split KV the splits of a tile follow each other, head groups
    // innermost.
    const int nhg = p.Hkv * (p.G / HP);
    const unsigned per_tile = (unsigned)nhg * (unsigned)p.kv_splits;
    const int tile = p.num_tiles - 1 - (int)(blockIdx.x / per_tile);
    const int rem = (int)(blockIdx.x % per_tile);
    const int split = rem / nhg;
    const int hg = rem - split * nhg;
    // Work map (packed, ragged Q) or the dense schedule: Lq rows per
    // sequence, tiles_per_seq tiles each.
    int b, ti;
    if (p.dense_lq > 0) {
        const int tps = (p.dense_lq + R - 1) / R;
        b = tile / tps;
        ti = tile - b * tps;
    } else {
        b = p.t2b[tile];
        ti = p.t2i[tile];
    }
    const int groups_per_kv = p.G / HP;
    const int g = hg / groups_per_kv;
    // Row offset (in the tile) and query head of each of the wave's row
    // blocks.
    int rboff[RB], hq[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int hbase = g * p.G + (hg % groups_per_kv) * HP;
        if constexpr (RB == 2) {
            rboff[rb] = HP <= 4 ? (w / HP) * 32 + 16 * rb : 0;
            hq[rb] = hbase + (HP <= 4 ? w % HP : 2 * w + rb);
        } else {
            rboff[rb] = (w / HP) * 16;
            hq[rb] = hbase + w % HP;
        }
    }
    // The sequence's row range, length and causal offset, loaded together:
    // an array the call does not give is read at a stand-in address (the
    // first word of Q, always readable) and its value replaced, so no load
    // waits behind another.
    const bool dense = p.dense_lq > 0;
    const int32_t *stand_in = reinterpret_cast<const int32_t *>(p.q);
    const int v_q0 = *(dense ? stand_in : p.qo_indptr + b);
    const int v_q1 = *(dense ? stand_in : p.qo_indptr + b + 1);
    const int v_n = *(p.kv_lens ? p.kv_lens + b : stand_in);
    const int v_c = *(p.causal ? p.causal + b : stand_in);
    const int q0 = dense ? 0 : v_q0;
    const int qn = dense ? p.dense_lq : v_q1 - q0;
    const int n = p.kv_lens ? v_n : p.kv_len_const;
    // Causality: an offset array (-1 = off for that sequence), or bottom-right
    // alignment c = n - qn for every sequence; key j is admitted for local row
    // i iff j <= c + i (c may be negative: early rows then see no key).
    const bool causal_on = p.causal ? v_c >= 0 : p.causal_br != 0;
    const int c = p.causal ? v_c : n - qn;
    const int64_t qrow0 = (int64_t)b * p.q_sb + (int64_t)q0 * p.q_st;   // Q row 0 of the sequence
    const int64_t orow0 = (int64_t)b * p.o_sb + (int64_t)q0 * p.o_st;
    const int row0 = ti * R;
    const int lq = lane >> 4;   // lane group 0..3
    int myrow[RB];
    bool row_ok[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        myrow[rb] = row0 + rboff[rb] + (lane & 15);   // local query row of this lane
        row_ok[rb] = myrow[rb] < qn;
    }

    // Keys the tile can see: all of the sequence, or up to its causal
    // frontier; this workgroup's share of them is [k_beg, k_end), whole
    // 64-key tiles except at the frontier.
    const int last_row = min(qn, row0 + R) - 1;
    const int kv_end = causal_on ? min(n, c + last_row + 1) : n;
    const int kt_all = kv_end > 0 ? (kv_end + BK - 1) / BK : 0;
    const int k_beg = (int)((int64_t)split * kt_all / p.kv_splits) * BK;
    const int k_end = min(kv_end, (int)((int64_t)(split + 1) * kt_all / p.kv_splits) * BK);

    // Q^T operands: row myrow[rb], d = 32s + 8*lq .. +8.  A negative scale
    // is applied as |scale| on negated Q (a sign flip, exact), so the row
    // maximum can be taken on the unscaled scores.
    // (A zero scale is taken as a tiny positive one: masked scores then stay
    // -inf instead of 0 * -inf, and every admitted key weighs 2^0.)
    const float sl2 = fmaxf(fabsf(p.sl2), 1e-30f);
    const uint32_t qsign = p.sl2 < 0.f ? 0x80008000u : 0u;
    bf16x8_t qf[RB][NS];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const uint16_t *qr =
            p.q + qrow0 + (int64_t)min(myrow[rb], qn - 1) * p.q_st + (int64_t)hq[rb] * p.q_sh + 8 * lq;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            uint4 v = *reinterpret_cast<const uint4 *>(qr + 32 * s);
            v.x ^= qsign; v.y ^= qsign; v.z ^= qsign; v.w ^= qsign;
            qf[rb][s] = as_bf16x8(v);
        }
    }

    // O^T accumulators, and row sums of P from an MFMA against a ones
    // operand (every entry of lacc[rb] holds the lane's row sum).
    f32x4_t oacc[RB][NM], lacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        lacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NM; ++m) oacc[rb][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const bf16x8_t ones = as_bf16x8(make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    // Softmax reference per row (scaled, log2 units), raised lazily: only
    // when a score exceeds it by more than 2^8, so P stays <= 256 and the
    // rescale of O is mostly skipped.
    float m_ref[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) m_ref[rb] = -INFINITY;
    const int wrow0 = row0 + rboff[0];   // first row of this wave

    // Staging assignment: chunk cc = ttid % CPR of the K and V rows of keys
    // 4kg .. 4kg+3, for key groups kg = ttid / CPR + KGS * pass < 16 (at
    // D = 256 a team's 256 threads cover the 16 groups in two passes).
    constexpr int KGS = 256 / CPR;                       // key groups per pass
    constexpr int NPASS = KGS >= 16 ? 1 : 16 / KGS;
    StageCtx sc;
    sc.cc = ttid % CPR;
    const int kg0 = ttid / CPR;
    const bool stager = kg0 < 16;
    // A sequence of one row tile whose KV head's query heads are all packed
    // here (G = HP) has its keys read by this workgroup alone: stream them
    // past the caches.  Otherwise other workgroups (the sequence's other row
    // tiles, or the KV head's other head groups) read the same keys, which
    // stay cached for them.
    sc.stream = qn <= R && p.G == HP;
    sc.pages = pages;
    const int64_t seq_base = PAGED ? 0 : (int64_t)b * p.k_sb;   // contiguous: the sequence's K/V
    sc.kbase = p.k + seq_base + (int64_t)g * p.s_head + sc.cc * 8;
    sc.vbase = p.v + seq_base + (int64_t)g * p.s_head + sc.cc * 8;
    const uint16_t *kseq = p.k + seq_base + (int64_t)g * p.s_head;   // LDS-copy staging: row starts
    const uint16_t *vseq = p.v + seq_base + (int64_t)g * p.s_head;
    const int32_t *bt_row = PAGED ? p.bt + b * p.bt_sb : nullptr;
    Stage st_regs[NPASS];
    auto load_tile = [&](int kt) {
        if (!stager) return;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) load_stage<PAGED>(p, sc, kg0 + KGS * ps, kt, st_regs[ps]);
    };
    auto store_tile = [&](uint16_t *k_lds, uint16_t *v_lds) {
        if (!stager) return;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) store_stage<D>(sc, kg0 + KGS * ps, st_regs[ps], k_lds, v_lds);
    };
    // LDS-copy staging of tile kt into buffer t (K rows, then V rows at
    // + BK * D): wave w copies keys 16 w .. 16 w + 15, four per instruction
    // (lane l: key 4 i + l / 16 of them, physical chunk l % 16).  Keys past
    // the chunk end read keys of the chunk at or below its last key.
    // The four key groups' offsets first (their page lookups from LDS go
    // out together and are waited for once), then the eight copies, under
    // one wave-uniform choice of the streaming hint.
    // Page size a multiple of 16, and slot index and slot stride below 2^24
    // (their product, below 2^32, then comes from a 24-bit multiply).
    const bool ps16 = (p.ps & 15) == 0 && p.ps < (1 << 24) && p.s_slot < (1 << 24);
    auto issue_tile = [&](int kt, uint16_t *t) __attribute__((always_inline)) {
        const int kr = lane >> 4, pc = lane & 15;
        uint64_t off[4];
        if constexpr (PAGED) {
            if (ps16) {
                // The wave's 16 keys start on a multiple of 16, so with a page
                // size that is one they share a page: one wave-uniform lookup.
                // Past the chunk's last key the group is moved back to the
                // last key's group (keys there are not admitted; they read
                // keys of the same tile).
                const int g = __builtin_amdgcn_readfirstlane(min(kt * BK + 16 * w, (sc.c1 - 1) & ~15));
                const uint32_t gpi = divu32((uint32_t)g, p.ps_div);
                const uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(sc.pages[gpi - sc.first_pg]);
                const uint64_t pbase = (uint64_t)pg * (uint32_t)p.s_page;
                const uint32_t kbase = gpi * (uint32_t)p.ps;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t key = (uint32_t)min(g + 4 * i + kr, sc.c1 - 1);
                    off[i] = pbase + ((key - kbase) & 0xffffffu) * ((uint32_t)p.s_slot & 0xffffffu);
                }
            } else {
                uint32_t pi[4], slot[4];
                int pg[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t key = (uint32_t)min(kt * BK + 16 * w + 4 * i + kr, sc.c1 - 1);
                    pi[i] = divu32(key, p.ps_div);
                    slot[i] = key - pi[i] * p.ps;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) pg[i] = sc.pages[pi[i] - sc.first_pg];
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    off[i] = (uint64_t)(uint32_t)pg[i] * (uint32_t)p.s_page + slot[i] * (uint32_t)p.s_slot;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                off[i] = (uint64_t)(uint32_t)min(kt * BK + 16 * w + 4 * i + kr, sc.c1 - 1) * (uint64_t)p.s_slot;
        }
        auto copies = [&](auto nt_c) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = 16 * w + 4 * i + kr;
                copy16_to_lds(kseq + off[i] + 8 * kchunk_swz(tk, pc), t + (16 * w + 4 * i) * D, decltype(nt_c)::value);
                copy16_to_lds(vseq + off[i] + 8 * vchunk_swz(tk, pc), t + BK * D + (16 * w + 4 * i) * D,
                              decltype(nt_c)::value);
            }
        };
        if (__builtin_amdgcn_readfirstlane((int)sc.stream)) copies(std::true_type{});
        else copies(std::false_type{});
    };

    MaskCtx mc;
    mc.base = p.mask + (int64_t)b * p.m_sb + (MASK == 3 ? (int64_t)row0 * p.m_sq : 0);
    mc.m_sq = p.m_sq;
    mc.rows = MASK == 3 ? min(R, qn - row0) : 1;
    MaskStage<MASK, NQ> mst;
    // Mask row (within the tile) of each of this lane's two query rows.
    int mloc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) mloc[rb] = MASK == 3 ? rboff[rb] + (lane & 15) : 0;

    // Keys row myrow[rb] admits: j < lim[rb] (length and causal frontier);
    // the wave's first row has the smallest limit.
    int lim[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lim[rb] = causal_on ? min(n, c + myrow[rb] + 1) : n;
    const int lim_wave = causal_on ? min(n, c + wrow0 + 1) : n;

    // One tile of math from LDS buffer `buf`.  FULL: every key of the tile is
    // admitted by every row of the wave (the common case), so the per-key
    // length and causal tests are skipped.
    auto kbuf = [&](int buf) { return stage_lds + (2 * team + buf) * SBUF; };
    auto vbuf = [&](int buf) { return stage_lds + (2 * team + buf) * SBUF + BK * KLD; };
    auto tile_math = [&](auto full_c, int kt, int buf, const uint16_t *kl, const uint16_t *vl)
        __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        // S^T blocks: keys 16kb + 4lq + i of the tile, rows myrow[rb].
        // Depth step outermost: eight independent accumulators per step, so
        // no MFMA waits on the result of the one before it.
        // The MFMA phases (S^T here, O^T below) run at a raised wave priority
        // and the softmax between them at the normal one, so a SIMD's other
        // wave, in its softmax, yields issue slots to the one feeding the
        // matrix core (measured 2-3% faster on dense and masked prefill).
        __builtin_amdgcn_s_setprio(2);
        f32x4_t st[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) st[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // K operand of depth step s, key block kb.
        auto kop = [&](int s, int kb) __attribute__((always_inline)) {
            const int krow = 16 * kb + (lane & 15);
            return as_bf16x8(*reinterpret_cast<const uint4 *>(
                kDma ? &kl[team * SBUF + krow * D + 8 * kchunk_swz(krow, 4 * s + lq)]
                     : &kl[krow * KLD + 32 * s + 8 * lq]));
        };
        // Operand reads run two depth steps ahead: step s + 2 is read while
        // step s's MFMAs run (scheduling barriers keep that order), so an
        // MFMA never waits on a read issued just before it.
        bf16x8_t ka[2][4];
#pragma unroll
        for (int j = 0; j < (NS < 2 ? NS : 2); ++j)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) ka[j][kb] = kop(j, kb);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) st[rb][kb] = mfma16(ka[s & 1][kb], qf[rb][s], st[rb][kb]);
            if (s + 2 < NS) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) ka[s & 1][kb] = kop(s + 2, kb);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // Scores of keys not admitted become -inf (then P = 0).
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int room = lim[rb] - (kt * BK + 4 * lq);   // admitted iff 16kb + i < room
            uint2 kbits = make_uint2(~0u, ~0u);               // keys 0..31, 32..63 of the tile
            if constexpr (MASK != 0) kbits = *reinterpret_cast<const uint2 *>(&mbits[team][buf][mloc[rb] * 8]);
            kbits.x >>= 4 * lq;
            kbits.y >>= 4 * lq;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (MASK != 0) {
                        // keep = all ones iff the key's mask bit is set (a
                        // sign-extended one-bit field), then a bitwise select
                        // of the score or -inf: two ALU ops per score.
                        uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe(
                            (int)(kb < 2 ? kbits.x : kbits.y), 16 * (kb & 1) + i, 1);
                        if constexpr (!FULL) keep = 16 * kb + i < room ? keep : 0u;
                        st[rb][kb][i] = __uint_as_float((__float_as_uint(st[rb][kb][i]) & keep) |
                                                        (~keep & 0xff800000u));
                    } else if constexpr (!FULL) {
                        st[rb][kb][i] = 16 * kb + i < room ? st[rb][kb][i] : -INFINITY;
                    }
                }
            }
        }
        // Row maxima of the unscaled scores, then the lazy reference.
        float mts[RB];
        bool raise[RB];
        bool any_raise = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                mt = fmaxf(fmaxf(mt, fmaxf(st[rb][kb][0], st[rb][kb][1])), fmaxf(st[rb][kb][2], st[rb][kb][3]));
            mts[rb] = max_over_rows(mt) * sl2;
            raise[rb] = mts[rb] > m_ref[rb] + 8.f;   // false for an all-masked tile
            any_raise = any_raise || raise[rb];
        }
        if (__builtin_amdgcn_ballot_w64(any_raise)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float alpha = raise[rb] ? exp2_fast(m_ref[rb] - mts[rb]) : 1.f;   // 0 from -inf
                m_ref[rb] = raise[rb] ? mts[rb] : m_ref[rb];
                lacc[rb] *= alpha;
#pragma unroll
                for (int m = 0; m < NM; ++m) oacc[rb][m] *= alpha;
            }
        }
        // V^T operand of 16-dim block m, key half s2.
        auto vop = [&](int m, int s2) __attribute__((always_inline)) {
            if constexpr (kDma) return vt_operand(kl, team * SBUF + BK * D, m, s2, lane);
            else return as_bf16x8(*reinterpret_cast<const uint4 *>(
                &vl[(16 * m + (lane & 15)) * VLD + v_col(16 * m, 4 * s2 + lq)]));
        };
        // O^T runs in stages of MB 16-dim blocks, two stages of V^T operands
        // in flight; the first two are read here, so that their latency hides
        // under the exponentials.
        constexpr int MB = NM >= 2 ? 2 : 1;
        constexpr int NMS = NM / MB;
        bf16x8_t va[2][MB][2];
#pragma unroll
        for (int j = 0; j < (NMS < 2 ? NMS : 2); ++j)
#pragma unroll
            for (int mm = 0; mm < MB; ++mm)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) va[j][mm][s2] = vop(MB * j + mm, s2);
        __builtin_amdgcn_sched_barrier(0);
        // P = 2^(s * scale * log2 e - reference), rounded to bf16 pairs.
        uint32_t pw[RB][2][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float neg_ref = m_ref[rb] == -INFINITY ? 0.f : -m_ref[rb];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kb = 2 * s2 + h;
#pragma unroll
                    for (int i = 0; i < 4; i += 2)
                        pw[rb][s2][2 * h + i / 2] = pack_bf16(exp2_fast(fmaf(st[rb][kb][i], sl2, neg_ref)),
                                                              exp2_fast(fmaf(st[rb][kb][i + 1], sl2, neg_ref)));
                }
        }
        __builtin_amdgcn_s_setprio(2);
        // O^T += V^T . P^T, stage j + 2's operands read while stage j's
        // MFMAs run; then the row sums.
        bf16x8_t pb[2][RB];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                pb[s2][rb] = as_bf16x8(make_uint4(pw[rb][s2][0], pw[rb][s2][1], pw[rb][s2][2], pw[rb][s2][3]));
#pragma unroll
        for (int j = 0; j < NMS; ++j) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mm = 0; mm < MB; ++mm)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        oacc[rb][MB * j + mm] = mfma16(va[j & 1][mm][s2], pb[s2][rb], oacc[rb][MB * j + mm]);
            if (j + 2 < NMS) {
#pragma unroll
                for (int mm = 0; mm < MB; ++mm)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) va[j & 1][mm][s2] = vop(MB * (j + 2) + mm, s2);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) lacc[rb] = mfma16(ones, pb[s2][rb], lacc[rb]);
        __builtin_amdgcn_s_setprio(0);
    };
    auto compute = [&](int kt, int buf) {
        if (kt * BK + BK <= lim_wave) tile_math(std::true_type{}, kt, buf, kbuf(buf), vbuf(buf));
        else tile_math(std::false_type{}, kt, buf, kbuf(buf), vbuf(buf));
    };
    // LDS-copy tiles: the buffer is a compile-time choice (bc), so each
    // instance reads one array.
    auto compute_dma = [&](int kt, auto bc) __attribute__((always_inline)) {
        constexpr int B = decltype(bc)::value;
        // the array itself: the team's offset is part of each read's index
        const uint16_t *t = B == 0 ? dma0 : dma1;
        if (kt * BK + BK <= lim_wave) tile_math(std::true_type{}, kt, B, t, t);
        else tile_math(std::false_type{}, kt, B, t, t);
    };

    // Keys in chunks whose pages fit the LDS slice; chunks start on tile
    // boundaries, so no tile straddles two.
    const int64_t ch_keys = PAGED ? (int64_t)(kPages - 2) * p.ps / BK * BK : (int64_t)1 << 30;
    const int CH = (int)min<int64_t>(ch_keys > 0 ? ch_keys : BK, 1 << 30);
    for (int c0 = k_beg; c0 < k_end; c0 += CH) {
        const int c1 = min(k_end, c0 + CH);
        const int t0 = c0 / BK, t1 = (c1 + BK - 1) / BK;
        sc.c1 = c1;
        __syncthreads();   // the previous chunk is done with the slice and the buffers
        if constexpr (PAGED) {
            sc.first_pg = (int)divu32((uint32_t)c0, p.ps_div);
            const int npg = (int)divu32((uint32_t)(c1 - 1), p.ps_div) - sc.first_pg + 1;
            for (int i = tid; i < npg; i += NT) pages[i] = bt_row[sc.first_pg + i];
        }
        __syncthreads();
        // This team's tiles of the chunk: t0 + team, t0 + team + TEAMS, ...
        const int kt0 = t0 + team;
        const int nit = (t1 - t0 + TEAMS - 1) / TEAMS;
        if constexpr (kDma) {
            // Tile kt + 1 lands in one buffer while tile kt is computed from
            // the other; tile kt + 2 goes out once every wave is past kt.
            // The copies are outside the compiler's register tracking, so
            // the wait for them (all of the wave's vector memory operations,
            // mask loads included) is explicit, before the barrier.
            if (kt0 < t1) {
                issue_tile(kt0, dma0 + team * SBUF);
                if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt0, mst);
                __builtin_amdgcn_s_waitcnt(kWaitVmem0);
                if constexpr (MASK != 0) store_mask<MASK, NQ, MROWS>(mst, ttid, mbits[team][0]);
            }
            if (kt0 + TEAMS < t1) {
                issue_tile(kt0 + TEAMS, dma1 + team * SBUF);
                if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt0 + TEAMS, mst);
            }
            __syncthreads();
            auto step = [&](auto bc, int it) __attribute__((always_inline)) {
                constexpr int B = decltype(bc)::value;
                const int kt = kt0 + TEAMS * it;
                if (kt < t1) compute_dma(kt, bc);
                if constexpr (MASK != 0)
                    if (kt + TEAMS < t1) store_mask<MASK, NQ, MROWS>(mst, ttid, mbits[team][B ^ 1]);
                __builtin_amdgcn_s_waitcnt(kWaitVmem0);
                __syncthreads();
                if (kt + 2 * TEAMS < t1) {
                    issue_tile(kt + 2 * TEAMS, (B == 0 ? dma0 : dma1) + team * SBUF);
                    if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt + 2 * TEAMS, mst);
                }
            };
            for (int it = 0; it < nit; it += 2) {
                step(std::integral_constant<int, 0>{}, it);
                if (it + 1 < nit) step(std::integral_constant<int, 1>{}, it + 1);
            }
            continue;
        }
        if (kt0 < t1) {
            load_tile(kt0);
            if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt0, mst);
            store_tile(kbuf(0), vbuf(0));
            if constexpr (MASK != 0) store_mask<MASK, NQ, MROWS>(mst, ttid, mbits[team][0]);
        }
        if (kt0 + TEAMS < t1) {
            load_tile(kt0 + TEAMS);
            if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt0 + TEAMS, mst);
        }
        __syncthreads();
        for (int it = 0; it < nit; ++it) {
            const int kt = kt0 + TEAMS * it;
            if (kt < t1) compute(kt, it & 1);
            if (kt + TEAMS < t1) {
                // The team's next tile into its other buffer (its readers
                // finished at the last barrier), then the one after goes out.
                store_tile(kbuf((it + 1) & 1), vbuf((it + 1) & 1));
                if constexpr (MASK != 0) store_mask<MASK, NQ, MROWS>(mst, ttid, mbits[team][(it + 1) & 1]);
                if (kt + 2 * TEAMS < t1) {
                    load_tile(kt + 2 * TEAMS);
                    if constexpr (MASK != 0) load_mask<MASK, NQ>(mc, ttid, n, kt + 2 * TEAMS, mst);
                }
            }
            __syncthreads();
        }
    }

    if constexpr (TEAMS == 2) {
        // Team 1's (O, reference, sum) go through the stage buffers (free
        // since the last barrier) to the matching wave of team 0, which merges.
        // With LDS-copy buffers, waves 0-1 use the first array, 2-3 the second.
        float *xch = kDma ? reinterpret_cast<float *>(w < 2 ? dma0 : dma1) + (w & 1) * (XCH * 64)
                          : reinterpret_cast<float *>(stage_lds) + w * (XCH * 64);
        if (team == 1) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) xch[(rb * (D / 4) + m * 4 + i) * 64 + lane] = oacc[rb][m][i];
                xch[(D / 2 + rb) * 64 + lane] = m_ref[rb];
                xch[(D / 2 + 2 + rb) * 64 + lane] = lacc[rb][0];
            }
        }
        __syncthreads();
        if (team == 1) return;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float mb = xch[(D / 2 + rb) * 64 + lane], lb = xch[(D / 2 + 2 + rb) * 64 + lane];
            const float mm = fmaxf(m_ref[rb], mb);
            const float aa = m_ref[rb] == -INFINITY ? 0.f : exp2_fast(m_ref[rb] - mm);
            const float ab = mb == -INFINITY ? 0.f : exp2_fast(mb - mm);
            lacc[rb][0] = lacc[rb][0] * aa + lb * ab;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    oacc[rb][m][i] = oacc[rb][m][i] * aa + xch[(rb * (D / 4) + m * 4 + i) * 64 + lane] * ab;
            m_ref[rb] = mm;   // the merged (O, l) are relative to 2^mm
        }
    }

    if (p.kv_splits > 1) {
        // Unnormalised partial: O^T column and (m, l), m back in natural-log
        // units of the scaled score.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int64_t t = (p.dense_lq > 0 ? (int64_t)b * p.dense_lq : (int64_t)q0) + myrow[rb];
            if (!row_ok[rb] || t >= p.part_rows) continue;
            const int64_t pr = ((int64_t)split * p.part_rows + t) * p.Hq + hq[rb];
            float *op = p.o_part + pr * D + 4 * lq;
#pragma unroll
            for (int m = 0; m < NM; ++m)
                *reinterpret_cast<float4 *>(op + 16 * m) =
                    make_float4(oacc[rb][m][0], oacc[rb][m][1], oacc[rb][m][2], oacc[rb][m][3]);
            if (lq == 0)
                *reinterpret_cast<float2 *>(p.ml_part + pr * 2) = make_float2(
                    m_ref[rb] == -INFINITY && !is_nan_bits(lacc[rb][0]) ? -INFINITY : partial_m(m_ref[rb], lacc[rb][0]),
                    lacc[rb][0]);
        }
        return;
    }
    // One team with 16-byte aligned output rows: each wave stages its
    // normalised rows in its own LDS region (rows padded by 8 elements, so
    // the 8-byte writes of a 16-row block hit distinct banks) and writes
    // whole rows back with 16-byte stores, four 256-byte rows (D = 128) per
    // instruction.  A block's 8-byte pieces scatter over 16 rows, and
    // issuing them took about 12 times as long.  The stage buffers are free
    // since the last barrier, and a wave reads back only what it wrote.
    if constexpr (TEAMS == 1) {
        const bool aligned16 = ((reinterpret_cast<uintptr_t>(p.o) | (uint64_t)orow0 * 2 | (uint64_t)p.o_st * 2 |
                                 (uint64_t)p.o_sh * 2) & 15) == 0;
        if (aligned16) {
            constexpr int SD = D + 8;                 // staged row stride (elements)
            constexpr int LU = D / 8;                 // lanes per row (16 bytes each)
            constexpr int UPI = 64 / LU;              // rows per store instruction
            constexpr int NI = RB * 16 / UPI;         // store instructions per wave
            uint16_t *stg = kDma ? (w < 2 ? dma0 : dma1) + (w & 1) * (RB * 16 * SD)
                                 : stage_lds + w * (RB * 16 * SD);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float l_row = lacc[rb][0];
                const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    uint2 wv;
                    wv.x = pack_bf16(oacc[rb][m][0] * inv, oacc[rb][m][1] * inv);
                    wv.y = pack_bf16(oacc[rb][m][2] * inv, oacc[rb][m][3] * inv);
                    *reinterpret_cast<uint2 *>(stg + (rb * 16 + (lane & 15)) * SD + 16 * m + 4 * lq) = wv;
                }
            }
#pragma unroll
            for (int k = 0; k < NI; ++k) {
                const int u = k * UPI + lane / LU, c = lane % LU;   // staged row, 16-byte chunk
                const int rb = u / 16, rr = u % 16;
                const uint4 v = *reinterpret_cast<const uint4 *>(stg + u * SD + 8 * c);
                const int row = row0 + (rb == 0 ? rboff[0] : rboff[RB - 1]) + rr;
                const int h = rb == 0 ? hq[0] : hq[RB - 1];
                if (row < qn)
                    *reinterpret_cast<uint4 *>(p.o + orow0 + (int64_t)row * p.o_st + (int64_t)h * p.o_sh + 8 * c) = v;
            }
            return;
        }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const float l_row = lacc[rb][0];
        if (!row_ok[rb]) continue;
        const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
        uint16_t *orow = p.o + orow0 + (int64_t)myrow[rb] * p.o_st + (int64_t)hq[rb] * p.o_sh + 4 * lq;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            uint2 wv;
            wv.x = pack_bf16(oacc[rb][m][0] * inv, oacc[rb][m][1] * inv);
            wv.y = pack_bf16(oacc[rb][m][2] * inv, oacc[rb][m][3] * inv);
            *reinterpret_cast<uint2 *>(orow + 16 * m) = wv;
        }
    }
}

template <int D, int HP, bool PAGED, int TEAMS>
hipError_t launch_teams(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)p.num_tiles * (unsigned)(p.Hkv * (p.G / HP)) * (unsigned)p.kv_splits);
    const dim3 block(256 * TEAMS);
    switch (p.mask_ndim) {
        case 0: hipLaunchKernelGGL((prefill_kernel<D, HP, 0, PAGED, TEAMS>), grid, block, 0, stream, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<D, HP, 2, PAGED, TEAMS>), grid, block, 0, stream, p); break;
        case 3: hipLaunchKernelGGL((prefill_kernel<D, HP, 3, PAGED, TEAMS>), grid, block, 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int HP, bool PAGED>
hipError_t launch_hp(const PrefillParams &p, hipStream_t stream) {
    if constexpr (D <= 128) {
        if (p.teams == 2) return launch_teams<D, HP, PAGED, 2>(p, stream);
    }
    return launch_teams<D, HP, PAGED, 1>(p, stream);
}

template <int D, bool PAGED>
hipError_t launch_paged(const PrefillParams &p, hipStream_t stream) {
    switch (prefill_heads_packed(p.G, D)) {
        case 1: return launch_hp<D, 1, PAGED>(p, stream);
        case 2: return launch_hp<D, 2, PAGED>(p, stream);
        case 4: return launch_hp<D, 4, PAGED>(p, stream);
        case 8:
            if constexpr (D <= 128) return launch_hp<D, 8, PAGED>(p, stream);
            else return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

// Split-KV combine: wave per (row t, head h); lanes hold EPL consecutive
// floats of the head row, eight partials in flight per step.
template <int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(const PrefillCombineParams p) {
    constexpr int EPL = D >= 64 ? D / 64 : 1;
    constexpr int NL = D / EPL;   // lanes that hold part of the row
    const int lane = threadIdx.x & 63;
    const int64_t RH = (int64_t)p.rows * p.Hq;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave_id();
    if (item >= RH) return;
    const int64_t t = item / p.Hq;
    const int h = (int)(item - t * p.Hq);
    float M = -INFINITY;
    for (int s = lane; s < p.S; s += 64) M = fmaxf(M, p.ml_part[((int64_t)s * RH + item) * 2]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, __shfl_xor(M, k));
    float acc[EPL], L = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    const int ln = min(lane, NL - 1);
    if (M != -INFINITY) {
        constexpr int U = 8;
        for (int s0 = 0; s0 < p.S; s0 += U) {
            float2 ml[U];
            float ov[U][EPL];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int64_t row = (int64_t)min(s0 + k, p.S - 1) * RH + item;
                ml[k] = *reinterpret_cast<const float2 *>(p.ml_part + row * 2);
#pragma unroll
                for (int e = 0; e < EPL; ++e) ov[k][e] = p.o_part[row * D + ln * EPL + e];
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const bool use = s0 + k < p.S && ml[k].x != -INFINITY;
                const float wgt = use ? exp2_fast((ml[k].x - M) * kLog2e) : 0.f;
                L = fmaf(wgt, use ? ml[k].y : 0.f, L);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] = fmaf(wgt, use ? ov[k][e] : 0.f, acc[e]);
            }
        }
    }
    if (lane >= NL) return;
    const float inv = L > 0.f ? 1.f / L : 0.f;
    int64_t off;
    if (p.dense_lq > 0) {
        const int64_t bb = t / p.dense_lq;
        off = bb * p.o_sb + (t - bb * p.dense_lq) * p.o_st;
    } else {
        off = t * p.o_st;
    }
    uint16_t *dst = p.o + off + (int64_t)h * p.o_sh + lane * EPL;
    if constexpr (EPL == 1) {
        dst[0] = (uint16_t)(pack_bf16(acc[0] * inv, 0.f) & 0xffffu);
    } else {
#pragma unroll
        for (int e = 0; e < EPL; e += 2) *reinterpret_cast<uint32_t *>(dst + e) = pack_bf16(acc[e] * inv, acc[e + 1] * inv);
    }
}

}  // namespace

int prefill_heads_packed(int G, int D) {
    const int cap = D <= 128 ? 8 : 4;   // row blocks of a workgroup's team: eight, or four at D = 256
    return (G & -G) < cap ? (G & -G) : cap;
}
int prefill_tile_rows(int G, int D) {
    const int hp = prefill_heads_packed(G, D);
    if (D > 128) return 64 / hp;
    return hp <= 4 ? 128 / hp : 16;
}

hipError_t launch_prefill_combine(const PrefillCombineParams &p, int D, hipStream_t stream) {
    const int64_t items = (int64_t)p.rows * p.Hq;
    if (items <= 0) return hipSuccess;
    const dim3 grid((unsigned)((items + 3) / 4));
    if (D == 32) hipLaunchKernelGGL((prefill_combine_kernel<32>), grid, dim3(256), 0, stream, p);
    else if (D == 64) hipLaunchKernelGGL((prefill_combine_kernel<64>), grid, dim3(256), 0, stream, p);
    else if (D == 128) hipLaunchKernelGGL((prefill_combine_kernel<128>), grid, dim3(256), 0, stream, p);
    else if (D == 256) hipLaunchKernelGGL((prefill_combine_kernel<256>), grid, dim3(256), 0, stream, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &p, int D, hipStream_t stream) {
    if (p.num_tiles <= 0) return hipSuccess;
    if (D == 32) return p.bt ? launch_paged<32, true>(p, stream) : launch_paged<32, false>(p, stream);
    if (D == 64) return p.bt ? launch_paged<64, true>(p, stream) : launch_paged<64, false>(p, stream);
    if (D == 128) return p.bt ? launch_paged<128, true>(p, stream) : launch_paged<128, false>(p, stream);
    if (D == 256) return p.bt ? launch_paged<256, true>(p, stream) : launch_paged<256, false>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
