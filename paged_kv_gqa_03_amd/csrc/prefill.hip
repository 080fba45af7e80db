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
// Work decomposition: one 256-thread workgroup per (work-map tile, group of
// HP query heads sharing one KV head).  Wave w handles 16 query rows of one
// head; the HP heads of a workgroup read every K/V tile once from LDS.  A
// tile has 64/HP rows (HP = min(G, 4)).
//
// Per KV tile of 64 keys the workgroup stages K row-major and V transposed
// (d-major, keys permuted) in LDS; the transpose is done in registers while
// staging.  Each wave then runs, with v_mfma_f32_16x16x32_bf16,
//   S^T (64 keys x 16 rows) = K (64 x 128) . Q^T (128 x 16)     16 MFMA
//   O^T (128 x 16)        += V^T (128 x 64) . P^T (64 x 16)     16 MFMA
// In this transposed form lane l always holds query row l % 16: its scores
// are 16 keys of that row (keys 4*(l/16) + i of each 16-key block), so the
// row max / sum need only two cross-lane steps, the softmax rescale of O is
// a per-lane scalar, and P^T feeds the second MFMA straight from registers
// (V^T is stored with the matching key order).  Scores are scaled in fp32
// after the dot product (csrc commit that moved the scale after Q.K^T).
// Keys past the causal frontier of the tile are never loaded.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;         // keys per KV tile
constexpr int KLD = 128 + 8;   // K tile row stride in LDS (elements): 272 B, conflict-free 16 B reads
constexpr int VLD = BK + 8;    // V^T row stride in LDS (elements): 144 B

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Position of key k (0..63) inside the transposed V tile: within each group
// of 32 keys, key 16h + 4q + i sits at 8q + 4h + i, so the eight keys that
// lane group q contributes to one P^T operand are contiguous.
__device__ __forceinline__ int v_phys(int k) {
    const int k32 = k & 31;
    return (k & ~31) + 8 * ((k32 & 15) >> 2) + 4 * (k32 >> 4) + (k32 & 3);
}

// Per-thread share of one KV tile in flight: four K chunks, four V chunks.
struct Stage {
    uint4 k0, k1, k2, k3, v0, v1, v2, v3;
};

struct StageCtx {
    int cc, kg, kv_end;
    const int32_t *bt_row;
    const uint16_t *kbase, *vbase;
};

__device__ __forceinline__ uint64_t key_off(const PrefillParams &p, const StageCtx &sc, int key) {
    const int kc = min(key, sc.kv_end - 1);
    const uint32_t pi = udiv_magic((uint32_t)kc, p.ps_magic);
    const int page = sc.bt_row[pi];
    const uint32_t slot = (uint32_t)kc - pi * p.ps;
    return (uint64_t)(uint32_t)page * (uint32_t)p.s_page + slot * (uint32_t)p.s_slot;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *ptr) { return *reinterpret_cast<const uint4 *>(ptr); }

__device__ __forceinline__ void load_stage(const PrefillParams &p, const StageCtx &sc, int kt, Stage &r) {
    const int kv0 = kt * BK;
    r.k0 = ld16(sc.kbase + key_off(p, sc, kv0 + sc.kg));
    r.k1 = ld16(sc.kbase + key_off(p, sc, kv0 + sc.kg + 16));
    r.k2 = ld16(sc.kbase + key_off(p, sc, kv0 + sc.kg + 32));
    r.k3 = ld16(sc.kbase + key_off(p, sc, kv0 + sc.kg + 48));
    r.v0 = ld16(sc.vbase + key_off(p, sc, kv0 + 4 * sc.kg));
    r.v1 = ld16(sc.vbase + key_off(p, sc, kv0 + 4 * sc.kg + 1));
    r.v2 = ld16(sc.vbase + key_off(p, sc, kv0 + 4 * sc.kg + 2));
    r.v3 = ld16(sc.vbase + key_off(p, sc, kv0 + 4 * sc.kg + 3));
}

// One 32-bit column pair of the 4 x 8 V block: dims (2j, 2j+1) of 4 keys.
__device__ __forceinline__ void store_v_pair(uint16_t *v_lds, int d, int ph, uint32_t a, uint32_t b, uint32_t c,
                                             uint32_t e) {
    uint2 lo, hi;
    lo.x = (a & 0xffffu) | (b << 16);
    lo.y = (c & 0xffffu) | (e << 16);
    hi.x = (a >> 16) | (b & 0xffff0000u);
    hi.y = (c >> 16) | (e & 0xffff0000u);
    *reinterpret_cast<uint2 *>(&v_lds[d * VLD + ph]) = lo;
    *reinterpret_cast<uint2 *>(&v_lds[(d + 1) * VLD + ph]) = hi;
}

__device__ __forceinline__ void store_stage(const StageCtx &sc, const Stage &r, uint16_t *k_lds, uint16_t *v_lds) {
    *reinterpret_cast<uint4 *>(&k_lds[(sc.kg + 0) * KLD + sc.cc * 8]) = r.k0;
    *reinterpret_cast<uint4 *>(&k_lds[(sc.kg + 16) * KLD + sc.cc * 8]) = r.k1;
    *reinterpret_cast<uint4 *>(&k_lds[(sc.kg + 32) * KLD + sc.cc * 8]) = r.k2;
    *reinterpret_cast<uint4 *>(&k_lds[(sc.kg + 48) * KLD + sc.cc * 8]) = r.k3;
    // 4 keys x 8 dims -> 8 dims x 4 keys
    const int ph = v_phys(4 * sc.kg), d0 = sc.cc * 8;
    store_v_pair(v_lds, d0 + 0, ph, r.v0.x, r.v1.x, r.v2.x, r.v3.x);
    store_v_pair(v_lds, d0 + 2, ph, r.v0.y, r.v1.y, r.v2.y, r.v3.y);
    store_v_pair(v_lds, d0 + 4, ph, r.v0.z, r.v1.z, r.v2.z, r.v3.z);
    store_v_pair(v_lds, d0 + 6, ph, r.v0.w, r.v1.w, r.v2.w, r.v3.w);
}

template <int HP, int MASK>
__global__ __launch_bounds__(256) void prefill_kernel(const PrefillParams p) {
    constexpr int RB = 4 / HP;   // 16-row blocks per workgroup
    constexpr int R = 16 * RB;   // rows per work-map tile
    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BK * KLD];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds[128 * VLD];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int tile = blockIdx.x;
    const int b = p.t2b[tile], ti = p.t2i[tile];
    const int groups_per_kv = p.G / HP;
    const int g = blockIdx.y / groups_per_kv;
    const int hq = g * p.G + (blockIdx.y % groups_per_kv) * HP + (w % HP);
    const int q0 = p.qo_indptr[b];
    const int qn = p.qo_indptr[b + 1] - q0;
    const int n = p.kv_lens[b];
    const int c = p.causal ? p.causal[b] : -1;
    const int row0 = ti * R;
    const int myrow = row0 + (w / HP) * 16 + (lane & 15);  // local query row of this lane
    const int lq = lane >> 4;                               // lane group 0..3
    const bool row_ok = myrow < qn;

    // Keys the tile can see: all of the sequence, or up to its causal frontier.
    const int last_row = min(qn, row0 + R) - 1;
    const int kv_end = (c >= 0) ? min(n, c + last_row + 1) : n;
    const int n_kt = (kv_end + BK - 1) / BK;

    // Q^T operand: row myrow, d = 32s + 8*lq .. +8.
    bf16x8_t qf[4];
    {
        const uint16_t *qr = p.q + (int64_t)(q0 + min(myrow, qn - 1)) * p.q_st + (int64_t)hq * p.q_sh + 8 * lq;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const uint4 *>(qr + 32 * s));
    }

    f32x4_t oacc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) oacc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_i = -INFINITY, l_i = 0.f;

    // Staging assignment: K rows kk = (tid >> 4) + 16 i, chunk cc = tid & 15;
    // V keys 4*(tid >> 4) + r, same chunk.
    StageCtx sc;
    sc.cc = tid & 15;
    sc.kg = tid >> 4;
    sc.bt_row = p.bt + b * p.bt_sb;
    sc.kbase = p.k + (int64_t)g * p.s_head + sc.cc * 8;
    sc.vbase = p.v + (int64_t)g * p.s_head + sc.cc * 8;
    sc.kv_end = kv_end;
    Stage st_regs;

    const int64_t mrow = MASK == 3 ? (int64_t)b * p.m_sb + (int64_t)myrow * p.m_sq : (int64_t)b * p.m_sb;
    if (n_kt > 0) load_stage(p, sc, 0, st_regs);
    for (int kt = 0; kt < n_kt; ++kt) {
        __syncthreads();   // every wave is done reading the previous tile
        store_stage(sc, st_regs, k_lds, v_lds);
        __syncthreads();
        // Next tile's loads are in flight during the math (the last
        // iteration reloads its own tile: in bounds, never stored).
        load_stage(p, sc, min(kt + 1, n_kt - 1), st_regs);
        const int kv0 = kt * BK;

        // S^T blocks: keys 16kb + 4lq + i of the tile, row myrow.
        f32x4_t st[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            st[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8_t a = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&k_lds[(16 * kb + (lane & 15)) * KLD + 32 * s + 8 * lq]));
                st[kb] = mfma16(a, qf[s], st[kb]);
            }
        }
        // Scale, causal frontier, keep-mask.
        float x[4][4];
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int j0 = kv0 + 16 * kb + 4 * lq;
            uint32_t keep4 = 0x01010101u;
            if constexpr (MASK != 0) {
                keep4 = 0;
                if (row_ok) {
                    const uint8_t *mp = p.mask + mrow + j0;
                    if (j0 + 4 <= n) {
                        keep4 = *reinterpret_cast<const uint32_t *>(mp);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (j0 + i < n) keep4 |= (uint32_t)mp[i] << (8 * i);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + i;
                const bool ok = j < n && (c < 0 || j <= c + myrow) && ((keep4 >> (8 * i)) & 0xffu);
                x[kb][i] = ok ? st[kb][i] * p.sl2 : -INFINITY;
                mt = fmaxf(mt, x[kb][i]);
            }
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_i, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2_fast(m_i - m_use);   // 0 while m_i is -inf
        m_i = m_new;
        uint32_t pw[2][4];
        float psum = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kb = 2 * s2 + h;
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const uint32_t pk = pack_bf16(exp2_fast(x[kb][i] - m_use), exp2_fast(x[kb][i + 1] - m_use));
                    psum += bf16_lo(pk) + bf16_hi(pk);
                    pw[s2][2 * h + i / 2] = pk;
                }
            }
        l_i = l_i * alpha + psum;
#pragma unroll
        for (int m = 0; m < 8; ++m) oacc[m] *= alpha;
        // O^T += V^T . P^T
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8_t pb = as_bf16x8(make_uint4(pw[s2][0], pw[s2][1], pw[s2][2], pw[s2][3]));
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const bf16x8_t a = as_bf16x8(
                    *reinterpret_cast<const uint4 *>(&v_lds[(16 * m + (lane & 15)) * VLD + 32 * s2 + 8 * lq]));
                oacc[m] = mfma16(a, pb, oacc[m]);
            }
        }
    }

    float l_row = l_i;
    l_row += __shfl_xor(l_row, 16);
    l_row += __shfl_xor(l_row, 32);
    if (!row_ok) return;
    const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
    uint16_t *orow = p.o + (int64_t)(q0 + myrow) * p.o_st + (int64_t)hq * p.o_sh + 4 * lq;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        uint2 wv;
        wv.x = pack_bf16(oacc[m][0] * inv, oacc[m][1] * inv);
        wv.y = pack_bf16(oacc[m][2] * inv, oacc[m][3] * inv);
        *reinterpret_cast<uint2 *>(orow + 16 * m) = wv;
    }
}

template <int HP>
hipError_t launch_hp(const PrefillParams &p, hipStream_t stream) {
    const dim3 grid(p.num_tiles, p.Hkv * (p.G / HP));
    switch (p.mask_ndim) {
        case 0: hipLaunchKernelGGL((prefill_kernel<HP, 0>), grid, dim3(256), 0, stream, p); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<HP, 2>), grid, dim3(256), 0, stream, p); break;
        case 3: hipLaunchKernelGGL((prefill_kernel<HP, 3>), grid, dim3(256), 0, stream, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int prefill_heads_packed(int G) { return G >= 4 ? 4 : G; }

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream) {
    if (p.num_tiles <= 0) return hipSuccess;
    switch (prefill_heads_packed(p.G)) {
        case 1: return launch_hp<1>(p, stream);
        case 2: return launch_hp<2>(p, stream);
        case 4: return launch_hp<4>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
