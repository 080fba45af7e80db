// swa.hip -- fp8 (OCP e4m3fn) sliding-window decode, MLA style (K = V),
// for gfx950.
//
// Method (native_swa_decode.py: the host wrapper's problem statement and the
// batched-SDPA fallback's steps): decode token t attends at most `window`
// cache slots listed in swa_indices[t]; position j is admitted iff
// j < swa_lens[t] and the slot index is >= 0; the slot is split into (block,
// offset), its 512 fp8 bytes are dequantised with the slot's inverse scale,
// and every query head of the token attends the same rows, which serve as
// both keys and values.
//
// Work decomposition (cf. the CuTeDSL stub's plan: one CTA per (token, group
// of 16 query heads), KV streamed in tiles): one workgroup per token and
// GPW adjacent 16-head groups (GPW = 2 when the group count is even, else
// 1), four waves per group.  The groups of a workgroup share one staged copy
// of the token's rows, which halves the row traffic from L2 (a token's
// groups otherwise each gather the same rows).  Per tile of up to 128
// window positions:
//   1. the rows (fp8, 512 B each) and inverse scales are staged in LDS in
//      two dependent load steps (indices, then rows and scales, all issued
//      before any LDS store); masked positions become zero rows;
//   2. wave w computes S^T for positions 32w..32w+31 with
//      v_mfma_f32_16x16x32_bf16 on rows converted fp8 -> bf16 exactly
//      (v_cvt_scalef32_pk_bf16_fp8), Q^T for the 16 heads held in registers;
//      the score is scale * inv_scale_j * (q . e4m3(x_j)), i.e. the exact
//      dequantised product, with the scale folded into one multiply;
//   3. the row max / sum across the four waves go through LDS;
//   4. P' = P * inv_scale_j (bf16) is written to LDS, and wave w computes
//      O^T for dims 128w..128w+127 = X^T P'^T, building the X^T operands by
//      a byte transpose (v_perm) of four dims x eight positions and the same
//      exact fp8 -> bf16 conversion.  Lane l then holds head l % 16 and four
//      consecutive dims per output block, written as 8-byte bf16 stores.
// Windows longer than 128 loop over tiles with an online softmax.
#include "device_common.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int HD = 512;
constexpr int KT = 128;        // window positions per tile
constexpr int XLD = HD + 16;   // staged row stride (bytes)
constexpr int PLD = KT + 8;    // P' row stride (elements)

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight e4m3fn codes (lo: codes 0..3, hi: codes 4..7) -> eight bf16, exact.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}

// v_perm_b32: result byte i = selector byte i, where 0..3 pick bytes of the
// second operand and 4..7 bytes of the first.
__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Transpose a 4-position x 4-byte block: w[e] holds bytes (d0..d3) of
// position e; out[m] holds byte d_m of positions 0..3.
__device__ __forceinline__ void transpose4x4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3, uint32_t (&out)[4]) {
    const uint32_t a01 = perm(w1, w0, 0x06020400u);  // w0.b0 w1.b0 w0.b2 w1.b2
    const uint32_t b01 = perm(w1, w0, 0x07030501u);  // w0.b1 w1.b1 w0.b3 w1.b3
    const uint32_t a23 = perm(w3, w2, 0x06020400u);
    const uint32_t b23 = perm(w3, w2, 0x07030501u);
    out[0] = perm(a23, a01, 0x05040100u);  // b0 of w0..w3
    out[2] = perm(a23, a01, 0x07060302u);  // b2
    out[1] = perm(b23, b01, 0x05040100u);  // b1
    out[3] = perm(b23, b01, 0x07060302u);  // b3
}

template <int GPW>
__global__ __launch_bounds__(256 * GPW, GPW == 1 ? 2 : 1) void swa_kernel(const SwaParams p) {
    constexpr int NTH = 256 * GPW;        // threads
    constexpr int RPT = KT * 32 / NTH;    // staged 16-byte row chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t x_lds[KT * XLD];
    __shared__ __attribute__((aligned(16))) int32_t admit[KT];   // window position admitted (1) or masked (0)
    __shared__ __attribute__((aligned(16))) float inv_lds[KT];
    __shared__ __attribute__((aligned(16))) uint16_t p_lds_all[GPW][16 * PLD];
    __shared__ float red_max_all[GPW][4][16], red_sum_all[GPW][4][16];

    const int tid = threadIdx.x, lane = tid & 63, w = (tid >> 6) & 3, gs = tid >> 8;
    const int r = lane & 15, q4 = lane >> 4;
    uint16_t *p_lds = p_lds_all[gs];
    float(*red_max)[16] = red_max_all[gs];
    float(*red_sum)[16] = red_sum_all[gs];
    // Workgroup (token t, head groups GPW c .. GPW c + GPW - 1) at
    // t * (NH / 16 / GPW) + c: the workgroups of a token are adjacent.
    const int nwg = (p.NH >> 4) / GPW;
    const int t = (int)(blockIdx.x / (unsigned)nwg);
    const int head = ((int)(blockIdx.x - (unsigned)t * (unsigned)nwg) * GPW + gs) * 16 + r;
    int64_t len = p.lens[t];
    len = len < 0 ? 0 : (len > p.W ? p.W : len);

    // Q^T operand: head r, dims 32s + 8*q4 .. +8.
    // Loaded right after the first tile's window indices: the loads complete
    // in order, so the index -> row chain must not queue behind 16 KB of Q.
    bf16x8_t qf[16];
    auto load_q = [&]() {
        const uint16_t *qr = p.q + (int64_t)t * p.q_st + (int64_t)head * p.q_sh + 8 * q4;
#pragma unroll
        for (int s = 0; s < 16; ++s) qf[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(qr + 32 * s));
    };
    f32x4_t oacc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int m = 0; m < 4; ++m) oacc[a][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, L = 0.f;

    // The first tile's window indices and Q go out with the token length:
    // positions below the window exist in the index row whatever the
    // length (those at or past it are dropped below).
    int64_t idx0[RPT], idx0_s = -1;
    if (p.W > 0) {
        const int64_t *irow = p.ind + (int64_t)t * p.i_st;
        const int wl = p.W - 1;
#pragma unroll
        for (int i = 0; i < RPT; ++i) idx0[i] = irow[min((tid >> 5) + (NTH / 32) * i, wl)];
        idx0_s = irow[min(tid, wl)];
    }
    load_q();
    const int ntile = (int)((len + KT - 1) / KT);
    for (int tile = 0; tile < ntile; ++tile) {
        const int j0 = tile * KT;
        const int nk = (int)min((int64_t)KT, len - j0);
        const int nkb = (nk + 31) >> 5;   // 32-position blocks in this tile
        __syncthreads();                  // the previous tile is fully consumed
        // Staging with two dependent steps: every thread first loads the
        // window indices of its RPT rows (keys (tid >> 5) + (NTH / 32) i,
        // chunk tid & 31) and, below 128, of key tid (for the scale); then all
        // row chunks and scales go out together, and only then are they
        // stored to LDS.
        {
            const int64_t *irow = p.ind + (int64_t)t * p.i_st + j0;
            const int ch = tid & 31;
            int64_t idx[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int key = (tid >> 5) + (NTH / 32) * i;
                idx[i] = key < nk ? (tile == 0 ? idx0[i] : irow[key]) : -1;
            }
            const int64_t idx_s = tid < nk ? (tile == 0 ? idx0_s : irow[tid]) : -1;
            uint4 v[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                v[i] = make_uint4(0u, 0u, 0u, 0u);
                if (idx[i] >= 0 && idx[i] < p.slots) {
                    const uint32_t blk = divu32((uint32_t)idx[i], p.bs_div);
                    const uint32_t off = (uint32_t)idx[i] - blk * (uint32_t)p.bs;
                    v[i] = *reinterpret_cast<const uint4 *>(p.cache + (int64_t)blk * p.c_sb + (int64_t)off * p.c_ss +
                                                             ch * 16);
                }
            }
            const bool ok_s = idx_s >= 0 && idx_s < p.slots;
            const float inv = ok_s ? bf16_lo((uint32_t)p.inv_scale[idx_s * p.s_ss]) : 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int key = (tid >> 5) + (NTH / 32) * i;
                if (key < nkb * 32) *reinterpret_cast<uint4 *>(&x_lds[key * XLD + ch * 16]) = v[i];
            }
            if (tid < KT) {
                admit[tid] = ok_s ? 1 : 0;
                inv_lds[tid] = inv;
            }
        }
        __syncthreads();

        // Scores of positions 32w .. 32w+31 (S^T blocks kb = 2w, 2w+1).
        float x[2][4];
        float mt = -INFINITY;
        // Admission and inverse scale of the lane's eight positions (keys
        // 16 (2w + h2) + 4 q4 + i), read as vectors: ahead of the MFMAs and
        // kept for P' in the two-group kernel; after them, and again for P',
        // in the one-group kernel, which has not the registers to hold them.
        constexpr bool EARLY = GPW == 2;
        int4 adm[2];
        float4 ivs[2];
        auto read_scales = [&](bool with_admit) __attribute__((always_inline)) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int key0 = 16 * (2 * w + h2) + 4 * q4;
                if (with_admit) adm[h2] = *reinterpret_cast<const int4 *>(&admit[key0]);
                ivs[h2] = *reinterpret_cast<const float4 *>(&inv_lds[key0]);
            }
        };
        if (w < nkb) {
            if constexpr (EARLY) read_scales(true);
            // The wave's two 16-position blocks side by side (two independent
            // accumulator chains); the operands of a group of depth steps are
            // read one group ahead of the MFMAs that use them, so no MFMA
            // waits on a read issued just before it.
            const uint8_t *xr0 = &x_lds[(32 * w + r) * XLD + 8 * q4];
            const uint8_t *xr1 = xr0 + 16 * XLD;
            f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
            constexpr int SG = GPW == 2 ? 4 : 2;   // depth steps per group (fewer registers at GPW = 1)
            constexpr int NG = 16 / SG;
            uint2 cb[2][2][SG];
#pragma unroll
            for (int i = 0; i < SG; ++i) {
                cb[0][0][i] = *reinterpret_cast<const uint2 *>(xr0 + 32 * i);
                cb[0][1][i] = *reinterpret_cast<const uint2 *>(xr1 + 32 * i);
            }
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                __builtin_amdgcn_sched_barrier(0);
                if (g + 1 < NG) {
#pragma unroll
                    for (int i = 0; i < SG; ++i) {
                        cb[(g + 1) & 1][0][i] = *reinterpret_cast<const uint2 *>(xr0 + 32 * (SG * (g + 1) + i));
                        cb[(g + 1) & 1][1][i] = *reinterpret_cast<const uint2 *>(xr1 + 32 * (SG * (g + 1) + i));
                    }
                }
#pragma unroll
                for (int i = 0; i < SG; ++i)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2)
                        acc[h2] = mfma16(fp8x8_to_bf16(cb[g & 1][h2][i].x, cb[g & 1][h2][i].y), qf[SG * g + i], acc[h2]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!EARLY) read_scales(true);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int a4[4] = {adm[h2].x, adm[h2].y, adm[h2].z, adm[h2].w};
                const float v4[4] = {ivs[h2].x, ivs[h2].y, ivs[h2].z, ivs[h2].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[h2][i] = a4[i] ? acc[h2][i] * p.sl2 * v4[i] : -INFINITY;
                    mt = fmaxf(mt, x[h2][i]);
                }
            }
        } else {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[h2][i] = -INFINITY;
        }
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        if (q4 == 0) red_max[w][r] = mt;
        __syncthreads();
        mt = fmaxf(fmaxf(red_max[0][r], red_max[1][r]), fmaxf(red_max[2][r], red_max[3][r]));
        const float M_new = fmaxf(M, mt);
        const float M_use = M_new == -INFINITY ? 0.f : M_new;
        const float alpha = exp2_fast(M - M_use);
        M = M_new;
        float psum = 0.f;
        if (w < nkb) {
            if constexpr (!EARLY) read_scales(false);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int key0 = 16 * (2 * w + h2) + 4 * q4;
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pv[i] = exp2_fast(x[h2][i] - M_use);
                    psum += pv[i];
                }
                uint2 pk;
                pk.x = pack_bf16(pv[0] * ivs[h2].x, pv[1] * ivs[h2].y);
                pk.y = pack_bf16(pv[2] * ivs[h2].z, pv[3] * ivs[h2].w);
                *reinterpret_cast<uint2 *>(&p_lds[r * PLD + key0]) = pk;
            }
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        if (q4 == 0) red_sum[w][r] = psum;
        __syncthreads();
        L = L * alpha + (red_sum[0][r] + red_sum[1][r] + red_sum[2][r] + red_sum[3][r]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int m = 0; m < 4; ++m) oacc[a][m] *= alpha;

        // O^T for dims 128w .. 128w+127: block (mb, mm) covers dims
        // 64mb + 4R + mm for A-row R.  The next 32-position block's operands
        // are read while this one's MFMAs run (reads past the tile's last
        // block stay inside the staged arrays and go unused).
        bf16x8_t bpb[2];
        uint32_t dwb[2][2][8];
        auto read_block = [&](int ks, int b) __attribute__((always_inline)) {
            bpb[b] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(&p_lds[r * PLD + 32 * ks + 8 * q4]));
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                const uint8_t *xc = &x_lds[(32 * ks + 8 * q4) * XLD + 64 * (2 * w + a) + 4 * r];
#pragma unroll
                for (int e = 0; e < 8; ++e) dwb[b][a][e] = *reinterpret_cast<const uint32_t *>(xc + e * XLD);
            }
        };
        // (The one-group kernel, at two workgroups per CU, has not the
        // registers for the second block's operands: it reads each block
        // just before its MFMAs.)
        constexpr bool AHEAD = GPW == 2;
        if constexpr (AHEAD) read_block(0, 0);
#pragma unroll
        for (int ks = 0; ks < KT / 32; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (AHEAD) {
                if (ks + 1 < KT / 32) read_block(ks + 1, (ks + 1) & 1);
            }
            if (ks < nkb) {
                if constexpr (!AHEAD) read_block(ks, ks & 1);
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const uint32_t *dw = dwb[ks & 1][a];
                    uint32_t lo[4], hi[4];
                    transpose4x4(dw[0], dw[1], dw[2], dw[3], lo);
                    transpose4x4(dw[4], dw[5], dw[6], dw[7], hi);
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm)
                        oacc[a][mm] = mfma16(fp8x8_to_bf16(lo[mm], hi[mm]), bpb[ks & 1], oacc[a][mm]);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    const float invL = L > 0.f ? 1.f / L : 0.f;
    uint16_t *orow = p.o + (int64_t)t * p.o_st + (int64_t)head * p.o_sh;
    // Lane (r, q4) holds dims 64 mb + 16 q4 + 4 i + mm of head r: 16
    // consecutive dims (32 bytes) per block mb = 2 w + a.  The output is not
    // read again here: non-temporal stores, 16 bytes each when the rows are
    // 16-byte aligned (8-byte pieces were written back to HBM as about 1.8x
    // the output's bytes).
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        uint32_t pk[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pk[2 * i] = pack_bf16(oacc[a][0][i] * invL, oacc[a][1][i] * invL);
            pk[2 * i + 1] = pack_bf16(oacc[a][2][i] * invL, oacc[a][3][i] * invL);
        }
        uint16_t *dst = orow + 64 * (2 * w + a) + 16 * q4;
        if (p.o16) {
            __builtin_nontemporal_store(u32x4{pk[0], pk[1], pk[2], pk[3]}, reinterpret_cast<u32x4 *>(dst));
            __builtin_nontemporal_store(u32x4{pk[4], pk[5], pk[6], pk[7]}, reinterpret_cast<u32x4 *>(dst + 8));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_nontemporal_store(u32x2{pk[2 * i], pk[2 * i + 1]}, reinterpret_cast<u32x2 *>(dst + 4 * i));
        }
    }
}

}  // namespace

hipError_t launch_swa(const SwaParams &p, hipStream_t stream) {
    if (p.T <= 0) return hipSuccess;
    const unsigned ngrp = (unsigned)(p.NH / 16);
    if (ngrp % 2 == 0)
        hipLaunchKernelGGL(swa_kernel<2>, dim3((unsigned)p.T * (ngrp / 2)), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL(swa_kernel<1>, dim3((unsigned)p.T * ngrp), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
