// kernels.hpp -- parameter blocks and launchers shared by the host entry
// points (api.hip) and the kernel translation units.  Library-internal.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace pa {

// Most block-table entries one decode sub-piece may span; the host caps a
// sub-piece at (kDecodeMaxSplitPages - 2) * page_size tokens.
constexpr int kDecodeMaxSplitPages = 512;

// Split-KV decode over one KV source (paged pool or contiguous strides),
// balanced partition: rows r = (sequence, group of HW KV heads) laid end to
// end, W equal slices of the line, partial of row r in wave w at slot r + w.
struct DecodeParams {
    const uint16_t *q;
    int64_t q_sb, q_sh;
    const uint16_t *k, *v;
    // contiguous source: (b, g, j) -> b*sb + g*sh + j*sl
    int64_t k_sb, k_sh, k_sl, v_sb, v_sh, v_sl;
    // paged source: (page, slot, g) -> page*s_page + slot*s_slot + g*s_head
    int64_t s_page, s_slot, s_head;
    const int32_t *bt;
    int64_t bt_sb;
    uint32_t ps;
    DivU32 ps_div;      // exact division by ps
    const int32_t *kv_lens;  // NULL: every sequence has kv_len_const keys
    int kv_len_const;
    uint16_t *o;
    int64_t o_sb, o_sh;
    float *o_part;   // [(B + W) * Hq, D]   partial of slot s, local head i at row s*HW*G + i
    float *ml_part;  // [(B + W) * Hq, 2]
    int32_t *ranges; // [R, 2]: first and last wave holding keys of row r (NULL when W = 1)
    int B, Hq, Hkv;
    int G_all;       // Hq / Hkv; a row's pass covers the kernel's G of them
    int passes;      // G_all / G: rows per (sequence, KV head); > 1 only with HW = 1
    int HW;          // KV heads per row (1, 2, 4, 8; divides Hkv)
    int ngrp;        // rows per sequence: Hkv / HW * passes
    int R;           // B * ngrp rows
    int W;           // slices of the line (one workgroup each)
    int NW;          // waves per workgroup: 1, or 4 (alternate tiles, merged in LDS; G <= 4)
    int NB;          // > 0: MFMA kernel with NB blocks of 16 query-head rows (decode_mfma.hip)
    int max_sub;     // longest sub-piece (tokens) one LDS page slice covers
    int direct;      // 1: a row covered by one piece is written normalised
    float sl2;       // scale * log2(e)
};

// Combine of the balanced partition (one wave per sequence x query head).
struct DecodeCombineParams {
    const float *o_part, *ml_part;
    const int32_t *ranges;   // [R, 2] first / last wave of each row with keys (unused when W = 1)
    const int32_t *kv_lens;
    int kv_len_const;
    int B, Hq, ngrp, R, W;
    int direct_single;   // 1: single-piece rows were written by the split kernel
    uint16_t *o;
    int64_t o_sb, o_sh;
};

// Generic combine: row r merges partials s*R + r, s = 0..S-1.
struct CombineParams {
    const float *o_part;   // [S, R, D]
    const float *ml_part;  // [S, R, 2]
    int S, R;
    float *out_f32;        // NULL or [R, D]
    uint16_t *out_bf16;    // NULL or [R, D]
    float *lse;            // NULL or [R]
};

// Ragged paged prefill (work-map tiles x groups of packed query heads).
// Prefill: packed ragged Q through a work map with a paged KV source, or the
// dense schedule (dense_lq rows per sequence, batch strides q_sb / o_sb) with
// a contiguous KV source (bt == NULL: key j of sequence b, head g at
// b*k_sb + g*s_head + j*s_slot).
struct PrefillParams {
    const uint16_t *q;
    int64_t q_sb, q_st, q_sh;
    const int32_t *qo_indptr, *t2b, *t2i;
    int num_tiles;
    int dense_lq;            // > 0: dense schedule, no work map
    const uint16_t *k, *v;
    int64_t k_sb, s_page, s_slot, s_head;
    const int32_t *bt;       // NULL: contiguous source
    int64_t bt_sb;
    uint32_t ps;
    DivU32 ps_div;
    const int32_t *kv_lens;  // NULL: kv_len_const for every sequence
    int kv_len_const;
    const int32_t *causal;   // causal offsets (-1 = off), or NULL
    int causal_br;           // with causal NULL: bottom-right causality (c = n - Lq)
    const uint8_t *mask;     // NULL when mask_ndim == 0
    int mask_ndim;           // 0, 2 or 3
    int64_t m_sb, m_sq;
    uint16_t *o;
    int64_t o_sb, o_st, o_sh;
    int B, Hq, Hkv, G;
    float sl2;               // scale * log2(e)
    // Split KV: with kv_splits > 1 each workgroup takes an equal share (in
    // 64-key tiles) of its tile's keys and writes an unnormalised partial
    // for split s, query row t (packed row, or b * dense_lq + i), head h at
    // row (s * part_rows + t) * Hq + h of o_part [.., D] and ml_part [.., 2]
    // (m in natural-log units of the scaled score, l); rows t >= part_rows
    // are not written.
    int kv_splits;
    int part_rows;
    float *o_part, *ml_part;
    int teams;               // 1 or 2 teams of four waves per workgroup (2 only for D <= 128)
};

// Query heads HP one prefill workgroup packs (they share a KV head): the
// largest power of two dividing G, at most 8 (4 at D = 256), so all G heads
// for G in {1, 2, 4, 8}; G / HP workgroups then cover a KV head.  Rows of a
// work-map tile: for D <= 128, 32 per wave, 128 / HP for HP <= 4 and 16 for
// HP = 8 (each wave then takes two heads of the same 16 rows); for D = 256,
// 16 per wave of one team, 64 / HP.
int prefill_heads_packed(int G, int D);
int prefill_tile_rows(int G, int D);

// Combine of split-KV prefill partials: one wave per (query row, head).
struct PrefillCombineParams {
    const float *o_part, *ml_part;
    int S, rows, Hq;
    int dense_lq;            // > 0: row t is (b, i) = (t / dense_lq, t % dense_lq)
    uint16_t *o;
    int64_t o_sb, o_st, o_sh;
};

// fp8 sliding-window decode (K = V), head dim 512, 16-head groups.
struct SwaParams {
    const uint16_t *q;
    int64_t q_st, q_sh;
    const uint8_t *cache;
    int64_t c_sb, c_ss;
    const uint16_t *inv_scale;
    int64_t s_ss;
    const int64_t *ind;
    int64_t i_st;
    const int64_t *lens;
    uint16_t *o;
    int64_t o_st, o_sh;
    int T, NH, W, bs;
    int slots;            // num_blocks * bs: indices at or above it are not admitted
    DivU32 bs_div;        // slot -> (block, offset): exact division by bs
    float sl2;            // scale * log2(e)
    int o16;              // output rows 16-byte aligned: 16-byte stores
};

// Paged KV append: packed new rows [N, Hkv, D] into their (page, slot).
struct KvAppendParams {
    const uint16_t *k_new, *v_new;
    int64_t n_st, n_sh;
    const int32_t *indptr, *start_pos;
    uint16_t *k_pool, *v_pool;
    int64_t s_page, s_slot, s_head;
    const int32_t *bt;
    int64_t bt_sb;
    int B, Hkv, D, ps, N, num_pages;
};

// fp8 quantize-on-write of sliding-window cache rows (HD = 512).
struct SwaQuantParams {
    const uint16_t *x;
    int64_t x_st;
    const int64_t *slots;
    const float *mult;     // NULL: 448 / amax per row
    uint8_t *cache;
    int64_t c_sb, c_ss;
    uint16_t *inv_scale;
    int64_t s_ss;
    float *amax;           // NULL: not reported
    int N, bs;
    int64_t num_slots;
    DivU32 bs_div;
};

// Rotary embedding of x [T, H, D] by fp32 cos / sin tables at positions.
struct RotaryParams {
    const uint16_t *x;
    int64_t x_st, x_sh;
    uint16_t *out;
    int64_t o_st, o_sh;
    const float *cos, *sin;
    int64_t tab_st;
    const int32_t *pos;
    int T, H, D, rows;
};

hipError_t launch_decode(const DecodeParams &p, int D, int G, bool paged, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams &p, int D, bool paged, hipStream_t stream);
hipError_t launch_swa(const SwaParams &p, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendParams &p, hipStream_t stream);
hipError_t launch_swa_quantize(const SwaQuantParams &p, hipStream_t stream);
hipError_t launch_rotary(const RotaryParams &p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, int D, hipStream_t stream);
hipError_t launch_prefill_combine(const PrefillCombineParams &p, int D, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeCombineParams &p, int D, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, int D, hipStream_t stream);
hipError_t launch_stream_read(const void *buf, uint64_t bytes, uint32_t *sink, int workgroups, hipStream_t stream);

}  // namespace pa
