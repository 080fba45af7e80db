// kernels.hpp -- parameter blocks and launchers shared by the host entry
// points (api.hip) and the kernel translation units.  Library-internal.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Most block-table entries one decode split may span; the host keeps
// chunk / page_size + 1 within it (one LDS slice per wave).
constexpr int kDecodeMaxSplitPages = 512;

// Split-KV decode over one KV source (paged pool or contiguous strides).
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
    uint64_t ps_magic;  // ceil(2^32 / ps)
    const int32_t *kv_lens;  // NULL: every sequence has kv_len_const keys
    int kv_len_const;
    uint16_t *o;
    int64_t o_sb, o_sh;
    float *o_part;   // [S, B, Hq, D]     (S > 1)
    float *ml_part;  // [S, B, Hq, 2]     (S > 1)
    int B, Hq, Hkv, S, chunk;
    int direct;      // 1: single split writes the normalised bf16 output
    int HW;          // KV heads per wave (1, 2, 4, 8; divides Hkv)
    int units;       // B * (Hkv / HW) * S
    float sl2;       // scale * log2(e)
};

struct CombineParams {
    const float *o_part;   // [S, R, D]
    const float *ml_part;  // [S, R, 2]
    int S, R;
    // Optional per-row split count: rows r of sequence r / rows_per_seq use
    // max(1, ceil(kv_lens[seq] / chunk)) splits (capped at S).
    const int32_t *kv_lens;
    int kv_len_const;      // used when kv_lens == NULL and chunk > 0
    int chunk;             // 0: every row uses all S partials
    int rows_per_seq;
    // Outputs (any may be NULL).  Row r of the bf16 output sits at
    // out_bf16 + (r / rows_per_seq) * o_sb + (r % rows_per_seq) * o_sh.
    float *out_f32;
    uint16_t *out_bf16;
    int64_t o_sb, o_sh;
    float *lse;
};

// Ragged paged prefill (work-map tiles x groups of packed query heads).
struct PrefillParams {
    const uint16_t *q;
    int64_t q_st, q_sh;
    const int32_t *qo_indptr, *t2b, *t2i;
    int num_tiles;
    const uint16_t *k, *v;
    int64_t s_page, s_slot, s_head;
    const int32_t *bt;
    int64_t bt_sb;
    uint32_t ps;
    uint64_t ps_magic;
    const int32_t *kv_lens;
    const int32_t *causal;   // NULL: no causality
    const uint8_t *mask;     // NULL when mask_ndim == 0
    int mask_ndim;           // 0, 2 or 3
    int64_t m_sb, m_sq;
    uint16_t *o;
    int64_t o_st, o_sh;
    int B, Hq, Hkv, G;
    float sl2;               // scale * log2(e)
};

// Query heads one prefill workgroup packs (they share a KV head); a work-map
// tile then has 64 / prefill_heads_packed(G) rows.
int prefill_heads_packed(int G);

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
    float sl2;   // scale * log2(e)
};

hipError_t launch_decode(const DecodeParams &p, int D, int G, bool paged, hipStream_t stream);
hipError_t launch_swa(const SwaParams &p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream);
hipError_t launch_combine(const CombineParams &p, int D, hipStream_t stream);

}  // namespace pa
