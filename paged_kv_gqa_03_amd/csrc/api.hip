// api.hip -- the C ABI declared in include/paged_attn.h: argument checks,
// the split planner, the ragged work map, workspace layout and launches.
// Every check runs before anything is enqueued; nothing here allocates
// device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "paged_attn.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return ATTN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool mult8(int64_t s) { return (s & 7) == 0; }

int launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(ATTN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Compute units of the current device, queried once per device.
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64 && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

constexpr int kMaxWaves = 1 << 16;     // upper bound on decode slices (num_splits)
// One-wave slices (group sizes above 4): waves per CU the planner aims at,
// three when a wave streams whole 2 KB token rows (eight KV heads), two when
// it streams one head (measured best for each on MI355X with non-temporal
// K/V loads).
constexpr int kWavesPerCuRows = 3;
constexpr int kWavesPerCuHead = 2;
constexpr int kMinSliceTokens = 64;    // shortest one-wave slice, in tokens of a row
// Four-wave slices (group sizes up to 4), one workgroup per CU at most: with
// eight KV heads per row, slices on three quarters of the CUs (768 waves;
// swept on MI355X, B = 128 and B = 32 over kv U[512, 4096]: 192 slices
// 195.6 / 60.4 us per call against 200.9 / 60.9 at 256 and 210 / 66 for 512
// slices, which put two workgroups on some CUs); with one head per row, one
// slice per CU.
constexpr int kSlicesPerCu4Rows_num = 3, kSlicesPerCu4Rows_den = 4;
constexpr int kMinSliceTokens4 = 256;  // shortest four-wave slice, in tokens of a row

// Waves per decode slice (one workgroup each): four take alternate tiles of
// every piece and merge their states in LDS, so the fp32 partials (one per
// piece) are four times fewer than with one-wave slices of the same total
// wave count; the kernel is built for that up to Gk = 4 query heads a pass.
int decode_waves_per_slice(int Gk) { return Gk <= 4 ? 4 : 1; }
constexpr int kMaxPrefillSplits = 256; // upper bound on prefill KV splits
constexpr int kPrefillWgPerCu = 1;     // prefill workgroups resident per CU (512 threads, up to 159 KB LDS)
constexpr int kMinSplitKeyTiles = 8;   // fewest 64-key tiles the prefill planner gives one split

// KV heads one decode wave covers: with the heads of a token adjacent in
// memory (head stride == D) a wave takes up to 8 of them (4 at D = 256,
// where 16 lanes share a head row) so each token's rows form one contiguous
// read; otherwise one head, whose tokens are then the contiguous direction.
int heads_per_wave(int Hkv, int64_t kv_s_head, int D) {
    if (kv_s_head != D) return 1;
    int hw = D == 256 ? 4 : 8;
    while (hw > 1 && Hkv % hw != 0) hw >>= 1;
    return hw;
}

// Longest sub-piece (tokens) whose block-table slice fits the kernel's LDS
// slice: c tokens span at most (c - 1) / ps + 2 pages.
int max_sub_piece(int page_size) {
    if (page_size <= 0) return 1 << 30;
    const long c = (long)(pa::kDecodeMaxSplitPages - 2) * page_size;
    return (int)(c > (1L << 30) ? (1L << 30) : c);
}

bool decode_dim(int D) { return D == 32 || D == 64 || D == 128 || D == 256; }

// Prefill takes any group size: a workgroup packs the largest power of two
// (at most 8) dividing G, and G / that many workgroups share a KV head.
int check_prefill_heads(int Hq, int Hkv, int *G) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
    *G = Hq / Hkv;
    return ATTN_OK;
}

int check_heads(int Hq, int Hkv, int *G) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
        return fail(ATTN_ERR_INVALID_ARG, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
    *G = Hq / Hkv;
    return ATTN_OK;
}

// Decode row layout for group size G.  Head dims 64 and 128 with G other
// than 1, 2 or 4 run the MFMA kernel: a KV head contributes Gk query heads
// to a row (the largest divisor of G that is at most 32, on NB = ceil(Gk /
// 16) blocks of 16 MFMA rows), G / Gk passes per KV head, and with one pass
// a row holds HW = 4 (else 2, else 1) adjacent KV heads, one wave each, so a
// workgroup reads those heads of each token together.  Otherwise the VALU
// kernel is built for Gk query heads per pass (the largest power of two
// dividing G, at most 8) and a (sequence, KV head) takes G / Gk passes, each
// a row of its own that streams the KV head again; with one pass, a row may
// hold HW > 1 adjacent KV heads.
struct DecodeLayout {
    int Gk, passes, HW, ngrp, NB;
};

DecodeLayout decode_layout(int Hkv, int G, int64_t kv_s_head, int D) {
    DecodeLayout L;
    if ((D == 64 || D == 128) && G != 1 && G != 2 && G != 4) {
        int gm = G < 32 ? G : 32;
        while (G % gm != 0) --gm;
        L.Gk = gm;
        L.passes = G / gm;
        L.HW = L.passes > 1 ? 1 : Hkv % 4 == 0 ? 4 : Hkv % 2 == 0 ? 2 : 1;
        L.ngrp = Hkv / L.HW * L.passes;
        L.NB = (gm + 15) / 16;
        return L;
    }
    L.NB = 0;
    L.Gk = (G & -G) < 8 ? (G & -G) : 8;
    L.passes = G / L.Gk;
    L.HW = L.passes > 1 ? 1 : heads_per_wave(Hkv, kv_s_head, D);
    L.ngrp = Hkv / L.HW * L.passes;
    return L;
}

// Workspace: o_part [(B + W) * Hq, D] f32, then ml_part [(B + W) * Hq, 2] f32
// at the next 256-byte boundary.  Partial of slot s (row r + wave w), local
// query head i of the row, sits at row s * heads_per_row + i < (B + W) * Hq.
size_t ws_rows(int B, int Hq, int W) { return ((size_t)B + (size_t)W) * (size_t)Hq; }
size_t ws_ml_offset(int B, int Hq, int D, int W) {
    const size_t o_bytes = ws_rows(B, Hq, W) * D * sizeof(float);
    return (o_bytes + 255) & ~(size_t)255;
}

// Row ranges after ml_part: int32 [B * Hq, 2] (rows per sequence <= Hq).
size_t ws_range_offset(int B, int Hq, int D, int W) {
    const size_t end = ws_ml_offset(B, Hq, D, W) + ws_rows(B, Hq, W) * 2 * sizeof(float);
    return (end + 255) & ~(size_t)255;
}

int check_workspace(const void *workspace, size_t workspace_bytes, int B, int Hq, int D, int W) {
    const size_t need = attn_decode_workspace_bytes(B, Hq, D, W);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "decode with %d slices needs %zu workspace bytes, got %zu", W, need,
                    workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return ATTN_OK;
}

pa::DecodeCombineParams combine_params(const void *workspace, int B, int Hq, int D, int W, int ngrp,
                                       const int32_t *kv_lens, int kv_len_const, void *o, int64_t o_sb,
                                       int64_t o_sh, int direct_single) {
    pa::DecodeCombineParams c{};
    c.o_part = static_cast<const float *>(workspace);
    c.ml_part = reinterpret_cast<const float *>(static_cast<const char *>(workspace) + ws_ml_offset(B, Hq, D, W));
    c.ranges = workspace ? reinterpret_cast<const int32_t *>(static_cast<const char *>(workspace) +
                                                              ws_range_offset(B, Hq, D, W))
                         : nullptr;
    c.kv_lens = kv_lens;
    c.kv_len_const = kv_len_const;
    c.B = B;
    c.Hq = Hq;
    c.ngrp = ngrp;
    c.R = B * c.ngrp;
    c.W = W;
    c.direct_single = direct_single;
    c.o = static_cast<uint16_t *>(o);
    c.o_sb = o_sb;
    c.o_sh = o_sh;
    return c;
}

// Decode workspace of attn_paged_decode_noalloc: a static device array, one
// copy per device, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): it looks up each device's address once with hipGetSymbolAddress
// and passes that.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Address of this device's copy of `scratch` (looked up on the first call on
// the device, with the device current), or nullptr with *rc set.
void *scratch_address(int *rc) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return *rc = fail(ATTN_ERR_LAUNCH, "attn_paged_decode_noalloc: no current HIP device"), nullptr;
    if (dev >= kMaxDevices)
        return *rc = fail(ATTN_ERR_UNSUPPORTED, "attn_paged_decode_noalloc: device %d beyond %d", dev, kMaxDevices),
               nullptr;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return *rc = fail(ATTN_ERR_LAUNCH, "attn_paged_decode_noalloc: hipGetSymbolAddress: %s",
                              hipGetErrorString(e)), nullptr;
        addr[dev] = ptr;
    }
    return addr[dev];
}

// Shared tail of the decode entry points: partition, workspace, launches.
// mode 0: split kernel (direct writes on) + combine;
// mode 1: split kernel only, every piece written as an fp32 partial.
int run_decode(pa::DecodeParams &p, int D, int G, bool paged, int max_kv_len, int num_splits,
               void *workspace, size_t workspace_bytes, int page_size, int64_t kv_s_head, hipStream_t stream,
               int mode) {
    const DecodeLayout L = decode_layout(p.Hkv, G, kv_s_head, D);
    int W = num_splits;
    if (W == 0) {
        W = attn_plan_splits(p.B, p.Hkv, G, D, max_kv_len, page_size, kv_s_head, 0);
        if (W < 0) return W;
        // One length for every row: when the rows number between half the
        // planned count and the count, one slice per row leaves the planned
        // waves at least half busy and needs no combine (contiguous decode
        // B = 16, 128 rows of 2048 keys: 30.3 against 31.1-31.9 us per call
        // at 256 slices on MI355X).
        const int64_t rows = (int64_t)p.B * L.ngrp;
        if (mode == 0 && !p.kv_lens && p.kv_len_const > 0 && rows <= W && 2 * rows >= W) W = (int)rows;
    }
    if (W < 1 || W > kMaxWaves) return fail(ATTN_ERR_INVALID_ARG, "num_splits %d outside [1, %d]", W, kMaxWaves);
    p.G_all = G;
    p.passes = L.passes;
    p.HW = L.HW;
    p.ngrp = L.ngrp;
    p.R = p.B * p.ngrp;
    p.W = W;
    p.NB = L.NB;
    p.NW = L.NB ? 4 : decode_waves_per_slice(L.Gk);
    if ((int64_t)p.R * (int64_t)max_kv_len >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "decode: rows * max_kv_len must stay below 2^31 tokens");
    if ((int64_t)p.B * p.Hq >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "decode: B * Hq must stay below 2^31");
    p.max_sub = max_sub_piece(paged ? page_size : 0);
    p.direct = mode == 0 ? 1 : 0;
    if (mode == 1 || W > 1) {
        const int rc = check_workspace(workspace, workspace_bytes, p.B, p.Hq, D, W);
        if (rc) return rc;
        p.o_part = static_cast<float *>(workspace);
        p.ml_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + ws_ml_offset(p.B, p.Hq, D, W));
        p.ranges = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + ws_range_offset(p.B, p.Hq, D, W));
    }
    if (p.B == 0) return ok();
    hipError_t e = L.NB ? pa::launch_decode_mfma(p, D, paged, stream) : pa::launch_decode(p, D, L.Gk, paged, stream);
    if (e != hipSuccess) return launch_status(e, "decode split kernel");
    // One length for every row (no kv_lens), not zero, and W dividing R:
    // every slice boundary falls on a row boundary, so each row lies in one
    // slice and was written directly; nothing is left to combine.
    const bool whole_rows = !p.kv_lens && p.kv_len_const > 0 && p.R % W == 0;
    if (mode == 0 && !whole_rows) {
        // Rows spanning several slices are merged; empty rows are zeroed;
        // rows written directly are left alone.
        pa::DecodeCombineParams c = combine_params(workspace, p.B, p.Hq, D, W, p.ngrp, p.kv_lens,
                                                   p.kv_len_const, p.o, p.o_sb, p.o_sh, 1);
        e = pa::launch_decode_combine(c, D, stream);
        if (e != hipSuccess) return launch_status(e, "combine kernel");
    }
    return ok();
}

}  // namespace

extern "C" {

const char *attn_last_error(void) { return g_err.c_str(); }

int attn_version(void) { return 100; }

int attn_plan_splits(int B, int Hkv, int G, int D, int max_kv_len, int page_size, int64_t kv_s_head,
                     int num_cus) {
    if (B < 0 || Hkv <= 0 || G <= 0 || D <= 0 || max_kv_len < 0 || page_size < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_plan_splits: bad sizes");
    if (num_cus <= 0) {
        num_cus = device_cus();
        if (num_cus <= 0) return fail(ATTN_ERR_LAUNCH, "attn_plan_splits: cannot query the device");
    }
    const DecodeLayout L = decode_layout(Hkv, G, kv_s_head, D);
    const int hw = L.HW;
    const long rows = (long)B * L.ngrp;
    const long line = rows * (long)max_kv_len;   // upper bound on the tokens of all rows
    const bool four = L.NB > 0 || decode_waves_per_slice(L.Gk) == 4;
    const long min_slice = four ? kMinSliceTokens4 : kMinSliceTokens;
    long W = (line + min_slice - 1) / min_slice;
    long cap;
    if (four) cap = hw == 8 ? ((long)num_cus * kSlicesPerCu4Rows_num + kSlicesPerCu4Rows_den - 1) / kSlicesPerCu4Rows_den
                            : (long)num_cus;
    else cap = (long)num_cus * (hw == 8 ? kWavesPerCuRows : kWavesPerCuHead);
    if (W > cap) W = cap;
    if (W > kMaxWaves) W = kMaxWaves;
    if (W < 1) W = 1;
    return (int)W;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
    if (B <= 0 || Hq <= 0 || D <= 0 || num_splits < 1) return 0;
    return ws_range_offset(B, Hq, D, num_splits) + (size_t)B * (size_t)Hq * 2 * sizeof(int32_t);
}

int attn_decode(const void *q, int64_t q_sb, int64_t q_sh,
                const void *k, int64_t k_sb, int64_t k_sh, int64_t k_sl,
                const void *v, int64_t v_sb, int64_t v_sh, int64_t v_sl,
                void *o, int64_t o_sb, int64_t o_sh,
                const int32_t *kv_lens, int kv_len,
                int B, int Hq, int Hkv, int D, float scale, int num_splits,
                void *workspace, size_t workspace_bytes, void *stream) {
    int G = 0, rc = check_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (B < 0 || kv_len < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_decode: negative B or kv_len");
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: head dim %d not built (32, 64, 128, 256)", D);
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "attn_decode: null tensor pointer");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_decode: scale is not finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        !mult8(q_sb) || !mult8(q_sh) || !mult8(k_sb) || !mult8(k_sh) || !mult8(k_sl) ||
        !mult8(v_sb) || !mult8(v_sh) || !mult8(v_sl) || !mult8(o_sb) || !mult8(o_sh))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: rows must be 16-byte aligned (pointers, strides %% 8)");
    if (k_sl < 0 || v_sl < 0 || (int64_t)kv_len * (k_sl > v_sl ? k_sl : v_sl) >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: kv_len * position stride must stay below 2^31");
    pa::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_sb = q_sb; p.q_sh = q_sh;
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.k_sb = k_sb; p.k_sh = k_sh; p.k_sl = k_sl;
    p.v_sb = v_sb; p.v_sh = v_sh; p.v_sl = v_sl;
    p.kv_lens = kv_lens;
    p.kv_len_const = kv_len;
    p.o = static_cast<uint16_t *>(o);
    p.o_sb = o_sb; p.o_sh = o_sh;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv;
    p.sl2 = scale * 1.4426950408889634f;
    // Any heads-per-wave choice is correct for any strides; it only decides
    // which direction one load instruction reads contiguously.
    return run_decode(p, D, G, false, kv_len, num_splits, workspace, workspace_bytes, 0, k_sh,
                      static_cast<hipStream_t>(stream), 0);
}

static int paged_decode_impl(const void *q, int64_t q_sb, int64_t q_sh,
                             const void *k_pool, const void *v_pool,
                             int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                             const int32_t *block_table, int64_t bt_sb,
                             const int32_t *kv_lens, int max_kv_len,
                             void *o, int64_t o_sb, int64_t o_sh,
                             int B, int Hq, int Hkv, int D, int page_size, float scale,
                             int num_splits, void *workspace, size_t workspace_bytes,
                             void *stream, int mode) {
    const char *fn = mode ? "attn_paged_decode_split" : "attn_paged_decode";
    int G = 0, rc = check_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (B < 0 || max_kv_len < 0) return fail(ATTN_ERR_INVALID_ARG, "%s: negative B or max_kv_len", fn);
    if (page_size <= 0) return fail(ATTN_ERR_INVALID_ARG, "%s: page_size must be >= 1", fn);
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d not built (32, 64, 128, 256)", fn, D);
    if (!q || !k_pool || !v_pool || (!o && mode == 0) || !block_table || !kv_lens)
        return fail(ATTN_ERR_INVALID_ARG, "%s: null pointer", fn);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "%s: scale is not finite", fn);
    if (bt_sb < 0) return fail(ATTN_ERR_INVALID_ARG, "%s: negative block-table stride", fn);
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) ||
        !mult8(q_sb) || !mult8(q_sh) || !mult8(kv_s_page) || !mult8(kv_s_slot) || !mult8(kv_s_head) ||
        !mult8(o_sb) || !mult8(o_sh))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: rows must be 16-byte aligned (pointers, strides %% 8)", fn);
    if (kv_s_page < 0 || kv_s_slot < 0 || kv_s_head < 0 || kv_s_page >= (1ll << 32) ||
        (int64_t)(page_size - 1) * kv_s_slot + (int64_t)(Hkv - 1) * kv_s_head + D >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: pool strides exceed the 32-bit page/slot addressing", fn);
    pa::DecodeParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_sb = q_sb; p.q_sh = q_sh;
    p.k = static_cast<const uint16_t *>(k_pool);
    p.v = static_cast<const uint16_t *>(v_pool);
    p.s_page = kv_s_page; p.s_slot = kv_s_slot; p.s_head = kv_s_head;
    p.bt = block_table;
    p.bt_sb = bt_sb;
    p.ps = (uint32_t)page_size;
    p.ps_div = pa::make_divu32((uint32_t)page_size);
    p.kv_lens = kv_lens;
    p.o = static_cast<uint16_t *>(o);
    p.o_sb = o_sb; p.o_sh = o_sh;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv;
    p.sl2 = scale * 1.4426950408889634f;
    return run_decode(p, D, G, true, max_kv_len, num_splits, workspace, workspace_bytes, page_size, kv_s_head,
                      static_cast<hipStream_t>(stream), mode);
}

int attn_paged_decode(const void *q, int64_t q_sb, int64_t q_sh,
                      const void *k_pool, const void *v_pool,
                      int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                      const int32_t *block_table, int64_t bt_sb,
                      const int32_t *kv_lens, int max_kv_len,
                      void *o, int64_t o_sb, int64_t o_sh,
                      int B, int Hq, int Hkv, int D, int page_size, float scale,
                      int num_splits, void *workspace, size_t workspace_bytes,
                      void *stream) {
    return paged_decode_impl(q, q_sb, q_sh, k_pool, v_pool, kv_s_page, kv_s_slot, kv_s_head, block_table,
                             bt_sb, kv_lens, max_kv_len, o, o_sb, o_sh, B, Hq, Hkv, D, page_size, scale,
                             num_splits, workspace, workspace_bytes, stream, 0);
}

int attn_paged_decode_noalloc(const void *q, int64_t q_sb, int64_t q_sh,
                              const void *k_pool, const void *v_pool,
                              int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                              const int32_t *block_table, int64_t bt_sb,
                              const int32_t *kv_lens, int max_kv_len,
                              void *o, int64_t o_sb, int64_t o_sh,
                              int B, int Hq, int Hkv, int D, int page_size, float scale,
                              int num_splits, void *stream) {
    const size_t cap = ATTN_NOALLOC_SCRATCH_BYTES;
    int W = num_splits;
    const bool plannable = B > 0 && Hkv > 0 && Hq > 0 && Hq % Hkv == 0 && decode_dim(D) && max_kv_len >= 0 &&
                           page_size > 0;
    if (W == 0 && plannable) {
        W = attn_plan_splits(B, Hkv, Hq / Hkv, D, max_kv_len, page_size, kv_s_head, 0);
        if (W < 0) return W;
        // The planner's count, lowered to the largest whose partials fit the
        // static buffer (one slice needs no workspace at all).
        if (attn_decode_workspace_bytes(B, Hq, D, W) > cap) {
            int lo = 1, hi = W;
            while (lo < hi) {
                const int mid = lo + (hi - lo + 1) / 2;
                if (attn_decode_workspace_bytes(B, Hq, D, mid) <= cap) lo = mid;
                else hi = mid - 1;
            }
            W = lo;
        }
    } else if (W > 1 && plannable && attn_decode_workspace_bytes(B, Hq, D, W) > cap) {
        return fail(ATTN_ERR_UNSUPPORTED,
                    "attn_paged_decode_noalloc: %d slices need %zu bytes of partials, above the %zu-byte static "
                    "scratch buffer", W, attn_decode_workspace_bytes(B, Hq, D, W), cap);
    }
    void *ws = nullptr;
    if (W > 1 && plannable) {
        int rc = ATTN_OK;
        ws = scratch_address(&rc);
        if (!ws) return rc;
    }
    return paged_decode_impl(q, q_sb, q_sh, k_pool, v_pool, kv_s_page, kv_s_slot, kv_s_head, block_table, bt_sb,
                             kv_lens, max_kv_len, o, o_sb, o_sh, B, Hq, Hkv, D, page_size, scale, W, ws,
                             ws ? cap : 0, stream, 0);
}

int attn_paged_decode_split(const void *q, int64_t q_sb, int64_t q_sh,
                            const void *k_pool, const void *v_pool,
                            int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                            const int32_t *block_table, int64_t bt_sb,
                            const int32_t *kv_lens, int max_kv_len,
                            int B, int Hq, int Hkv, int D, int page_size, float scale,
                            int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    const void *o_dummy = q;  // never written in split-only mode; keeps the shared checks uniform
    return paged_decode_impl(q, q_sb, q_sh, k_pool, v_pool, kv_s_page, kv_s_slot, kv_s_head, block_table,
                             bt_sb, kv_lens, max_kv_len, const_cast<void *>(o_dummy), q_sb, q_sh, B, Hq, Hkv,
                             D, page_size, scale, num_splits, workspace, workspace_bytes, stream, 1);
}

int attn_decode_combine(const void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int D,
                        int num_splits, int64_t kv_s_head, const int32_t *kv_lens, int max_kv_len, void *o,
                        int64_t o_sb, int64_t o_sh, void *stream) {
    int G = 0, rc = check_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (B < 0 || max_kv_len < 0 || num_splits < 1 || num_splits > kMaxWaves)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode_combine: bad sizes");
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_combine: head dim %d not built", D);
    if (!o) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_combine: null output");
    if (!aligned16(o) || !mult8(o_sb) || !mult8(o_sh))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_combine: output rows must be 16-byte aligned");
    rc = check_workspace(workspace, workspace_bytes, B, Hq, D, num_splits);
    if (rc) return rc;
    if (B == 0) return ok();
    const DecodeLayout L = decode_layout(Hkv, G, kv_s_head, D);
    pa::DecodeCombineParams c = combine_params(workspace, B, Hq, D, num_splits, L.ngrp, kv_lens, max_kv_len, o,
                                               o_sb, o_sh, 0);
    return launch_status(pa::launch_decode_combine(c, D, static_cast<hipStream_t>(stream)), "combine kernel");
}

int attn_split_combine(const float *o_part, const float *ml_part, int S, int R, int D,
                       float *out_f32, void *out_bf16, float *lse, void *stream) {
    if (S < 1 || R < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_split_combine: bad S or R");
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_split_combine: head dim %d not built", D);
    if (!o_part || !ml_part) return fail(ATTN_ERR_INVALID_ARG, "attn_split_combine: null partials");
    if (!out_f32 && !out_bf16 && !lse) return fail(ATTN_ERR_INVALID_ARG, "attn_split_combine: no output");
    if (((uintptr_t)ml_part & 7u) || ((uintptr_t)o_part & 7u) || (out_bf16 && ((uintptr_t)out_bf16 & 3u)))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_split_combine: misaligned buffers");
    pa::CombineParams c{};
    c.o_part = o_part;
    c.ml_part = ml_part;
    c.S = S;
    c.R = R;
    c.out_f32 = out_f32;
    c.out_bf16 = static_cast<uint16_t *>(out_bf16);
    c.lse = lse;
    return launch_status(pa::launch_combine(c, D, static_cast<hipStream_t>(stream)), "combine kernel");
}

int attn_prefill_plan(const int32_t *q_lens_host, int B, int tile_rows,
                      int32_t *qo_indptr_host, int32_t *tile_to_batch_host,
                      int32_t *tile_to_index_host, int cap, int *num_tiles) {
    if (B < 0 || tile_rows <= 0 || !qo_indptr_host || !num_tiles || (B > 0 && !q_lens_host))
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_plan: bad arguments");
    int t = 0;
    qo_indptr_host[0] = 0;
    for (int b = 0; b < B; ++b) {
        if (q_lens_host[b] < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_plan: negative q_len");
        qo_indptr_host[b + 1] = qo_indptr_host[b] + q_lens_host[b];
        const int tiles = (q_lens_host[b] + tile_rows - 1) / tile_rows;
        for (int i = 0; i < tiles; ++i) {
            if (t >= cap) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_plan: more than cap=%d tiles", cap);
            tile_to_batch_host[t] = b;
            tile_to_index_host[t] = i;
            ++t;
        }
    }
    *num_tiles = t;
    return ok();
}

int attn_prefill_tile_rows(int D, int G) {
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_tile_rows: head dim %d not built (32, 64, 128, 256)", D);
    if (G < 1) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_tile_rows: group size %d", G);
    return pa::prefill_tile_rows(G, D);
}

}  // extern "C"

namespace {

// Split-KV prefill workspace: o_part [S, rows, Hq, D] f32, then ml_part
// [S, rows, Hq, 2] f32 at the next 256-byte boundary.
size_t pf_ml_offset(int rows, int Hq, int D, int S) {
    const size_t o_bytes = (size_t)S * (size_t)rows * (size_t)Hq * (size_t)D * sizeof(float);
    return (o_bytes + 255) & ~(size_t)255;
}

// Checks the split arguments and fills the split fields of p; S == 1 needs
// no workspace.  rows: query rows the partials hold.
int prefill_split_setup(pa::PrefillParams &p, const char *who, int rows, int Hq, int D, int S, void *workspace,
                        size_t workspace_bytes) {
    if (S < 1 || S > kMaxPrefillSplits)
        return fail(ATTN_ERR_INVALID_ARG, "%s: num_splits %d outside [1, %d]", who, S, kMaxPrefillSplits);
    if (rows < 0) return fail(ATTN_ERR_INVALID_ARG, "%s: negative row count", who);
    p.kv_splits = S;
    p.part_rows = rows;
    if (S == 1) return ATTN_OK;
    const size_t need = attn_prefill_workspace_bytes(rows, Hq, D, S);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "%s with %d splits needs %zu workspace bytes, got %zu", who, S, need,
                    workspace ? workspace_bytes : (size_t)0);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", who);
    if ((int64_t)S * rows * Hq >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: num_splits * rows * Hq must stay below 2^31", who);
    p.o_part = static_cast<float *>(workspace);
    p.ml_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + pf_ml_offset(rows, Hq, D, S));
    return ATTN_OK;
}

// Teams per prefill workgroup.  One team uses half the LDS, so two
// independent workgroups share a CU and their waves' MFMA and softmax
// phases overlap: measured on MI355X 5-10% faster on ragged and dense
// prefill, even on grids of about one workgroup per CU.  Two teams halve a
// workgroup's serial walk over the keys and keep twice the K/V loads in
// flight, which wins only on grids of a few long walks (short query runs
// over long contexts, split or not).  Hence: two teams when the grid before
// any KV split holds at most one workgroup per two CUs.  D = 256 always runs
// one team.
int prefill_teams_for(int64_t base_workgroups, int D) {
    if (D > 128) return 1;
    const int cus = device_cus();
    return (cus > 0 && 2 * base_workgroups <= cus) ? 2 : 1;
}

// Split kernel, then (S > 1) the combine into o.
int run_prefill(pa::PrefillParams &p, int D, hipStream_t stream) {
    const int64_t base = (int64_t)p.num_tiles * p.Hkv * (p.G / pa::prefill_heads_packed(p.G, D));
    p.teams = prefill_teams_for(base, D);
    hipError_t e = pa::launch_prefill(p, D, stream);
    if (e != hipSuccess) return launch_status(e, "prefill kernel");
    if (p.kv_splits > 1) {
        pa::PrefillCombineParams c{};
        c.o_part = p.o_part;
        c.ml_part = p.ml_part;
        c.S = p.kv_splits;
        c.rows = p.part_rows;
        c.Hq = p.Hq;
        c.dense_lq = p.dense_lq;
        c.o = p.o;
        c.o_sb = p.o_sb; c.o_st = p.o_st; c.o_sh = p.o_sh;
        e = pa::launch_prefill_combine(c, D, stream);
        if (e != hipSuccess) return launch_status(e, "prefill combine kernel");
    }
    return ok();
}

int paged_prefill_impl(const void *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                       const int32_t *tile_to_batch, const int32_t *tile_to_index, int num_tiles, int tile_rows,
                       const void *k_pool, const void *v_pool,
                       int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                       const int32_t *block_table, int64_t bt_sb, const int32_t *kv_lens,
                       const int32_t *causal_offset,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_st, int64_t o_sh,
                       int B, int Hq, int Hkv, int D, int page_size, float scale,
                       int total_q, int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    int G = 0, rc = check_prefill_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_prefill: head dim %d not built (32, 64, 128, 256)", D);
    if (B < 0 || num_tiles < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: negative B or num_tiles");
    // The kernel's tile height is fixed per (D, G); a work map built for
    // another height would leave rows unwritten or computed twice.
    if (tile_rows != pa::prefill_tile_rows(G, D))
        return fail(ATTN_ERR_INVALID_ARG,
                    "attn_paged_prefill: work map built for tile_rows=%d, the kernel takes %d at D=%d, G=%d "
                    "(attn_prefill_tile_rows)", tile_rows, pa::prefill_tile_rows(G, D), D, G);
    if (page_size <= 0) return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: page_size must be >= 1");
    if (!q || !qo_indptr || !k_pool || !v_pool || !block_table || !kv_lens || !o ||
        (num_tiles > 0 && (!tile_to_batch || !tile_to_index)))
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: null pointer");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: scale is not finite");
    if (mask && mask_ndim != 2 && mask_ndim != 3)
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: mask_ndim must be 2 or 3");
    if (mask && (m_sb < 0 || m_sq < 0))
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_prefill: negative mask stride");
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || ((uintptr_t)o & 7u) ||
        !mult8(q_st) || !mult8(q_sh) || !mult8(kv_s_page) || !mult8(kv_s_slot) || !mult8(kv_s_head) ||
        (o_st & 3) || (o_sh & 3))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_prefill: q/k/v rows must be 16-byte and o rows 8-byte aligned");
    if (kv_s_page < 0 || kv_s_slot < 0 || kv_s_head < 0 || kv_s_page >= (1ll << 32) ||
        (int64_t)(page_size - 1) * kv_s_slot + (int64_t)(Hkv - 1) * kv_s_head + D >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_prefill: pool strides exceed the 32-bit page/slot addressing");
    const int64_t groups = (int64_t)Hkv * (G / pa::prefill_heads_packed(G, D));   // workgroups per tile and split
    if ((int64_t)num_tiles * groups * (num_splits > 0 ? num_splits : 1) >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_prefill: num_tiles * Hkv * num_splits too large for one grid");
    pa::PrefillParams p{};
    rc = prefill_split_setup(p, "attn_paged_prefill", total_q, Hq, D, num_splits, workspace, workspace_bytes);
    if (rc) return rc;
    if (B == 0 || num_tiles == 0) return ok();
    p.q = static_cast<const uint16_t *>(q);
    p.q_st = q_st; p.q_sh = q_sh;
    p.qo_indptr = qo_indptr; p.t2b = tile_to_batch; p.t2i = tile_to_index; p.num_tiles = num_tiles;
    p.k = static_cast<const uint16_t *>(k_pool);
    p.v = static_cast<const uint16_t *>(v_pool);
    p.s_page = kv_s_page; p.s_slot = kv_s_slot; p.s_head = kv_s_head;
    p.bt = block_table; p.bt_sb = bt_sb;
    p.ps = (uint32_t)page_size;
    p.ps_div = pa::make_divu32((uint32_t)page_size);
    p.kv_lens = kv_lens;
    p.causal = causal_offset;
    p.mask = mask;
    p.mask_ndim = mask ? mask_ndim : 0;
    p.m_sb = m_sb; p.m_sq = m_sq;
    p.o = static_cast<uint16_t *>(o);
    p.o_st = o_st; p.o_sh = o_sh;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = G;
    p.sl2 = scale * 1.4426950408889634f;
    return run_prefill(p, D, static_cast<hipStream_t>(stream));
}

int dense_prefill_impl(const void *q, int64_t q_sb, int64_t q_sl, int64_t q_sh,
                       const void *k, const void *v, int64_t k_sb, int64_t k_sl, int64_t k_sh,
                       const int32_t *kv_lens, int kv_len, int is_causal,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_sb, int64_t o_sl, int64_t o_sh,
                       int B, int Lq, int Hq, int Hkv, int D, float scale,
                       int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    int G = 0, rc = check_prefill_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (!decode_dim(D)) return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: head dim %d not built (32, 64, 128, 256)", D);
    if (B < 0 || Lq < 0 || kv_len < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: negative size");
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: null pointer");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: scale is not finite");
    if (mask && mask_ndim != 2 && mask_ndim != 3)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: mask_ndim must be 2 or 3");
    if (mask && (m_sb < 0 || m_sq < 0))
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: negative mask stride");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || ((uintptr_t)o & 7u) || !mult8(q_sb) || !mult8(q_sl) ||
        !mult8(q_sh) || !mult8(k_sb) || !mult8(k_sl) || !mult8(k_sh) || (o_sb & 3) || (o_sl & 3) || (o_sh & 3))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: q/k/v rows must be 16-byte and o rows 8-byte aligned");
    if (q_sb < 0 || q_sl < 0 || q_sh < 0 || k_sb < 0 || k_sl < 0 || k_sh < 0 || o_sb < 0 || o_sl < 0 || o_sh < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: negative stride");
    const int R = pa::prefill_tile_rows(G, D);
    const int64_t tiles = (int64_t)B * ((Lq + R - 1) / R);
    const int64_t groups = (int64_t)Hkv * (G / pa::prefill_heads_packed(G, D));
    if (tiles * groups * (num_splits > 0 ? num_splits : 1) >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: too many tiles for one grid");
    if ((int64_t)B * Lq >= (1ll << 31)) return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: B * Lq must stay below 2^31");
    pa::PrefillParams p{};
    rc = prefill_split_setup(p, "attn_prefill", B * Lq, Hq, D, num_splits, workspace, workspace_bytes);
    if (rc) return rc;
    if (B == 0 || Lq == 0) return ok();
    p.q = static_cast<const uint16_t *>(q);
    p.q_sb = q_sb; p.q_st = q_sl; p.q_sh = q_sh;
    p.num_tiles = (int)tiles;
    p.dense_lq = Lq;
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.k_sb = k_sb; p.s_slot = k_sl; p.s_head = k_sh;
    p.bt = nullptr;
    p.ps = 1;
    p.kv_lens = kv_lens; p.kv_len_const = kv_len;
    p.causal = nullptr; p.causal_br = is_causal ? 1 : 0;
    p.mask = mask;
    p.mask_ndim = mask ? mask_ndim : 0;
    p.m_sb = m_sb; p.m_sq = m_sq;
    p.o = static_cast<uint16_t *>(o);
    p.o_sb = o_sb; p.o_st = o_sl; p.o_sh = o_sh;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = G;
    p.sl2 = scale * 1.4426950408889634f;
    return run_prefill(p, D, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

size_t attn_prefill_workspace_bytes(int rows, int Hq, int D, int num_splits) {
    if (rows < 0 || Hq <= 0 || D <= 0 || num_splits < 1) return 0;
    if (num_splits == 1) return 0;
    return pf_ml_offset(rows, Hq, D, num_splits) +
           (size_t)num_splits * (size_t)rows * (size_t)Hq * 2 * sizeof(float);
}

int attn_prefill_plan_splits(int num_tiles, int Hq, int Hkv, int D, int max_kv_len, int target_workgroups) {
    int G = 0, rc = check_prefill_heads(Hq, Hkv, &G);
    if (rc) return rc;
    if (num_tiles < 0 || max_kv_len < 0 || target_workgroups < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_plan_splits: negative argument");
    if (target_workgroups == 0) {
        const int cus = device_cus();
        if (cus <= 0) return fail(ATTN_ERR_LAUNCH, "attn_prefill_plan_splits: no HIP device");
        target_workgroups = kPrefillWgPerCu * cus;
    }
    const int64_t base = (int64_t)num_tiles * Hkv * (G / pa::prefill_heads_packed(G, D));
    if (base == 0) return 1;
    int64_t S = target_workgroups / base;
    const int64_t key_tiles = ((int64_t)max_kv_len + 63) / 64;
    S = std::min<int64_t>(S, key_tiles / kMinSplitKeyTiles);
    S = std::min<int64_t>(S, kMaxPrefillSplits);
    return (int)std::max<int64_t>(S, 1);
}

int attn_paged_prefill(const void *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                       const int32_t *tile_to_batch, const int32_t *tile_to_index, int num_tiles, int tile_rows,
                       const void *k_pool, const void *v_pool,
                       int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                       const int32_t *block_table, int64_t bt_sb, const int32_t *kv_lens,
                       const int32_t *causal_offset,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_st, int64_t o_sh,
                       int B, int Hq, int Hkv, int D, int page_size, float scale,
                       void *stream) {
    return paged_prefill_impl(q, q_st, q_sh, qo_indptr, tile_to_batch, tile_to_index, num_tiles, tile_rows,
                              k_pool, v_pool,
                              kv_s_page, kv_s_slot, kv_s_head, block_table, bt_sb, kv_lens, causal_offset, mask,
                              mask_ndim, m_sb, m_sq, o, o_st, o_sh, B, Hq, Hkv, D, page_size, scale, 0, 1, nullptr,
                              0, stream);
}

int attn_paged_prefill_split(const void *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                             const int32_t *tile_to_batch, const int32_t *tile_to_index, int num_tiles, int tile_rows,
                             const void *k_pool, const void *v_pool,
                             int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                             const int32_t *block_table, int64_t bt_sb, const int32_t *kv_lens,
                             const int32_t *causal_offset,
                             const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                             void *o, int64_t o_st, int64_t o_sh,
                             int B, int Hq, int Hkv, int D, int page_size, float scale,
                             int total_q, int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    return paged_prefill_impl(q, q_st, q_sh, qo_indptr, tile_to_batch, tile_to_index, num_tiles, tile_rows,
                              k_pool, v_pool,
                              kv_s_page, kv_s_slot, kv_s_head, block_table, bt_sb, kv_lens, causal_offset, mask,
                              mask_ndim, m_sb, m_sq, o, o_st, o_sh, B, Hq, Hkv, D, page_size, scale, total_q,
                              num_splits, workspace, workspace_bytes, stream);
}

int attn_prefill(const void *q, int64_t q_sb, int64_t q_sl, int64_t q_sh,
                 const void *k, const void *v, int64_t k_sb, int64_t k_sl, int64_t k_sh,
                 const int32_t *kv_lens, int kv_len, int is_causal,
                 const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                 void *o, int64_t o_sb, int64_t o_sl, int64_t o_sh,
                 int B, int Lq, int Hq, int Hkv, int D, float scale, void *stream) {
    return dense_prefill_impl(q, q_sb, q_sl, q_sh, k, v, k_sb, k_sl, k_sh, kv_lens, kv_len, is_causal, mask,
                              mask_ndim, m_sb, m_sq, o, o_sb, o_sl, o_sh, B, Lq, Hq, Hkv, D, scale, 1, nullptr, 0,
                              stream);
}

int attn_prefill_split(const void *q, int64_t q_sb, int64_t q_sl, int64_t q_sh,
                       const void *k, const void *v, int64_t k_sb, int64_t k_sl, int64_t k_sh,
                       const int32_t *kv_lens, int kv_len, int is_causal,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_sb, int64_t o_sl, int64_t o_sh,
                       int B, int Lq, int Hq, int Hkv, int D, float scale,
                       int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    return dense_prefill_impl(q, q_sb, q_sl, q_sh, k, v, k_sb, k_sl, k_sh, kv_lens, kv_len, is_causal, mask,
                              mask_ndim, m_sb, m_sq, o, o_sb, o_sl, o_sh, B, Lq, Hq, Hkv, D, scale, num_splits,
                              workspace, workspace_bytes, stream);
}

int attn_swa_fp8_decode(const void *q, int64_t q_st, int64_t q_sh,
                        const uint8_t *kv_cache, int64_t c_sb, int64_t c_ss,
                        const void *inv_scale, int64_t s_ss,
                        const int64_t *swa_indices, int64_t i_st, const int64_t *swa_lens,
                        void *o, int64_t o_st, int64_t o_sh,
                        int T, int NH, int HD, int window, int block_size, int num_blocks,
                        float scale, void *stream) {
    if (T < 0 || NH <= 0 || window < 0 || block_size <= 0 || num_blocks < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_decode: bad sizes");
    if (HD != 512) return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_decode: head dim %d not built (512)", HD);
    if (NH % 16 != 0) return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_decode: NH=%d is not a multiple of 16", NH);
    if (window > 1024) return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_decode: window %d above 1024", window);
    if (!q || !kv_cache || !inv_scale || !swa_indices || !swa_lens || !o)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_decode: null pointer");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_decode: scale is not finite");
    if (!aligned16(q) || !mult8(q_st) || !mult8(q_sh) || !aligned16(kv_cache) || (c_sb & 15) || (c_ss & 15) ||
        ((uintptr_t)o & 7u) || (o_st & 3) || (o_sh & 3) || ((uintptr_t)inv_scale & 1u))
        return fail(ATTN_ERR_UNSUPPORTED,
                    "attn_swa_fp8_decode: q rows and cache rows must be 16-byte aligned, o rows 8-byte aligned");
    if (c_sb < 0 || c_ss < 0 || s_ss < 0 || i_st < window)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_decode: bad strides");
    if ((int64_t)num_blocks * block_size >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_decode: num_blocks * block_size must stay below 2^31 slots");
    if ((int64_t)T * (NH / 16) >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_decode: T * NH / 16 must stay below 2^31");
    if (T == 0) return ok();
    pa::SwaParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.q_st = q_st; p.q_sh = q_sh;
    p.cache = kv_cache; p.c_sb = c_sb; p.c_ss = c_ss;
    p.inv_scale = static_cast<const uint16_t *>(inv_scale); p.s_ss = s_ss;
    p.ind = swa_indices; p.i_st = i_st; p.lens = swa_lens;
    p.o = static_cast<uint16_t *>(o); p.o_st = o_st; p.o_sh = o_sh;
    p.T = T; p.NH = NH; p.W = window; p.bs = block_size;
    p.slots = num_blocks * block_size;
    p.bs_div = pa::make_divu32((uint32_t)block_size);
    p.sl2 = scale * 1.4426950408889634f;
    p.o16 = (((uintptr_t)o & 15u) == 0 && (o_st & 7) == 0 && (o_sh & 7) == 0) ? 1 : 0;
    return launch_status(pa::launch_swa(p, static_cast<hipStream_t>(stream)), "swa kernel");
}

int attn_paged_kv_append(const void *k_new, const void *v_new, int64_t n_st, int64_t n_sh,
                         const int32_t *new_indptr, const int32_t *start_pos, int num_new,
                         void *k_pool, void *v_pool, int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                         int num_pages, const int32_t *block_table, int64_t bt_sb,
                         int B, int Hkv, int D, int page_size, void *stream) {
    if (B < 0 || num_new < 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || num_pages < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_kv_append: bad sizes");
    if (D % 8 != 0) return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_kv_append: D=%d is not a multiple of 8", D);
    if (num_new == 0 || B == 0) return ok();
    if (!k_new || !v_new || !new_indptr || !start_pos || !k_pool || !v_pool || !block_table)
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_kv_append: null pointer");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) || !mult8(n_st) ||
        !mult8(n_sh) || !mult8(kv_s_page) || !mult8(kv_s_slot) || !mult8(kv_s_head))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_paged_kv_append: rows must be 16-byte aligned");
    if (n_st < 0 || n_sh < 0 || kv_s_page < 0 || kv_s_slot < 0 || kv_s_head < 0 || bt_sb < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_paged_kv_append: negative stride");
    pa::KvAppendParams p{};
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.n_st = n_st; p.n_sh = n_sh;
    p.indptr = new_indptr; p.start_pos = start_pos;
    p.k_pool = static_cast<uint16_t *>(k_pool);
    p.v_pool = static_cast<uint16_t *>(v_pool);
    p.s_page = kv_s_page; p.s_slot = kv_s_slot; p.s_head = kv_s_head;
    p.bt = block_table; p.bt_sb = bt_sb;
    p.B = B; p.Hkv = Hkv; p.D = D; p.ps = page_size; p.N = num_new; p.num_pages = num_pages;
    return launch_status(pa::launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv append kernel");
}

int attn_swa_fp8_append(const void *x, int64_t x_st, const int64_t *slots, const float *multiplier, int N, int HD,
                        uint8_t *kv_cache, int64_t c_sb, int64_t c_ss, void *inv_scale, int64_t s_ss,
                        int block_size, int num_blocks, float *amax_out, void *stream) {
    if (N < 0 || block_size <= 0 || num_blocks < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_append: bad sizes");
    if (HD != 512) return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_append: head dim %d not built (512)", HD);
    if ((int64_t)num_blocks * block_size >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_append: num_blocks * block_size must stay below 2^31 slots");
    if (N == 0) return ok();
    if (!x || !slots || !kv_cache || !inv_scale)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_append: null pointer");
    if (!aligned16(x) || !mult8(x_st) || !aligned16(kv_cache) || (c_sb & 15) || (c_ss & 15) ||
        ((uintptr_t)inv_scale & 1u))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_swa_fp8_append: x rows and cache rows must be 16-byte aligned");
    if (x_st < 0 || c_sb < 0 || c_ss < 0 || s_ss < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_swa_fp8_append: negative stride");
    pa::SwaQuantParams p{};
    p.x = static_cast<const uint16_t *>(x); p.x_st = x_st;
    p.slots = slots; p.mult = multiplier;
    p.cache = kv_cache; p.c_sb = c_sb; p.c_ss = c_ss;
    p.inv_scale = static_cast<uint16_t *>(inv_scale); p.s_ss = s_ss;
    p.amax = amax_out;
    p.N = N; p.bs = block_size;
    p.num_slots = (int64_t)num_blocks * block_size;
    p.bs_div = pa::make_divu32((uint32_t)block_size);
    return launch_status(pa::launch_swa_quantize(p, static_cast<hipStream_t>(stream)), "swa quantize kernel");
}

int attn_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink, int workgroups, void *stream) {
    if (!buf || !sink) return fail(ATTN_ERR_INVALID_ARG, "attn_hbm_read_probe: null pointer");
    if (workgroups < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_hbm_read_probe: negative workgroup count");
    if (!aligned16(buf) || (bytes & 15) || ((uintptr_t)sink & 15u))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_hbm_read_probe: buffer, size and sink must be 16-byte aligned");
    if (workgroups == 0) {
        workgroups = device_cus();
        if (workgroups <= 0) return fail(ATTN_ERR_LAUNCH, "attn_hbm_read_probe: cannot query the device");
    }
    if (workgroups > (1 << 20)) return fail(ATTN_ERR_INVALID_ARG, "attn_hbm_read_probe: too many workgroups");
    return launch_status(pa::launch_stream_read(buf, bytes, sink, workgroups, static_cast<hipStream_t>(stream)),
                         "stream read probe");
}

int attn_rotary_embed(const void *x, int64_t x_st, int64_t x_sh, void *out, int64_t o_st, int64_t o_sh,
                      int T, int H, int D, const float *cos_table, const float *sin_table, int64_t tab_st,
                      int table_rows, const int32_t *positions, void *stream) {
    if (T < 0 || H <= 0 || D <= 0 || table_rows < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_rotary_embed: bad sizes");
    if (D % 8 != 0) return fail(ATTN_ERR_UNSUPPORTED, "attn_rotary_embed: D=%d is not a multiple of 8", D);
    if ((int64_t)T * H * (D / 8) >= (1ll << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_rotary_embed: T * H * D / 8 must stay below 2^31");
    if ((int64_t)H * (D / 8) > 65535ll * 256)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_rotary_embed: H * D / 8 must stay at or below 65535 * 256");
    if (T == 0) return ok();
    if (!x || !out || !cos_table || !sin_table || !positions)
        return fail(ATTN_ERR_INVALID_ARG, "attn_rotary_embed: null pointer");
    if (!aligned16(x) || !aligned16(out) || !mult8(x_st) || !mult8(x_sh) || !mult8(o_st) || !mult8(o_sh) ||
        !aligned16(cos_table) || !aligned16(sin_table) || (tab_st & 3))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_rotary_embed: rows must be 16-byte aligned");
    if (tab_st < D / 2) return fail(ATTN_ERR_INVALID_ARG, "attn_rotary_embed: table stride below D/2");
    pa::RotaryParams p{};
    p.x = static_cast<const uint16_t *>(x); p.x_st = x_st; p.x_sh = x_sh;
    p.out = static_cast<uint16_t *>(out); p.o_st = o_st; p.o_sh = o_sh;
    p.cos = cos_table; p.sin = sin_table; p.tab_st = tab_st;
    p.pos = positions;
    p.T = T; p.H = H; p.D = D; p.rows = table_rows;
    return launch_status(pa::launch_rotary(p, static_cast<hipStream_t>(stream)), "rotary kernel");
}

}  // extern "C"
