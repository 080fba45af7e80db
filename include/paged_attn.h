/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged GQA attention library.
 *
 * Grouped-query attention over a paged KV cache, as the AstrAI "CUDA
 * Kernels" developer doc describes it (Overview table: attn_decode,
 * attn_paged_decode, attn_paged_prefill), plus the fp8 sliding-window decode
 * of native_swa_decode.py (nvfp4-megamoe-kernel).  Every function computes
 * out = softmax(scale * q K^T + mask) V exactly, up to rounding.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, except
 *     where a parameter name ends in _host.  The library never allocates or
 *     frees device memory, never synchronises the stream, and keeps no
 *     state between calls besides the per-thread error message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs on the calling thread's current HIP device.
 *   - Element types: q, k, v and outputs are bf16 (stored as uint16 bit
 *     patterns); indices and lengths are int32 unless stated otherwise.
 *   - Strides are in ELEMENTS of the tensor they describe.  The innermost
 *     (head-dim) stride is 1.  Rows of bf16 data must start at 16-byte
 *     aligned addresses: base pointers 16-byte aligned and every stride a
 *     multiple of 8 elements; otherwise ATTN_ERR_UNSUPPORTED is returned
 *     (there is no scalar fallback path).
 *   - GQA head mapping: query head h reads KV head h / (Hq / Hkv), so
 *     consecutive query heads share a KV head.
 *   - A query row with no admissible key (empty sequence, everything masked)
 *     produces an all-zero output row.
 *   - Non-finite inputs are not checked; inputs are expected to be finite.
 *     What the kernels do with a NaN (pinned by the tests): a NaN in a
 *     query row, or in the K row of a key that the query row admits, makes
 *     that output row NaN, as softmax attention does, whatever the split
 *     count (a split piece whose sum l is NaN carries m = +inf, so every
 *     merge through it is NaN).  A NaN in the V row of an admitted key makes
 *     the rows that admit it NaN.  The K row of a key a query row does not
 *     admit (past its length or causal frontier, or masked out) never
 *     reaches that row; the V row of such a key may still reach rows that
 *     share its 64-key prefill tile.  Infinite inputs are not supported.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code; then
 *     attn_last_error() gives a message.  Argument checks happen before any
 *     device work is enqueued, so a failed call leaves outputs untouched.
 *     Bad device-side data (a block-table entry outside the pool, a length
 *     above the stated maximum, a slot index beyond the cache) is undefined
 *     behaviour: it is not checked on the device.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad stride ... */
#define ATTN_ERR_UNSUPPORTED (-2) /* valid but not built: head dim, alignment   */
#define ATTN_ERR_WORKSPACE (-3)   /* workspace missing or too small              */
#define ATTN_ERR_LAUNCH (-4)      /* the HIP runtime refused a launch            */

/* Message for the last failed call on this thread ("" if none).  The
 * pointer stays valid until the next call on the same thread. */
const char *attn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

/* ------------------------------------------------------------ split plan */

/*
 * Decode work partition (AstrAI csrc commit history: the commit that
 * partitions KV across gridDim.z and sizes the split count to fill the
 * device, and the later one that retargets it at a fixed total block count
 * after a grid search).  Decode runs one workgroup per slice of a balanced
 * partition: the rows are laid end to end and the line of all their tokens is
 * cut into `num_splits` = W equal slices, whatever the spread of kv_lens.
 * Rows (see attn_decode for the kernels):
 *   - G = 1, 2, 4 (any D), VALU kernel: a row is (sequence, group of up to 8
 *     adjacent KV heads, 4 at D = 256) when the KV head stride `kv_s_head`
 *     equals D (heads of a token contiguous), else one KV head;
 *   - other G at D = 64 or 128, MFMA kernel: a row is (sequence, group of 4,
 *     2 or 1 adjacent KV heads -- the largest dividing Hkv -- and up to 32
 *     query heads each), or with G > 32 (sequence, KV head, pass of G / Gk);
 *   - other G at D = 32 or 256, VALU kernel: (sequence, KV head, pass over
 *     a power-of-two share of its G query heads).
 * Slices are four-wave workgroups for the first two (a slice of at least 256
 * tokens; at most 3/4 of the compute units when a row holds 8 KV heads, one
 * per unit otherwise) and one-wave workgroups for the third (at least 64
 * tokens; three per unit with 8-head rows, two otherwise).  This planner
 * returns W for `num_cus` compute units (0 = query the current device) and
 * the longest row max_kv_len.  page_size 0 stands for a contiguous source
 * (pass its K head stride as kv_s_head).  Host-only and deterministic;
 * returns W >= 1, or a negative error code.
 */
int attn_plan_splits(int B, int Hkv, int G, int D, int max_kv_len, int page_size, int64_t kv_s_head,
                     int num_cus);

/*
 * Bytes of device workspace decode needs with W = num_splits slices:
 *   o_part  float [(B + W) * Hq, D]  unnormalised partial outputs
 *   ml_part float [(B + W) * Hq, 2]  (m, l) per partial, starting at the
 *                                    first 256-byte boundary after o_part
 *   ranges  int32 [B * Hq, 2]        per row with keys, the first and last
 *                                    slice holding them (written by the split
 *                                    kernel, read by the combine), at the
 *                                    first 256-byte boundary after ml_part
 * The piece of row r in slice w is stored at slot r + w (every row or slice
 * boundary along the line advances r or w, so slots are unique); local query
 * head i of the row sits at partial row slot * heads_per_row + i.  m is a
 * reference value in natural-log units of the scaled score (every
 * exp(score - m) <= e^(8 ln 2)); l = sum exp(score - m), o = sum exp(score -
 * m) v over the piece (m = +inf marks a piece whose l is NaN, see the
 * non-finite inputs convention).  The split kernel writes every slot it owns, so the
 * workspace needs no initialisation (cf. the commit that switched
 * alloc_split_partials to torch::empty).  attn_decode / attn_paged_decode
 * with W = 1 need no workspace.  Returns 0 for empty shapes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits);

/* ---------------------------------------------------------------- decode */

/*
 * Contiguous GQA decode, one query token per sequence (AstrAI "CUDA Kernels"
 * doc, Overview: attn_decode, GQA decode with split-KV; layout-agnostic
 * stride addressing from the csrc commit that added bhld/blhd strides).
 *   q   [B, Hq, D]: element (b, h, d) at q + b*q_sb + h*q_sh + d
 *   k,v [B, Hkv, L, D] logical: (b, g, j, d) at k + b*k_sb + g*k_sh + j*k_sl + d
 *       (bhld and blhd are both stride choices)
 *   o   [B, Hq, D]: (b, h, d) at o + b*o_sb + h*o_sh + d
 *   kv_lens  device int32 [B], each in [0, kv_len]; NULL = all equal kv_len
 *   scale    multiplies q.k before the softmax (normally 1/sqrt(D))
 *   num_splits  slices W of the balanced partition; 0 = attn_plan_splits()
 *               on the current device, except that with kv_lens NULL and
 *               kv_len > 0, when the rows (B times the KV head groups) number
 *               between half that count and the count, W = the rows (one
 *               slice per row; never above the planner's count)
 *   workspace   >= attn_decode_workspace_bytes(B, Hq, D, W) bytes, device,
 *               256-byte aligned (may be NULL when W = 1)
 * With kv_lens NULL, kv_len > 0 and W dividing the rows, every slice holds
 * whole rows, each written directly, and no combine kernel is launched.
 * Supported: D in {32, 64, 128, 256}, any G = Hq/Hkv.  G = 1, 2 and 4 run the
 * VALU kernel (dot products on the vector ALUs, a wave holding all G query
 * heads of its KV heads).  Other G at D = 64 and 128 run the MFMA kernel:
 * the Gm query heads of a KV head (the largest divisor of G that is at most
 * 32) sit on the rows of bf16 16x16x32 MFMAs, so each KV head is read once
 * (G / Gm times for G > 32).  Other G at D = 32 and 256 take passes over
 * power-of-two shares of at most 8 heads, reading each KV head once per pass.
 * Launches the split kernel, then the combine kernel, which merges rows
 * spread over several slices and zeroes rows without keys.
 */
int attn_decode(const void *q, int64_t q_sb, int64_t q_sh,
                const void *k, int64_t k_sb, int64_t k_sh, int64_t k_sl,
                const void *v, int64_t v_sb, int64_t v_sh, int64_t v_sl,
                void *o, int64_t o_sb, int64_t o_sh,
                const int32_t *kv_lens, int kv_len,
                int B, int Hq, int Hkv, int D, float scale, int num_splits,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Paged GQA decode (AstrAI "CUDA Kernels" doc, Overview: attn_paged_decode;
 * per-element page lookup from the csrc commit that replaced the per-tile
 * lookup, which works for any page size).
 *   q      [B, Hq, D] as in attn_decode
 *   k_pool, v_pool  paged pools sharing one addressing: element
 *          (page, slot, g, d) at pool + page*kv_s_page + slot*kv_s_slot
 *          + g*kv_s_head + d  ([P, ps, Hkv, D] and [P, Hkv, ps, D] both fit)
 *   block_table  int32, row b at block_table + b*bt_sb; logical token j of
 *          sequence b lives in page block_table[b*bt_sb + j/page_size] at
 *          slot j % page_size.  Entries past a sequence's last page are
 *          never read.
 *   kv_lens  int32 [B], each in [0, max_kv_len]
  *   max_kv_len  host-side bound on kv_lens, used by the planner
 *   o      [B, Hq, D] bf16 output
 * Supported: D in {32, 64, 128, 256}, any G (as attn_decode), any page_size >= 1.
 * A slice longer than 510 pages is processed as consecutive sub-pieces.
 */
int attn_paged_decode(const void *q, int64_t q_sb, int64_t q_sh,
                      const void *k_pool, const void *v_pool,
                      int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                      const int32_t *block_table, int64_t bt_sb,
                      const int32_t *kv_lens, int max_kv_len,
                      void *o, int64_t o_sb, int64_t o_sh,
                      int B, int Hq, int Hkv, int D, int page_size, float scale,
                      int num_splits, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * attn_paged_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as attn_paged_decode without the
 * workspace: the split partials go to a static device buffer of
 * ATTN_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library, one copy per
 * device, held until the process ends; the call itself allocates nothing
 * (no hipMalloc, no allocating library routine).  Its device address is
 * looked up once per device, on the first call with that device current.
 *   num_splits  0 = the planner's count, lowered if needed to the largest
 *               whose partials fit the buffer (attn_decode_workspace_bytes
 *               <= ATTN_NOALLOC_SCRATCH_BYTES; one slice needs none); an
 *               explicit count whose partials do not fit returns
 *               ATTN_ERR_UNSUPPORTED.
 * The buffer keeps the last call's contents; nothing in it needs to start
 * at zero (the split kernel writes every slot the combine reads).  Calls
 * that overlap in time on one device (several streams or threads) share
 * the buffer and race: serialise them.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_paged_decode_noalloc(const void *q, int64_t q_sb, int64_t q_sh,
                              const void *k_pool, const void *v_pool,
                              int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                              const int32_t *block_table, int64_t bt_sb,
                              const int32_t *kv_lens, int max_kv_len,
                              void *o, int64_t o_sb, int64_t o_sh,
                              int B, int Hq, int Hkv, int D, int page_size, float scale,
                              int num_splits, void *stream);

/*
 * The two halves of attn_paged_decode, for callers that schedule them
 * separately (e.g. to time each kernel).  attn_paged_decode_split takes the
 * arguments of attn_paged_decode minus the output and writes every piece as
 * an fp32 partial into `workspace` (layout at attn_decode_workspace_bytes),
 * together with the `ranges` region: for each row with keys, the first and
 * last slice holding them.  attn_decode_combine then writes o [B, Hq, D]
 * bf16 from that workspace: it reads the ranges region to find each row's
 * pieces (slots r + first .. r + last), so the whole workspace written by the
 * split call, ranges included, is its input.  It must be given the same B,
 * Hq, Hkv, D, num_splits (after planning, i.e. the explicit W) and KV head
 * stride as the split call, which fix the row layout; kv_lens (NULL = all
 * max_kv_len) only marks the rows without keys, which are written as zeros.
 * Partials produced elsewhere (another device's share of the keys) can be
 * merged this way only if they come with a ranges region consistent with
 * the same W and row layout; attn_split_combine merges partials stored
 * densely instead.
 */
int attn_paged_decode_split(const void *q, int64_t q_sb, int64_t q_sh,
                            const void *k_pool, const void *v_pool,
                            int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                            const int32_t *block_table, int64_t bt_sb,
                            const int32_t *kv_lens, int max_kv_len,
                            int B, int Hq, int Hkv, int D, int page_size, float scale,
                            int num_splits, void *workspace, size_t workspace_bytes, void *stream);

int attn_decode_combine(const void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int D,
                        int num_splits, int64_t kv_s_head, const int32_t *kv_lens, int max_kv_len, void *o,
                        int64_t o_sb, int64_t o_sh, void *stream);

/*
 * Log-sum-exp combine of split partials (AstrAI csrc commit history: the
 * combine kernel that reduces the unnormalised (O, m, l) partials; one
 * combine kernel serves every decode path).  Rows are independent:
 *   o_part  float [S, R, D], ml_part float [S, R, 2] = (m, l), natural log
 *   out_f32  NULL or float [R, D];  out_bf16 NULL or bf16 [R, D]
 *   lse      NULL or float [R]: M + log(sum_s exp(m_s - M) l_s)
 * out = sum_s exp(m_s - M) o_s / sum_s exp(m_s - M) l_s with M = max_s m_s;
 * a partial with m = -inf contributes nothing; a row whose partials are all
 * empty gives 0 (lse = -inf).  D in {32, 64, 128, 256}.
 */
int attn_split_combine(const float *o_part, const float *ml_part, int S, int R, int D,
                       float *out_f32, void *out_bf16, float *lse, void *stream);

/* --------------------------------------------------------------- prefill */

/*
 * Ragged work map (AstrAI "CUDA Kernels" doc, section "Q Scheduling and KV
 * Addressing"): from per-sequence query lengths builds qo_indptr (prefix sum,
 * B + 1 entries) and, for every tile of `tile_rows` query rows, the sequence
 * it belongs to and its index inside that sequence, in sequence order.  All
 * arrays are HOST memory.  Writes *num_tiles; fails with ATTN_ERR_INVALID_ARG
 * if more than `cap` tiles would be needed.
 */
int attn_prefill_plan(const int32_t *q_lens_host, int B, int tile_rows,
                      int32_t *qo_indptr_host, int32_t *tile_to_batch_host,
                      int32_t *tile_to_index_host, int cap, int *num_tiles);

/* Query rows per tile that attn_paged_prefill expects in its work map for
 * head dim D and group size G = Hq / Hkv.  A workgroup packs HP query heads
 * that share a KV head (csrc commit on GQA head packing: K/V tiles are
 * streamed once per block, not once per query head): HP is the largest power
 * of two dividing G, at most 8, i.e. all G heads for G in {1, 2, 4, 8}.  A
 * tile holds 128 / HP rows for HP <= 4 (32 rows of one head per wave) and 16
 * rows for HP = 8 (two heads of the same 16 rows per wave).  At D = 256 a
 * workgroup has four waves of 16 rows: HP is at most 4 and a tile holds
 * 64 / HP rows. */
int attn_prefill_tile_rows(int D, int G);

/*
 * Ragged paged prefill (AstrAI "CUDA Kernels" doc, Overview:
 * attn_paged_prefill; "Q Scheduling and KV Addressing": packed Q schedule +
 * paged KV source; csrc commits on the unified causal_offset and on 2-D/3-D
 * masks that coexist with causality).
 *   q  packed [total_q, Hq, D]: row r, head h at q + r*q_st + h*q_sh
 *   qo_indptr  device int32 [B + 1]; sequence b owns rows
 *          qo_indptr[b] .. qo_indptr[b+1]
 *   tile_to_batch, tile_to_index  device copies of attn_prefill_plan's
 *          output; num_tiles tiles
 *   tile_rows  the tile height the work map was built with; it must equal
 *          attn_prefill_tile_rows(D, Hq / Hkv), the height this kernel
 *          computes (a map of another height, e.g. the 64-row tiles of the
 *          doc's worked example at G = 4, D = 128, would leave rows unwritten
 *          or computed twice), else ATTN_ERR_INVALID_ARG
 *   k_pool, v_pool, kv_s_*, block_table, bt_sb, page_size  as in
 *          attn_paged_decode; kv_lens [B] = keys held by each sequence
 *          (prior context plus the new rows)
 *   causal_offset  NULL = no causality; else device int32 [B]: -1 turns it
 *          off for that sequence, c >= 0 admits key j for local row i iff
 *          j <= c + i (c is the absolute position of the sequence's first
 *          new row)
 *   mask   NULL, or uint8 keep-mask (nonzero = keep): mask_ndim 2 reads
 *          mask[b*m_sb + j], mask_ndim 3 reads mask[b*m_sb + i*m_sq + j]
 *          with i the local row; combined with causality by AND
 *   o      packed [total_q, Hq, D] bf16: row r, head h at o + r*o_st + h*o_sh
 * Alignment: q/k/v rows 16-byte aligned, o rows 8-byte aligned; mask rows
 * may start at any byte (e.g. a plain bool [B, q, kv] tensor with kv odd);
 * mask bytes at key positions >= kv_lens[b] are never used.  Supported: D in {32, 64, 128, 256}, any G = Hq / Hkv.
 */
int attn_paged_prefill(const void *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                       const int32_t *tile_to_batch, const int32_t *tile_to_index, int num_tiles, int tile_rows,
                       const void *k_pool, const void *v_pool,
                       int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                       const int32_t *block_table, int64_t bt_sb, const int32_t *kv_lens,
                       const int32_t *causal_offset,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_st, int64_t o_sh,
                       int B, int Hq, int Hkv, int D, int page_size, float scale,
                       void *stream);

/*
 * Dense prefill over a contiguous KV source (AstrAI "CUDA Kernels" doc:
 * attention kernels combine a Q schedule, DenseQSchedule or PackedQSchedule,
 * with a KV source, ContigKV or PagedKV; Python Wrappers interface note:
 * is_causal and a 2-D [batch, kv] or 3-D [batch, q, kv] keep-mask).
 *   q   [B, Lq, Hq, D] by strides: (b, i, h) at q + b*q_sb + i*q_sl + h*q_sh
 *       (any of blhd / bhld)
 *   k, v  [B, Lk, Hkv, D] by the same strides for both: (b, j, g) at
 *       k + b*k_sb + j*k_sl + g*k_sh
 *   kv_lens  device int32 [B] keys of each sequence, or NULL for kv_len
 *   is_causal  nonzero: query row i of sequence b admits key j iff
 *       j <= n_b - Lq + i (bottom-right alignment: the Lq queries are the
 *       sequence's last Lq positions); rows that admit no key give zeros
 *   mask, mask_ndim, m_sb, m_sq  as in attn_paged_prefill
 *   o   [B, Lq, Hq, D] bf16: (b, i, h) at o + b*o_sb + i*o_sl + h*o_sh
 * Same kernel and numerics as attn_paged_prefill; no work map is needed.
 * Supported: D in {32, 64, 128, 256}, any G; alignment as attn_paged_prefill.
 */
int attn_prefill(const void *q, int64_t q_sb, int64_t q_sl, int64_t q_sh,
                 const void *k, const void *v, int64_t k_sb, int64_t k_sl, int64_t k_sh,
                 const int32_t *kv_lens, int kv_len, int is_causal,
                 const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                 void *o, int64_t o_sb, int64_t o_sl, int64_t o_sh,
                 int B, int Lq, int Hq, int Hkv, int D, float scale, void *stream);

/*
 * Split-KV prefill, for short query runs over long contexts, where the
 * tiles x KV heads of the plain prefill leave the device mostly idle (csrc
 * commit on GQA head packing, measured on short-q / long-kv prefill; the
 * unnormalised partials and their log-sum-exp combine are those of split-KV
 * decode, AstrAI "CUDA Kernels" doc, Overview).  num_splits workgroups
 * share each tile's visible keys in equal runs of 64-key tiles; each writes
 * an unnormalised fp32 partial (o, m, l) per query row and head into the
 * workspace, and a combine kernel merges them into o by log-sum-exp.  The
 * arguments and results are those of attn_paged_prefill / attn_prefill,
 * plus:
 *   total_q     (paged) rows of the packed Q, i.e. qo_indptr[B] (host int);
 *               the partials cover rows < total_q
 *   num_splits  >= 1, e.g. from attn_prefill_plan_splits; 1 runs the plain
 *               kernel and needs no workspace
 *   workspace   device, 256-byte aligned, at least
 *               attn_prefill_workspace_bytes(rows, Hq, D, num_splits) bytes
 *               with rows = total_q (paged) or B * Lq (dense); its contents
 *               need no initialisation and are scratch after the call.
 * Layout: o_part f32 [num_splits, rows, Hq, D], then at the next 256-byte
 * boundary ml_part f32 [num_splits, rows, Hq, 2] (m in natural-log units of
 * the scaled score, l).  Errors: ATTN_ERR_WORKSPACE if the workspace is
 * missing or short; ATTN_ERR_INVALID_ARG if num_splits is outside [1, 256].
 */
size_t attn_prefill_workspace_bytes(int rows, int Hq, int D, int num_splits);

/* Host planner for the split count: with W0 = num_tiles * Hkv * (G / HP)
 * workgroups of the plain kernel (HP as in attn_prefill_tile_rows), returns the largest S <= target_workgroups / W0 that
 * leaves every split at least 8 key tiles of 64 at max_kv_len (at least 1,
 * at most 256).  target_workgroups = 0 uses one per compute unit of the
 * current device.  Negative on error. */
int attn_prefill_plan_splits(int num_tiles, int Hq, int Hkv, int D, int max_kv_len, int target_workgroups);

int attn_paged_prefill_split(const void *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                             const int32_t *tile_to_batch, const int32_t *tile_to_index, int num_tiles, int tile_rows,
                             const void *k_pool, const void *v_pool,
                             int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                             const int32_t *block_table, int64_t bt_sb, const int32_t *kv_lens,
                             const int32_t *causal_offset,
                             const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                             void *o, int64_t o_st, int64_t o_sh,
                             int B, int Hq, int Hkv, int D, int page_size, float scale,
                             int total_q, int num_splits, void *workspace, size_t workspace_bytes, void *stream);

int attn_prefill_split(const void *q, int64_t q_sb, int64_t q_sl, int64_t q_sh,
                       const void *k, const void *v, int64_t k_sb, int64_t k_sl, int64_t k_sh,
                       const int32_t *kv_lens, int kv_len, int is_causal,
                       const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                       void *o, int64_t o_sb, int64_t o_sl, int64_t o_sh,
                       int B, int Lq, int Hq, int Hkv, int D, float scale,
                       int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/* --------------------------------------------------- fp8 sliding window */

/*
 * fp8 sliding-window decode, MLA style with K = V (native_swa_decode.py:
 * the host wrapper's signature and the batched-SDPA fallback's steps).
 *   q       [T, NH, HD] bf16: (t, h, d) at q + t*q_st + h*q_sh + d
 *   kv_cache  uint8 OCP e4m3fn codes; slot idx lives at
 *           kv_cache + (idx / block_size)*c_sb + (idx % block_size)*c_ss
 *   inv_scale  bf16 per slot at inv_scale + idx*s_ss; the dequantised row
 *           is e4m3(code) * inv_scale (exact product)
 *   swa_indices int64 [T, W], row t at swa_indices + t*i_st
 *   swa_lens    int64 [T]; window position j of token t is admitted iff
 *           j < swa_lens[t] and 0 <= swa_indices[t, j] < num_blocks*block_size
 *           (an index outside the pool is treated like -1 and never read)
 *   o       [T, NH, HD] bf16
 * Every head of a token attends the same rows (K = V).  Supported: HD = 512,
 * NH a multiple of 16, W <= 1024, num_blocks*block_size < 2^31.
 */
int attn_swa_fp8_decode(const void *q, int64_t q_st, int64_t q_sh,
                        const uint8_t *kv_cache, int64_t c_sb, int64_t c_ss,
                        const void *inv_scale, int64_t s_ss,
                        const int64_t *swa_indices, int64_t i_st, const int64_t *swa_lens,
                        void *o, int64_t o_st, int64_t o_sh,
                        int T, int NH, int HD, int window, int block_size, int num_blocks,
                        float scale, void *stream);

/* --------------------------------------------- cache writes and rotary */

/*
 * Paged KV append: the cache write that precedes paged decode and prefill
 * (AstrAI "CUDA Kernels" doc, Backend Layer: the attention backend owns the
 * KV cache writes).
 *   k_new, v_new  packed new rows [num_new, Hkv, D] bf16: row i, head g at
 *          + i*n_st + g*n_sh (same strides for both)
 *   new_indptr    device int32 [B + 1]: sequence b owns new rows
 *          new_indptr[b] .. new_indptr[b+1]
 *   start_pos     device int32 [B]: position of sequence b's first new token
 *          (its length before the append)
 *   k_pool, v_pool, kv_s_*, block_table, bt_sb, page_size  as in
 *          attn_paged_decode; num_pages = pages in the pool
 * New token i of sequence b is written to position start_pos[b] + i, i.e.
 * page block_table[b][pos / page_size], slot pos % page_size, as an exact
 * copy.  A token whose block-table entry is negative or >= num_pages is not
 * written.  The block table must cover the new positions.  Supported: D a
 * multiple of 8, 16-byte aligned rows.
 */
int attn_paged_kv_append(const void *k_new, const void *v_new, int64_t n_st, int64_t n_sh,
                         const int32_t *new_indptr, const int32_t *start_pos, int num_new,
                         void *k_pool, void *v_pool, int64_t kv_s_page, int64_t kv_s_slot, int64_t kv_s_head,
                         int num_pages, const int32_t *block_table, int64_t bt_sb,
                         int B, int Hkv, int D, int page_size, void *stream);

/*
 * fp8 quantize-on-write of sliding-window cache rows (native_swa_decode.py:
 * the cache holds OCP e4m3fn codes and a bf16 inverse scale per slot;
 * AstrAI "CUDA Kernels" doc, FP8 section: quantize takes the quantization
 * multiplier and multiplies by it, amax is reported in the input domain).
 *   x         [N, HD] bf16, row n at x + n*x_st
 *   slots     device int64 [N]: cache slot of row n (block = slot / block_size,
 *             offset = slot % block_size, as in attn_swa_fp8_decode)
 *   multiplier  device float [N], or NULL for 448 / amax of the row (1 when
 *             the row is all zeros)
 *   kv_cache, c_sb, c_ss, inv_scale, s_ss  as in attn_swa_fp8_decode
 *   amax_out  device float [N] (max |x| of each row), or NULL
 * Row n's codes are e4m3fn(x * m): the product in binary32, rounded to the
 * nearest code with ties to even, magnitudes >= 448 saturated to 448, the
 * sign kept (-0 gives 0x80), NaN giving 0x7F; the slot's inverse scale is
 * bf16(1 / m) (nearest-even), so decode dequantises code * inv_scale.  A row
 * whose slot is negative or >= num_blocks*block_size is not written (its
 * amax is still reported).  Supported: HD = 512.
 */
int attn_swa_fp8_append(const void *x, int64_t x_st, const int64_t *slots, const float *multiplier, int N, int HD,
                        uint8_t *kv_cache, int64_t c_sb, int64_t c_ss, void *inv_scale, int64_t s_ss,
                        int block_size, int num_blocks, float *amax_out, void *stream);

/*
 * Rotary embedding (AstrAI "CUDA Kernels" doc, Rotary Embedding Kernel: a
 * fused cos/sin lookup and rotation; Rotary Backend: the fallback multiplies
 * adjacent pairs, viewed as complex numbers, by the table's cos + i sin).
 *   x, out     [T, H, D] bf16 (out may be x: in place)
 *   cos_table, sin_table  fp32 [table_rows, D/2], row p at + p*tab_st
 *   positions  device int32 [T]: table row of token t
 * out[t, h, 2i] = x[2i] cos - x[2i+1] sin, out[t, h, 2i+1] = x[2i] sin +
 * x[2i+1] cos with (cos, sin) = table row positions[t], column i; the math is
 * fp32 and each output is rounded to bf16 once.  Tokens whose position is
 * outside [0, table_rows) are left untouched.  Supported: D a multiple of 8,
 * 16-byte aligned rows, tab_st a multiple of 4, T * H * D/8 below 2^31 and
 * H * D/8 at most 65535 * 256 (else ATTN_ERR_UNSUPPORTED).
 */
int attn_rotary_embed(const void *x, int64_t x_st, int64_t x_sh, void *out, int64_t o_st, int64_t o_sh,
                      int T, int H, int D, const float *cos_table, const float *sin_table, int64_t tab_st,
                      int table_rows, const int32_t *positions, void *stream);

/* ----------------------------------------------------------- measurement */

/*
 * Pure-read HBM streaming probe: the measured ceiling that decode's achieved
 * bandwidth is compared against (beside the 8 TB/s specification).  Reads
 * every 16-byte word of buf [bytes] exactly once with non-temporal loads,
 * the grid sweeping the buffer front to back, and writes the XOR of the words
 * each wave read to sink (uint32 [workgroups * 4 waves * 4], 16-byte
 * aligned), so that no load is dropped and the XOR over sink equals the XOR
 * of every 16-byte word of the buffer.  workgroups 0 = one per compute unit
 * (256 threads each).  buf and bytes must be 16-byte aligned.
 */
int attn_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink, int workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
