"""GPU parity of the ragged paged prefill (MFMA) against the CPU oracle.

Bar: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| on the bf16 outputs."""
import math

import pytest
import torch

import oracle
import paged_kv_gqa_03_amd as pa
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def assert_close(got, ref, atol=1e-2, rtol=1e-2, what=""):
    got = got.detach().to("cpu", torch.float64)
    err = (got - ref).abs()
    bad = err > atol + rtol * ref.abs()
    assert not bool(bad.any()), "%s: %d of %d elements off, max err %.4g" % (
        what, int(bad.sum()), bad.numel(), float(err.max()))


def run_prefill(case, causal=True):
    G = case["Hq"] // case["Hkv"]
    R = pa.attn_prefill_tile_rows(case["D"], G)
    indptr, t2b, t2i = pa.attn_prefill_plan(case["q_lens"], R)
    assert torch.equal(indptr, case["qo_indptr"].cpu())
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "qo_indptr",
                                     "causal_offset")}
    mask = case["mask"].to(DEV) if case["mask"] is not None else None
    out = torch.full_like(d["q"], float("nan"))
    pa.attn_paged_prefill(d["q"], d["qo_indptr"], t2b.to(DEV), t2i.to(DEV), d["k_pool"], d["v_pool"],
                          d["block_table"], d["kv_lens"], out, case["page_size"], case["scale"],
                          causal_offset=d["causal_offset"] if causal else None, mask=mask, tile_rows=R)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, causal=True):
    out, _ = oracle.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"],
                                  case["block_table"], case["kv_lens"], case["scale"],
                                  causal_offset=case["causal_offset"] if causal else None, mask=case["mask"])
    return out


@pytest.mark.parametrize("masked", [False, True])
def test_ragged_prefill_config(masked):
    """Config 4 at full size, every row and head.  Besides the 1e-2 pass bar,
    a secondary absolute bar of 2e-3: outputs average up to 2560 values and
    are ~0.02-0.05 in size, where 1e-2 alone would be loose."""
    case = workloads.ragged_prefill(masked=masked)
    out, ref = run_prefill(case), oracle_prefill(case)
    assert_close(out, ref, what="ragged prefill masked=%s" % masked)
    assert_close(out, ref, atol=2e-3, what="ragged prefill masked=%s, secondary bar" % masked)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("ps", [1, 16, 5])
def test_prefill_group_sizes_and_pages(G, ps):
    case = workloads.prefill_case(300 + G + ps, 3, 2 * G, 2, 128, (0, 150), (1, 90), ps)
    assert_close(run_prefill(case), oracle_prefill(case), what="G=%d ps=%d" % (G, ps))


@pytest.mark.parametrize("ndim", [2, 3])
def test_prefill_masks_without_causality(ndim):
    case = workloads.prefill_case(310 + ndim, 4, 8, 2, 128, (0, 100), (1, 70), 16, mask_frac=0.3,
                                  mask_ndim=ndim, causal=False)
    assert_close(run_prefill(case, causal=False), oracle_prefill(case, causal=False), what="mask %dD" % ndim)


def test_prefill_mixed_causal_off_and_single_rows():
    case = workloads.prefill_case(320, 5, 16, 4, 128, None, None, 16, q_lens=[1, 17, 64, 1, 33],
                                  ctx_lens=[0, 5, 100, 300, 63], mask_frac=0.1)
    case["causal_offset"][1] = -1          # this sequence attends every key
    case["causal_offset"][3] = -1
    assert_close(run_prefill(case), oracle_prefill(case))


def test_prefill_fully_masked_rows_give_zero():
    case = workloads.prefill_case(330, 2, 8, 2, 128, None, None, 16, q_lens=[20, 9], ctx_lens=[40, 0],
                                  mask_frac=0.0, mask_ndim=3)
    case["mask"][0, 3, :] = False
    case["mask"][1, :, :] = False
    out = run_prefill(case).cpu()
    assert torch.equal(out[3], torch.zeros_like(out[3]))
    assert torch.equal(out[20:29], torch.zeros_like(out[20:29]))
    assert_close(out, oracle_prefill(case))


def test_prefill_skips_empty_sequences():
    case = workloads.prefill_case(340, 4, 8, 2, 128, None, None, 16, q_lens=[5, 0, 12, 0], ctx_lens=[3, 7, 0, 9])
    assert_close(run_prefill(case), oracle_prefill(case))


def test_prefill_page_head_slot_pool_layout():
    case = workloads.prefill_case(350, 3, 8, 2, 128, (0, 60), (1, 40), 16)
    # re-lay the pools as [P, Hkv, ps, D] and hand over the (page, slot, head, dim) view
    case["k_pool"] = case["k_pool"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    case["v_pool"] = case["v_pool"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    assert_close(run_prefill(case), oracle_prefill(case))


def test_prefill_repeat_runs_are_bit_identical():
    case = workloads.ragged_prefill(masked=True, seed=1015)
    a = run_prefill(case).clone()
    b = run_prefill(case)
    assert torch.equal(a, b)


@pytest.mark.parametrize("ps,G", [(1, 4), (3, 2), (1, 1)])
def test_prefill_long_context_spans_several_page_slices(ps, G):
    """The kernel stages at most 510 block-table entries at a time; with page
    size 1 that is 448 keys, with page size 3 1472 keys, so these contexts
    cross several slices, with ragged ends and a 3-D mask."""
    case = workloads.prefill_case(360 + ps + G, 2, 2 * G, 2, 128, None, None, ps,
                                  q_lens=[70, 37], ctx_lens=[1500, 1333], mask_frac=0.05)
    assert_close(run_prefill(case), oracle_prefill(case), what="ps=%d G=%d" % (ps, G))


# ------------------------------------------------ dense Q, contiguous KV
def dense_case(seed, B, Lq, Lk, Hq, Hkv, D=128, layout="blhd", mask_ndim=0, mask_frac=0.1):
    g = torch.Generator().manual_seed(seed)
    if layout == "blhd":
        q = torch.randn(B, Lq, Hq, D, generator=g).to(torch.bfloat16)
        k = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
        v = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
    else:   # bhld storage, (b, i, h, d) views
        q = torch.randn(B, Hq, Lq, D, generator=g).to(torch.bfloat16).permute(0, 2, 1, 3)
        k = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16).permute(0, 2, 1, 3)
        v = torch.randn(B, Hkv, Lk, D, generator=g).to(torch.bfloat16).permute(0, 2, 1, 3)
    mask = None
    if mask_ndim:
        pad = (Lk + 3) // 4 * 4
        shape = (B, Lq, pad) if mask_ndim == 3 else (B, pad)
        mask = torch.rand(*shape, generator=g) >= mask_frac
    return q, k, v, mask


def oracle_dense(q, k, v, kv_lens, is_causal, mask, scale):
    """The dense problem restated for the oracle's paged prefill: packed Q
    rows b*Lq + i, each sequence's K/V one page of Lk slots.  Bottom-right
    causality (key j for row i iff j <= n_b - Lq + i, which may admit no key
    when n_b < Lq) is given to the oracle as a 3-D keep-mask, ANDed with the
    caller's mask."""
    B, Lq, Hq, D = q.shape
    Lk = k.shape[1]
    qp = q.contiguous().reshape(B * Lq, Hq, D)
    bt = torch.arange(B, dtype=torch.int32).reshape(B, 1)
    indptr = torch.arange(0, (B + 1) * Lq, Lq, dtype=torch.int32)
    m = mask
    if is_causal:
        width = mask.shape[-1] if mask is not None else (Lk + 3) // 4 * 4
        j = torch.arange(width)[None, None, :]
        i = torch.arange(Lq)[None, :, None]
        keep = j <= (kv_lens.long() - Lq)[:, None, None] + i
        if mask is not None:
            keep = keep & (mask if mask.dim() == 3 else mask[:, None, :])
        m = keep.contiguous()
    out, _ = oracle.paged_prefill(qp, indptr, k.contiguous(), v.contiguous(), bt, kv_lens, scale,
                                  causal_offset=None, mask=m)
    return out.reshape(B, Lq, Hq, D)


@pytest.mark.parametrize("B,Lq,Lk,G,layout,causal,ndim", [
    (2, 200, 200, 4, "blhd", True, 0),
    (3, 70, 300, 4, "bhld", True, 0),
    (2, 130, 130, 1, "blhd", False, 0),
    (1, 64, 500, 8, "blhd", True, 2),
    (2, 33, 97, 2, "bhld", True, 3),
])
def test_dense_prefill_matches_oracle(B, Lq, Lk, G, layout, causal, ndim):
    Hkv = 2
    q, k, v, mask = dense_case(800 + B + Lq + G, B, Lq, Lk, Hkv * G, Hkv, layout=layout, mask_ndim=ndim)
    scale = 1.0 / math.sqrt(128)
    kv_lens = torch.full((B,), Lk, dtype=torch.int32)
    ref = oracle_dense(q, k, v, kv_lens, causal, mask, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=causal,
                    mask=None if mask is None else mask.to(DEV))
    torch.cuda.synchronize()
    assert_close(out, ref, what="dense B=%d Lq=%d Lk=%d G=%d %s" % (B, Lq, Lk, G, layout))


def test_dense_prefill_ragged_kv_lengths_and_short_sequences():
    """Per-sequence key counts below the stored Lk, one of them shorter than
    Lq under causality (its first rows admit no key and give zeros)."""
    B, Lq, Lk, Hkv, G = 3, 40, 260, 2, 4
    q, k, v, _ = dense_case(820, B, Lq, Lk, Hkv * G, Hkv)
    kv_lens = torch.tensor([260, 100, 25], dtype=torch.int32)
    scale = 1.0 / math.sqrt(128)
    ref = oracle_dense(q, k, v, kv_lens, True, None, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True, kv_lens=kv_lens.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out[2, :15].cpu(), torch.zeros(15, Hkv * G, 128, dtype=torch.bfloat16))
    assert_close(out, ref, what="ragged kv")


def test_decode_with_2d_mask_via_paged_prefill():
    """A decode step under a 2-D keep-mask [B, kv] runs as a paged prefill
    with one query row per sequence: equal to the oracle's masked decode."""
    case = workloads.paged_decode_case(860, 6, 32, 8, 128, [1, 300, 77, 1024, 5, 640], 16)
    B = case["B"]
    g = torch.Generator().manual_seed(861)
    width = (case["max_kv_len"] + 3) // 4 * 4
    mask = torch.rand(B, width, generator=g) >= 0.3
    mask[4, :] = False                                   # a sequence with every key masked
    ref, _ = oracle.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                 case["kv_lens"], case["scale"], mask=mask)
    R = pa.attn_prefill_tile_rows(128, 4)
    q_lens = [1] * B
    indptr, t2b, t2i = pa.attn_prefill_plan(q_lens, R)
    out = torch.full((B, 32, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_paged_prefill(case["q"].to(DEV), indptr.to(DEV), t2b.to(DEV), t2i.to(DEV), case["k_pool"].to(DEV),
                          case["v_pool"].to(DEV), case["block_table"].to(DEV), case["kv_lens"].to(DEV), out, 16,
                          case["scale"], causal_offset=None, mask=mask.to(DEV), tile_rows=R)
    torch.cuda.synchronize()
    assert torch.equal(out[4].cpu(), torch.zeros(32, 128, dtype=torch.bfloat16))
    assert_close(out, ref, what="masked decode")


@pytest.mark.parametrize("G,ps,mask_ndim", [(4, 16, None), (2, 5, 3), (8, 16, 2), (1, 1, None)])
def test_prefill_head_dim_64(G, ps, mask_ndim):
    case = workloads.prefill_case(880 + G + ps, 3, 2 * G, 2, 64, (0, 300), (1, 140), ps,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    assert_close(run_prefill(case), oracle_prefill(case), what="D=64 G=%d ps=%d" % (G, ps))


def test_dense_prefill_head_dim_64():
    B, Lq, Lk, Hkv, G = 2, 150, 400, 2, 4
    q, k, v, _ = dense_case(890, B, Lq, Lk, Hkv * G, Hkv, D=64, layout="bhld")
    kv_lens = torch.full((B,), Lk, dtype=torch.int32)
    scale = 1.0 / math.sqrt(64)
    ref = oracle_dense(q, k, v, kv_lens, True, None, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True)
    torch.cuda.synchronize()
    assert_close(out, ref, what="dense D=64")


@pytest.mark.parametrize("G,ps,mask_ndim", [(4, 16, None), (2, 3, 2), (8, 16, 3)])
def test_prefill_head_dim_32(G, ps, mask_ndim):
    case = workloads.prefill_case(895 + G + ps, 3, 2 * G, 2, 32, (0, 300), (1, 140), ps,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    assert_close(run_prefill(case), oracle_prefill(case), what="D=32 G=%d ps=%d" % (G, ps))


# ------------------------------------------------------------ split KV
def nan_workspace(nbytes):
    """Workspace filled with 0xFF bytes (every float a NaN): a partial the
    kernel failed to write would poison the combine."""
    return torch.full((max(nbytes, 1),), 0xFF, dtype=torch.uint8, device=DEV)


def run_prefill_split(case, S, causal=True):
    G = case["Hq"] // case["Hkv"]
    R = pa.attn_prefill_tile_rows(case["D"], G)
    _, t2b, t2i = pa.attn_prefill_plan(case["q_lens"], R)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "qo_indptr",
                                     "causal_offset")}
    mask = case["mask"].to(DEV) if case["mask"] is not None else None
    total_q = d["q"].shape[0]
    ws = nan_workspace(pa.attn_prefill_workspace_bytes(total_q, case["Hq"], case["D"], S))
    out = torch.full_like(d["q"], float("nan"))
    pa.attn_paged_prefill_split(d["q"], d["qo_indptr"], t2b.to(DEV), t2i.to(DEV), d["k_pool"], d["v_pool"],
                                d["block_table"], d["kv_lens"], out, case["page_size"], case["scale"],
                                max(case["kv_lens"].tolist() + [0]),
                                causal_offset=d["causal_offset"] if causal else None, mask=mask,
                                num_splits=S, workspace=ws, tile_rows=R)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G,ps,S,D,mask_ndim", [
    (8, 16, 4, 128, None),
    (4, 16, 3, 128, 3),
    (2, 5, 7, 128, 2),
    (1, 1, 2, 128, None),
    (8, 3, 5, 64, 3),
    (4, 16, 6, 32, None),
    (8, 16, 1, 128, None),
])
def test_split_prefill_matches_oracle(G, ps, S, D, mask_ndim):
    """Short query runs over long contexts, keys split over S workgroups per
    tile (S = 1 runs the plain kernel through the split entry point)."""
    case = workloads.prefill_case(900 + G + ps + S + D, 3, 2 * G, 2, D, None, None, ps,
                                  q_lens=[16, 5, 1], ctx_lens=[1200, 777, 1600],
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    # Over ~1000 keys the outputs are ~0.03 in size; the absolute bar is
    # tightened to 2e-3 (rounding of P to bf16 contributes ~1e-4 here).
    assert_close(run_prefill_split(case, S), oracle_prefill(case), atol=2e-3,
                 what="split G=%d ps=%d S=%d D=%d" % (G, ps, S, D))


def test_split_prefill_more_splits_than_key_tiles():
    """Splits past a tile's last key tile hold no key: they write an empty
    partial (m = -inf, l = 0) that the combine ignores; causal frontiers and a
    sequence without keys give the oracle's zeros."""
    case = workloads.prefill_case(930, 4, 16, 2, 128, None, None, 16, q_lens=[40, 3, 70, 9],
                                  ctx_lens=[10, 0, 200, 0])
    case["causal_offset"][3] = -1
    out = run_prefill_split(case, 9)
    assert_close(out, oracle_prefill(case), what="S=9 short contexts")


def test_split_prefill_fully_masked_rows_give_zero():
    case = workloads.prefill_case(935, 2, 8, 2, 128, None, None, 16, q_lens=[20, 9], ctx_lens=[900, 500],
                                  mask_frac=0.0, mask_ndim=3)
    case["mask"][0, 3, :] = False
    case["mask"][1, :, :] = False
    out = run_prefill_split(case, 4).cpu()
    assert torch.equal(out[3], torch.zeros_like(out[3]))
    assert torch.equal(out[20:29], torch.zeros_like(out[20:29]))
    assert_close(out, oracle_prefill(case))


@pytest.mark.parametrize("B,Lq,Lk,G,layout,S,ndim", [
    (2, 16, 1500, 8, "blhd", 4, 0),
    (3, 40, 900, 4, "bhld", 3, 3),
    (2, 1, 2000, 2, "blhd", 8, 2),
])
def test_dense_split_prefill_matches_oracle(B, Lq, Lk, G, layout, S, ndim):
    Hkv = 2
    q, k, v, mask = dense_case(940 + B + Lq + S, B, Lq, Lk, Hkv * G, Hkv, layout=layout, mask_ndim=ndim)
    scale = 1.0 / math.sqrt(128)
    kv_lens = torch.tensor([Lk - 7 * b for b in range(B)], dtype=torch.int32)
    ref = oracle_dense(q, k, v, kv_lens, True, mask, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = nan_workspace(pa.attn_prefill_workspace_bytes(B * Lq, Hkv * G, 128, S))
    pa.attn_prefill_split(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True, kv_lens=kv_lens.to(DEV),
                          mask=None if mask is None else mask.to(DEV), num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, ref, atol=2e-3, what="dense split B=%d Lq=%d Lk=%d G=%d S=%d" % (B, Lq, Lk, G, S))


def test_split_prefill_short_q_long_kv_workload():
    """G = 8, 16 sequences of 16 new rows after 16368 cached keys (Hq = 32,
    Hkv = 4, D = 128, page size 16), planner-chosen splits, in the launch
    configuration the benchmark times.  Every row of all 16 sequences is
    checked against the oracle, for the split and the unsplit kernel, at
    the 1e-2 bar and at a secondary absolute bar of 1e-3: the outputs
    average 16384 values (~0.01 in size), so 1e-2 alone would hide a
    mis-weighted split piece."""
    case = workloads.short_q_prefill(device=DEV)
    G = case["Hq"] // case["Hkv"]
    R = pa.attn_prefill_tile_rows(128, G)
    _, t2b, t2i = pa.attn_prefill_plan(case["q_lens"], R)
    t2b, t2i = t2b.to(DEV), t2i.to(DEV)
    args = (case["q"], case["qo_indptr"], t2b, t2i, case["k_pool"], case["v_pool"], case["block_table"],
            case["kv_lens"])
    S = pa.attn_prefill_plan_splits(t2b.numel(), case["Hq"], case["Hkv"], 128, max(case["kv_lens"].tolist()))
    assert S > 1
    out_s = torch.full_like(case["q"], float("nan"))
    pa.attn_paged_prefill_split(*args, out_s, 16, case["scale"], max(case["kv_lens"].tolist()),
                                causal_offset=case["causal_offset"], num_splits=S, tile_rows=R)
    out_1 = torch.full_like(case["q"], float("nan"))
    pa.attn_paged_prefill(*args, out_1, 16, case["scale"], causal_offset=case["causal_offset"], tile_rows=R)
    torch.cuda.synchronize()
    # every row of every sequence against the oracle, split and unsplit
    cpu = {k: case[k].cpu() for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "causal_offset",
                                     "qo_indptr")}
    ref, _ = oracle.paged_prefill(cpu["q"], cpu["qo_indptr"], cpu["k_pool"], cpu["v_pool"], cpu["block_table"],
                                  cpu["kv_lens"], case["scale"], causal_offset=cpu["causal_offset"], mask=None)
    for label, out in (("split S=%d" % S, out_s), ("unsplit", out_1)):
        assert_close(out, ref, what=label + " vs oracle")
        assert_close(out, ref, atol=1e-3, rtol=1e-2, what=label + " vs oracle, secondary bar")


# ------------------------------------------ group sizes beyond 1, 2, 4, 8
@pytest.mark.parametrize("Hq,Hkv,ps,mask_ndim", [
    (6, 2, 16, None),      # G = 3: one head per workgroup, three workgroups per KV head
    (12, 2, 5, 3),         # G = 6: two heads packed
    (24, 2, 16, 2),        # G = 12: four heads packed
    (32, 1, 16, None),     # G = 32: eight heads packed, four workgroups per KV head
    (16, 1, 3, 3),         # G = 16
])
def test_prefill_any_group_size(Hq, Hkv, ps, mask_ndim):
    """The pages verify head packing for G in {1, 2, 3, 4, 8, 32}; any G runs
    here, packing the largest power of two dividing it (at most 8)."""
    case = workloads.prefill_case(960 + Hq + ps, 3, Hq, Hkv, 128, (0, 300), (1, 140), ps,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    assert_close(run_prefill(case), oracle_prefill(case), what="Hq=%d Hkv=%d" % (Hq, Hkv))


@pytest.mark.parametrize("Hq,Hkv,S", [(32, 1, 4), (6, 2, 3)])
def test_split_prefill_any_group_size(Hq, Hkv, S):
    case = workloads.prefill_case(970 + Hq + S, 3, Hq, Hkv, 128, None, None, 16,
                                  q_lens=[16, 3, 9], ctx_lens=[1000, 2000, 50])
    assert_close(run_prefill_split(case, S), oracle_prefill(case), atol=2e-3, what="split Hq=%d Hkv=%d" % (Hq, Hkv))


def test_dense_prefill_group_size_3():
    B, Lq, Lk, Hkv, G = 2, 50, 300, 2, 3
    q, k, v, _ = dense_case(980, B, Lq, Lk, Hkv * G, Hkv)
    kv_lens = torch.full((B,), Lk, dtype=torch.int32)
    scale = 1.0 / math.sqrt(128)
    ref = oracle_dense(q, k, v, kv_lens, True, None, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True)
    torch.cuda.synchronize()
    assert_close(out, ref, what="dense G=3")


# ------------------------------------------------------------ head dim 256
@pytest.mark.parametrize("G,ps,mask_ndim", [(4, 16, None), (8, 5, 3), (1, 1, 2), (2, 16, 3), (3, 16, None)])
def test_prefill_head_dim_256(G, ps, mask_ndim):
    """D = 256 runs one team of four waves with one 16-row block each (at
    most four heads packed; G = 8 takes two workgroups per KV head)."""
    case = workloads.prefill_case(990 + G + ps, 3, 2 * G, 2, 256, (0, 300), (1, 140), ps,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    assert_close(run_prefill(case), oracle_prefill(case), what="D=256 G=%d ps=%d" % (G, ps))


def test_prefill_head_dim_256_long_context():
    case = workloads.prefill_case(995, 2, 8, 2, 256, None, None, 3, q_lens=[70, 37], ctx_lens=[1500, 1333],
                                  mask_frac=0.05)
    assert_close(run_prefill(case), oracle_prefill(case), atol=2e-3, what="D=256 long")


@pytest.mark.parametrize("S", [1, 5])
def test_split_prefill_head_dim_256(S):
    case = workloads.prefill_case(996 + S, 3, 16, 2, 256, None, None, 16, q_lens=[16, 5, 1],
                                  ctx_lens=[1200, 777, 1600])
    assert_close(run_prefill_split(case, S), oracle_prefill(case), atol=2e-3, what="split D=256 S=%d" % S)


def test_dense_prefill_head_dim_256():
    B, Lq, Lk, Hkv, G = 2, 90, 300, 2, 4
    q, k, v, mask = dense_case(997, B, Lq, Lk, Hkv * G, Hkv, D=256, layout="bhld", mask_ndim=3)
    kv_lens = torch.tensor([300, 120], dtype=torch.int32)
    scale = 1.0 / math.sqrt(256)
    ref = oracle_dense(q, k, v, kv_lens, True, mask, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True, kv_lens=kv_lens.to(DEV),
                    mask=mask.to(DEV))
    torch.cuda.synchronize()
    assert_close(out, ref, what="dense D=256")


# ------------------------------------- one team per workgroup (full grids)
def grid_workgroups(case, S=1):
    G = case["Hq"] // case["Hkv"]
    R = pa.attn_prefill_tile_rows(case["D"], G)
    if case["D"] <= 128:
        hp = 8 if R == 16 else 128 // R      # heads packed per workgroup
    else:
        hp = 64 // R
    tiles = sum((q + R - 1) // R for q in case["q_lens"])
    return tiles * case["Hkv"] * (G // hp) * S


@pytest.mark.parametrize("G,D,mask_ndim,ps", [
    (4, 128, None, 16), (4, 128, 3, 5), (8, 128, 2, 16), (2, 64, 3, 16), (1, 32, None, 3), (3, 128, None, 16),
])
def test_prefill_full_grid_one_team(G, D, mask_ndim, ps):
    """Grids of more than one workgroup per two compute units run one team of
    four waves per workgroup (two workgroups share a CU); many short
    sequences give such a grid at a size the oracle finishes quickly.  (The
    small cases above run two teams.)"""
    Hkv = 8
    case = workloads.prefill_case(1100 + G * D + ps, 96, Hkv * G, Hkv, D, (0, 120), (20, 70), ps,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert grid_workgroups(case) >= 2 * cus
    assert_close(run_prefill(case), oracle_prefill(case), what="full grid G=%d D=%d" % (G, D))


@pytest.mark.parametrize("G,D,mask_ndim", [(4, 128, None), (2, 64, 3), (1, 32, None)])
def test_prefill_one_team_output_rows_only_8_byte_aligned(G, D, mask_ndim):
    """One-team grids stage each wave's output rows in LDS and write whole
    rows with 16-byte stores when the output rows are 16-byte aligned.  Here
    the output is a view 4 elements into a flat buffer (rows 8-byte aligned
    only), so the kernel writes its 8-byte pieces directly: same result, and
    nothing written outside the view.  The aligned path is the one every
    other one-team test above takes."""
    Hkv = 8
    case = workloads.prefill_case(1200 + G * D, 96, Hkv * G, Hkv, D, (0, 120), (20, 70), 16,
                                  mask_frac=None if mask_ndim is None else 0.2, mask_ndim=mask_ndim or 3)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert grid_workgroups(case) >= 2 * cus
    R = pa.attn_prefill_tile_rows(D, G)
    _, t2b, t2i = pa.attn_prefill_plan(case["q_lens"], R)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "qo_indptr",
                                     "causal_offset")}
    mask = case["mask"].to(DEV) if case["mask"] is not None else None
    n = d["q"].numel()
    flat = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)
    out = flat[4:4 + n].view(d["q"].shape)
    assert out.data_ptr() % 16 == 8
    pa.attn_paged_prefill(d["q"], d["qo_indptr"], t2b.to(DEV), t2i.to(DEV), d["k_pool"], d["v_pool"],
                          d["block_table"], d["kv_lens"], out, 16, case["scale"],
                          causal_offset=d["causal_offset"], mask=mask, tile_rows=R)
    torch.cuda.synchronize()
    assert_close(out, oracle_prefill(case), what="8-byte aligned output G=%d D=%d" % (G, D))
    assert torch.equal(flat[:4].cpu(), torch.zeros(4, dtype=torch.bfloat16))
    assert torch.equal(flat[4 + n:].cpu(), torch.zeros(4, dtype=torch.bfloat16))


def test_split_prefill_full_grid_one_team():
    case = workloads.prefill_case(1150, 64, 32, 8, 128, (100, 900), (1, 40), 16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert grid_workgroups(case, 4) >= 2 * cus
    assert_close(run_prefill_split(case, 4), oracle_prefill(case), atol=2e-3, what="split full grid")


def test_dense_split_prefill_rows_without_keys():
    """Bottom-right causality with sequences shorter than Lq: early rows admit
    no key in any split, so every partial is empty and the combine writes 0."""
    B, Lq, Lk, Hkv, G, S = 2, 48, 600, 2, 4, 3
    q, k, v, _ = dense_case(1200, B, Lq, Lk, Hkv * G, Hkv)
    kv_lens = torch.tensor([600, 20], dtype=torch.int32)
    scale = 1.0 / math.sqrt(128)
    ref = oracle_dense(q, k, v, kv_lens, True, None, scale)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = nan_workspace(pa.attn_prefill_workspace_bytes(B * Lq, Hkv * G, 128, S))
    pa.attn_prefill_split(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True, kv_lens=kv_lens.to(DEV),
                          num_splits=S, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out[1, :28].cpu(), torch.zeros(28, Hkv * G, 128, dtype=torch.bfloat16))
    assert_close(out, ref, what="dense split, rows without keys")
