"""Seeded random shapes across the supported space, each checked against the
CPU oracle: decode (paged and contiguous) and prefill (paged and dense,
split and unsplit) with random head dims, group sizes, page sizes, pool
layouts, lengths, split counts, masks and causality.  Same bar as the other
parity tests (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|)."""
import math
import random

import pytest
import torch

import oracle
import paged_kv_gqa_03_amd as pa
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
DIMS = [32, 64, 128, 256]
GROUPS = [1, 2, 3, 4, 6, 8, 16]


def assert_close(got, ref, what):
    got = got.detach().to("cpu", torch.float64)
    err = (got - ref).abs()
    bad = err > 1e-2 + 1e-2 * ref.abs()
    assert not bool(bad.any()), "%s: %d of %d off, max err %.4g" % (what, int(bad.sum()), bad.numel(),
                                                                    float(err.max()))


@pytest.mark.parametrize("seed", range(40))
def test_random_paged_decode(seed):
    r = random.Random(7000 + seed)
    D, G, Hkv = r.choice(DIMS), r.choice(GROUPS), r.choice([1, 2, 4, 8])
    ps = r.choice([1, 3, 8, 16, 32])
    B = r.randint(1, 9)
    lens = [r.choice([0, 1, r.randint(2, 64), r.randint(65, 1500)]) for _ in range(B)]
    layout = r.choice(["page_slot_head", "page_head_slot"])
    S = r.choice([0, 1, r.randint(2, 40)])
    what = "D=%d G=%d Hkv=%d ps=%d lens=%s %s S=%d" % (D, G, Hkv, ps, lens, layout, S)
    case = workloads.paged_decode_case(7100 + seed, B, Hkv * G, Hkv, D, lens, ps, layout=layout)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens")}
    out = torch.full_like(d["q"], float("nan"))
    pa.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"], case["max_kv_len"], out,
                         ps, case["scale"], num_splits=S)
    torch.cuda.synchronize()
    ref, _ = oracle.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"], case["kv_lens"],
                                 case["scale"])
    assert_close(out, ref, what)


@pytest.mark.parametrize("seed", range(16))
def test_random_contiguous_decode(seed):
    r = random.Random(7200 + seed)
    D, G, Hkv = r.choice(DIMS), r.choice(GROUPS), r.choice([1, 2, 4, 8])
    B, L = r.randint(1, 6), r.randint(1, 900)
    lens = [r.randint(0, L) for _ in range(B)]
    layout = r.choice(["bhld", "blhd"])
    what = "D=%d G=%d Hkv=%d L=%d lens=%s %s" % (D, G, Hkv, L, lens, layout)
    case = workloads.contig_decode_case(7300 + seed, B, Hkv * G, Hkv, D, L, device=DEV, layout=layout, kv_lens=lens)
    # Half the cases give no kv_lens (every row has L keys): the planner may
    # then take one slice per row, and a slice count dividing the rows
    # launches no combine.
    one_length = r.random() < 0.5
    S = r.choice([0, 0, 1, 2, 3, 4, 6, 7, 8, 12, 16])
    what += " one_length=%s S=%d" % (one_length, S)
    out = torch.full_like(case["q"], float("nan"))
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"],
                   kv_lens=None if one_length else case["kv_lens"], num_splits=S)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"],
                           kv_lens=None if one_length else case["kv_lens"].cpu())
    assert_close(out, ref, what)


@pytest.mark.parametrize("seed", range(40))
def test_random_paged_prefill(seed):
    r = random.Random(7400 + seed)
    D, G, Hkv = r.choice(DIMS), r.choice(GROUPS), r.choice([1, 2, 4])
    Hkv = max(1, min(Hkv, 32 // G))      # at most 32 query heads (oracle time)
    ps = r.choice([1, 4, 5, 16])
    B = r.randint(1, 5)
    q_lens = [r.choice([0, 1, r.randint(2, 40), r.randint(41, 200)]) for _ in range(B)]
    ctx = [r.choice([0, r.randint(1, 100), r.randint(101, 900)]) for _ in range(B)]
    mask_ndim = r.choice([0, 2, 3])
    causal = r.random() < 0.7
    S = r.choice([1, 1, 2, r.randint(3, 9)])
    what = "D=%d G=%d Hkv=%d ps=%d q=%s ctx=%s mask=%d causal=%s S=%d" % (D, G, Hkv, ps, q_lens, ctx, mask_ndim,
                                                                      causal, S)
    case = workloads.prefill_case(7500 + seed, B, Hkv * G, Hkv, D, None, None, ps, q_lens=q_lens, ctx_lens=ctx,
                                  mask_frac=0.2 if mask_ndim else None, mask_ndim=mask_ndim or 3, causal=causal)
    R = pa.attn_prefill_tile_rows(D, G)
    _, t2b, t2i = pa.attn_prefill_plan(q_lens, R)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "qo_indptr",
                                     "causal_offset")}
    mask = case["mask"].to(DEV) if case["mask"] is not None else None
    out = torch.full_like(d["q"], float("nan"))
    if sum(q_lens) > 0:
        pa.attn_paged_prefill_split(d["q"], d["qo_indptr"], t2b.to(DEV), t2i.to(DEV), d["k_pool"], d["v_pool"],
                                    d["block_table"], d["kv_lens"], out, ps, case["scale"],
                                    max(case["kv_lens"].tolist()), causal_offset=d["causal_offset"], mask=mask,
                                    num_splits=S, tile_rows=R)
    torch.cuda.synchronize()
    ref, _ = oracle.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"], case["block_table"],
                                  case["kv_lens"], case["scale"], causal_offset=case["causal_offset"],
                                  mask=case["mask"])
    assert_close(out, ref, what)


@pytest.mark.parametrize("seed", range(16))
def test_random_dense_prefill(seed):
    r = random.Random(7600 + seed)
    D, G, Hkv = r.choice(DIMS), r.choice(GROUPS), r.choice([1, 2])
    B, Lq = r.randint(1, 3), r.randint(1, 150)
    Lk = r.randint(max(1, Lq // 2), 600)
    lens = [r.randint(0, Lk) for _ in range(B)]
    causal = r.random() < 0.7
    S = r.choice([1, 1, r.randint(2, 6)])
    what = "D=%d G=%d B=%d Lq=%d Lk=%d lens=%s causal=%s S=%d" % (D, G, B, Lq, Lk, lens, causal, S)
    g = torch.Generator().manual_seed(7700 + seed)
    q = torch.randn(B, Lq, Hkv * G, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
    kv_lens = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(D)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill_split(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=causal, kv_lens=kv_lens.to(DEV),
                          num_splits=S)
    torch.cuda.synchronize()
    # the oracle's paged prefill over one page of Lk slots per sequence;
    # bottom-right causality given as a 3-D keep-mask
    qp = q.reshape(B * Lq, Hkv * G, D)
    bt = torch.arange(B, dtype=torch.int32).reshape(B, 1)
    indptr = torch.arange(0, (B + 1) * Lq, Lq, dtype=torch.int32)
    m = None
    if causal:
        width = (Lk + 3) // 4 * 4
        j = torch.arange(width)[None, None, :]
        i = torch.arange(Lq)[None, :, None]
        m = (j <= (kv_lens.long() - Lq)[:, None, None] + i).contiguous()
    ref, _ = oracle.paged_prefill(qp, indptr, k, v, bt, kv_lens, scale, causal_offset=None, mask=m)
    assert_close(out, ref.reshape(B, Lq, Hkv * G, D), what)


@pytest.mark.parametrize("seed", range(16))
def test_random_swa_fp8_decode(seed):
    """fp8 sliding-window decode (K = V, head dim 512): random token counts,
    head groups, windows (several 128-position tiles), lengths, masked slots
    and block sizes."""
    r = random.Random(7800 + seed)
    T, NH = r.randint(1, 12), 16 * r.randint(1, 4)
    W = r.choice([1, 17, 64, 128, 200, 384])
    bs, nb = r.choice([16, 64, 256]), r.randint(1, 6)
    slots = bs * nb
    lens = [r.choice([0, 1, r.randint(1, W), W, W + r.randint(1, 50)]) for _ in range(T)]
    lens = [min(n, slots) for n in lens]        # distinct slots per token
    neg = r.choice([0.0, 0.0, 0.2])
    what = "T=%d NH=%d W=%d bs=%d nb=%d lens=%s neg=%.1f" % (T, NH, W, bs, nb, lens, neg)
    case = workloads.swa_case(7900 + seed, T, NH, 512, W, bs, nb, lens=lens, neg_frac=neg)
    d = {k: case[k].to(DEV) for k in ("q", "cache", "inv_scale", "indices", "lens")}
    out = torch.full_like(d["q"], float("nan"))
    pa.attn_swa_fp8_decode(d["q"], d["cache"], d["inv_scale"], d["indices"], d["lens"], out, bs, case["scale"])
    torch.cuda.synchronize()
    ref, _ = oracle.swa_fp8_decode(case["q"], case["cache"], case["inv_scale"], case["indices"], case["lens"], bs,
                                   case["scale"])
    assert_close(out, ref, what)
