"""GPU parity of split-KV decode and the combine against the CPU oracle.

Bar: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise on bf16 outputs; the
fp32 combine is held to 1e-5 + 1e-5 |ref| against the oracle's fp64 combine
of the same fp32 partials."""
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


def assert_decode_close(got, ref, lens, what=""):
    """The 1e-2 + 1e-2 |ref| bar on every element, and the secondary 2e-3
    absolute bar on sequences of at least 256 keys, whose outputs are long
    averages.  Softmax weights are rounded to bf16 (u = 2^-8) before P.V, so
    a row's error is a weighted mean of independent relative errors: its
    standard deviation is about u / sqrt(3 n) times the spread of V, near
    2e-4 at n = 256, while a row of a few keys can err by u max|v - out|."""
    assert_close(got, ref, what=what)
    long_rows = torch.tensor([int(n) >= 256 for n in lens], dtype=torch.bool)
    if bool(long_rows.any()):
        assert_close(got.detach().cpu()[long_rows], ref[long_rows], atol=2e-3, what=what + ", rows >= 256 keys")


def to_dev(case, keys):
    return {k: (case[k].to(DEV) if torch.is_tensor(case[k]) else case[k]) for k in keys}


def run_paged(case, S=0, workspace=None, out=None):
    d = to_dev(case, ["q", "k_pool", "v_pool", "block_table", "kv_lens"])
    out = torch.empty_like(d["q"]) if out is None else out
    pa.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"],
                         case["max_kv_len"], out, case["page_size"], case["scale"], num_splits=S,
                         workspace=workspace)
    torch.cuda.synchronize()
    return out


def oracle_paged(case):
    return oracle.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                               case["kv_lens"], case["scale"])


@pytest.mark.parametrize("S", [0, 1, 2, 3, 19])
def test_tiny_paged_decode(S):
    case = workloads.tiny_paged_decode()
    ref, _ = oracle_paged(case)
    assert_close(run_paged(case, S), ref, what="tiny S=%d" % S)


@pytest.mark.parametrize("G,D,ps,lens", [
    (1, 64, 16, [1, 15, 16, 17, 100]),
    (2, 128, 1, [33, 7, 250]),
    (4, 128, 3, [0, 5, 48, 301]),
    (8, 128, 16, [64, 200, 1000]),
    (8, 64, 64, [700, 63, 65]),
    (4, 64, 7, [129, 1]),
    (4, 128, 32, [513, 2000, 1]),
])
@pytest.mark.parametrize("S", [0, 1, 4])
def test_paged_decode_shapes(G, D, ps, lens, S):
    Hkv = 2
    case = workloads.paged_decode_case(100 + G * 7 + D + ps, len(lens), Hkv * G, Hkv, D, lens, ps)
    ref, _ = oracle_paged(case)
    assert_close(run_paged(case, S), ref, what="G=%d D=%d ps=%d S=%d" % (G, D, ps, S))


def test_paged_decode_empty_sequences_give_zero():
    case = workloads.paged_decode_case(7, 3, 8, 2, 128, [0, 40, 0], 16)
    for S in (1, 3):
        out = run_paged(case, S)
        assert torch.equal(out[0].cpu(), torch.zeros_like(out[0].cpu()))
        assert torch.equal(out[2].cpu(), torch.zeros_like(out[2].cpu()))
        ref, _ = oracle_paged(case)
        assert_close(out, ref)


def test_paged_decode_page_head_slot_layout():
    case = workloads.paged_decode_case(8, 4, 32, 8, 128, [77, 512, 1, 333], 16, layout="page_head_slot")
    ref, _ = oracle_paged(case)
    assert_close(run_paged(case, 0), ref)


@pytest.mark.parametrize("B", [32, 128])
def test_serving_paged_decode(B):
    """Config 3 at B = 32 and at B = 128 (the timed configuration, planner
    split count), every sequence and head against the oracle.  Besides the
    1e-2 pass bar, a secondary absolute bar of 2e-3: outputs average up to
    4096 values and are ~0.02 in size, where 1e-2 alone would hide a
    mis-weighted piece."""
    case = workloads.serving_paged_decode(B, device=DEV)
    out = run_paged(case, 0)
    cpu = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in case.items()}
    ref, _ = oracle_paged(cpu)
    assert_close(out, ref, what="B=%d serving" % B)
    assert_close(out, ref, atol=2e-3, what="B=%d serving, secondary bar" % B)


@pytest.mark.parametrize("Hq,Hkv,seed", [(64, 8, 1012), (32, 1, 1013)])
def test_mfma_serving_paged_decode(Hq, Hkv, seed):
    """The MFMA decode at the size its bench lines time: B = 128, kv_lens
    U[512, 4096], page size 16, planner split count; G = 8 (four KV heads a
    row, one wave each) and G = 32 (one KV head a row, 32 query heads on two
    16-row blocks).  Every sequence and head against the oracle, at the pass
    bar and the secondary 2e-3 bar (every row has at least 512 keys)."""
    case = workloads.paged_decode_case(seed, 128, Hq, Hkv, 128, (512, 4096), 16, device=DEV)
    out = run_paged(case, 0)
    cpu = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in case.items()}
    ref, _ = oracle_paged(cpu)
    assert_close(out, ref, what="Hq=%d Hkv=%d serving" % (Hq, Hkv))
    assert_close(out, ref, atol=2e-3, what="Hq=%d Hkv=%d serving, secondary bar" % (Hq, Hkv))


def partition_bounds(lens, rows_per_seq, W):
    """Per row: (slot, first key, end key) of each piece under the balanced
    partition (rows laid end to end, W equal slices of the line, the piece of
    row r in slice w at slot r + w)."""
    n_rows = [n for n in lens for _ in range(rows_per_seq)]
    T = sum(n_rows)
    bounds = [w * T // W for w in range(W + 1)]
    out, P = [], 0
    for r, n in enumerate(n_rows):
        pieces = []
        for w in range(W):
            lo, hi = max(bounds[w], P), min(bounds[w + 1], P + n)
            if lo < hi:
                pieces.append((r + w, lo - P, hi - P))
        out.append(pieces)
        P += n
    return out


@pytest.mark.parametrize("B,Hkv,G,layout,W", [
    (32, 8, 4, "page_slot_head", 0),     # config 3 B = 32, planner slices: eight KV heads per row
    (5, 2, 4, "page_head_slot", 23),     # one KV head per row
    (5, 2, 8, "page_slot_head", 23),     # MFMA rows: both KV heads (a wave each), 16 query heads per row
])
def test_split_pieces_match_oracle_partials(B, Hkv, G, layout, W):
    """Each piece the split kernel leaves in the workspace (read through the
    documented slot layout) against the oracle's fp64 partial over the same
    key range: lse = m + ln l and o / l per piece (m is a lazily raised
    reference, so only these two are unique)."""
    Hq, D = Hkv * G, 128
    if B == 32:
        case = workloads.serving_paged_decode(32)
    else:
        case = workloads.paged_decode_case(120, B, Hq, Hkv, D, [1, 700, 0, 2500, 65], 16, layout=layout)
    lens = case["kv_lens"].tolist()
    if G in (1, 2, 4):
        hw = Hkv if layout == "page_slot_head" else 1    # KV heads per row, VALU kernel
    else:
        hw = 4 if Hkv % 4 == 0 else 2 if Hkv % 2 == 0 else 1   # MFMA kernel, one pass
    W = W or pa.attn_plan_splits(B, Hkv, G, D, case["max_kv_len"], 16, case["k_pool"].stride(2))
    d = to_dev(case, ["q", "k_pool", "v_pool", "block_table", "kv_lens"])
    nbytes = pa.attn_decode_workspace_bytes(B, Hq, D, W)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    pa.attn_paged_decode_split(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"],
                               case["max_kv_len"], 16, case["scale"], W, ws)
    torch.cuda.synchronize()
    rows_total = (B + W) * Hq
    o_bytes = rows_total * D * 4
    ml_off = (o_bytes + 255) // 256 * 256
    o_all = ws[:o_bytes].view(torch.float32).view(rows_total, D).cpu().double()
    ml_all = ws[ml_off:ml_off + rows_total * 8].view(torch.float32).view(rows_total, 2).cpu().double()
    ngrp = Hkv // hw
    heads_per_row = hw * G
    pieces = partition_bounds(lens, ngrp, W)
    S = max(1, max(len(p) for p in pieces))
    # oracle partials: per sequence and row group the same chunk bounds; rows
    # of one sequence share its keys, so one bounds row per (sequence, group)
    # is evaluated as its own oracle call on that group's heads
    n_checked = 0
    for grp in range(ngrp):
        bnd = torch.zeros(B, S + 1, dtype=torch.int32)
        for b in range(B):
            ps_ = pieces[b * ngrp + grp]
            edges = [0] + [hi for _, _, hi in ps_]
            edges = edges + [edges[-1]] * (S + 1 - len(edges))
            bnd[b] = torch.tensor(edges, dtype=torch.int32)
        o_ref, m_ref, l_ref = oracle.paged_decode_partials(case["q"], case["k_pool"], case["v_pool"],
                                                           case["block_table"], case["kv_lens"], bnd, case["scale"])
        for b in range(B):
            for s_i, (slot, lo, hi) in enumerate(pieces[b * ngrp + grp]):
                h0 = grp * heads_per_row
                rows = slice(slot * heads_per_row, (slot + 1) * heads_per_row)
                m_g, l_g, o_g = ml_all[rows, 0], ml_all[rows, 1], o_all[rows]
                lse_g = m_g + torch.log(l_g)
                mr, lr, orf = (m_ref[s_i, b, h0:h0 + heads_per_row], l_ref[s_i, b, h0:h0 + heads_per_row],
                               o_ref[s_i, b, h0:h0 + heads_per_row])
                lse_r = mr + torch.log(lr)
                what = "b=%d grp=%d piece %d [%d, %d)" % (b, grp, s_i, lo, hi)
                # The kernel rounds each weight exp(s - m) to bf16 (unit
                # roundoff 2^-8) and sums the rounded weights into l, so lse
                # is within ln(1 + 2^-8) < 2^-8 of the exact value; o / l is
                # a convex combination of V rows with weights perturbed by
                # <= 2^-8, within the 1e-2 pass bar, and pieces of >= 256
                # keys (where the perturbations average out) also within
                # the secondary 2e-3 bar.
                assert_close(lse_g, lse_r, atol=2.0 ** -8, rtol=0, what=what + " lse")
                assert_close(o_g / l_g[:, None], orf / lr[:, None], what=what + " o / l")
                if hi - lo >= 256:
                    assert_close(o_g / l_g[:, None], orf / lr[:, None], atol=2e-3, what=what + " o / l, 2e-3")
                n_checked += 1
    assert n_checked >= B * ngrp


@pytest.mark.parametrize("layout", ["bhld", "blhd"])
def test_contiguous_decode(layout):
    if layout == "bhld":
        case = workloads.contiguous_decode(device=DEV)
    else:
        case = workloads.contig_decode_case(9, 4, 32, 8, 128, 600, device=DEV, layout="blhd")
    out = torch.empty_like(case["q"])
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"])
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"])
    assert_close(out, ref, what="contiguous " + layout)
    assert_close(out, ref, atol=2e-3, what="contiguous %s, secondary bar" % layout)


@pytest.mark.parametrize("S", [1, 3])
def test_contiguous_decode_ragged_lengths(S):
    case = workloads.contig_decode_case(10, 5, 16, 4, 64, 300, device=DEV, kv_lens=[300, 0, 1, 17, 256])
    out = torch.empty_like(case["q"])
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], kv_lens=case["kv_lens"],
                   num_splits=S)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"],
                           kv_lens=case["kv_lens"].cpu())
    assert_close(out, ref)


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 4, 64), (32, 4, 128)])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 6, 8, 12, 24])
def test_contiguous_decode_one_length_every_split_count(Hq, Hkv, D, S):
    """No kv_lens, so every row has kv_len keys: when S divides the row count
    every slice holds whole rows, all written by the split kernel, and no
    combine runs; other S merge split rows.  The output starts as NaN, so a
    row left unwritten fails.  (16, 4, 64) runs the VALU kernel, (32, 4, 128)
    the MFMA one (G = 8)."""
    case = workloads.contig_decode_case(31 + S, 6, Hq, Hkv, D, 300, device=DEV)
    out = torch.full_like(case["q"], float("nan"))
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], num_splits=S)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"])
    assert_close(out, ref, what="contiguous one length, S=%d" % S)
    assert_close(out, ref, atol=2e-3, what="contiguous one length, S=%d, secondary bar" % S)


@pytest.mark.parametrize("S", [1, 4])
def test_contiguous_decode_zero_length_rows_are_zeroed(S):
    case = workloads.contig_decode_case(41, 4, 16, 4, 64, 8, device=DEV)
    out = torch.full_like(case["q"], float("nan"))
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], kv_len=0, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), torch.zeros(out.shape))


def test_workspace_poisoned_with_nan_is_fully_overwritten():
    case = workloads.paged_decode_case(12, 6, 32, 8, 128, [1, 100, 900, 1500, 16, 1024], 16)
    S = 7
    n = pa.attn_decode_workspace_bytes(6, 32, 128, S)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)   # all-ones bytes are NaNs
    ref, _ = oracle_paged(case)
    assert_close(run_paged(case, S, workspace=ws), ref)


def test_repeat_runs_are_bit_identical():
    case = workloads.paged_decode_case(13, 8, 32, 8, 128, (100, 3000), 16)
    a = run_paged(case, 0).clone()
    b = run_paged(case, 0)
    assert torch.equal(a, b)


def partition_pieces(lens, rows_per_seq, W):
    """Slots of each row's pieces under the balanced partition: rows laid end
    to end, W equal slices of the line, piece of row r in slice w at r + w."""
    n_rows = [n for n in lens for _ in range(rows_per_seq)]
    T = sum(n_rows)
    bounds = [w * T // W for w in range(W + 1)]
    out, P = [], 0
    for r, n in enumerate(n_rows):
        ws = [w for w in range(W) if n > 0 and bounds[w] < P + n and bounds[w + 1] > P]
        out.append([r + w for w in ws])
        P += n
    return out


@pytest.mark.parametrize("lens", [[1000] * 4, [5, 700, 1, 1500]])
def test_combine_of_decode_partials_matches_oracle_combine(lens):
    """The fp32 partials the split kernel leaves in the workspace (located by
    the documented slot rule) are combined on the GPU and by the oracle in
    fp64; the partials are also a valid split of the exact result."""
    B, Hq, Hkv, D, W = len(lens), 32, 8, 128, 9
    case = workloads.paged_decode_case(14, B, Hq, Hkv, D, lens, 16)
    d = to_dev(case, ["q", "k_pool", "v_pool", "block_table", "kv_lens"])
    nbytes = pa.attn_decode_workspace_bytes(B, Hq, D, W)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    pa.attn_paged_decode_split(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"],
                               case["max_kv_len"], 16, case["scale"], W, ws)
    torch.cuda.synchronize()
    rows_total = (B + W) * Hq
    o_bytes = rows_total * D * 4
    ml_off = (o_bytes + 255) // 256 * 256
    o_all = ws[:o_bytes].view(torch.float32).view(rows_total, D).cpu()
    ml_all = ws[ml_off:ml_off + rows_total * 8].view(torch.float32).view(rows_total, 2).cpu()
    pieces = partition_pieces(lens, 1, W)       # 8 adjacent heads per row: one row per sequence
    S = max(len(p) for p in pieces)
    o_part = torch.zeros(S, B * Hq, D)
    ml_part = torch.zeros(S, B * Hq, 2)
    ml_part[..., 0] = float("-inf")
    for b, slots in enumerate(pieces):
        for s_i, slot in enumerate(slots):
            for h in range(Hq):
                o_part[s_i, b * Hq + h] = o_all[slot * Hq + h]
                ml_part[s_i, b * Hq + h] = ml_all[slot * Hq + h]
    out = torch.empty(B * Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B * Hq, dtype=torch.float32, device=DEV)
    pa.attn_split_combine(o_part.to(DEV).contiguous(), ml_part.to(DEV).contiguous(), out_f32=out, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.combine_f32(o_part, ml_part)
    assert_close(out, ref, atol=1e-5, rtol=1e-5, what="combine")
    assert_close(lse, ref_lse, atol=1e-5, rtol=1e-5, what="lse")
    full, full_lse = oracle_paged(case)
    assert_close(out.view(B, Hq, D), full, atol=1e-2, rtol=1e-2)
    assert_close(lse.view(B, Hq), full_lse, atol=1e-2, rtol=1e-2)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_combine_random_partials_with_empty_splits(D):
    g = torch.Generator().manual_seed(D)
    S, R = 9, 300
    o = torch.randn(S, R, D, generator=g) * 5
    m = torch.randn(S, R, generator=g) * 3
    l = torch.rand(S, R, generator=g) * 10 + 0.1
    empty = torch.rand(S, R, generator=g) < 0.3
    m[empty] = -math.inf
    l[empty] = 0
    o[empty] = 0
    m[:, 0] = -math.inf                      # a row with no partial at all
    l[:, 0] = 0
    ml = torch.stack([m, l], dim=-1).float().contiguous()
    o = o.float().contiguous()
    out = torch.empty(R, D, dtype=torch.float32, device=DEV)
    outb = torch.empty(R, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(R, dtype=torch.float32, device=DEV)
    pa.attn_split_combine(o.to(DEV), ml.to(DEV), out_f32=out, out_bf16=outb, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.combine_f32(o, ml)
    assert_close(out, ref, atol=1e-5, rtol=1e-5)
    assert_close(outb, ref, atol=1e-2, rtol=1e-2)
    fin = torch.isfinite(ref_lse)
    assert_close(lse[fin.to(DEV)], ref_lse[fin], atol=1e-5, rtol=1e-5)
    assert bool(torch.isneginf(lse.cpu()[~fin]).all())


@pytest.mark.parametrize("S", [1, 6, 40])
def test_split_then_combine_equals_fused_call(S):
    case = workloads.paged_decode_case(15, 6, 32, 8, 128, [5, 300, 1200, 0, 77, 2000], 16)
    d = to_dev(case, ["q", "k_pool", "v_pool", "block_table", "kv_lens"])
    ws = torch.empty(pa.attn_decode_workspace_bytes(6, 32, 128, S), dtype=torch.uint8, device=DEV)
    fused = run_paged(case, S, workspace=ws).clone()
    pa.attn_paged_decode_split(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"],
                               case["max_kv_len"], 16, case["scale"], S, ws)
    out = torch.empty_like(d["q"])
    pa.attn_decode_combine(ws, 6, 32, 8, 128, S, d["k_pool"].stride(2), d["kv_lens"], case["max_kv_len"], out)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)


@pytest.mark.parametrize("Hkv,G,layout", [
    (1, 4, "page_slot_head"),    # one head per wave
    (4, 2, "page_slot_head"),    # four adjacent heads per wave
    (16, 2, "page_slot_head"),   # eight heads per wave, two head groups
    (4, 8, "page_head_slot"),    # head stride != D: one head per wave
])
@pytest.mark.parametrize("S", [1, 5])
def test_paged_decode_heads_per_wave(Hkv, G, layout, S):
    case = workloads.paged_decode_case(200 + Hkv + G, 3, Hkv * G, Hkv, 128, [1, 250, 700], 16, layout=layout)
    ref, _ = oracle_paged(case)
    assert_close(run_paged(case, S), ref, what="Hkv=%d G=%d %s S=%d" % (Hkv, G, layout, S))


def nan_workspace(B, Hq, D, S):
    n = max(256, pa.attn_decode_workspace_bytes(B, Hq, D, S))
    return torch.full((n,), 0xFF, dtype=torch.uint8, device=DEV)   # all-ones bytes are NaNs


@pytest.mark.parametrize("Hkv,layout", [(8, "page_slot_head"), (2, "page_head_slot")])
def test_partition_every_slice_count(Hkv, layout):
    """Every slice count from 1 to past the total key count, so slices that
    hold nothing (inside a row and at the ends) are covered, on a batch with
    empty and one-token sequences; the workspace starts as NaN."""
    lens = [0, 9, 1, 0, 23, 2, 0]
    G, D = 4, 64
    case = workloads.paged_decode_case(260 + Hkv, len(lens), Hkv * G, Hkv, D, lens, 4, layout=layout)
    ref, _ = oracle_paged(case)
    groups = 1 if layout == "page_slot_head" else Hkv     # KV-head groups per sequence
    T = sum(lens) * groups
    for S in list(range(1, T + 8)):
        got = run_paged(case, S, workspace=nan_workspace(len(lens), Hkv * G, D, S))
        assert_close(got, ref, what="S=%d of T=%d" % (S, T))


@pytest.mark.parametrize("S", [0, 150])
def test_planner_on_mostly_empty_batch(S):
    """128 sequences of which one holds keys: the planner sizes its slice
    count from max_kv_len (128 x 100 keys), far more than the 100 keys there
    are; with 150 slices most of them are empty."""
    lens = [0] * 128
    lens[77] = 100
    case = workloads.paged_decode_case(270, 128, 32, 8, 128, lens, 16)
    S = S or pa.attn_plan_splits(128, 8, 4, 128, 100, 16, case["k_pool"].stride(2))
    ref, _ = oracle_paged(case)
    got = run_paged(case, S, workspace=nan_workspace(128, 32, 128, S))
    assert_close(got, ref, what="S=%d" % S)


# ------------------------------------------------ head dims 32 and 256
@pytest.mark.parametrize("D", [32, 256])
@pytest.mark.parametrize("Hkv,G,layout", [
    (8, 4, "page_slot_head"),    # D=32: eight heads per wave; D=256: four (two head groups)
    (2, 8, "page_slot_head"),
    (4, 2, "page_head_slot"),    # one head per wave
    (1, 1, "page_slot_head"),
])
@pytest.mark.parametrize("S", [0, 1, 5])
def test_paged_decode_head_dims_32_and_256(D, Hkv, G, layout, S):
    """Head dims beyond 64 and 128: 4 chunk lanes per head row at D=32, 16 at
    D=256 (one more DPP step in the row sum).  Contexts up to 1500 keys;
    outputs are ~0.03 in size there, so rows of 256 keys or more are also
    held to 2e-3."""
    lens = [1, 200, 0, 777, 1500]
    case = workloads.paged_decode_case(300 + D + Hkv * G, len(lens), Hkv * G, Hkv, D, lens, 16, layout=layout)
    ref, _ = oracle_paged(case)
    assert_decode_close(run_paged(case, S), ref, lens, what="D=%d Hkv=%d G=%d %s S=%d" % (D, Hkv, G, layout, S))


@pytest.mark.parametrize("D,ps", [(32, 1), (32, 5), (256, 3), (256, 64)])
def test_paged_decode_head_dims_page_sizes(D, ps):
    case = workloads.paged_decode_case(330 + D + ps, 4, 32, 8, D, [17, 1024, 333, 2], ps)
    ref, _ = oracle_paged(case)
    assert_decode_close(run_paged(case, 0), ref, case["kv_lens"].tolist(), what="D=%d ps=%d" % (D, ps))


@pytest.mark.parametrize("D", [32, 256])
@pytest.mark.parametrize("layout", ["bhld", "blhd"])
def test_contiguous_decode_head_dims_32_and_256(D, layout):
    case = workloads.contig_decode_case(340 + D, 3, 16, 4, D, 900, device=DEV, layout=layout,
                                        kv_lens=[900, 1, 450])
    out = torch.empty_like(case["q"])
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], kv_lens=case["kv_lens"])
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"],
                           kv_lens=case["kv_lens"].cpu())
    assert_decode_close(out, ref, case["kv_lens"].tolist(), what="contiguous D=%d %s" % (D, layout))


@pytest.mark.parametrize("D", [32, 256])
def test_partition_every_slice_count_head_dims(D):
    """Every slice count up to past the key total at D = 32 (eight heads per
    wave) and D = 256 (four heads per wave, so two head groups per
    sequence), empty and one-token sequences, NaN workspace."""
    lens = [0, 9, 1, 0, 23, 2, 0]
    Hkv, G = 8, 2
    case = workloads.paged_decode_case(350 + D, len(lens), Hkv * G, Hkv, D, lens, 4)
    ref, _ = oracle_paged(case)
    groups = 1 if D == 32 else 2
    T = sum(lens) * groups
    for S in range(1, T + 8):
        got = run_paged(case, S, workspace=nan_workspace(len(lens), Hkv * G, D, S))
        assert_close(got, ref, what="D=%d S=%d of T=%d" % (D, S, T))


# ---------------------------------------- group sizes beyond 1, 2, 4, 8
@pytest.mark.parametrize("Hq,Hkv,layout", [
    (6, 2, "page_slot_head"),     # G = 3: three passes of one query head
    (12, 2, "page_head_slot"),    # G = 6: three passes of two
    (24, 2, "page_slot_head"),    # G = 12: three passes of four
    (32, 1, "page_slot_head"),    # G = 32: four passes of eight
    (16, 1, "page_head_slot"),    # G = 16
    (40, 8, "page_slot_head"),    # G = 5
])
@pytest.mark.parametrize("S", [0, 1, 7])
def test_paged_decode_any_group_size(Hq, Hkv, layout, S):
    """Group sizes the pages verify head packing for (3, 32) and others: a
    (sequence, KV head) is streamed once per pass of Gk query heads."""
    lens = [1, 300, 0, 1200]
    case = workloads.paged_decode_case(400 + Hq + Hkv, len(lens), Hq, Hkv, 128, lens, 16, layout=layout)
    ref, _ = oracle_paged(case)
    assert_decode_close(run_paged(case, S), ref, lens, what="Hq=%d Hkv=%d %s S=%d" % (Hq, Hkv, layout, S))


def test_contiguous_decode_group_size_32():
    case = workloads.contig_decode_case(420, 3, 32, 1, 64, 500, device=DEV, layout="blhd", kv_lens=[500, 7, 260])
    out = torch.empty_like(case["q"])
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], kv_lens=case["kv_lens"])
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"],
                           kv_lens=case["kv_lens"].cpu())
    assert_decode_close(out, ref, case["kv_lens"].tolist(), what="contiguous G=32")


@pytest.mark.parametrize("S", [3, 11])
def test_split_then_combine_group_size_6(S):
    """attn_paged_decode_split + attn_decode_combine locate a row's pieces from
    the same pass layout as the fused call."""
    case = workloads.paged_decode_case(430, 4, 12, 2, 128, [5, 300, 0, 900], 16)
    d = to_dev(case, ["q", "k_pool", "v_pool", "block_table", "kv_lens"])
    ws = torch.empty(pa.attn_decode_workspace_bytes(4, 12, 128, S), dtype=torch.uint8, device=DEV)
    fused = run_paged(case, S, workspace=ws).clone()
    pa.attn_paged_decode_split(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"],
                               case["max_kv_len"], 16, case["scale"], S, ws)
    out = torch.empty_like(d["q"])
    pa.attn_decode_combine(ws, 4, 12, 2, 128, S, d["k_pool"].stride(2), d["kv_lens"], case["max_kv_len"], out)
    torch.cuda.synchronize()
    assert torch.equal(fused, out)
    ref, _ = oracle_paged(case)
    assert_decode_close(out, ref, case["kv_lens"].tolist(), what="split + combine G=6")


def test_partition_every_slice_count_group_size_3():
    lens = [0, 9, 1, 0, 23, 2, 0]
    Hkv, G, D = 2, 3, 64
    case = workloads.paged_decode_case(440, len(lens), Hkv * G, Hkv, D, lens, 4)
    ref, _ = oracle_paged(case)
    T = sum(lens) * Hkv * G          # one row per (sequence, KV head, pass)
    for S in range(1, T + 8):
        got = run_paged(case, S, workspace=nan_workspace(len(lens), Hkv * G, D, S))
        assert_close(got, ref, what="G=3 S=%d of T=%d" % (S, T))


# ------------------------------------------ MFMA rows (D 64 / 128, G not 1, 2, 4)
@pytest.mark.parametrize("G,D,ps,layout,lens", [
    (8, 128, 1, "page_slot_head", [1300, 3, 0, 511]),     # per-key V loads, three sub-pieces at S = 1
    (8, 64, 3, "page_head_slot", [97, 1, 640]),
    (24, 128, 5, "page_slot_head", [33, 777, 2]),        # second block half used (heads 16..23)
    (20, 64, 16, "page_head_slot", [450, 0, 31, 64]),
    (64, 128, 8, "page_slot_head", [300, 129]),          # two passes of 32 heads
    (7, 128, 2, "page_head_slot", [1030, 5]),            # prime group size: one block of 7
    (32, 64, 4, "page_slot_head", [1, 2, 3, 4, 250]),
    (16, 128, 12, "page_head_slot", [100, 1]),
    (48, 64, 32, "page_slot_head", [700, 2100]),         # 24 heads a row, two passes
])
@pytest.mark.parametrize("S", [0, 1, 5])
def test_mfma_decode_shapes(G, D, ps, layout, lens, S):
    """Query heads of a KV head on bf16 MFMA rows: partly used 16-row blocks,
    page sizes not a multiple of 4, several passes and sub-pieces."""
    Hkv = 2 if G <= 32 else 1
    case = workloads.paged_decode_case(4500 + G * 3 + D + ps, len(lens), Hkv * G, Hkv, D, lens, ps, layout=layout)
    ref, _ = oracle_paged(case)
    out = torch.full_like(case["q"], float("nan"), device=DEV)
    assert_decode_close(run_paged(case, S, out=out), ref, lens, what="G=%d D=%d ps=%d S=%d" % (G, D, ps, S))


@pytest.mark.parametrize("G,D,layout", [(8, 128, "bhld"), (12, 64, "blhd"), (32, 128, "blhd")])
@pytest.mark.parametrize("S", [0, 1, 6])
def test_mfma_contiguous_decode(G, D, layout, S):
    """Contiguous K/V on the MFMA rows: rows of one sequence back to back in
    a slice, so the merge area of one row is followed by the next row's V^T."""
    lens = [700, 3, 260, 0, 1]
    case = workloads.contig_decode_case(4600 + G + D, len(lens), 2 * G, 2, D, 700, device=DEV, layout=layout,
                                        kv_lens=lens)
    out = torch.full_like(case["q"], float("nan"))
    pa.attn_decode(case["q"], case["k"], case["v"], out, case["scale"], kv_lens=case["kv_lens"], num_splits=S)
    torch.cuda.synchronize()
    ref, _ = oracle.decode(case["q"].cpu(), case["k"].cpu(), case["v"].cpu(), case["scale"],
                           kv_lens=case["kv_lens"].cpu())
    assert_decode_close(out, ref, lens, what="contiguous G=%d D=%d %s S=%d" % (G, D, layout, S))


def test_mfma_partition_every_slice_count():
    """Every slice count from 1 to past the token count for G = 8, D = 64 on
    MFMA rows: empty slices inside rows, rows of one key, several rows in
    one slice; the workspace starts as NaN."""
    lens = [0, 9, 1, 0, 23, 2, 40, 0]
    Hkv, G, D = 2, 8, 64
    case = workloads.paged_decode_case(4700, len(lens), Hkv * G, Hkv, D, lens, 4)
    ref, _ = oracle_paged(case)
    T = sum(lens) * Hkv          # one row per (sequence, KV head)
    for S in range(1, T + 8):
        got = run_paged(case, S, workspace=nan_workspace(len(lens), Hkv * G, D, S))
        assert_close(got, ref, what="G=8 S=%d of T=%d" % (S, T))


# ------------------------------------------------------- long slices
@pytest.mark.parametrize("ps,S", [(1, 1), (1, 3), (2, 1), (16, 1)])
def test_paged_decode_slices_longer_than_the_page_slice(ps, S):
    """A wave stages at most 510 block-table entries in LDS at a time, so a
    slice longer than 510 pages runs as consecutive sub-pieces that carry
    the softmax state across: with page size 1 a 5000-token sequence is ten
    of them at S = 1; page size 16 covers 8160 tokens per sub-piece."""
    lens = [5000, 1200, 17] if ps < 16 else [20000, 9000]
    case = workloads.paged_decode_case(500 + ps + S, len(lens), 32, 8, 128, lens, ps)
    ref, _ = oracle_paged(case)
    assert_decode_close(run_paged(case, S), ref, lens, what="ps=%d S=%d" % (ps, S))


@pytest.mark.parametrize("layout,S", [("page_slot_head", 0), ("page_head_slot", 0), ("page_slot_head", 5000)])
def test_paged_decode_large_batch(layout, S):
    """2048 sequences of 0..200 keys: the partition's scan of kv_lens walks
    32 rows per lane (256 with one KV head per row), and S = 5000 leaves
    many slices inside single rows.  Sampled sequences vs the oracle."""
    g = torch.Generator().manual_seed(600)
    lens = torch.randint(0, 201, (2048,), generator=g).tolist()
    case = workloads.paged_decode_case(601, 2048, 16, 4, 64, lens, 16, layout=layout)
    S = S or pa.attn_plan_splits(2048, 4, 4, 64, case["max_kv_len"], 16, case["k_pool"].stride(2))
    out = run_paged(case, S, workspace=nan_workspace(2048, 16, 64, S)).cpu()
    idx = torch.tensor([0, 1, 2, 511, 1000, 1023, 1024, 2000, 2046, 2047] +
                       [i for i, n in enumerate(lens) if n == 0][:3])
    sub = dict(q=case["q"][idx], k_pool=case["k_pool"], v_pool=case["v_pool"], block_table=case["block_table"][idx],
               kv_lens=case["kv_lens"][idx], scale=case["scale"])
    ref, _ = oracle_paged(sub)
    assert_close(out[idx], ref, what="B=2048 %s S=%d" % (layout, S))


def test_binding_rejects_wrong_element_types():
    """Arguments whose element type differs from the C ABI's are refused by
    the binding (int64 lengths, fp32 queries) instead of being reinterpreted."""
    case = workloads.tiny_paged_decode(device=DEV)
    out = torch.empty_like(case["q"])
    with pytest.raises(TypeError, match="kv_lens must be torch.int32"):
        pa.attn_paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                             case["kv_lens"].long(), case["max_kv_len"], out, case["page_size"], case["scale"])
    with pytest.raises(TypeError, match="q must be torch.bfloat16"):
        pa.attn_paged_decode(case["q"].float(), case["k_pool"], case["v_pool"], case["block_table"],
                             case["kv_lens"], case["max_kv_len"], out, case["page_size"], case["scale"])
