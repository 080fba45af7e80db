"""Pins for the CPU oracle: each test checks it against something other than
itself -- a library routine (torch SDPA in fp64, torch's fp8/bf16 casts), a
closed form, an invariant of softmax attention, or a value the pages print.
No test here needs a GPU."""
import json
import math
import os

import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def dense_kv(pool, bt_row, n, ps):
    """Logical sequence [n, Hkv, D] of a paged pool, gathered token by token
    with plain Python indexing (independent of the oracle's gather)."""
    rows = [pool[int(bt_row[j // ps]), j % ps] for j in range(n)]
    if not rows:
        return pool.new_zeros((0,) + tuple(pool.shape[2:]))
    return torch.stack(rows)


def sdpa64(q, k, v, scale, keep=None):
    """torch SDPA in float64.  q [H, R, D]; k/v [H, n, D]; keep [R, n] bool."""
    mask = None if keep is None else keep.unsqueeze(0).expand(q.shape[0], -1, -1)
    return torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), attn_mask=mask, scale=scale)


def sdpa_decode_ref(case, mask=None):
    q, kp, vp, bt, lens = case["q"], case["k_pool"], case["v_pool"], case["block_table"], case["kv_lens"]
    B, Hq, D = q.shape
    G = Hq // kp.shape[2]
    out = torch.empty(B, Hq, D, dtype=torch.float64)
    for b in range(B):
        n = int(lens[b])
        k = dense_kv(kp, bt[b], n, case["page_size"]).permute(1, 0, 2)   # [Hkv, n, D]
        v = dense_kv(vp, bt[b], n, case["page_size"]).permute(1, 0, 2)
        k = k.repeat_interleave(G, dim=0)
        v = v.repeat_interleave(G, dim=0)
        keep = None if mask is None else mask[b, :n].bool().unsqueeze(0)
        out[b] = sdpa64(q[b].unsqueeze(1), k, v, case["scale"], keep)[:, 0, :]
    return out


# ------------------------------------------------------------ element types
def test_e4m3fn_all_256_codes_match_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(256):
        got = orc.e4m3fn_to_f64(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(float(ref[c]))
        else:
            assert got == float(ref[c]), (c, got, float(ref[c]))


def test_e4m3fn_spec_points(orc):
    # OCP 8-bit FP spec, E4M3: max normal 448, min subnormal 2^-9, one at 0x38.
    assert orc.e4m3fn_to_f64(0x7E) == 448.0
    assert orc.e4m3fn_to_f64(0xFE) == -448.0
    assert orc.e4m3fn_to_f64(0x01) == 2.0 ** -9
    assert orc.e4m3fn_to_f64(0x08) == 2.0 ** -6
    assert orc.e4m3fn_to_f64(0x38) == 1.0
    assert orc.e4m3fn_to_f64(0x80) == 0.0


def test_bf16_widening_matches_torch(orc):
    g = torch.Generator().manual_seed(7)
    bits = torch.randint(0, 1 << 16, (4096,), generator=g, dtype=torch.int32)
    vals = bits.to(torch.int16).view(torch.bfloat16).to(torch.float64)
    for b, v in zip(bits.tolist(), vals.tolist()):
        got = orc.bf16_to_f64(b)
        assert (math.isnan(got) and math.isnan(v)) or got == v


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("G,D,ps,lens", [
    (4, 64, 16, [256, 300]),
    (1, 64, 3, [1, 17, 40]),
    (2, 128, 1, [5, 33]),
    (8, 128, 16, [15, 16, 17, 100]),
    (4, 32, 7, [50]),
])
def test_paged_decode_matches_sdpa(orc, G, D, ps, lens):
    Hkv = 2
    case = workloads.paged_decode_case(11 + G + D + ps, len(lens), Hkv * G, Hkv, D, lens, ps)
    out, lse = orc.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                case["kv_lens"], case["scale"])
    ref = sdpa_decode_ref(case)
    assert torch.allclose(out, ref, atol=1e-12, rtol=1e-12)
    assert torch.isfinite(lse).all()


def test_tiny_config_matches_sdpa(orc):
    case = workloads.tiny_paged_decode()
    out, _ = orc.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                              case["kv_lens"], case["scale"])
    assert torch.allclose(out, sdpa_decode_ref(case), atol=1e-12, rtol=1e-12)


def test_paged_decode_2d_mask_matches_sdpa(orc):
    case = workloads.paged_decode_case(21, 3, 8, 2, 64, [30, 47, 64], 16)
    g = torch.Generator().manual_seed(3)
    mask = torch.rand(3, 64, generator=g) >= 0.3
    mask[:, 0] = True
    out, _ = orc.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                              case["kv_lens"], case["scale"], mask=mask)
    assert torch.allclose(out, sdpa_decode_ref(case, mask), atol=1e-12, rtol=1e-12)


def test_paged_decode_page_head_slot_layout(orc):
    """A [P, Hkv, ps, D] pool addressed through strides gives the same
    result as SDPA on its logical sequence."""
    case = workloads.paged_decode_case(31, 2, 8, 2, 64, [40, 77], 16, layout="page_head_slot")
    out, _ = orc.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                              case["kv_lens"], case["scale"])
    assert torch.allclose(out, sdpa_decode_ref(case), atol=1e-12, rtol=1e-12)


def _decode(orc, case, **kw):
    return orc.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                            case["kv_lens"], case["scale"], **kw)


def test_zero_query_gives_mean_of_v(orc):
    case = workloads.paged_decode_case(41, 2, 4, 2, 64, [9, 23], 4)
    case["q"].zero_()
    out, lse = _decode(orc, case)
    for b in range(2):
        n = int(case["kv_lens"][b])
        v = dense_kv(case["v_pool"], case["block_table"][b], n, 4).double()   # [n, Hkv, D]
        mean = v.mean(dim=0)                                                   # [Hkv, D]
        for h in range(4):
            assert torch.allclose(out[b, h], mean[h // 2], atol=1e-13, rtol=0)
            assert abs(float(lse[b, h]) - math.log(n)) < 1e-13


def test_constant_v_returns_v(orc):
    case = workloads.paged_decode_case(42, 2, 8, 2, 64, [31, 64], 16)
    row = torch.randn(64).to(torch.bfloat16)
    case["v_pool"][:] = row
    out, _ = _decode(orc, case)
    assert torch.allclose(out, row.double().expand_as(out), atol=1e-14, rtol=0)


def test_single_key_returns_its_v(orc):
    case = workloads.paged_decode_case(43, 3, 8, 2, 64, [1, 1, 1], 16)
    out, lse = _decode(orc, case)
    for b in range(3):
        v = case["v_pool"][int(case["block_table"][b, 0]), 0].double()   # [Hkv, D]
        for h in range(8):
            assert torch.equal(out[b, h], v[h // 4])


def test_two_keys_closed_form(orc):
    """n = 2: out = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2."""
    case = workloads.paged_decode_case(44, 1, 2, 1, 64, [2], 16)
    out, lse = _decode(orc, case)
    page = int(case["block_table"][0, 0])
    k = case["k_pool"][page, :2, 0].double()
    v = case["v_pool"][page, :2, 0].double()
    for h in range(2):
        qh = case["q"][0, h].double()
        s1, s2 = case["scale"] * float(qh @ k[0]), case["scale"] * float(qh @ k[1])
        a = 1.0 / (1.0 + math.exp(s2 - s1))
        ref = a * v[0] + (1.0 - a) * v[1]
        assert torch.allclose(out[0, h], ref, atol=1e-14, rtol=0)
        ref_lse = max(s1, s2) + math.log(math.exp(s1 - max(s1, s2)) + math.exp(s2 - max(s1, s2)))
        assert abs(float(lse[0, h]) - ref_lse) < 1e-13


def test_page_permutation_invariance(orc):
    """Relabelling physical pages (pool order + block table) changes nothing."""
    case = workloads.paged_decode_case(45, 3, 8, 2, 64, [70, 5, 33], 8)
    out, lse = _decode(orc, case)
    P = case["k_pool"].shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(9))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    bt2 = case["block_table"].clone()
    valid = bt2 >= 0
    bt2[valid] = inv[bt2[valid].long()].to(torch.int32)
    case2 = dict(case, k_pool=case["k_pool"][perm].contiguous(),
                 v_pool=case["v_pool"][perm].contiguous(), block_table=bt2)
    out2, lse2 = _decode(orc, case2)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_paged_with_whole_sequence_page_equals_contiguous(orc):
    """page_size = n with an identity table is the contiguous layout."""
    B, Hq, Hkv, D, n = 2, 8, 2, 64, 37
    c = workloads.contig_decode_case(46, B, Hq, Hkv, D, n)
    out_c, lse_c = orc.decode(c["q"], c["k"], c["v"], c["scale"])
    kp = c["k4"].permute(0, 2, 1, 3).contiguous()     # [B pages, n slots, Hkv, D]
    vp = c["v4"].permute(0, 2, 1, 3).contiguous()
    bt = torch.arange(B, dtype=torch.int32).unsqueeze(1)
    out_p, lse_p = orc.paged_decode(c["q"], kp, vp, bt, torch.full((B,), n, dtype=torch.int32), c["scale"])
    assert torch.equal(out_c, out_p) and torch.equal(lse_c, lse_p)


def test_contiguous_decode_blhd_and_ragged_lengths_match_sdpa(orc):
    c = workloads.contig_decode_case(47, 3, 8, 4, 64, 50, layout="blhd", kv_lens=[50, 1, 23])
    out, _ = orc.decode(c["q"], c["k"], c["v"], c["scale"], kv_lens=c["kv_lens"])
    for b in range(3):
        n = int(c["kv_lens"][b])
        k = c["k"][b, :, :n].repeat_interleave(2, dim=0)
        v = c["v"][b, :, :n].repeat_interleave(2, dim=0)
        ref = sdpa64(c["q"][b].unsqueeze(1), k, v, c["scale"])[:, 0]
        assert torch.allclose(out[b], ref, atol=1e-12, rtol=1e-12)


def test_empty_sequence_gives_zero_and_neg_inf(orc):
    case = workloads.paged_decode_case(48, 2, 4, 2, 64, [0, 5], 16)
    out, lse = _decode(orc, case)
    assert torch.equal(out[0], torch.zeros_like(out[0]))
    assert torch.isneginf(lse[0]).all() and torch.isfinite(lse[1]).all()


# ------------------------------------------------------------ split/combine
@pytest.mark.parametrize("S", [1, 2, 3, 7, 40])
def test_split_count_invariance(orc, S):
    case = workloads.paged_decode_case(50 + S, 3, 8, 2, 64, [1, 40, 97], 16)
    out, lse = _decode(orc, case)
    g = torch.Generator().manual_seed(S)
    bounds = torch.zeros(3, S + 1, dtype=torch.int32)
    for b in range(3):
        n = int(case["kv_lens"][b])
        cuts = torch.sort(torch.randint(0, n + 1, (S - 1,), generator=g)).values
        bounds[b, 1:S] = cuts.to(torch.int32)
        bounds[b, S] = n
    o, m, l = orc.paged_decode_partials(case["q"], case["k_pool"], case["v_pool"],
                                        case["block_table"], case["kv_lens"], bounds, case["scale"])
    R = 3 * 8
    cout, clse = orc.combine(o.reshape(S, R, 64), m.reshape(S, R), l.reshape(S, R))
    assert torch.allclose(cout.reshape(3, 8, 64), out, atol=1e-12, rtol=1e-12)
    assert torch.allclose(clse.reshape(3, 8), lse, atol=1e-12, rtol=1e-12)


def test_combine_closed_form_two_partials(orc):
    """Two partials that are exactly the two halves of a 2-key softmax."""
    s1, s2 = 0.3, -1.1
    v1, v2 = torch.tensor([[1.0, 2.0]]), torch.tensor([[-3.0, 0.5]])
    o = torch.stack([v1, v2])                                  # l = 1, m = s
    m = torch.tensor([[s1], [s2]], dtype=torch.float64)
    l = torch.ones(2, 1, dtype=torch.float64)
    out, lse = orc.combine(o, m, l)
    a = 1.0 / (1.0 + math.exp(s2 - s1))
    assert torch.allclose(out[0], (a * v1 + (1 - a) * v2)[0].double(), atol=1e-15)
    assert abs(float(lse[0]) - math.log(math.exp(s1) + math.exp(s2))) < 1e-15


def test_combine_skips_empty_partials(orc):
    o = torch.tensor([[[2.0, 4.0]], [[99.0, 99.0]]])
    ml = torch.tensor([[[0.5, 2.0]], [[-math.inf, 0.0]]], dtype=torch.float32)
    out, lse = orc.combine_f32(o, ml)
    assert torch.equal(out[0], torch.tensor([1.0, 2.0], dtype=torch.float64))
    assert abs(float(lse[0]) - (0.5 + math.log(2.0))) < 1e-15
    out, lse = orc.combine_f32(o[1:], ml[1:])
    assert torch.equal(out[0], torch.zeros(2, dtype=torch.float64)) and math.isinf(float(lse[0]))


# ----------------------------------------------------------------- prefill
def sdpa_prefill_ref(case):
    q, kp, vp, bt = case["q"], case["k_pool"], case["v_pool"], case["block_table"]
    Hq, D = q.shape[1], q.shape[2]
    G = Hq // kp.shape[2]
    out = torch.empty(q.shape, dtype=torch.float64)
    for b in range(case["B"]):
        r0, r1 = int(case["qo_indptr"][b]), int(case["qo_indptr"][b + 1])
        n, c = int(case["kv_lens"][b]), int(case["causal_offset"][b])
        qn = r1 - r0
        keep = torch.ones(qn, n, dtype=torch.bool)
        if c >= 0:
            i = torch.arange(qn).unsqueeze(1)
            j = torch.arange(n).unsqueeze(0)
            keep &= j <= c + i
        if case["mask"] is not None:
            m = case["mask"]
            keep &= (m[b, :qn, :n] if m.dim() == 3 else m[b, :n].unsqueeze(0).expand(qn, n)).bool()
        k = dense_kv(kp, bt[b], n, case["page_size"]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        v = dense_kv(vp, bt[b], n, case["page_size"]).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = q[r0:r1].permute(1, 0, 2)                                      # [Hq, qn, D]
        ref = sdpa64(qb, k, v, case["scale"], keep)                         # rows w/o keys -> nan
        ref = torch.where(keep.any(dim=1).view(1, qn, 1), ref, torch.zeros_like(ref))
        out[r0:r1] = ref.permute(1, 0, 2)
    return out


def _prefill(orc, case):
    return orc.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"],
                             case["block_table"], case["kv_lens"], case["scale"],
                             causal_offset=case["causal_offset"], mask=case["mask"])


@pytest.mark.parametrize("kw", [
    dict(mask_frac=None, causal=True),
    dict(mask_frac=0.1, mask_ndim=3, causal=True),
    dict(mask_frac=0.3, mask_ndim=2, causal=False),
    dict(mask_frac=0.5, mask_ndim=3, causal=False),
])
def test_paged_prefill_matches_sdpa(orc, kw):
    case = workloads.prefill_case(61, 3, 8, 2, 64, (0, 40), (1, 30), 16, **kw)
    out, lse = _prefill(orc, case)
    assert torch.allclose(out, sdpa_prefill_ref(case), atol=1e-12, rtol=1e-12)


def test_prefill_causal_row_sees_only_its_prefix(orc):
    """Perturbing K/V at positions after c_b + i leaves row i unchanged."""
    case = workloads.prefill_case(62, 2, 4, 2, 64, (3, 20), (5, 12), 4)
    out, _ = _prefill(orc, case)
    b, i = 1, 2
    c = int(case["causal_offset"][b])
    n = int(case["kv_lens"][b])
    kp, vp = case["k_pool"].clone(), case["v_pool"].clone()
    for j in range(c + i + 1, n):
        page, slot = int(case["block_table"][b, j // 4]), j % 4
        kp[page, slot] = torch.randn(2, 64).to(torch.bfloat16)
        vp[page, slot] = torch.randn(2, 64).to(torch.bfloat16)
    out2, _ = _prefill(orc, dict(case, k_pool=kp, v_pool=vp))
    row = int(case["qo_indptr"][b]) + i
    assert torch.equal(out[row], out2[row])
    assert not torch.equal(out[row + 1:int(case["qo_indptr"][b + 1])],
                           out2[row + 1:int(case["qo_indptr"][b + 1])])


def test_prefill_last_row_equals_decode(orc):
    """With causality, the last new row of a sequence sees all n_b keys, which
    is the decode problem for that query."""
    case = workloads.prefill_case(63, 3, 8, 2, 64, (0, 30), (1, 9), 16)
    out, _ = _prefill(orc, case)
    last = case["qo_indptr"][1:] - 1
    q_last = case["q"][last.long()]
    dout, _ = orc.paged_decode(q_last, case["k_pool"], case["v_pool"], case["block_table"],
                               case["kv_lens"], case["scale"])
    assert torch.equal(out[last.long()], dout)


def test_prefill_fully_masked_rows_are_zero(orc):
    case = workloads.prefill_case(64, 2, 4, 2, 64, (0, 0), (3, 5), 16, mask_frac=0.0, mask_ndim=3)
    case["mask"][0, 0, :] = False
    out, lse = _prefill(orc, case)
    assert torch.equal(out[0], torch.zeros_like(out[0])) and torch.isneginf(lse[0]).all()


# ---------------------------------------------------------------- work map
def test_work_map_matches_worked_example(orc):
    with open(os.path.join(GOLDEN, "ragged_work_map.json")) as f:
        ex = json.load(f)
    indptr, t2b, t2i = orc.prefill_plan(ex["q_lens"], ex["tile_rows"])
    assert indptr.tolist() == ex["qo_indptr"]
    assert t2b.tolist() == ex["q_tile_to_batch"]
    assert t2i.tolist() == ex["q_tile_to_index"]
    assert t2b.numel() == ex["grid_x"]


def test_work_map_covers_every_row_exactly_once(orc):
    g = torch.Generator().manual_seed(5)
    for trial in range(50):
        B = int(torch.randint(1, 9, (1,), generator=g))
        lens = torch.randint(0, 300, (B,), generator=g).tolist()
        R = int(torch.randint(1, 130, (1,), generator=g))
        indptr, t2b, t2i = orc.prefill_plan(lens, R)
        seen = []
        for b, i in zip(t2b.tolist(), t2i.tolist()):
            lo = int(indptr[b]) + i * R
            hi = min(lo + R, int(indptr[b + 1]))
            assert lo < hi
            seen.extend(range(lo, hi))
        assert seen == list(range(sum(lens)))


# ---------------------------------------------------------- fp8 sliding window
def swa_torch_ref(case, exact=True):
    """The SWA fallback's steps restated with torch CPU ops: clamp the slot,
    split it into (block, offset), gather, view as e4m3fn, multiply by the
    slot's inverse scale, mask positions >= len or with index < 0, SDPA with
    K = V over every head."""
    q, cache, inv, ind, lens = case["q"], case["cache"], case["inv_scale"], case["indices"], case["lens"]
    T, NH, HD = q.shape
    W = ind.shape[1]
    bs = case["block_size"]
    safe = ind.clamp(min=0)
    raw = cache[safe // bs, safe % bs].view(torch.float8_e4m3fn)           # [T, W, HD]
    if exact:
        kv = raw.to(torch.float64) * inv[safe].to(torch.float64)
    else:
        kv = (raw.to(torch.bfloat16) * inv[safe]).to(torch.bfloat16).to(torch.float64)
    keep = (torch.arange(W).unsqueeze(0) < lens.unsqueeze(1)) & (ind >= 0)  # [T, W]
    out = torch.empty(T, NH, HD, dtype=torch.float64)
    for t in range(T):
        if not keep[t].any():
            out[t] = 0
            continue
        kvt = kv[t].unsqueeze(0).expand(NH, W, HD)
        out[t] = sdpa64(q[t].unsqueeze(1), kvt, kvt, case["scale"], keep[t].unsqueeze(0))[:, 0]
    return out


@pytest.mark.parametrize("neg_frac", [0.0, 0.2])
def test_swa_matches_torch_fallback_steps(orc, neg_frac):
    case = workloads.swa_case(71, 6, 32, 512, 128, 256, 4, len_range=(1, 128), neg_frac=neg_frac)
    case["lens"][0] = 128
    out, _ = orc.swa_fp8_decode(case["q"], case["cache"], case["inv_scale"], case["indices"],
                                case["lens"], case["block_size"], case["scale"])
    assert torch.allclose(out, swa_torch_ref(case, exact=True), atol=1e-12, rtol=1e-12)


def test_swa_bf16_dequant_emulation_matches_fallback_rounding(orc):
    case = workloads.swa_case(72, 4, 16, 512, 64, 256, 2, len_range=(1, 64))
    out, _ = orc.swa_fp8_decode(case["q"], case["cache"], case["inv_scale"], case["indices"],
                                case["lens"], case["block_size"], case["scale"],
                                emulate_bf16_dequant=True)
    assert torch.allclose(out, swa_torch_ref(case, exact=False), atol=1e-12, rtol=1e-12)


def test_swa_no_valid_position_gives_zero(orc):
    case = workloads.swa_case(73, 3, 16, 512, 16, 256, 1, lens=[0, 4, 3])
    case["indices"][2, :] = -1
    out, lse = orc.swa_fp8_decode(case["q"], case["cache"], case["inv_scale"], case["indices"],
                                  case["lens"], case["block_size"], case["scale"])
    assert torch.equal(out[0], torch.zeros_like(out[0])) and torch.isneginf(lse[0]).all()
    assert torch.equal(out[2], torch.zeros_like(out[2]))
    assert torch.isfinite(lse[1]).all()
