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
    (3, 256, 16, [40, 90]),
    (32, 64, 4, [33, 7]),
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


@pytest.mark.parametrize("Hq,Hkv,D", [(6, 2, 128), (8, 2, 256), (32, 1, 32)])
def test_paged_prefill_group_sizes_and_head_dims_match_sdpa(orc, Hq, Hkv, D):
    case = workloads.prefill_case(62 + Hq + D, 2, Hq, Hkv, D, (0, 40), (1, 30), 5, mask_frac=0.2, mask_ndim=3)
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


# ------------------------------------------------------- paged KV append
def test_kv_append_hand_placed_tokens(orc):
    """Page size 4, sequence 0 starts at position 6: its three new tokens go
    to (bt[0][1], slot 2), (bt[0][1], slot 3), (bt[0][2], slot 0); sequence 1
    starts at 0 with one token at (bt[1][0], slot 0)."""
    P, ps, Hkv, D = 7, 4, 2, 8
    g = torch.Generator().manual_seed(5)
    kp = torch.randn(P, ps, Hkv, D, generator=g).to(torch.bfloat16)
    vp = torch.randn(P, ps, Hkv, D, generator=g).to(torch.bfloat16)
    bt = torch.tensor([[5, 2, 6], [3, -1, -1]], dtype=torch.int32)
    kn = torch.randn(4, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(4, Hkv, D, generator=g).to(torch.bfloat16)
    k2, v2 = orc.kv_append(kp, vp, bt, kn, vn, torch.tensor([0, 3, 4], dtype=torch.int32),
                           torch.tensor([6, 0], dtype=torch.int32))
    placed = [(2, 2, 0), (2, 3, 1), (6, 0, 2), (3, 0, 3)]   # (page, slot, new row)
    for page, slot, i in placed:
        assert torch.equal(k2[page, slot], kn[i]) and torch.equal(v2[page, slot], vn[i])
    touched = torch.zeros(P, ps, dtype=torch.bool)
    for page, slot, _ in placed:
        touched[page, slot] = True
    assert torch.equal(k2[~touched], kp[~touched]) and torch.equal(v2[~touched], vp[~touched])


@pytest.mark.parametrize("layout", ["page_slot_head", "page_head_slot"])
def test_kv_append_reads_back_through_block_table(orc, layout):
    """After appending n_b rows at position c_b, the tokens c_b .. c_b+n_b of
    each sequence, gathered with plain indexing, are the new rows; all other
    pool bytes are unchanged."""
    case = workloads.paged_decode_case(71, 5, 8, 2, 64, [37, 0, 16, 100, 3], 16, layout=layout)
    g = torch.Generator().manual_seed(72)
    ctx = [5, 0, 16, 60, 0]
    new = [int(n) - c for n, c in zip(case["kv_lens"].tolist(), ctx)]
    indptr = torch.tensor([0] + list(torch.tensor(new).cumsum(0).tolist()), dtype=torch.int32)
    N = int(indptr[-1])
    kn = torch.randn(N, 2, 64, generator=g).to(torch.bfloat16)
    vn = torch.randn(N, 2, 64, generator=g).to(torch.bfloat16)
    k2, v2 = orc.kv_append(case["k_pool"], case["v_pool"], case["block_table"], kn, vn, indptr,
                           torch.tensor(ctx, dtype=torch.int32))
    assert k2.stride() == case["k_pool"].stride()
    written = torch.zeros(k2.shape[0], k2.shape[1], dtype=torch.bool)
    for b in range(5):
        seq_k = dense_kv(k2, case["block_table"][b], ctx[b] + new[b], 16)[ctx[b]:]
        seq_v = dense_kv(v2, case["block_table"][b], ctx[b] + new[b], 16)[ctx[b]:]
        assert torch.equal(seq_k, kn[indptr[b]:indptr[b + 1]])
        assert torch.equal(seq_v, vn[indptr[b]:indptr[b + 1]])
        for j in range(ctx[b], ctx[b] + new[b]):
            written[int(case["block_table"][b][j // 16]), j % 16] = True
    assert torch.equal(k2[~written], case["k_pool"][~written])
    assert torch.equal(v2[~written], case["v_pool"][~written])


# ---------------------------------------------------------------- rotary
def rope_tables(rows, D, base=10000.0):
    i = torch.arange(D // 2, dtype=torch.float64)
    theta = base ** (-2.0 * i / D)
    ang = torch.arange(rows, dtype=torch.float64)[:, None] * theta[None, :]
    return ang.cos().float(), ang.sin().float(), ang


def test_rotary_matches_numpy_complex_product(orc):
    """The pages' fallback: view adjacent pairs as complex numbers and
    multiply by cos + i sin.  numpy complex128 here, rounded to bf16."""
    import numpy as np
    T, H, D = 9, 3, 64
    g = torch.Generator().manual_seed(80)
    x = torch.randn(T, H, D, generator=g).to(torch.bfloat16)
    cos, sin, _ = rope_tables(50, D)
    pos = torch.tensor([0, 1, 2, 7, 49, 13, 13, 30, 5], dtype=torch.int32)
    out = orc.rotary(x, cos, sin, pos)
    xc = x.double().numpy().reshape(T, H, D // 2, 2)
    z = xc[..., 0] + 1j * xc[..., 1]
    w = (cos.double().numpy() + 1j * sin.double().numpy())[pos.numpy()][:, None, :]
    r = z * w
    ref = torch.from_numpy(np.stack([r.real, r.imag], -1).reshape(T, H, D)).to(torch.bfloat16)
    diff = (out.double() - ref.double()).abs()
    # both are one rounding of (nearly) the same product: at most one bf16 step apart
    assert float((diff / ref.double().abs().clamp_min(1e-30)).max()) <= 2 ** -7
    assert (out == ref).float().mean() > 0.99


def test_rotary_identity_at_angle_zero_and_pair_norms(orc):
    T, H, D = 6, 2, 32
    g = torch.Generator().manual_seed(81)
    x = torch.randn(T, H, D, generator=g).to(torch.bfloat16)
    cos, sin, _ = rope_tables(20, D)
    assert torch.equal(orc.rotary(x, cos, sin, torch.zeros(T, dtype=torch.int32)), x)
    out = orc.rotary(x, cos, sin, torch.arange(T, dtype=torch.int32) * 3).double()
    n_in = x.double().reshape(T, H, D // 2, 2).pow(2).sum(-1).sqrt()
    n_out = out.reshape(T, H, D // 2, 2).pow(2).sum(-1).sqrt()
    assert torch.allclose(n_in, n_out, rtol=2 ** -7, atol=1e-6)


def test_rotary_dot_products_depend_on_relative_position(orc):
    """(R_m q) . (R_n k) depends on n - m only (the property rotary
    embeddings are built for): shifting both positions leaves it unchanged."""
    D = 64
    g = torch.Generator().manual_seed(82)
    q = torch.randn(1, 1, D, generator=g).to(torch.bfloat16)
    k = torch.randn(1, 1, D, generator=g).to(torch.bfloat16)
    cos, sin, _ = rope_tables(200, D)
    def dot(m, n):
        a = orc.rotary(q, cos, sin, torch.tensor([m], dtype=torch.int32)).double()
        b = orc.rotary(k, cos, sin, torch.tensor([n], dtype=torch.int32)).double()
        return float((a * b).sum())
    scale = float(q.double().norm() * k.double().norm())
    for m, n, d in [(3, 10, 50), (0, 7, 100), (40, 41, 120)]:
        assert abs(dot(m, n) - dot(m + d, n + d)) <= 2 ** -6 * scale


# ------------------------------------------------------ fp8 quantize-on-write
def test_fp8_quantize_matches_torch_cast(orc):
    """Codes = torch's float8_e4m3fn cast (round to nearest even) of the
    binary32 product, after clamping to +-448 (the saturating reading)."""
    N, HD = 16, 512
    g = torch.Generator().manual_seed(90)
    x = (torch.randn(N, HD, generator=g) * torch.logspace(-3, 2, N)[:, None]).to(torch.bfloat16)
    mult = torch.logspace(-1, 3, N).float()
    codes, inv, amax = orc.fp8_quantize(x, mult)
    prod = x.float() * mult[:, None]
    ref = prod.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    assert torch.equal(codes, ref)
    assert torch.equal(inv, (1.0 / mult).to(torch.bfloat16))
    assert torch.equal(amax, x.float().abs().amax(1))


def test_fp8_quantize_dynamic_scale_and_round_trip(orc):
    """mult = 448 / amax: the largest magnitude of a row maps to 448 (code
    0x7E / 0xFE); values that are e4m3 codes times 1/m come back exactly."""
    N, HD = 8, 512
    g = torch.Generator().manual_seed(91)
    x = torch.randn(N, HD, generator=g).to(torch.bfloat16)
    codes, inv, amax = orc.fp8_quantize(x)
    arg = x.float().abs().argmax(1)
    for n in range(N):
        assert int(codes[n, arg[n]]) & 0x7F == 0x7E
    m = (448.0 / amax)
    assert torch.equal(inv, (1.0 / m).to(torch.bfloat16))
    # exact round trip: representable codes scaled by a power of two
    vals = torch.tensor([orc.e4m3fn_to_f64(c) for c in range(0x7F)], dtype=torch.float64)
    y = torch.cat([vals, -vals])[:HD].reshape(1, -1) / 4.0      # exact in bf16
    yb = y.to(torch.bfloat16)
    assert torch.equal(yb.double(), y)
    c2, _, _ = orc.fp8_quantize(yb, torch.tensor([4.0]))
    back = torch.tensor([orc.e4m3fn_to_f64(int(c)) for c in c2[0]], dtype=torch.float64) / 4.0
    assert torch.equal(back, y[0])


def test_fp8_quantize_saturates_and_keeps_signed_zero(orc):
    x = torch.tensor([[1000.0, -1000.0, 449.0, 464.0, -0.0, 0.0, 1e-4, -1e-4] + [0.0] * 8]).to(torch.bfloat16)
    codes, _, _ = orc.fp8_quantize(x, torch.tensor([1.0]))
    assert codes[0, :8].tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x80, 0x00, 0x00, 0x80]


def test_fp8_quantize_ties_go_to_even_code(orc):
    """Every midpoint between two adjacent finite e4m3 magnitudes (exact in
    bf16) rounds to the code with an even mantissa, as torch's cast does."""
    vals = [orc.e4m3fn_to_f64(c) for c in range(0x7F)]
    mids = [(vals[c] + vals[c + 1]) / 2 for c in range(0x7E)]
    x = torch.tensor(mids + [-m for m in mids], dtype=torch.float64)
    assert torch.equal(x.to(torch.bfloat16).double(), x)          # exact in bf16
    pad = 512 - x.numel()
    xb = torch.cat([x, torch.zeros(pad, dtype=torch.float64)]).to(torch.bfloat16).reshape(1, -1)
    codes, _, _ = orc.fp8_quantize(xb, torch.tensor([1.0]))
    got = codes[0, :x.numel()]
    for i, c in enumerate(got.tolist()):
        assert (c & 1) == 0, (float(x[i]), hex(c))
    assert torch.equal(got, x.float().to(torch.float8_e4m3fn).view(torch.uint8))


def test_fp8_quantize_decides_on_the_binary32_product(orc):
    """The code is chosen from the product rounded to binary32 (the precision
    the kernel decides in): a product just above the 1.0 / 1.125 midpoint
    that rounds onto it in binary32 gives the even code 1.0 (0x38), whereas
    rounding the exact product would give 1.125 (0x39)."""
    import numpy as np
    found = None
    for xi in range(1, 128):
        x = 1.0 + xi / 128.0                                   # bf16-exact
        m0 = np.float32(1.0625 / x)
        for k in range(-8, 9):
            m = np.nextafter(m0, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            m = np.float32(m0 + (m - m0) * abs(k)) if k else m0
            exact = x * float(m)                               # exact in double (24 x 8 bits)
            if exact > 1.0625 and np.float32(x) * m == np.float32(1.0625):
                found = (x, m)
                break
        if found:
            break
    assert found is not None
    x, m = found
    xb = torch.tensor([[x] + [0.0] * 511], dtype=torch.float64).to(torch.bfloat16)
    codes, _, _ = orc.fp8_quantize(xb, torch.tensor([float(m)], dtype=torch.float32))
    assert int(codes[0, 0]) == 0x38
