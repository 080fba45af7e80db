"""GPU parity of the cache writes and the rotary embedding against the oracle.

Bars: the paged KV append is a copy and the fp8 quantize decides integer
codes, so both are compared bit for bit (codes, inverse scales, amax, every
pool byte); rotary outputs are bf16 results of one rounding each, held to one
bf16 step (2^-7 relative) with at least 99% identical."""
import math

import pytest
import torch

import oracle
import paged_kv_gqa_03_amd as pa
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


# ------------------------------------------------------------ KV append
def append_case(seed, B, Hkv, D, ps, ctx, new, layout="page_slot_head"):
    lens = [c + n for c, n in zip(ctx, new)]
    case = workloads.paged_decode_case(seed, B, Hkv * 4, Hkv, D, lens, ps, layout=layout)
    g = torch.Generator().manual_seed(seed + 1)
    N = sum(new)
    kn = torch.randn(N, Hkv, D, generator=g).to(torch.bfloat16)
    vn = torch.randn(N, Hkv, D, generator=g).to(torch.bfloat16)
    indptr = torch.tensor([0] + list(torch.tensor(new, dtype=torch.int64).cumsum(0).tolist()), dtype=torch.int32)
    return case, kn, vn, indptr, torch.tensor(ctx, dtype=torch.int32)


def run_append(case, kn, vn, indptr, start):
    kp = case["k_pool"].to(DEV)
    vp = case["v_pool"].to(DEV)
    pa.attn_paged_kv_append(kn.to(DEV), vn.to(DEV), indptr.to(DEV), start.to(DEV), kp, vp,
                            case["block_table"].to(DEV), case["page_size"])
    torch.cuda.synchronize()
    return kp.cpu(), vp.cpu()


@pytest.mark.parametrize("ps,layout", [(16, "page_slot_head"), (1, "page_slot_head"), (5, "page_slot_head"),
                                       (16, "page_head_slot")])
def test_kv_append_matches_oracle(ps, layout):
    ctx, new = [0, 5, 16, 300, 31, 7], [1, 40, 16, 1, 0, 100]
    case, kn, vn, indptr, start = append_case(500 + ps, 6, 8, 128, ps, ctx, new, layout)
    k_ref, v_ref = oracle.kv_append(case["k_pool"], case["v_pool"], case["block_table"], kn, vn, indptr, start)
    k_got, v_got = run_append(case, kn, vn, indptr, start)
    assert torch.equal(k_got.view(torch.int16), k_ref.view(torch.int16))
    assert torch.equal(v_got.view(torch.int16), v_ref.view(torch.int16))


def test_kv_append_decode_step_then_decode():
    """One new token per sequence (a decode step), then paged decode over the
    grown cache equals the oracle on the oracle-appended cache."""
    B = 16
    ctx = [int(x) for x in torch.randint(1, 600, (B,), generator=torch.Generator().manual_seed(9))]
    case, kn, vn, indptr, start = append_case(520, B, 8, 128, 16, ctx, [1] * B)
    k_ref, v_ref = oracle.kv_append(case["k_pool"], case["v_pool"], case["block_table"], kn, vn, indptr, start)
    k_got, v_got = run_append(case, kn, vn, indptr, start)
    assert torch.equal(k_got.view(torch.int16), k_ref.view(torch.int16))
    ref, _ = oracle.paged_decode(case["q"], k_ref, v_ref, case["block_table"], case["kv_lens"], case["scale"])
    out = torch.empty_like(case["q"]).to(DEV)
    pa.attn_paged_decode(case["q"].to(DEV), k_got.to(DEV), v_got.to(DEV), case["block_table"].to(DEV),
                         case["kv_lens"].to(DEV), case["max_kv_len"], out, 16, case["scale"])
    torch.cuda.synchronize()
    err = (out.cpu().double() - ref).abs()
    assert bool((err <= 1e-2 + 1e-2 * ref.abs()).all())


def test_kv_append_skips_tokens_without_a_page():
    """A block-table entry of -1 (or past the pool) means no page: that token
    is not written and nothing else changes."""
    case, kn, vn, indptr, start = append_case(530, 2, 8, 64, 16, [10, 0], [10, 5])
    bt = case["block_table"].clone()
    bt[0, 1] = -1                       # positions 16..19 of sequence 0 have no page
    bt[1, 0] = case["k_pool"].shape[0] + 3
    case = dict(case, block_table=bt)
    k_got, v_got = run_append(case, kn, vn, indptr, start)
    # the oracle rejects a negative entry, so build the expectation by hand
    exp_k = case["k_pool"].clone()
    for i in range(10):
        pos = 10 + i
        if pos // 16 == 1:
            continue
        exp_k[int(bt[0, pos // 16]), pos % 16] = kn[i]
    assert torch.equal(k_got.view(torch.int16), exp_k.view(torch.int16))


def test_kv_append_empty_and_zero_sequences():
    case, kn, vn, indptr, start = append_case(540, 3, 8, 128, 16, [4, 4, 4], [0, 0, 0])
    k_got, v_got = run_append(case, kn, vn, indptr, start)
    assert torch.equal(k_got.view(torch.int16), case["k_pool"].view(torch.int16))


# ------------------------------------------------- fp8 quantize-on-write
def quant_rows(seed, N, spread=True):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(N, 512, generator=g)
    if spread:
        x = x * torch.logspace(-4, 3, N)[:, None]
    return x.to(torch.bfloat16)


def run_quant(x, slots, num_blocks, mult=None, cache=None, inv=None):
    bs = 256
    cache = torch.zeros(num_blocks, bs, 512, dtype=torch.uint8) if cache is None else cache
    inv = torch.zeros(num_blocks * bs, 1, dtype=torch.bfloat16) if inv is None else inv
    c_d, i_d = cache.to(DEV), inv.to(DEV)
    amax = torch.full((x.shape[0],), float("nan"), device=DEV)
    pa.attn_swa_fp8_append(x.to(DEV), slots.to(DEV), c_d, i_d, bs,
                           multiplier=None if mult is None else mult.to(DEV), amax=amax)
    torch.cuda.synchronize()
    return c_d.cpu(), i_d.cpu(), amax.cpu()


@pytest.mark.parametrize("explicit", [False, True])
def test_fp8_append_matches_oracle_bit_for_bit(explicit):
    N = 96
    x = quant_rows(600 + explicit, N)
    g = torch.Generator().manual_seed(601)
    slots = torch.randperm(8 * 256, generator=g)[:N].to(torch.int64)
    mult = torch.logspace(-2, 4, N).float() if explicit else None
    cache, inv, amax = run_quant(x, slots, 8, mult)
    codes, inv_ref, amax_ref = oracle.fp8_quantize(x, mult)
    flat = cache.view(-1, 512)
    assert torch.equal(flat[slots], codes)
    assert torch.equal(inv.view(-1)[slots].view(torch.int16), inv_ref.view(torch.int16))
    assert torch.equal(amax, amax_ref)
    untouched = torch.ones(8 * 256, dtype=torch.bool)
    untouched[slots] = False
    assert int(flat[untouched].abs().sum()) == 0


def test_fp8_append_special_values():
    """Midpoints (ties to even), saturation (finite and infinite), signed
    zeros, tiny values and NaN: the same codes as the oracle."""
    vals = [oracle.e4m3fn_to_f64(c) for c in range(0x7F)]
    mids = [(vals[c] + vals[c + 1]) / 2 for c in range(0x7E)]
    row = mids + [-m for m in mids] + [1000.0, -1000.0, 449.0, -0.0, 0.0, 1e-6, -1e-6, 2.0 ** -10,
                                       float("nan"), 3 * 2.0 ** -10, float("inf"), float("-inf"), 464.0,
                                       -464.0, 480.0]
    row = row + [0.0] * (512 - len(row))
    x = torch.tensor([row], dtype=torch.float64).to(torch.bfloat16)
    slots = torch.tensor([5], dtype=torch.int64)
    cache, inv, amax = run_quant(x, slots, 1, torch.tensor([1.0]))
    codes, _, amax_ref = oracle.fp8_quantize(x, torch.tensor([1.0]))
    assert torch.equal(cache.view(-1, 512)[5], codes[0])
    assert torch.equal(amax, amax_ref)


def test_fp8_append_skips_slots_outside_the_cache():
    x = quant_rows(610, 4)
    slots = torch.tensor([3, -1, 2 * 256, 7], dtype=torch.int64)   # cache has 2 blocks
    cache, inv, amax = run_quant(x, slots, 2)
    codes, inv_ref, amax_ref = oracle.fp8_quantize(x)
    flat = cache.view(-1, 512)
    assert torch.equal(flat[3], codes[0]) and torch.equal(flat[7], codes[3])
    others = torch.ones(512, dtype=torch.bool)
    others[3] = others[7] = False
    assert int(flat[others].abs().sum()) == 0
    assert torch.equal(amax, amax_ref)      # amax is reported for every row


def test_fp8_append_then_swa_decode():
    """Rows quantized by the kernel into the cache, then the sliding-window
    decode over that cache, equals the oracle decode over the same bytes."""
    case = workloads.swa_case(620, 12, 32, 512, 128, 256, 8, len_range=(1, 128))
    slots_used = case["indices"][case["indices"] >= 0].unique()
    x = quant_rows(621, slots_used.numel(), spread=False)
    cache, inv, _ = run_quant(x, slots_used, 8, cache=case["cache"].clone(), inv=case["inv_scale"].clone())
    case = dict(case, cache=cache, inv_scale=inv)
    ref, _ = oracle.swa_fp8_decode(case["q"], cache, inv, case["indices"], case["lens"], 256, case["scale"])
    out = torch.empty(case["q"].shape, dtype=torch.bfloat16, device=DEV)
    pa.attn_swa_fp8_decode(case["q"].to(DEV), cache.to(DEV), inv.to(DEV), case["indices"].to(DEV),
                           case["lens"].to(DEV), out, 256, case["scale"])
    torch.cuda.synchronize()
    err = (out.cpu().double() - ref).abs()
    assert bool((err <= 1e-2 + 1e-2 * ref.abs()).all())


# ---------------------------------------------------------------- rotary
def rope_tables(rows, D, base=10000.0):
    i = torch.arange(D // 2, dtype=torch.float64)
    ang = torch.arange(rows, dtype=torch.float64)[:, None] * (base ** (-2.0 * i / D))[None, :]
    return ang.cos().float(), ang.sin().float()


def assert_rotary_close(got, ref):
    got, ref = got.cpu().double(), ref.double()
    err = (got - ref).abs()
    assert bool((err <= 2.0 ** -7 * ref.abs() + 1e-30).all()), float(err.max())
    assert float((got == ref).double().mean()) >= 0.99


@pytest.mark.parametrize("T,H,D", [(37, 32, 128), (200, 8, 128), (5, 4, 64), (1, 1, 8)])
def test_rotary_matches_oracle(T, H, D):
    g = torch.Generator().manual_seed(700 + T + H + D)
    x = torch.randn(T, H, D, generator=g).to(torch.bfloat16)
    cos, sin = rope_tables(4096, D)
    pos = torch.randint(0, 4096, (T,), generator=g, dtype=torch.int32)
    ref = oracle.rotary(x, cos, sin, pos)
    out = torch.empty(T, H, D, dtype=torch.bfloat16, device=DEV)
    pa.attn_rotary_embed(x.to(DEV), cos.to(DEV), sin.to(DEV), pos.to(DEV), out=out)
    torch.cuda.synchronize()
    assert_rotary_close(out, ref)


def test_rotary_in_place_on_strided_rows_leaves_other_columns():
    """q is a column slice of a fused [T, 48 heads, D] buffer: rotating it in
    place touches only its heads; tokens at positions outside the table are
    left as they are."""
    T, D = 24, 128
    g = torch.Generator().manual_seed(710)
    big = torch.randn(T, 48, D, generator=g).to(torch.bfloat16)
    cos, sin = rope_tables(100, D)
    pos = torch.randint(0, 100, (T,), generator=g, dtype=torch.int32)
    pos[3] = -1
    pos[7] = 100
    q = big[:, 8:40]
    ref = oracle.rotary(q.contiguous(), cos, sin, pos.clamp(0, 99))
    ref[3] = q[3]
    ref[7] = q[7]
    bd = big.to(DEV)
    pa.attn_rotary_embed(bd[:, 8:40], cos.to(DEV), sin.to(DEV), pos.to(DEV))
    torch.cuda.synchronize()
    got = bd.cpu()
    assert_rotary_close(got[:, 8:40], ref)
    assert torch.equal(got[:, :8], big[:, :8]) and torch.equal(got[:, 40:], big[:, 40:])
