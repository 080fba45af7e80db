"""GPU tests of the input-domain edges stated in include/paged_attn.h:
keep-masks whose rows start at any byte, the non-finite input policy, and
cache slots far past 2^32 / block_size (exact division of a slot by a block
size that is not a power of two)."""
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


def run_paged_prefill(case, mask, S=1):
    G = case["Hq"] // case["Hkv"]
    R = pa.attn_prefill_tile_rows(case["D"], G)
    _, t2b, t2i = pa.attn_prefill_plan(case["q_lens"], R)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens", "qo_indptr",
                                     "causal_offset")}
    out = torch.full_like(d["q"], float("nan"))
    pa.attn_paged_prefill_split(d["q"], d["qo_indptr"], t2b.to(DEV), t2i.to(DEV), d["k_pool"], d["v_pool"],
                                d["block_table"], d["kv_lens"], out, case["page_size"], case["scale"],
                                max(case["kv_lens"].tolist()), causal_offset=d["causal_offset"], mask=mask,
                                num_splits=S, tile_rows=R)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------- unaligned mask rows
@pytest.mark.parametrize("ndim,S", [(3, 1), (2, 1), (3, 3)])
def test_paged_prefill_mask_rows_at_any_byte(ndim, S):
    """A plain bool keep-mask [B, q, kv] / [B, kv] whose key dimension is odd
    (rows start at every byte offset mod 4), no padding."""
    case = workloads.prefill_case(1100 + ndim + S, 3, 8, 2, 128, None, None, 16, q_lens=[37, 6, 70],
                                  ctx_lens=[250, 901, 3], mask_frac=0.25, mask_ndim=ndim, mask_pad=1)
    assert case["mask"].shape[-1] == 907 and case["mask"].dtype == torch.bool
    ref, _ = oracle.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"],
                                  case["block_table"], case["kv_lens"], case["scale"],
                                  causal_offset=case["causal_offset"], mask=case["mask"])
    out = run_paged_prefill(case, case["mask"].to(DEV), S)
    assert_close(out, ref, what="mask ndim=%d S=%d" % (ndim, S))


def test_paged_prefill_mask_view_at_odd_offset():
    """The mask is a view starting one byte into its storage (odd pointer,
    odd row strides)."""
    case = workloads.prefill_case(1110, 2, 8, 2, 128, None, None, 16, q_lens=[40, 17], ctx_lens=[600, 33],
                                  mask_frac=0.2, mask_ndim=3, mask_pad=1)
    B, Q, N = case["mask"].shape
    big = torch.zeros(B, Q, N + 2, dtype=torch.bool)
    big[:, :, 1:N + 1] = case["mask"]
    view = big.to(DEV)[:, :, 1:N + 1]
    assert view.data_ptr() % 4 != 0 and view.stride(1) % 4 != 0
    ref, _ = oracle.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"],
                                  case["block_table"], case["kv_lens"], case["scale"],
                                  causal_offset=case["causal_offset"], mask=case["mask"])
    assert_close(run_paged_prefill(case, view), ref, what="odd-offset mask view")


def test_dense_prefill_mask_rows_at_any_byte():
    B, Lq, Lk, Hq, Hkv, D = 2, 33, 301, 8, 2, 64
    g = torch.Generator().manual_seed(1120)
    q = torch.randn(B, Lq, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Lk, Hkv, D, generator=g).to(torch.bfloat16)
    mask = torch.rand(B, Lq, Lk, generator=g) >= 0.3
    scale = 1.0 / math.sqrt(D)
    # the oracle's ragged prefill over one page per sequence is the dense case
    kp = k.reshape(B, Lk, Hkv, D)
    bt = torch.arange(B, dtype=torch.int32).view(B, 1)
    kv_lens = torch.full((B,), Lk, dtype=torch.int32)
    qo = torch.arange(0, (B + 1) * Lq, Lq, dtype=torch.int32)
    ref, _ = oracle.paged_prefill(q.reshape(B * Lq, Hq, D), qo, kp, v.reshape(B, Lk, Hkv, D), bt, kv_lens, scale,
                                  causal_offset=torch.full((B,), Lk - Lq, dtype=torch.int32), mask=mask)
    out = torch.full((B, Lq, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), out, scale, is_causal=True, mask=mask.to(DEV))
    torch.cuda.synchronize()
    assert_close(out.reshape(B * Lq, Hq, D), ref, what="dense, mask kv=301")


# ------------------------------------------------- non-finite input policy
NAN = float("nan")


# Hq = 32 over 8 KV heads runs the VALU kernel (4 heads a row), 64 over 8 the
# MFMA kernel (8 heads a row on one 16-row block)
@pytest.mark.parametrize("Hq", [32, 64])
def test_decode_nan_query_poisons_only_its_row(Hq):
    case = workloads.paged_decode_case(1130, 4, Hq, 8, 128, [300, 1000, 17, 2500], 16)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens")}
    for S in (1, 9):
        clean = torch.empty_like(d["q"])
        pa.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"], case["max_kv_len"],
                             clean, 16, case["scale"], num_splits=S)
        qn = d["q"].clone()
        qn[1, 5, 77] = NAN
        out = torch.empty_like(d["q"])
        pa.attn_paged_decode(qn, d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"], case["max_kv_len"],
                             out, 16, case["scale"], num_splits=S)
        torch.cuda.synchronize()
        assert bool(torch.isnan(out[1, 5]).all()), "S=%d" % S
        keep = torch.ones(4, Hq, dtype=torch.bool)
        keep[1, 5] = False
        assert torch.equal(out.cpu()[keep], clean.cpu()[keep]), "S=%d" % S


@pytest.mark.parametrize("Hq", [32, 64])
def test_decode_nan_key_poisons_the_heads_that_read_it(Hq):
    case = workloads.paged_decode_case(1131, 3, Hq, 8, 128, [400, 1500, 64], 16)
    d = {k: case[k].to(DEV) for k in ("q", "k_pool", "v_pool", "block_table", "kv_lens")}
    j, b, g = 700, 1, 3
    page = int(case["block_table"][b, j // 16])
    kp = d["k_pool"].clone()
    kp[page, j % 16, g, 5] = NAN
    for S in (1, 7):
        clean = torch.empty_like(d["q"])
        pa.attn_paged_decode(d["q"], d["k_pool"], d["v_pool"], d["block_table"], d["kv_lens"], case["max_kv_len"],
                             clean, 16, case["scale"], num_splits=S)
        out = torch.empty_like(d["q"])
        pa.attn_paged_decode(d["q"], kp, d["v_pool"], d["block_table"], d["kv_lens"], case["max_kv_len"],
                             out, 16, case["scale"], num_splits=S)
        torch.cuda.synchronize()
        G = Hq // 8
        assert bool(torch.isnan(out[b, g * G:(g + 1) * G]).all()), "S=%d" % S
        keep = torch.ones(3, Hq, dtype=torch.bool)
        keep[b, g * G:(g + 1) * G] = False
        assert torch.equal(out.cpu()[keep], clean.cpu()[keep]), "S=%d" % S


@pytest.mark.parametrize("S", [1, 3])
def test_prefill_nan_query_poisons_only_its_row(S):
    case = workloads.prefill_case(1140, 3, 8, 2, 128, None, None, 16, q_lens=[50, 7, 130], ctx_lens=[100, 900, 0])
    clean = run_paged_prefill(case, None, S).cpu()
    r, h = 60, 6
    case["q"] = case["q"].clone()
    case["q"][r, h, 3] = NAN
    out = run_paged_prefill(case, None, S).cpu()
    assert bool(torch.isnan(out[r, h]).all())
    keep = torch.ones(out.shape[:2], dtype=torch.bool)
    keep[r, h] = False
    assert torch.equal(out[keep], clean[keep])


@pytest.mark.parametrize("masked", [False, True])
def test_prefill_nan_key_reaches_exactly_the_rows_that_admit_it(masked):
    """A NaN in the K row of key j of one sequence and KV head: causal rows
    that admit j (and keep it in the mask) become NaN for the KV head's query
    heads; every other output is unchanged, bit for bit (a key a row does not
    admit has its score replaced, never used)."""
    case = workloads.prefill_case(1150, 2, 8, 2, 128, None, None, 16, q_lens=[90, 20], ctx_lens=[300, 50],
                                  mask_frac=0.3 if masked else None, mask_ndim=3)
    mask = case["mask"].to(DEV) if masked else None
    clean = run_paged_prefill(case, mask).cpu()
    b, j, g, G = 0, 340, 1, 4            # key 340 of sequence 0: admitted from local row 40 on
    page = int(case["block_table"][b, j // 16])
    case["k_pool"] = case["k_pool"].clone()
    case["k_pool"][page, j % 16, g, 9] = NAN
    out = run_paged_prefill(case, mask).cpu()
    c = case["ctx_lens"][b]
    poisoned = torch.zeros(out.shape[:2], dtype=torch.bool)
    for i in range(case["q_lens"][b]):
        admits = j <= c + i and (not masked or bool(case["mask"][b, i, j]))
        if admits:
            poisoned[i, g * G:(g + 1) * G] = True
    assert int(poisoned.sum()) > 0 and int((~poisoned).sum()) > 0
    assert bool(torch.isnan(out[poisoned]).all())
    assert torch.equal(out[~poisoned], clean[~poisoned])


# ------------------------------------ slots past 2^32 / block size
def big_slot_cache(block_size, num_blocks, rows_per_block_step, g):
    """A cache view [num_blocks, block_size, 512] whose block stride holds
    only rows_per_block_step rows (blocks overlap in memory), so slot indices
    up to num_blocks * block_size address a buffer of a few tens of MB."""
    c_ss, c_sb = 512, rows_per_block_step * 512
    n = (num_blocks - 1) * c_sb + (block_size - 1) * c_ss + 512
    x = torch.randn(n // 512, 512, generator=g)
    inv = (0.01 + 0.09 * torch.rand(num_blocks * block_size, 1, generator=g)).to(torch.bfloat16)
    codes = (x / 0.05).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).reshape(-1)
    return codes, (num_blocks, block_size, 512), (c_sb, c_ss, 1), inv


@pytest.mark.parametrize("block_size,num_blocks", [(1000, 7000), (3000, 2400)])
def test_swa_decode_slots_past_the_old_magic_range(block_size, num_blocks):
    """Slots from 6.1M up with a block size of 1000 or 3000: the division of
    a slot by the block size must be exact there (a rounded-up 2^32 / d
    reciprocal gave block + 1 and an offset near 2^32 from slot 6,101,999 on)."""
    g = torch.Generator().manual_seed(1160 + block_size)
    flat, shape, strides, inv = big_slot_cache(block_size, num_blocks, 16, g)
    cache = flat.as_strided(shape, strides)
    T, NH, W = 8, 16, 64
    slots = num_blocks * block_size
    q = torch.randn(T, NH, 512, generator=g).to(torch.bfloat16)
    ind = torch.randint(6_100_000, slots, (T, W), generator=g, dtype=torch.int64)
    ind[0, :8] = torch.arange(6_100_990, 6_100_998)      # around the first failing slot
    ind[1, :4] = torch.tensor([slots - 1, slots - 2, 6_101_999, 6_101_000])
    lens = torch.tensor([W, 13, 64, 1, 40, 64, 7, 50], dtype=torch.int64)
    scale = 1.0 / math.sqrt(512)
    ref, _ = oracle.swa_fp8_decode(q, cache, inv, ind, lens, block_size, scale)
    cache_d = flat.to(DEV).as_strided(shape, strides)
    out = torch.full((T, NH, 512), NAN, dtype=torch.bfloat16, device=DEV)
    pa.attn_swa_fp8_decode(q.to(DEV), cache_d, inv.to(DEV), ind.to(DEV), lens.to(DEV), out, block_size, scale)
    torch.cuda.synchronize()
    assert_close(out, ref, what="bs=%d slots %d" % (block_size, slots))


def test_fp8_append_slots_past_the_old_magic_range():
    block_size, num_blocks = 1000, 7000
    g = torch.Generator().manual_seed(1170)
    flat, shape, strides, _ = big_slot_cache(block_size, num_blocks, 16, g)
    cand = torch.randint(6_100_000, num_blocks * block_size, (4000,), generator=g, dtype=torch.int64)
    cand = torch.cat([torch.tensor([6_101_999, 6_100_999, num_blocks * block_size - 1]), cand])
    row = (cand // block_size) * 16 + cand % block_size      # memory row of each slot in the overlapping view
    seen, pick = set(), []
    for i, r in enumerate(row.tolist()):
        if r not in seen:
            seen.add(r)
            pick.append(i)
    slots = cand[pick][:512]
    N = slots.numel()
    assert N == 512
    x = torch.randn(N, 512, generator=g).to(torch.bfloat16)
    cache_d = torch.zeros_like(flat, device=DEV)
    inv_d = torch.zeros(num_blocks * block_size, 1, dtype=torch.bfloat16, device=DEV)
    pa.attn_swa_fp8_append(x.to(DEV), slots.to(DEV), cache_d.as_strided(shape, strides), inv_d, block_size)
    torch.cuda.synchronize()
    codes, inv_ref, _ = oracle.fp8_quantize(x)
    got = cache_d.cpu().view(-1, 512)
    rows = ((slots // block_size) * 16 + slots % block_size).tolist()
    assert torch.equal(got[rows], codes)
    assert torch.equal(inv_d.cpu()[slots, 0].view(torch.int16), inv_ref.view(torch.int16).reshape(-1))
