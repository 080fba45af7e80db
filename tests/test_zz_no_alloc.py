"""attn_paged_decode_noalloc (the decode entry point that allocates nothing)
against attn_paged_decode, through the C ABI: same split count, outputs
bit-identical, on two calls in a row (the second smaller, so the static
scratch holds the first call's partials when it starts), plus the oracle at
the 1e-2 bar, and no device allocation by the call."""
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


def dev_case(case):
    return {k: (case[k].to(DEV) if torch.is_tensor(case[k]) else case[k]) for k in case}


def both(c, S):
    """(no-alloc output, attn_paged_decode output) for split count S (0 =
    planner) and the device bytes torch allocated around the no-alloc call."""
    ref = torch.empty_like(c["q"])
    W = S or pa.attn_plan_splits(c["B"], c["Hkv"], c["Hq"] // c["Hkv"], c["D"], c["max_kv_len"], c["page_size"],
                                 c["k_pool"].stride(2))
    pa.attn_paged_decode(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["kv_lens"], c["max_kv_len"], ref,
                         c["page_size"], c["scale"], num_splits=W)
    out = torch.full_like(c["q"], float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    pa.attn_paged_decode_noalloc(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["kv_lens"], c["max_kv_len"],
                                 out, c["page_size"], c["scale"], num_splits=S)
    after = torch.cuda.memory_allocated(DEV)
    torch.cuda.synchronize()
    return out, ref, after - before


@pytest.mark.parametrize("S", [0, 9])
def test_noalloc_matches_paged_decode_on_two_calls(S):
    big = workloads.serving_paged_decode(32)            # config 3, B = 32
    small = workloads.paged_decode_case(1190, 5, 16, 4, 64, [300, 0, 1, 77, 1000], 16)
    for name, case in (("B=32 serving", big), ("B=5 small", small)):
        c = dev_case(case)
        out, ref, grew = both(c, S)
        assert grew == 0, "%s: the call allocated %d bytes" % (name, grew)
        assert torch.equal(out, ref), "%s S=%d: differs from attn_paged_decode" % (name, S)
        want, _ = oracle.paged_decode(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                      case["kv_lens"], case["scale"])
        assert_close(out, want, what="%s S=%d vs oracle" % (name, S))


def test_noalloc_lowers_the_planner_count_to_fit_and_refuses_an_explicit_one():
    """B = 128 over 32 heads of 128: the planner's 768 slices need 15 MB of
    partials, which fits; 4000 explicit slices (71 MB) do not and are
    refused; with 2048 sequences the planner's count is lowered to fit."""
    case = dev_case(workloads.paged_decode_case(1191, 128, 32, 8, 128, (1, 300), 16))
    W = pa.attn_plan_splits(128, 8, 4, 128, case["max_kv_len"], 16, case["k_pool"].stride(2))
    assert pa.attn_decode_workspace_bytes(128, 32, 128, W) <= pa.NOALLOC_SCRATCH_BYTES
    assert pa.attn_decode_workspace_bytes(128, 32, 128, 4000) > pa.NOALLOC_SCRATCH_BYTES
    out = torch.empty_like(case["q"])
    with pytest.raises(pa.AttnError, match="static"):
        pa.attn_paged_decode_noalloc(case["q"], case["k_pool"], case["v_pool"], case["block_table"],
                                     case["kv_lens"], case["max_kv_len"], out, 16, case["scale"], num_splits=4000)
    big = workloads.paged_decode_case(1192, 2048, 32, 8, 128, (1, 40), 16)
    c = dev_case(big)
    out = torch.empty_like(c["q"])
    pa.attn_paged_decode_noalloc(c["q"], c["k_pool"], c["v_pool"], c["block_table"], c["kv_lens"],
                                 c["max_kv_len"], out, 16, c["scale"])
    torch.cuda.synchronize()
    assert pa.attn_decode_workspace_bytes(2048, 32, 128, 1) > 0
    idx = torch.arange(0, 2048, 97)
    want, _ = oracle.paged_decode(big["q"][idx], big["k_pool"], big["v_pool"], big["block_table"][idx],
                                  big["kv_lens"][idx], big["scale"])
    assert_close(out.cpu()[idx], want, what="B=2048 lowered count")
