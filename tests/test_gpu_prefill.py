"""GPU parity of the ragged paged prefill (MFMA) against the CPU oracle.

Bar: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| on the bf16 outputs."""
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
                          causal_offset=d["causal_offset"] if causal else None, mask=mask)
    torch.cuda.synchronize()
    return out


def oracle_prefill(case, causal=True):
    out, _ = oracle.paged_prefill(case["q"], case["qo_indptr"], case["k_pool"], case["v_pool"],
                                  case["block_table"], case["kv_lens"], case["scale"],
                                  causal_offset=case["causal_offset"] if causal else None, mask=case["mask"])
    return out


@pytest.mark.parametrize("masked", [False, True])
def test_ragged_prefill_config(masked):
    case = workloads.ragged_prefill(masked=masked)
    assert_close(run_prefill(case), oracle_prefill(case), what="ragged prefill masked=%s" % masked)


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
