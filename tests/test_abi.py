"""Host-side checks of the C ABI: the library loads and exports every symbol
the header declares, host-only helpers (planner, chunking, workspace size,
ragged work map) behave, and bad arguments are rejected before any device
work.  No test here needs a GPU or makes a compute call."""
import ctypes
import json
import os
import re

import pytest
import torch

import paged_kv_gqa_03_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_path_entry_points():
    names = declared_functions()
    for n in ("attn_decode", "attn_paged_decode", "attn_paged_prefill", "attn_swa_fp8_decode",
              "attn_split_combine", "attn_plan_splits", "attn_prefill_plan", "attn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    l = ctypes.CDLL(pa.LIB_PATH)
    for n in declared_functions():
        assert hasattr(l, n), n
    assert set(declared_functions()) == set(pa.EXPORTED_SYMBOLS)


def test_version():
    assert pa.attn_version() >= 100


@pytest.mark.parametrize("B,Hkv,max_len", [(2, 2, 300), (16, 8, 2048), (32, 8, 4096), (128, 8, 4096),
                                           (1, 1, 100000), (512, 8, 4096), (4, 8, 16), (3, 1, 0)])
@pytest.mark.parametrize("s_head", [128, 16 * 128])
def test_planner_bounds(B, Hkv, max_len, s_head):
    # G = 4: four-wave slices, at most one per CU
    W = pa.attn_plan_splits(B, Hkv, 4, 128, max_len, 16, s_head, 256)
    hw = min(8, Hkv) if s_head == 128 else 1
    assert 1 <= W <= (192 if hw == 8 else 256)
    rows = B * (Hkv // hw)
    # no slice shorter than 256 tokens of a row, given the longest possible line
    assert W == 1 or rows * max_len >= 256 * (W - 1)
    # a larger batch never asks for fewer slices
    assert pa.attn_plan_splits(2 * B, Hkv, 4, 128, max_len, 16, s_head, 256) >= W


def test_planner_waves_per_cu_target():
    # G <= 4, eight KV heads per row (whole 2 KB token rows): four-wave
    # slices on three quarters of the CUs (768 waves on 256 CUs)
    assert pa.attn_plan_splits(128, 8, 4, 128, 4096, 16, 128, 256) == 192
    assert pa.attn_plan_splits(32, 8, 4, 128, 4096, 16, 128, 304) == 228
    # one KV head per row (head-major source): one four-wave slice per CU
    assert pa.attn_plan_splits(16, 8, 4, 128, 2048, 0, 2048 * 128, 256) == 256
    assert pa.attn_plan_splits(2, 2, 4, 64, 300, 16, 64, 256) == 3   # 600 tokens / 256
    # G = 8 at D = 128: the MFMA kernel, one KV head per row, one four-wave
    # slice per CU; at D = 256 the VALU kernel, one-wave slices, three waves
    # per CU with four heads per row... (two waves per CU for one head)
    assert pa.attn_plan_splits(128, 8, 8, 128, 4096, 16, 128, 256) == 256
    assert pa.attn_plan_splits(128, 8, 8, 256, 4096, 16, 256, 256) == 512


def test_workspace_bytes_layout():
    assert pa.attn_decode_workspace_bytes(0, 32, 128, 4) == 0
    n = pa.attn_decode_workspace_bytes(32, 32, 128, 100)
    rows = (32 + 100) * 32
    ml_end = ((rows * 128 * 4 + 255) // 256) * 256 + rows * 2 * 4
    assert n == (ml_end + 255) // 256 * 256 + 32 * 32 * 2 * 4


def test_work_map_matches_worked_example():
    with open(os.path.join(GOLDEN, "ragged_work_map.json")) as f:
        ex = json.load(f)
    indptr, t2b, t2i = pa.attn_prefill_plan(ex["q_lens"], ex["tile_rows"])
    assert indptr.tolist() == ex["qo_indptr"]
    assert t2b.tolist() == ex["q_tile_to_batch"] and t2i.tolist() == ex["q_tile_to_index"]


def test_work_map_matches_oracle_on_random_batches(orc):
    g = torch.Generator().manual_seed(11)
    for _ in range(40):
        B = int(torch.randint(1, 12, (1,), generator=g))
        lens = torch.randint(0, 700, (B,), generator=g).tolist()
        R = int(torch.randint(1, 129, (1,), generator=g))
        a = pa.attn_prefill_plan(lens, R)
        b = orc.prefill_plan(lens, R)
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_work_map_rejects_small_cap():
    lib = pa.lib()
    lens = torch.tensor([70, 10, 130], dtype=torch.int32)
    indptr = torch.empty(4, dtype=torch.int32)
    t = torch.empty(8, dtype=torch.int32)
    n = ctypes.c_int(0)
    rc = lib.attn_prefill_plan(ctypes.c_void_p(lens.data_ptr()), 3, 64, ctypes.c_void_p(indptr.data_ptr()),
                               ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(t.data_ptr()), 5, ctypes.byref(n))
    assert rc == pa.ATTN_ERR_INVALID_ARG and "cap" in pa.attn_last_error()


# --- argument validation (rejected on the host; no HIP call is made) -----
FAKE = 1 << 20  # 16-byte aligned fake device address, never dereferenced


def paged_args(**over):
    a = dict(q=FAKE, q_sb=256, q_sh=64, k=FAKE, v=FAKE, s_page=16 * 2 * 64, s_slot=2 * 64, s_head=64,
             bt=FAKE, bt_sb=32, lens=FAKE, max_len=300, o=FAKE, o_sb=256, o_sh=64,
             B=2, Hq=8, Hkv=2, D=64, ps=16, scale=0.125, S=1, ws=None, ws_bytes=0)
    a.update(over)
    return a


def call_paged(a):
    return pa.lib().attn_paged_decode(
        a["q"], a["q_sb"], a["q_sh"], a["k"], a["v"], a["s_page"], a["s_slot"], a["s_head"],
        a["bt"], a["bt_sb"], a["lens"], a["max_len"], a["o"], a["o_sb"], a["o_sh"],
        a["B"], a["Hq"], a["Hkv"], a["D"], a["ps"], a["scale"], a["S"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("over,code,word", [
    (dict(Hq=7), pa.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(D=96), pa.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(q=None), pa.ATTN_ERR_INVALID_ARG, "null"),
    (dict(bt=None), pa.ATTN_ERR_INVALID_ARG, "null"),
    (dict(q=FAKE + 2), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(s_slot=100), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(ps=0), pa.ATTN_ERR_INVALID_ARG, "page_size"),
    (dict(B=-1), pa.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(scale=float("nan")), pa.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(S=1 << 20), pa.ATTN_ERR_INVALID_ARG, "num_splits"),
    (dict(S=4), pa.ATTN_ERR_WORKSPACE, "workspace"),
    (dict(S=4, ws=FAKE + 16, ws_bytes=1 << 30), pa.ATTN_ERR_INVALID_ARG, "aligned"),
    (dict(B=1 << 20, max_len=1 << 12, q_sb=256), pa.ATTN_ERR_UNSUPPORTED, "2^31"),
])
def test_paged_decode_rejects_bad_arguments(over, code, word):
    rc = call_paged(paged_args(**over))
    assert rc == code
    assert word in pa.attn_last_error()


def test_decode_rejects_bad_arguments():
    lib = pa.lib()
    rc = lib.attn_decode(FAKE, 256, 64, FAKE, 4096, 2048, 64, FAKE, 4096, 2048, 63,
                         FAKE, 256, 64, None, 32, 2, 8, 2, 64, 0.125, 1, None, 0, None)
    assert rc == pa.ATTN_ERR_UNSUPPORTED and "aligned" in pa.attn_last_error()
    rc = lib.attn_decode(FAKE, 256, 64, FAKE, 4096, 2048, 64, FAKE, 4096, 2048, 64,
                         FAKE, 256, 64, None, -1, 2, 8, 2, 64, 0.125, 1, None, 0, None)
    assert rc == pa.ATTN_ERR_INVALID_ARG


def test_combine_rejects_bad_arguments():
    lib = pa.lib()
    assert lib.attn_split_combine(FAKE, FAKE, 0, 4, 128, FAKE, None, None, None) == pa.ATTN_ERR_INVALID_ARG
    assert lib.attn_split_combine(FAKE, FAKE, 2, 4, 96, FAKE, None, None, None) == pa.ATTN_ERR_UNSUPPORTED
    assert lib.attn_split_combine(FAKE, FAKE, 2, 4, 128, None, None, None, None) == pa.ATTN_ERR_INVALID_ARG


def test_binding_refuses_non_unit_inner_stride():
    x = torch.zeros(2, 8, 128, dtype=torch.bfloat16)[:, :, ::2]
    with pytest.raises(ValueError):
        pa._unit_inner(x)


# --- split-KV prefill: host planner, workspace size, argument checks ------
def test_prefill_tile_rows_pack_every_head_of_a_group():
    # 32 rows of one head per wave for G <= 4; G = 8: two heads of 16 rows
    assert [pa.attn_prefill_tile_rows(128, G) for G in (1, 2, 4, 8)] == [128, 64, 32, 16]


def test_prefill_split_planner():
    # the short-q / long-kv workload: 16 tiles x 4 KV heads = 64 workgroups
    assert pa.attn_prefill_plan_splits(16, 32, 4, 128, 16384, 256) == 4
    assert pa.attn_prefill_plan_splits(16, 32, 4, 128, 16384, 1024) == 16
    # at least 8 key tiles of 64 per split
    assert pa.attn_prefill_plan_splits(16, 32, 4, 128, 1024, 1024) == 2
    assert pa.attn_prefill_plan_splits(16, 32, 4, 128, 511, 1024) == 1
    # enough workgroups already: no split
    assert pa.attn_prefill_plan_splits(72, 32, 8, 128, 2560, 256) == 1
    assert pa.attn_prefill_plan_splits(0, 32, 8, 128, 2560, 256) == 1
    # capped at 256
    assert pa.attn_prefill_plan_splits(1, 8, 8, 128, 1 << 22, 1 << 20) == 256
    assert pa.lib().attn_prefill_plan_splits(1, 6, 4, 128, 100, 256) == pa.ATTN_ERR_INVALID_ARG


def test_prefill_workspace_bytes_layout():
    assert pa.attn_prefill_workspace_bytes(100, 32, 128, 1) == 0
    rows, Hq, D, S = 256, 32, 128, 4
    o_bytes = S * rows * Hq * D * 4
    assert pa.attn_prefill_workspace_bytes(rows, Hq, D, S) == (o_bytes + 255) // 256 * 256 + S * rows * Hq * 2 * 4
    assert pa.attn_prefill_workspace_bytes(3, 2, 32, 3) == (3 * 3 * 2 * 32 * 4 + 255) // 256 * 256 + 3 * 3 * 2 * 8


def call_paged_prefill_split(S, ws=None, ws_bytes=0, total_q=40):
    # 2 sequences, Hq=8, Hkv=2, D=128, page size 16, fake device addresses
    return pa.lib().attn_paged_prefill_split(
        FAKE, 8 * 128, 128, FAKE, FAKE, FAKE, 2, 32, FAKE, FAKE, 16 * 2 * 128, 2 * 128, 128, FAKE, 64, FAKE, None,
        None, 0, 0, 0, FAKE, 8 * 128, 128, 2, 8, 2, 128, 16, 0.088, total_q, S, ws, ws_bytes, None)


@pytest.mark.parametrize("S,ws,ws_bytes,total_q,code,word", [
    (0, None, 0, 40, pa.ATTN_ERR_INVALID_ARG, "num_splits"),
    (257, None, 0, 40, pa.ATTN_ERR_INVALID_ARG, "num_splits"),
    (4, None, 0, 40, pa.ATTN_ERR_WORKSPACE, "workspace"),
    (4, FAKE, 1000, 40, pa.ATTN_ERR_WORKSPACE, "workspace"),
    (4, FAKE + 16, 1 << 30, 40, pa.ATTN_ERR_INVALID_ARG, "aligned"),
    (4, FAKE, 1 << 30, -1, pa.ATTN_ERR_INVALID_ARG, "row"),
])
def test_paged_prefill_split_rejects_bad_arguments(S, ws, ws_bytes, total_q, code, word):
    assert call_paged_prefill_split(S, ws, ws_bytes, total_q) == code
    assert word in pa.attn_last_error()


def test_dense_prefill_split_rejects_short_workspace():
    lib = pa.lib()
    rc = lib.attn_prefill_split(FAKE, 16 * 8 * 128, 8 * 128, 128, FAKE, FAKE, 500 * 2 * 128, 2 * 128, 128,
                                None, 500, 1, None, 0, 0, 0, FAKE, 16 * 8 * 128, 8 * 128, 128,
                                2, 16, 8, 2, 128, 0.088, 3, FAKE, 4096, None)
    assert rc == pa.ATTN_ERR_WORKSPACE and "workspace" in pa.attn_last_error()


def test_prefill_tile_rows_any_group_size():
    # packed heads = largest power of two dividing G, at most 8
    assert [pa.attn_prefill_tile_rows(128, G) for G in (3, 5, 6, 12, 16, 32, 24)] == [128, 128, 64, 32, 16, 16, 16]
    # G = 32 over one KV head: four workgroups of eight heads per tile
    assert pa.attn_prefill_plan_splits(16, 32, 1, 128, 16384, 256) == 4
    assert pa.attn_prefill_plan_splits(16, 32, 1, 128, 16384, 1024) == 16


def test_planner_counts_one_row_per_pass_for_other_group_sizes():
    # D = 128, G = 32 over 1 KV head: one MFMA row of 32 query heads per
    # (sequence, KV head), four-wave slices of >= 256 tokens
    assert pa.attn_plan_splits(2, 1, 32, 128, 640, 16, 128, 256) == 2 * 640 // 256
    assert pa.attn_plan_splits(2, 1, 64, 128, 640, 16, 128, 256) == 2 * 2 * 640 // 256   # two passes of 32
    # G = 3 over 2 KV heads: one pass, so both KV heads share a row (a wave
    # each): one row of 640 tokens, slices of >= 256 tokens
    assert pa.attn_plan_splits(1, 2, 3, 128, 640, 16, 128, 256) == (640 + 255) // 256
    # D = 256 keeps the VALU kernel: G = 32 is four passes of 8 (one-wave
    # slices of >= 64 tokens), G = 3 three passes of one head (four-wave)
    assert pa.attn_plan_splits(2, 1, 32, 256, 640, 16, 256, 256) == 2 * 4 * 640 // 64
    assert pa.attn_plan_splits(1, 2, 3, 256, 640, 16, 256, 256) == 2 * 3 * 640 // 256


def test_prefill_tile_rows_head_dim_256():
    # one team of four 16-row waves: at most four heads packed
    assert [pa.attn_prefill_tile_rows(256, G) for G in (1, 2, 4, 8, 3, 32)] == [64, 32, 16, 16, 64, 16]


# --- argument checks of the remaining entry points (host only) -----------
def swa_args(**over):
    a = dict(q=FAKE, q_st=128 * 512, q_sh=512, cache=FAKE, c_sb=256 * 512, c_ss=512, inv=FAKE, s_ss=1,
             ind=FAKE, i_st=128, lens=FAKE, o=FAKE, o_st=128 * 512, o_sh=512, T=4, NH=128, HD=512, W=128,
             bs=256, nb=8, scale=0.044)
    a.update(over)
    return a


def call_swa(a):
    return pa.lib().attn_swa_fp8_decode(a["q"], a["q_st"], a["q_sh"], a["cache"], a["c_sb"], a["c_ss"], a["inv"],
                                        a["s_ss"], a["ind"], a["i_st"], a["lens"], a["o"], a["o_st"], a["o_sh"],
                                        a["T"], a["NH"], a["HD"], a["W"], a["bs"], a["nb"], a["scale"], None)


@pytest.mark.parametrize("over,code,word", [
    (dict(HD=256), pa.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(NH=24), pa.ATTN_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(W=2048), pa.ATTN_ERR_UNSUPPORTED, "window"),
    (dict(T=-1), pa.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(bs=0), pa.ATTN_ERR_INVALID_ARG, "sizes"),
    (dict(cache=None), pa.ATTN_ERR_INVALID_ARG, "null"),
    (dict(scale=float("inf")), pa.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(q=FAKE + 8), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(c_ss=520), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(i_st=64), pa.ATTN_ERR_INVALID_ARG, "strides"),
    (dict(bs=1 << 16, nb=1 << 16), pa.ATTN_ERR_UNSUPPORTED, "2^31"),
    (dict(T=1 << 27, NH=512), pa.ATTN_ERR_UNSUPPORTED, "2^31"),
])
def test_swa_rejects_bad_arguments(over, code, word):
    assert call_swa(swa_args(**over)) == code
    assert word in pa.attn_last_error()


def test_kv_append_rejects_bad_arguments():
    lib = pa.lib()
    good = [FAKE, FAKE, 8 * 128, 128, FAKE, FAKE, 10, FAKE, FAKE, 16 * 8 * 128, 8 * 128, 128, 100, FAKE, 32,
            2, 8, 128, 16, None]
    assert lib.attn_paged_kv_append(*good[:17], 100, *good[18:]) == pa.ATTN_ERR_UNSUPPORTED   # D % 8
    assert "multiple of 8" in pa.attn_last_error()
    bad = list(good); bad[0] = None
    assert lib.attn_paged_kv_append(*bad) == pa.ATTN_ERR_INVALID_ARG and "null" in pa.attn_last_error()
    bad = list(good); bad[3] = 100                                                            # head stride % 8
    assert lib.attn_paged_kv_append(*bad) == pa.ATTN_ERR_UNSUPPORTED and "aligned" in pa.attn_last_error()
    bad = list(good); bad[18] = 0                                                             # page size
    assert lib.attn_paged_kv_append(*bad) == pa.ATTN_ERR_INVALID_ARG
    bad = list(good); bad[6] = 0                                                              # nothing to write
    assert lib.attn_paged_kv_append(*bad) == pa.ATTN_OK


def test_fp8_append_rejects_bad_arguments():
    lib = pa.lib()
    good = [FAKE, 512, FAKE, None, 4, 512, FAKE, 256 * 512, 512, FAKE, 1, 256, 8, None, None]
    bad = list(good); bad[5] = 256
    assert lib.attn_swa_fp8_append(*bad) == pa.ATTN_ERR_UNSUPPORTED and "head dim" in pa.attn_last_error()
    bad = list(good); bad[2] = None
    assert lib.attn_swa_fp8_append(*bad) == pa.ATTN_ERR_INVALID_ARG and "null" in pa.attn_last_error()
    bad = list(good); bad[1] = 100
    assert lib.attn_swa_fp8_append(*bad) == pa.ATTN_ERR_UNSUPPORTED and "aligned" in pa.attn_last_error()
    bad = list(good); bad[11] = 0
    assert lib.attn_swa_fp8_append(*bad) == pa.ATTN_ERR_INVALID_ARG
    bad = list(good); bad[4] = 0
    assert lib.attn_swa_fp8_append(*bad) == pa.ATTN_OK


def test_rotary_rejects_bad_arguments():
    lib = pa.lib()
    good = [FAKE, 32 * 128, 128, FAKE, 32 * 128, 128, 10, 32, 128, FAKE, FAKE, 64, 4096, FAKE, None]
    bad = list(good); bad[8] = 100
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_UNSUPPORTED and "multiple of 8" in pa.attn_last_error()
    bad = list(good); bad[11] = 32
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_INVALID_ARG and "table stride" in pa.attn_last_error()
    bad = list(good); bad[13] = None
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_INVALID_ARG and "null" in pa.attn_last_error()
    bad = list(good); bad[0] = FAKE + 4
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_UNSUPPORTED and "aligned" in pa.attn_last_error()
    bad = list(good); bad[6] = 1 << 28
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_UNSUPPORTED and "2^31" in pa.attn_last_error()
    # one token with more head chunks than a grid column of 65535 workgroups holds
    bad = list(good); bad[6] = 1; bad[7] = 65535 * 256 // 16 + 1
    assert lib.attn_rotary_embed(*bad) == pa.ATTN_ERR_UNSUPPORTED and "65535" in pa.attn_last_error()


def paged_prefill_args(**over):
    a = dict(q=FAKE, q_st=8 * 128, q_sh=128, indptr=FAKE, t2b=FAKE, t2i=FAKE, nt=2, tr=32, k=FAKE, v=FAKE,
             s_page=16 * 2 * 128, s_slot=2 * 128, s_head=128, bt=FAKE, bt_sb=64, lens=FAKE, causal=None,
             mask=None, ndim=0, m_sb=0, m_sq=0, o=FAKE, o_st=8 * 128, o_sh=128, B=2, Hq=8, Hkv=2, D=128,
             ps=16, scale=0.088)
    a.update(over)
    return a


def call_paged_prefill(a):
    return pa.lib().attn_paged_prefill(
        a["q"], a["q_st"], a["q_sh"], a["indptr"], a["t2b"], a["t2i"], a["nt"], a["tr"], a["k"], a["v"], a["s_page"],
        a["s_slot"], a["s_head"], a["bt"], a["bt_sb"], a["lens"], a["causal"], a["mask"], a["ndim"], a["m_sb"],
        a["m_sq"], a["o"], a["o_st"], a["o_sh"], a["B"], a["Hq"], a["Hkv"], a["D"], a["ps"], a["scale"], None)


@pytest.mark.parametrize("over,code,word", [
    (dict(D=96), pa.ATTN_ERR_UNSUPPORTED, "head dim"),
    (dict(Hq=7), pa.ATTN_ERR_INVALID_ARG, "multiple"),
    (dict(ps=0), pa.ATTN_ERR_INVALID_ARG, "page_size"),
    (dict(nt=-1), pa.ATTN_ERR_INVALID_ARG, "negative"),
    (dict(t2b=None), pa.ATTN_ERR_INVALID_ARG, "null"),
    (dict(lens=None), pa.ATTN_ERR_INVALID_ARG, "null"),
    (dict(scale=float("nan")), pa.ATTN_ERR_INVALID_ARG, "scale"),
    (dict(mask=FAKE, ndim=4), pa.ATTN_ERR_INVALID_ARG, "mask_ndim"),
    (dict(mask=FAKE, ndim=3, m_sb=4096, m_sq=-30), pa.ATTN_ERR_INVALID_ARG, "negative mask"),
    (dict(q=FAKE + 8), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(o_sh=130), pa.ATTN_ERR_UNSUPPORTED, "aligned"),
    (dict(s_page=1 << 33), pa.ATTN_ERR_UNSUPPORTED, "32-bit"),
    (dict(tr=0), pa.ATTN_ERR_INVALID_ARG, "tile_rows"),
    (dict(tr=128), pa.ATTN_ERR_INVALID_ARG, "tile_rows"),
])
def test_paged_prefill_rejects_bad_arguments(over, code, word):
    assert call_paged_prefill(paged_prefill_args(**over)) == code
    assert word in pa.attn_last_error()


def test_paged_prefill_refuses_the_worked_examples_64_row_map():
    """The doc's worked work map (q lens [70, 10, 130] in 64-row tiles) at
    G = 4, D = 128, where the kernel computes 32-row tiles: the map's height
    is refused instead of leaving rows 32..63 of every tile unwritten."""
    ex = json.load(open(os.path.join(GOLDEN, "ragged_work_map.json")))
    assert ex["tile_rows"] == 64 and pa.attn_prefill_tile_rows(128, 4) == 32
    _, t2b, _ = pa.attn_prefill_plan(ex["q_lens"], ex["tile_rows"])
    a = paged_prefill_args(B=3, nt=int(t2b.numel()), tr=ex["tile_rows"], Hq=8, Hkv=2, D=128)
    assert call_paged_prefill(a) == pa.ATTN_ERR_INVALID_ARG
    assert "tile_rows=64" in pa.attn_last_error() and "takes 32" in pa.attn_last_error()
    # the split entry point checks the same contract
    assert pa.lib().attn_paged_prefill_split(
        FAKE, 8 * 128, 128, FAKE, FAKE, FAKE, int(t2b.numel()), 64, FAKE, FAKE, 16 * 2 * 128, 2 * 128, 128, FAKE,
        64, FAKE, None, None, 0, 0, 0, FAKE, 8 * 128, 128, 3, 8, 2, 128, 16, 0.088, 210, 2, FAKE, 1 << 30,
        None) == pa.ATTN_ERR_INVALID_ARG
    assert "tile_rows" in pa.attn_last_error()


def test_dense_prefill_rejects_bad_arguments():
    lib = pa.lib()

    def call(**over):
        a = dict(q=FAKE, q_sb=40 * 8 * 128, q_sl=8 * 128, q_sh=128, k=FAKE, v=FAKE, k_sb=500 * 2 * 128,
                 k_sl=2 * 128, k_sh=128, lens=None, kv=500, causal=1, mask=None, ndim=0, m_sb=0, m_sq=0, o=FAKE,
                 o_sb=40 * 8 * 128, o_sl=8 * 128, o_sh=128, B=2, Lq=40, Hq=8, Hkv=2, D=128, scale=0.088)
        a.update(over)
        return lib.attn_prefill(*a.values(), None)
    assert call(D=48) == pa.ATTN_ERR_UNSUPPORTED and "head dim" in pa.attn_last_error()
    assert call(Lq=-1) == pa.ATTN_ERR_INVALID_ARG and "negative" in pa.attn_last_error()
    assert call(k=None) == pa.ATTN_ERR_INVALID_ARG and "null" in pa.attn_last_error()
    assert call(k_sl=100) == pa.ATTN_ERR_UNSUPPORTED and "aligned" in pa.attn_last_error()
    assert call(mask=FAKE, ndim=1) == pa.ATTN_ERR_INVALID_ARG and "mask_ndim" in pa.attn_last_error()
    assert call(B=0) == pa.ATTN_OK


def test_decode_combine_rejects_bad_arguments():
    lib = pa.lib()
    # workspace too small for 4 slices of B=2, Hq=8, D=128
    rc = lib.attn_decode_combine(FAKE, 1024, 2, 8, 2, 128, 4, 128, FAKE, 300, FAKE, 8 * 128, 128, None)
    assert rc == pa.ATTN_ERR_WORKSPACE
    rc = lib.attn_decode_combine(FAKE, 1 << 30, 2, 8, 2, 96, 4, 128, FAKE, 300, FAKE, 8 * 128, 128, None)
    assert rc == pa.ATTN_ERR_UNSUPPORTED
    rc = lib.attn_decode_combine(FAKE, 1 << 30, 2, 8, 2, 128, 0, 128, FAKE, 300, FAKE, 8 * 128, 128, None)
    assert rc == pa.ATTN_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    """The binding passes device pointers only: a host tensor is refused
    before any library call (its pointer would otherwise reach a kernel)."""
    B, Hq, Hkv, D, ps = 2, 8, 2, 64, 16
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16)
    pool = torch.zeros(4, ps, Hkv, D, dtype=torch.bfloat16)
    bt = torch.zeros(B, 2, dtype=torch.int32)
    lens = torch.full((B,), 20, dtype=torch.int32)
    with pytest.raises(ValueError, match="q must be a device tensor"):
        pa.attn_paged_decode(q, pool, pool, bt, lens, 32, torch.empty_like(q), ps, 0.125, num_splits=1)
    x = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    tab = torch.zeros(8, 32, dtype=torch.float32)
    with pytest.raises(ValueError, match="x must be a device tensor"):
        pa.attn_rotary_embed(x, tab, tab, torch.zeros(3, dtype=torch.int32))


def test_probe_rejects_bad_arguments():
    lib = pa.lib()
    assert lib.attn_hbm_read_probe(None, 1024, FAKE, 4, None) == pa.ATTN_ERR_INVALID_ARG
    assert lib.attn_hbm_read_probe(FAKE, 1000, FAKE, 4, None) == pa.ATTN_ERR_UNSUPPORTED
    assert lib.attn_hbm_read_probe(FAKE + 8, 1024, FAKE, 4, None) == pa.ATTN_ERR_UNSUPPORTED
    assert lib.attn_hbm_read_probe(FAKE, 1024, FAKE, -1, None) == pa.ATTN_ERR_INVALID_ARG
