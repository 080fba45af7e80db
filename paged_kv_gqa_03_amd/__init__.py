"""Python binding of libpaged_attn.so (gfx950 paged GQA attention).

Argument marshalling only: every function below forwards device pointers,
element strides and sizes of torch tensors to the C entry point of the same
name (include/paged_attn.h) and raises AttnError when it returns an error.
All compute runs in the HIP kernels.  There is no fallback: if the library is
not built, every call raises.
"""
import ctypes
import os

import torch

__all__ = [
    "AttnError", "lib", "attn_version", "attn_last_error", "attn_plan_splits",
    "attn_decode_workspace_bytes", "attn_decode", "attn_paged_decode", "attn_paged_decode_split",
    "attn_paged_decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "attn_decode_combine", "attn_split_combine",
    "attn_prefill_plan", "attn_prefill_tile_rows", "attn_paged_prefill", "attn_swa_fp8_decode",
    "attn_prefill", "attn_paged_kv_append", "attn_swa_fp8_append", "attn_rotary_embed",
    "attn_prefill_workspace_bytes", "attn_prefill_plan_splits", "attn_paged_prefill_split",
    "attn_prefill_split", "attn_hbm_read_probe", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_LAUNCH = -4

_P, _I, _L, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "attn_last_error": ([], ctypes.c_char_p),
    "attn_version": ([], _I),
    "attn_plan_splits": ([_I, _I, _I, _I, _I, _I, _L, _I], _I),
    "attn_decode_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "attn_decode": ([_P, _L, _L, _P, _L, _L, _L, _P, _L, _L, _L, _P, _L, _L, _P, _I,
                     _I, _I, _I, _I, _F, _I, _P, _Z, _P], _I),
    "attn_paged_decode": ([_P, _L, _L, _P, _P, _L, _L, _L, _P, _L, _P, _I, _P, _L, _L,
                           _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P], _I),
    "attn_paged_decode_noalloc": ([_P, _L, _L, _P, _P, _L, _L, _L, _P, _L, _P, _I, _P, _L, _L,
                                   _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "attn_paged_decode_split": ([_P, _L, _L, _P, _P, _L, _L, _L, _P, _L, _P, _I,
                                 _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P], _I),
    "attn_decode_combine": ([_P, _Z, _I, _I, _I, _I, _I, _L, _P, _I, _P, _L, _L, _P], _I),
    "attn_split_combine": ([_P, _P, _I, _I, _I, _P, _P, _P, _P], _I),
    "attn_prefill_plan": ([_P, _I, _I, _P, _P, _P, _I, _P], _I),
    "attn_prefill_tile_rows": ([_I, _I], _I),
    "attn_paged_prefill": ([_P, _L, _L, _P, _P, _P, _I, _I, _P, _P, _L, _L, _L, _P, _L, _P, _P,
                            _P, _I, _L, _L, _P, _L, _L, _I, _I, _I, _I, _I, _F, _P], _I),
    "attn_swa_fp8_decode": ([_P, _L, _L, _P, _L, _L, _P, _L, _P, _L, _P, _P, _L, _L,
                             _I, _I, _I, _I, _I, _I, _F, _P], _I),
    "attn_prefill": ([_P, _L, _L, _L, _P, _P, _L, _L, _L, _P, _I, _I, _P, _I, _L, _L, _P, _L, _L, _L,
                      _I, _I, _I, _I, _I, _F, _P], _I),
    "attn_paged_kv_append": ([_P, _P, _L, _L, _P, _P, _I, _P, _P, _L, _L, _L, _I, _P, _L,
                              _I, _I, _I, _I, _P], _I),
    "attn_swa_fp8_append": ([_P, _L, _P, _P, _I, _I, _P, _L, _L, _P, _L, _I, _I, _P, _P], _I),
    "attn_rotary_embed": ([_P, _L, _L, _P, _L, _L, _I, _I, _I, _P, _P, _L, _I, _P, _P], _I),
    "attn_prefill_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "attn_prefill_plan_splits": ([_I, _I, _I, _I, _I, _I], _I),
    "attn_paged_prefill_split": ([_P, _L, _L, _P, _P, _P, _I, _I, _P, _P, _L, _L, _L, _P, _L, _P, _P,
                                  _P, _I, _L, _L, _P, _L, _L, _I, _I, _I, _I, _I, _F,
                                  _I, _I, _P, _Z, _P], _I),
    "attn_prefill_split": ([_P, _L, _L, _L, _P, _P, _L, _L, _L, _P, _I, _I, _P, _I, _L, _L, _P, _L, _L, _L,
                            _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P], _I),
    "attn_hbm_read_probe": ([_P, _Z, _P, _I, _P], _I),
}
EXPORTED_SYMBOLS = tuple(_SIGS)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpaged_attn.so is not built (python -m paged_kv_gqa_03_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def attn_last_error():
    return lib().attn_last_error().decode()


def _check(rc):
    if rc != ATTN_OK:
        raise AttnError(rc, attn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


_BF16 = (torch.bfloat16,)
_I32 = (torch.int32,)
_I64 = (torch.int64,)
_F32 = (torch.float32,)


def _dev(**named):
    """Every tensor argument the library reads or writes through a device
    pointer must live on the GPU (a host pointer would reach a kernel) and
    have the element type the C ABI declares.  Values are (tensor, dtypes)
    or (tensor, None) for any dtype; a None tensor is an absent optional."""
    for name, (t, dtypes) in named.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if dtypes is not None and t.dtype not in dtypes:
            raise TypeError("%s must be %s, got %s" % (name, " or ".join(str(d) for d in dtypes), t.dtype))


def _unit_inner(*ts):
    for t in ts:
        if t is not None and t.stride(-1) != 1:
            raise ValueError("innermost stride must be 1")


def attn_version():
    return lib().attn_version()


def attn_plan_splits(B, Hkv, G, D, max_kv_len, page_size, kv_s_head, num_cus=0):
    rc = lib().attn_plan_splits(B, Hkv, G, D, max_kv_len, page_size, kv_s_head, num_cus)
    if rc < 0:
        _check(rc)
    return rc


def attn_decode_workspace_bytes(B, Hq, D, num_splits):
    return int(lib().attn_decode_workspace_bytes(B, Hq, D, num_splits))


def _workspace(workspace, B, Hq, D, S, device):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    if S <= 1:
        return None, 0
    n = attn_decode_workspace_bytes(B, Hq, D, S)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws, n


def attn_paged_decode(q, k_pool, v_pool, block_table, kv_lens, max_kv_len, out, page_size, scale,
                      num_splits=0, workspace=None, stream=None, num_cus=0):
    """q [B, Hq, D]; k_pool / v_pool 4-D (page, slot, head, dim) views with
    identical strides; block_table [B, *] int32; kv_lens [B] int32; out
    [B, Hq, D] bf16.  num_splits 0 asks the planner."""
    _dev(q=(q, _BF16), k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16), block_table=(block_table, _I32),
         kv_lens=(kv_lens, _I32), out=(out, _BF16), workspace=(workspace, None))
    _unit_inner(q, k_pool, v_pool, out, block_table)
    assert k_pool.stride() == v_pool.stride(), "K and V pools must share strides"
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    S = num_splits or attn_plan_splits(B, Hkv, Hq // Hkv, D, max_kv_len, page_size, k_pool.stride(2), num_cus)
    ws, nbytes = _workspace(workspace, B, Hq, D, S, q.device)
    _check(lib().attn_paged_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens), int(max_kv_len),
        _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv, D, int(page_size), float(scale),
        int(S), _ptr(ws), nbytes, _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # ATTN_NOALLOC_SCRATCH_BYTES


def attn_paged_decode_noalloc(q, k_pool, v_pool, block_table, kv_lens, max_kv_len, out, page_size, scale,
                              num_splits=0, stream=None):
    """attn_paged_decode with the split partials in the library's static
    per-device scratch buffer: nothing is allocated (no workspace tensor)."""
    _dev(q=(q, _BF16), k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16), block_table=(block_table, _I32),
         kv_lens=(kv_lens, _I32), out=(out, _BF16))
    _unit_inner(q, k_pool, v_pool, out, block_table)
    assert k_pool.stride() == v_pool.stride(), "K and V pools must share strides"
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    _check(lib().attn_paged_decode_noalloc(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens), int(max_kv_len),
        _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv, D, int(page_size), float(scale),
        int(num_splits), _stream(stream)))
    return out


def attn_paged_decode_split(q, k_pool, v_pool, block_table, kv_lens, max_kv_len, page_size, scale,
                            num_splits, workspace, stream=None):
    """Split kernel only: fp32 partials for `num_splits` splits into the
    workspace (a uint8 device tensor of attn_decode_workspace_bytes)."""
    _dev(q=(q, _BF16), k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16), block_table=(block_table, _I32),
         kv_lens=(kv_lens, _I32), workspace=(workspace, None))
    _unit_inner(q, k_pool, v_pool, block_table)
    assert k_pool.stride() == v_pool.stride()
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    _check(lib().attn_paged_decode_split(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens), int(max_kv_len),
        B, Hq, Hkv, D, int(page_size), float(scale), int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode_combine(workspace, B, Hq, Hkv, D, num_splits, kv_s_head, kv_lens, max_kv_len, out, stream=None):
    """Combine step of decode over a workspace filled by attn_paged_decode_split."""
    _dev(workspace=(workspace, None), kv_lens=(kv_lens, _I32), out=(out, _BF16))
    _unit_inner(out)
    _check(lib().attn_decode_combine(
        _ptr(workspace), workspace.numel() * workspace.element_size(), int(B), int(Hq), int(Hkv), int(D),
        int(num_splits), int(kv_s_head), _ptr(kv_lens), int(max_kv_len), _ptr(out), out.stride(0), out.stride(1),
        _stream(stream)))
    return out


def attn_decode(q, k, v, out, scale, kv_lens=None, kv_len=None, num_splits=0, workspace=None,
                stream=None, num_cus=0):
    """q [B, Hq, D]; k, v 4-D (b, head, pos, dim) views; out [B, Hq, D]."""
    _dev(q=(q, _BF16), k=(k, _BF16), v=(v, _BF16), out=(out, _BF16), kv_lens=(kv_lens, _I32),
         workspace=(workspace, None))
    _unit_inner(q, k, v, out)
    B, Hq, D = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    kv_len = L if kv_len is None else kv_len
    S = num_splits or attn_plan_splits(B, Hkv, Hq // Hkv, D, kv_len, 0, k.stride(1), num_cus)
    ws, nbytes = _workspace(workspace, B, Hq, D, S, q.device)
    _check(lib().attn_decode(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(k), k.stride(0), k.stride(1), k.stride(2),
        _ptr(v), v.stride(0), v.stride(1), v.stride(2),
        _ptr(out), out.stride(0), out.stride(1), _ptr(kv_lens), int(kv_len),
        B, Hq, Hkv, D, float(scale), int(num_splits or (S if num_cus else 0)), _ptr(ws), nbytes,
        _stream(stream)))
    return out


def attn_split_combine(o_part, ml_part, out_f32=None, out_bf16=None, lse=None, stream=None):
    """o_part [S, R, D] float32, ml_part [S, R, 2] float32 (contiguous)."""
    _dev(o_part=(o_part, _F32), ml_part=(ml_part, _F32), out_f32=(out_f32, _F32), out_bf16=(out_bf16, _BF16),
         lse=(lse, _F32))
    S, R, D = o_part.shape
    assert o_part.is_contiguous() and ml_part.is_contiguous()
    for t in (out_f32, out_bf16, lse):
        assert t is None or t.is_contiguous()
    _check(lib().attn_split_combine(_ptr(o_part), _ptr(ml_part), S, R, D, _ptr(out_f32),
                                    _ptr(out_bf16), _ptr(lse), _stream(stream)))


def attn_prefill_tile_rows(D, G):
    rc = lib().attn_prefill_tile_rows(D, G)
    if rc < 0:
        _check(rc)
    return rc


def attn_prefill_plan(q_lens, tile_rows):
    """Host work map: returns (qo_indptr, tile_to_batch, tile_to_index) as
    int32 CPU tensors."""
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).contiguous()
    B = q_lens.numel()
    cap = sum((int(x) + tile_rows - 1) // tile_rows for x in q_lens.tolist() if x > 0) + 1
    indptr = torch.empty(B + 1, dtype=torch.int32)
    t2b = torch.empty(cap, dtype=torch.int32)
    t2i = torch.empty(cap, dtype=torch.int32)
    n = ctypes.c_int(0)
    _check(lib().attn_prefill_plan(_ptr(q_lens), B, int(tile_rows), _ptr(indptr), _ptr(t2b),
                                   _ptr(t2i), cap, ctypes.byref(n)))
    return indptr, t2b[:n.value].clone(), t2i[:n.value].clone()


def attn_paged_prefill(q, qo_indptr, tile_to_batch, tile_to_index, k_pool, v_pool, block_table,
                       kv_lens, out, page_size, scale, causal_offset=None, mask=None, stream=None, *, tile_rows):
    """q / out packed [total_q, Hq, D]; work map and index arrays on the
    device (int32), built by attn_prefill_plan with `tile_rows` rows per
    tile (the library refuses a height other than attn_prefill_tile_rows);
    mask None, [B, kv] or [B, q, kv] uint8/bool keep-mask."""
    _dev(q=(q, _BF16), qo_indptr=(qo_indptr, _I32), tile_to_batch=(tile_to_batch, _I32),
         tile_to_index=(tile_to_index, _I32), k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16),
         block_table=(block_table, _I32), kv_lens=(kv_lens, _I32), out=(out, _BF16),
         causal_offset=(causal_offset, _I32), mask=(mask, (torch.bool, torch.uint8)))
    _unit_inner(q, k_pool, v_pool, out, block_table)
    assert k_pool.stride() == v_pool.stride()
    total_q, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    B = qo_indptr.numel() - 1
    mask, ndim, m_sb, m_sq = _mask_args(mask)
    _check(lib().attn_paged_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(qo_indptr), _ptr(tile_to_batch), _ptr(tile_to_index),
        int(tile_to_batch.numel()), int(tile_rows), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2), _ptr(block_table), block_table.stride(0),
        _ptr(kv_lens), _ptr(causal_offset), _ptr(mask), ndim, m_sb, m_sq,
        _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv, D, int(page_size), float(scale),
        _stream(stream)))
    return out


def attn_swa_fp8_decode(q, kv_cache, inv_scale, swa_indices, swa_lens, out, block_size, scale,
                        stream=None):
    """q / out [T, NH, HD] bf16; kv_cache [num_blocks, block_size, HD] uint8
    e4m3fn codes; inv_scale [max_slots, 1] bf16; swa_indices [T, W] int64;
    swa_lens [T] int64."""
    _dev(q=(q, _BF16), kv_cache=(kv_cache, (torch.uint8,)), inv_scale=(inv_scale, _BF16),
         swa_indices=(swa_indices, _I64), swa_lens=(swa_lens, _I64), out=(out, _BF16))
    _unit_inner(q, kv_cache, swa_indices, out)
    T, NH, HD = q.shape
    W = swa_indices.shape[1]
    num_blocks = kv_cache.shape[0]
    _check(lib().attn_swa_fp8_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(kv_cache), kv_cache.stride(0), kv_cache.stride(1),
        _ptr(inv_scale), inv_scale.stride(0), _ptr(swa_indices), swa_indices.stride(0), _ptr(swa_lens),
        _ptr(out), out.stride(0), out.stride(1), T, NH, HD, W, int(block_size), num_blocks,
        float(scale), _stream(stream)))
    return out


def attn_paged_kv_append(k_new, v_new, new_indptr, start_pos, k_pool, v_pool, block_table, page_size,
                         stream=None):
    """k_new / v_new packed [N, Hkv, D] bf16 (identical strides); new_indptr
    int32 [B + 1], start_pos int32 [B] on the device; pools are the 4-D
    (page, slot, head, dim) views of attn_paged_decode."""
    _dev(k_new=(k_new, _BF16), v_new=(v_new, _BF16), new_indptr=(new_indptr, _I32), start_pos=(start_pos, _I32),
         k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16), block_table=(block_table, _I32))
    _unit_inner(k_new, v_new, k_pool, v_pool, block_table)
    assert k_new.stride() == v_new.stride() and k_pool.stride() == v_pool.stride()
    N, Hkv, D = k_new.shape
    _check(lib().attn_paged_kv_append(
        _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1), _ptr(new_indptr), _ptr(start_pos), N,
        _ptr(k_pool), _ptr(v_pool), k_pool.stride(0), k_pool.stride(1), k_pool.stride(2), k_pool.shape[0],
        _ptr(block_table), block_table.stride(0), new_indptr.numel() - 1, Hkv, D, int(page_size),
        _stream(stream)))


def attn_swa_fp8_append(x, slots, kv_cache, inv_scale, block_size, multiplier=None, amax=None, stream=None):
    """x [N, HD] bf16; slots int64 [N]; kv_cache [num_blocks, block_size, HD]
    uint8; inv_scale [slots, 1] bf16; multiplier float32 [N] or None;
    amax float32 [N] output or None."""
    _dev(x=(x, _BF16), slots=(slots, _I64), kv_cache=(kv_cache, (torch.uint8,)), inv_scale=(inv_scale, _BF16),
         multiplier=(multiplier, _F32), amax=(amax, _F32))
    _unit_inner(x, kv_cache)
    N, HD = x.shape
    _check(lib().attn_swa_fp8_append(
        _ptr(x), x.stride(0), _ptr(slots), _ptr(multiplier), N, HD, _ptr(kv_cache), kv_cache.stride(0),
        kv_cache.stride(1), _ptr(inv_scale), inv_scale.stride(0), int(block_size), kv_cache.shape[0],
        _ptr(amax), _stream(stream)))


def attn_rotary_embed(x, cos_table, sin_table, positions, out=None, stream=None):
    """x [T, H, D] bf16; cos_table / sin_table float32 [rows, D/2];
    positions int32 [T].  Writes out (default: x, in place) and returns it."""
    out = x if out is None else out
    _dev(x=(x, _BF16), out=(out, _BF16), cos_table=(cos_table, _F32), sin_table=(sin_table, _F32),
         positions=(positions, _I32))
    _unit_inner(x, out, cos_table, sin_table)
    assert cos_table.stride() == sin_table.stride()
    T, H, D = x.shape
    _check(lib().attn_rotary_embed(
        _ptr(x), x.stride(0), x.stride(1), _ptr(out), out.stride(0), out.stride(1), T, H, D,
        _ptr(cos_table), _ptr(sin_table), cos_table.stride(0), cos_table.shape[0], _ptr(positions),
        _stream(stream)))
    return out


def attn_prefill(q, k, v, out, scale, is_causal=False, kv_lens=None, mask=None, stream=None):
    """Dense prefill, contiguous KV.  q / out are (b, i, h, d)-indexed views
    [B, Lq, Hq, D] (any strides with unit innermost); k / v are (b, j, g, d)
    views [B, Lk, Hkv, D] with identical strides; kv_lens int32 [B] or None
    (all Lk); mask None, [B, Lk] or [B, Lq, Lk] keep-mask."""
    _dev(q=(q, _BF16), k=(k, _BF16), v=(v, _BF16), out=(out, _BF16), kv_lens=(kv_lens, _I32),
         mask=(mask, (torch.bool, torch.uint8)))
    _unit_inner(q, k, v, out)
    assert k.stride() == v.stride(), "K and V must share strides"
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    mask, ndim, m_sb, m_sq = _mask_args(mask)
    _check(lib().attn_prefill(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2), _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(kv_lens), int(Lk), 1 if is_causal else 0, _ptr(mask), ndim, m_sb, m_sq,
        _ptr(out), out.stride(0), out.stride(1), out.stride(2), B, Lq, Hq, Hkv, D, float(scale), _stream(stream)))
    return out


def _mask_args(mask):
    """(mask as uint8, ndim, batch stride, row stride) of a keep-mask or None."""
    if mask is None:
        return None, 0, 0, 0
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _unit_inner(mask)
    ndim = mask.dim()
    return mask, ndim, mask.stride(0), (mask.stride(1) if ndim == 3 else 0)


def attn_prefill_workspace_bytes(rows, Hq, D, num_splits):
    return int(lib().attn_prefill_workspace_bytes(rows, Hq, D, num_splits))


def attn_prefill_plan_splits(num_tiles, Hq, Hkv, D, max_kv_len, target_workgroups=0):
    rc = lib().attn_prefill_plan_splits(num_tiles, Hq, Hkv, D, max_kv_len, target_workgroups)
    if rc < 0:
        _check(rc)
    return rc


def _prefill_workspace(workspace, rows, Hq, D, S, device):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    if S <= 1:
        return None, 0
    n = attn_prefill_workspace_bytes(rows, Hq, D, S)
    return torch.empty(n, dtype=torch.uint8, device=device), n


def attn_paged_prefill_split(q, qo_indptr, tile_to_batch, tile_to_index, k_pool, v_pool, block_table,
                             kv_lens, out, page_size, scale, max_kv_len, causal_offset=None, mask=None,
                             num_splits=0, workspace=None, stream=None, target_workgroups=0, *, tile_rows):
    """attn_paged_prefill with the keys of each tile split over num_splits
    workgroups (0 asks the planner with max_kv_len) and merged by a combine."""
    _dev(q=(q, _BF16), qo_indptr=(qo_indptr, _I32), tile_to_batch=(tile_to_batch, _I32),
         tile_to_index=(tile_to_index, _I32), k_pool=(k_pool, _BF16), v_pool=(v_pool, _BF16),
         block_table=(block_table, _I32), kv_lens=(kv_lens, _I32), out=(out, _BF16),
         causal_offset=(causal_offset, _I32), mask=(mask, (torch.bool, torch.uint8)), workspace=(workspace, None))
    _unit_inner(q, k_pool, v_pool, out, block_table)
    assert k_pool.stride() == v_pool.stride()
    total_q, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    B = qo_indptr.numel() - 1
    num_tiles = int(tile_to_batch.numel())
    S = num_splits or attn_prefill_plan_splits(num_tiles, Hq, Hkv, D, max_kv_len, target_workgroups)
    ws, nbytes = _prefill_workspace(workspace, total_q, Hq, D, S, q.device)
    mask, ndim, m_sb, m_sq = _mask_args(mask)
    _check(lib().attn_paged_prefill_split(
        _ptr(q), q.stride(0), q.stride(1), _ptr(qo_indptr), _ptr(tile_to_batch), _ptr(tile_to_index),
        num_tiles, int(tile_rows), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2), _ptr(block_table), block_table.stride(0),
        _ptr(kv_lens), _ptr(causal_offset), _ptr(mask), ndim, m_sb, m_sq,
        _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv, D, int(page_size), float(scale),
        total_q, S, _ptr(ws), nbytes, _stream(stream)))
    return out


def attn_prefill_split(q, k, v, out, scale, is_causal=False, kv_lens=None, mask=None, num_splits=0,
                       workspace=None, stream=None, target_workgroups=0):
    """attn_prefill with split KV and a combine; num_splits 0 asks the
    planner (the tile count of the dense schedule, max_kv_len = Lk)."""
    _dev(q=(q, _BF16), k=(k, _BF16), v=(v, _BF16), out=(out, _BF16), kv_lens=(kv_lens, _I32),
         mask=(mask, (torch.bool, torch.uint8)), workspace=(workspace, None))
    _unit_inner(q, k, v, out)
    assert k.stride() == v.stride(), "K and V must share strides"
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if num_splits:
        S = num_splits
    else:
        R = attn_prefill_tile_rows(D, Hq // Hkv)
        S = attn_prefill_plan_splits(B * ((Lq + R - 1) // R), Hq, Hkv, D, Lk, target_workgroups)
    ws, nbytes = _prefill_workspace(workspace, B * Lq, Hq, D, S, q.device)
    mask, ndim, m_sb, m_sq = _mask_args(mask)
    _check(lib().attn_prefill_split(
        _ptr(q), q.stride(0), q.stride(1), q.stride(2), _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(kv_lens), int(Lk), 1 if is_causal else 0, _ptr(mask), ndim, m_sb, m_sq,
        _ptr(out), out.stride(0), out.stride(1), out.stride(2), B, Lq, Hq, Hkv, D, float(scale),
        S, _ptr(ws), nbytes, _stream(stream)))
    return out


def attn_hbm_read_probe(buf, sink, workgroups=0, stream=None):
    """Read every byte of the device tensor buf once (HBM streaming probe);
    sink: uint32 device tensor of at least workgroups * 16 entries (0 = one
    workgroup per CU: 16 * CU count), which receives per-wave XORs."""
    _dev(buf=(buf, None), sink=(sink, (torch.int32,)))
    assert buf.is_contiguous() and sink.is_contiguous()
    nbytes = buf.numel() * buf.element_size()
    _check(lib().attn_hbm_read_probe(_ptr(buf), nbytes, _ptr(sink), int(workgroups), _stream(stream)))
