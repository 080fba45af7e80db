"""CPU fp64 oracle for paged GQA attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU baseline
may import this package.  It wraps ``liboracle.so`` (plain C, built from
``oracle.c`` with gcc and OpenMP) and shares no code with the HIP library.

Inputs are torch CPU tensors whose raw bytes are handed to C: bf16 tensors
as ``torch.bfloat16``, fp8 cache bytes as ``torch.uint8``, indices as int32
or int64.  Outputs are float64 tensors.  Strides are in elements and follow
the tensors passed in, so any strided view works.
"""
import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose=False):
    """Compile liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", _LIB, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_D = ctypes.c_double


def _declare(l):
    l.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    l.orc_bf16_to_f64.restype = _D
    l.orc_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    l.orc_e4m3fn_to_f64.restype = _D
    l.orc_paged_decode.argtypes = [_P, _L, _L, _P, _P, _L, _L, _L, _P, _L, _P, _P, _L,
                                   _I, _I, _I, _I, _I, _D, _P, _P]
    l.orc_decode.argtypes = [_P, _L, _L, _P, _L, _L, _L, _P, _L, _L, _L, _P, _I,
                             _I, _I, _I, _I, _D, _P, _P]
    l.orc_paged_decode_partials.argtypes = [_P, _L, _L, _P, _P, _L, _L, _L, _P, _L, _P,
                                            _P, _I, _I, _I, _I, _I, _I, _D, _P, _P, _P]
    l.orc_combine.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P]
    l.orc_combine_f32.argtypes = [_P, _P, _I, _I, _I, _P, _P]
    l.orc_paged_prefill.argtypes = [_P, _L, _L, _P, _P, _P, _L, _L, _L, _P, _L, _P, _P,
                                    _P, _I, _L, _L, _I, _I, _I, _I, _I, _D, _P, _P]
    l.orc_prefill_plan.argtypes = [_P, _I, _I, _P, _P, _P, _I]
    l.orc_swa_fp8_decode.argtypes = [_P, _L, _L, _P, _L, _L, _P, _L, _P, _L, _P,
                                     _I, _I, _I, _I, _I, _D, _I, _P, _P]
    l.orc_kv_append.argtypes = [_P, _P, _L, _L, _P, _P, _P, _P, _L, _L, _L, _P, _L, _I, _I, _I, _I]
    l.orc_rotary.argtypes = [_P, _L, _L, _I, _I, _I, _P, _P, _L, _P, _P, _L, _L]
    l.orc_fp8_quantize.argtypes = [_P, _L, _I, _I, _P, _P, _L, _P, _P]
    l.orc_num_threads.argtypes = []
    for name in ("orc_paged_decode", "orc_decode", "orc_paged_decode_partials", "orc_combine",
                 "orc_combine_f32", "orc_paged_prefill", "orc_prefill_plan",
                 "orc_swa_fp8_decode", "orc_kv_append", "orc_rotary", "orc_fp8_quantize",
                 "orc_num_threads"):
        getattr(l, name).restype = _I


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)


def _cpu(t, dtype=None):
    assert t is None or t.device.type == "cpu", "oracle takes CPU tensors"
    if t is not None and dtype is not None:
        assert t.dtype == dtype, (t.dtype, dtype)
    return t


def bf16_to_f64(bits):
    return lib().orc_bf16_to_f64(int(bits) & 0xFFFF)


def e4m3fn_to_f64(bits):
    return lib().orc_e4m3fn_to_f64(int(bits) & 0xFF)


def num_threads():
    return lib().orc_num_threads()


def paged_decode(q, k_pool, v_pool, block_table, kv_lens, scale, mask=None):
    """q [B, Hq, D] bf16 (any strides with unit inner stride); k_pool/v_pool
    [P, ps, Hkv, D] or any 4-D view (page, slot, head, dim) with unit inner
    stride and identical strides; block_table [B, *] int32; kv_lens [B] int32;
    optional 2-D keep-mask [B, >=max n] uint8/bool.  Returns (out, lse)."""
    _cpu(q, torch.bfloat16), _cpu(block_table, torch.int32), _cpu(kv_lens, torch.int32)
    B, Hq, D = q.shape
    P, ps, Hkv, D2 = k_pool.shape
    assert D2 == D and q.stride(2) == 1 and k_pool.stride(3) == 1
    assert k_pool.stride() == v_pool.stride() and block_table.stride(1) == 1
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
    out = torch.empty(B, Hq, D, dtype=torch.float64)
    lse = torch.empty(B, Hq, dtype=torch.float64)
    kv_lens = kv_lens.contiguous()
    _check(lib().orc_paged_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens),
        _ptr(mask), mask.stride(0) if mask is not None else 0,
        B, Hq, Hkv, D, ps, float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def decode(q, k, v, scale, kv_lens=None):
    """Contiguous decode.  q [B, Hq, D]; k, v [B, Hkv, L, D] views (bhld) or
    any 4-D (b, head, pos, dim) view with unit inner stride."""
    _cpu(q, torch.bfloat16)
    B, Hq, D = q.shape
    _, Hkv, L, _ = k.shape
    assert q.stride(2) == 1 and k.stride(3) == 1 and v.stride(3) == 1
    if kv_lens is not None:
        kv_lens = _cpu(kv_lens, torch.int32).contiguous()
    out = torch.empty(B, Hq, D, dtype=torch.float64)
    lse = torch.empty(B, Hq, dtype=torch.float64)
    _check(lib().orc_decode(
        _ptr(q), q.stride(0), q.stride(1),
        _ptr(k), k.stride(0), k.stride(1), k.stride(2),
        _ptr(v), v.stride(0), v.stride(1), v.stride(2),
        _ptr(kv_lens), L, B, Hq, Hkv, D, float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def paged_decode_partials(q, k_pool, v_pool, block_table, kv_lens, bounds, scale):
    """fp64 split partials for chunk boundaries bounds [B, S+1] (int32).
    Returns (o_part [S,B,Hq,D], m_part [S,B,Hq], l_part [S,B,Hq])."""
    B, Hq, D = q.shape
    P, ps, Hkv, _ = k_pool.shape
    bounds = _cpu(bounds, torch.int32).contiguous()
    S = bounds.shape[1] - 1
    o = torch.empty(S, B, Hq, D, dtype=torch.float64)
    m = torch.empty(S, B, Hq, dtype=torch.float64)
    l = torch.empty(S, B, Hq, dtype=torch.float64)
    _check(lib().orc_paged_decode_partials(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens.contiguous()),
        _ptr(bounds), S, B, Hq, Hkv, D, ps, float(scale), _ptr(o), _ptr(m), _ptr(l)))
    return o, m, l


def combine(o_part, m_part, l_part):
    """fp64 log-sum-exp combine; o_part [S, R, D], m/l [S, R] float64."""
    o_part = o_part.to(torch.float64).contiguous()
    m_part = m_part.to(torch.float64).contiguous()
    l_part = l_part.to(torch.float64).contiguous()
    S, R, D = o_part.shape
    out = torch.empty(R, D, dtype=torch.float64)
    lse = torch.empty(R, dtype=torch.float64)
    _check(lib().orc_combine(_ptr(o_part), _ptr(m_part), _ptr(l_part), S, R, D,
                             _ptr(out), _ptr(lse)))
    return out, lse


def combine_f32(o_part, ml_part):
    """fp64 combine of float32 partials o_part [S, R, D], ml_part [S, R, 2]."""
    o_part = _cpu(o_part, torch.float32).contiguous()
    ml_part = _cpu(ml_part, torch.float32).contiguous()
    S, R, D = o_part.shape
    out = torch.empty(R, D, dtype=torch.float64)
    lse = torch.empty(R, dtype=torch.float64)
    _check(lib().orc_combine_f32(_ptr(o_part), _ptr(ml_part), S, R, D, _ptr(out), _ptr(lse)))
    return out, lse


def paged_prefill(q, qo_indptr, k_pool, v_pool, block_table, kv_lens, scale,
                  causal_offset=None, mask=None):
    """q [total_q, Hq, D] bf16 packed; qo_indptr [B+1] int32; mask None, 2-D
    [B, kv] or 3-D [B, q, kv] (keep = nonzero).  Returns (out, lse)."""
    _cpu(q, torch.bfloat16)
    total_q, Hq, D = q.shape
    P, ps, Hkv, _ = k_pool.shape
    B = qo_indptr.numel() - 1
    qo_indptr = _cpu(qo_indptr, torch.int32).contiguous()
    kv_lens = _cpu(kv_lens, torch.int32).contiguous()
    if causal_offset is not None:
        causal_offset = _cpu(causal_offset, torch.int32).contiguous()
    ndim, m_sb, m_sq = 0, 0, 0
    if mask is not None:
        mask = mask.to(torch.uint8)
        assert mask.stride(-1) == 1
        ndim = mask.dim()
        m_sb = mask.stride(0)
        m_sq = mask.stride(1) if ndim == 3 else 0
    out = torch.empty(total_q, Hq, D, dtype=torch.float64)
    lse = torch.empty(total_q, Hq, dtype=torch.float64)
    _check(lib().orc_paged_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(qo_indptr), _ptr(k_pool), _ptr(v_pool),
        k_pool.stride(0), k_pool.stride(1), k_pool.stride(2),
        _ptr(block_table), block_table.stride(0), _ptr(kv_lens), _ptr(causal_offset),
        _ptr(mask), ndim, m_sb, m_sq, B, Hq, Hkv, D, ps, float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def prefill_plan(q_lens, tile_rows=64):
    """Work map for a ragged batch: (qo_indptr, tile_to_batch, tile_to_index)."""
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).contiguous()
    B = q_lens.numel()
    cap = int(sum((int(x) + tile_rows - 1) // tile_rows for x in q_lens.tolist())) + 1
    indptr = torch.empty(B + 1, dtype=torch.int32)
    t2b = torch.empty(cap, dtype=torch.int32)
    t2i = torch.empty(cap, dtype=torch.int32)
    n = lib().orc_prefill_plan(_ptr(q_lens), B, tile_rows, _ptr(indptr), _ptr(t2b), _ptr(t2i), cap)
    if n < 0:
        raise ValueError("bad work-map arguments")
    return indptr, t2b[:n].clone(), t2i[:n].clone()


def swa_fp8_decode(q, cache, inv_scale, indices, lens, block_size, scale,
                   emulate_bf16_dequant=False):
    """q [T, NH, HD] bf16; cache [num_blocks, block_size, HD] uint8 (e4m3fn
    bytes); inv_scale [max_slots, 1] or [max_slots] bf16; indices [T, W]
    int64; lens [T] int64.  Returns (out [T, NH, HD], lse [T, NH])."""
    _cpu(q, torch.bfloat16), _cpu(cache, torch.uint8)
    _cpu(indices, torch.int64), _cpu(lens, torch.int64)
    T, NH, HD = q.shape
    W = indices.shape[1]
    assert cache.stride(2) == 1 and indices.stride(1) == 1
    lens = lens.contiguous()
    out = torch.empty(T, NH, HD, dtype=torch.float64)
    lse = torch.empty(T, NH, dtype=torch.float64)
    _check(lib().orc_swa_fp8_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(cache), cache.stride(0), cache.stride(1),
        _ptr(inv_scale), inv_scale.stride(0), _ptr(indices), indices.stride(0), _ptr(lens),
        T, NH, HD, W, block_size, float(scale), 1 if emulate_bf16_dequant else 0,
        _ptr(out), _ptr(lse)))
    return out, lse


def kv_append(k_pool, v_pool, block_table, k_new, v_new, new_indptr, start_pos):
    """Return copies of the (page, slot, head, dim) pools with the packed new
    rows k_new / v_new [N, Hkv, D] written at positions start_pos[b] + i of
    sequence b (rows new_indptr[b] .. new_indptr[b+1]).  The pools' strides
    are kept (a strided view is copied into a tensor of the same layout)."""
    kp = torch.empty_strided(k_pool.shape, k_pool.stride(), dtype=k_pool.dtype)
    vp = torch.empty_strided(v_pool.shape, v_pool.stride(), dtype=v_pool.dtype)
    kp.copy_(k_pool.cpu())
    vp.copy_(v_pool.cpu())
    kn, vn = _cpu(k_new), _cpu(v_new)
    assert kn.stride() == vn.stride() and kn.stride(2) == 1
    bt = _cpu(block_table, torch.int32)
    ind = _cpu(new_indptr, torch.int32)
    st = _cpu(start_pos, torch.int32)
    _check(lib().orc_kv_append(_ptr(kn), _ptr(vn), kn.stride(0), kn.stride(1), _ptr(ind), _ptr(st),
                               _ptr(kp), _ptr(vp), kp.stride(0), kp.stride(1), kp.stride(2), _ptr(bt),
                               bt.stride(0), ind.numel() - 1, kp.shape[2], kp.shape[3], kp.shape[1]))
    return kp, vp


def rotary(x, cos_tab, sin_tab, positions):
    """x [T, H, D] bf16; cos_tab / sin_tab float32 [rows, D/2]; positions
    int [T].  Returns the rotated [T, H, D] bf16 tensor."""
    xc = _cpu(x)
    assert xc.stride(2) == 1
    c, s = _cpu(cos_tab, torch.float32), _cpu(sin_tab, torch.float32)
    assert c.stride() == s.stride() and c.stride(1) == 1
    pos = _cpu(positions, torch.int32)
    T, H, D = xc.shape
    out = torch.empty(T, H, D, dtype=torch.bfloat16)
    _check(lib().orc_rotary(_ptr(xc), xc.stride(0), xc.stride(1), T, H, D, _ptr(c), _ptr(s), c.stride(0),
                            _ptr(pos), _ptr(out), out.stride(0), out.stride(1)))
    return out


def fp8_quantize(x, mult=None):
    """x [N, HD] bf16; mult float32 [N] or None (448 / amax per row).
    Returns (codes uint8 [N, HD], inv_scale bf16 [N], amax float32 [N])."""
    xc = _cpu(x)
    assert xc.stride(1) == 1
    N, HD = xc.shape
    m = None if mult is None else _cpu(mult, torch.float32)
    codes = torch.empty(N, HD, dtype=torch.uint8)
    inv = torch.empty(N, dtype=torch.bfloat16)
    amax = torch.empty(N, dtype=torch.float32)
    _check(lib().orc_fp8_quantize(_ptr(xc), xc.stride(0), N, HD, _ptr(m), _ptr(codes), codes.stride(0),
                                  _ptr(inv), _ptr(amax)))
    return codes, inv, amax
