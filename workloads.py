"""Seeded synthetic inputs for paged GQA attention.

This module only draws random inputs and lays them out; it computes nothing
of the attention method.  Both the HIP path and the CPU oracle consume the
tensors it returns (the oracle on CPU copies of the same bytes).

Value recipe (shared by every case): Q, K and V are N(0, 1) draws rounded to
bf16 (round-to-nearest-even, torch's conversion).  Page placement is a seeded
random permutation of a pool; block-table entries past a sequence's last page
are -1 and must never be read.  Generation runs on ``device`` with a torch
generator seeded on that device, so a seed reproduces the same bytes on the
same kind of device.
"""
import math

import torch


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def _randint(lo, hi, n, g, device):
    """n integers uniform in [lo, hi] inclusive."""
    return torch.randint(lo, hi + 1, (n,), generator=g, device=device, dtype=torch.int64)


def scatter_pages(kv_lens, page_size, g, device, pool_pages=None, pool_factor=1.5):
    """Block table [B, max_pages] int32 whose rows are disjoint draws without
    replacement from a random permutation of the pool.  Returns (bt, P)."""
    need = [(int(n) + page_size - 1) // page_size for n in kv_lens]
    total = sum(need)
    P = pool_pages if pool_pages is not None else max(1, math.ceil(pool_factor * total))
    assert P >= total
    perm = torch.randperm(P, generator=g, device=device).to(torch.int32)
    width = max(1, max(need) if need else 1)
    bt = torch.full((len(need), width), -1, dtype=torch.int32, device=device)
    off = 0
    for b, k in enumerate(need):
        bt[b, :k] = perm[off:off + k]
        off += k
    return bt, P


def paged_decode_case(seed, B, Hq, Hkv, D, kv_lens, page_size, pool_pages=None,
                      pool_factor=1.5, device="cpu", layout="page_slot_head"):
    """Paged decode inputs.  kv_lens: list of ints or (lo, hi) for a uniform
    draw.  Pool layout 'page_slot_head' is [P, ps, Hkv, D]; 'page_head_slot'
    allocates [P, Hkv, ps, D] and returns the (page, slot, head, dim) view."""
    g = _gen(seed, device)
    if isinstance(kv_lens, tuple):
        lo, hi = kv_lens
        kv_lens = _randint(lo, hi, B, g, device).tolist()
    kv_lens = [int(n) for n in kv_lens]
    bt, P = scatter_pages(kv_lens, page_size, g, device, pool_pages, pool_factor)
    q = _randn_bf16((B, Hq, D), g, device)
    if layout == "page_slot_head":
        k_pool = _randn_bf16((P, page_size, Hkv, D), g, device)
        v_pool = _randn_bf16((P, page_size, Hkv, D), g, device)
    elif layout == "page_head_slot":
        k_pool = _randn_bf16((P, Hkv, page_size, D), g, device).permute(0, 2, 1, 3)
        v_pool = _randn_bf16((P, Hkv, page_size, D), g, device).permute(0, 2, 1, 3)
    else:
        raise ValueError(layout)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                kv_lens=torch.tensor(kv_lens, dtype=torch.int32, device=device),
                max_kv_len=max(kv_lens) if kv_lens else 0, page_size=page_size,
                B=B, Hq=Hq, Hkv=Hkv, D=D, scale=1.0 / math.sqrt(D))


def contig_decode_case(seed, B, Hq, Hkv, D, kv_len, device="cpu", layout="bhld", kv_lens=None):
    """Contiguous decode inputs.  q is [B, Hq, 1, D] (bhld) or [B, 1, Hq, D]
    (blhd); K/V are [B, Hkv, L, D] (bhld) or [B, L, Hkv, D] (blhd).  The
    returned q/k/v entries are views indexed (b, head, [pos,] dim)."""
    g = _gen(seed, device)
    if layout == "bhld":
        q4 = _randn_bf16((B, Hq, 1, D), g, device)
        k4 = _randn_bf16((B, Hkv, kv_len, D), g, device)
        v4 = _randn_bf16((B, Hkv, kv_len, D), g, device)
        q, k, v = q4[:, :, 0, :], k4, v4
    elif layout == "blhd":
        q4 = _randn_bf16((B, 1, Hq, D), g, device)
        k4 = _randn_bf16((B, kv_len, Hkv, D), g, device)
        v4 = _randn_bf16((B, kv_len, Hkv, D), g, device)
        q, k, v = q4[:, 0, :, :], k4.permute(0, 2, 1, 3), v4.permute(0, 2, 1, 3)
    else:
        raise ValueError(layout)
    if kv_lens is not None:
        kv_lens = torch.tensor([int(n) for n in kv_lens], dtype=torch.int32, device=device)
    return dict(q=q, k=k, v=v, q4=q4, k4=k4, v4=v4, kv_len=kv_len, kv_lens=kv_lens,
                B=B, Hq=Hq, Hkv=Hkv, D=D, scale=1.0 / math.sqrt(D), layout=layout)


def prefill_case(seed, B, Hq, Hkv, D, ctx_range, q_range, page_size, mask_frac=None,
                 mask_ndim=3, causal=True, device="cpu", q_lens=None, ctx_lens=None,
                 pool_factor=1.5, mask_pad=4):
    """Ragged paged prefill inputs: prior context c_b ~ U[ctx_range], new rows
    q_b ~ U[q_range]; the new tokens' K/V are already in the cache, so the
    sequence holds n_b = c_b + q_b keys and causal_offset[b] = c_b.  With
    mask_frac, a keep-mask (True = keep) drops that fraction of entries at
    random: 3-D [B, max_q, max_n] or 2-D [B, max_n], its key dimension padded
    to a multiple of mask_pad (1: no padding)."""
    g = _gen(seed, device)
    if ctx_lens is None:
        ctx_lens = _randint(ctx_range[0], ctx_range[1], B, g, device).tolist()
    if q_lens is None:
        q_lens = _randint(q_range[0], q_range[1], B, g, device).tolist()
    ctx_lens = [int(c) for c in ctx_lens]
    q_lens = [int(x) for x in q_lens]
    kv_lens = [c + x for c, x in zip(ctx_lens, q_lens)]
    bt, P = scatter_pages(kv_lens, page_size, g, device, pool_factor=pool_factor)
    total_q = sum(q_lens)
    q = _randn_bf16((total_q, Hq, D), g, device)
    k_pool = _randn_bf16((P, page_size, Hkv, D), g, device)
    v_pool = _randn_bf16((P, page_size, Hkv, D), g, device)
    qo_indptr = torch.tensor([0] + list(_cumsum(q_lens)), dtype=torch.int32, device=device)
    mask = None
    if mask_frac is not None:
        # key dimension padded to a multiple of mask_pad; entries past a
        # sequence's keys are never used
        max_n = (max(max(kv_lens) if kv_lens else 1, 1) + mask_pad - 1) // mask_pad * mask_pad
        max_q = max(q_lens) if q_lens else 1
        shape = (B, max_q, max_n) if mask_ndim == 3 else (B, max_n)
        mask = torch.rand(*shape, generator=g, device=device) >= mask_frac
    causal_offset = torch.tensor(ctx_lens if causal else [-1] * B, dtype=torch.int32, device=device)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                kv_lens=torch.tensor(kv_lens, dtype=torch.int32, device=device),
                qo_indptr=qo_indptr, q_lens=q_lens, ctx_lens=ctx_lens,
                causal_offset=causal_offset, mask=mask, page_size=page_size,
                B=B, Hq=Hq, Hkv=Hkv, D=D, scale=1.0 / math.sqrt(D))


def _cumsum(xs):
    s = 0
    for x in xs:
        s += x
        yield s


def swa_case(seed, T, NH, HD, W, block_size, num_blocks, len_range=None, lens=None,
             neg_frac=0.0, device="cpu"):
    """fp8 sliding-window decode inputs.  For window position j < len_t the
    slot index is a distinct random slot of the pool (a neg_frac fraction of
    them replaced by -1); positions j >= len_t hold -1.  inv_scale ~ U[0.01,
    0.1] rounded to bf16.  Cache bytes are e4m3fn codes of x / inv_scale with
    x ~ N(0, 1), saturated to +-448 and rounded to nearest-even, so the
    dequantised rows are close to N(0, 1)."""
    g = _gen(seed, device)
    slots = num_blocks * block_size
    if lens is None:
        lo, hi = len_range if len_range is not None else (1, W)
        lens = _randint(lo, hi, T, g, device).tolist()
    lens = [int(x) for x in lens]
    q = _randn_bf16((T, NH, HD), g, device)
    inv = (0.01 + 0.09 * torch.rand(slots, 1, generator=g, device=device)).to(torch.bfloat16)
    x = torch.randn(slots, HD, generator=g, device=device)
    codes = (x / inv.float()).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    cache = codes.view(torch.uint8).reshape(num_blocks, block_size, HD)
    ind = torch.full((T, W), -1, dtype=torch.int64, device=device)
    for t in range(T):
        n = min(lens[t], W)   # a length above the window admits the whole window
        if n > 0:
            pick = torch.randperm(slots, generator=g, device=device)[:n]
            ind[t, :n] = pick
    if neg_frac > 0:
        drop = torch.rand(T, W, generator=g, device=device) < neg_frac
        ind[drop] = -1
    return dict(q=q, cache=cache, inv_scale=inv, indices=ind,
                lens=torch.tensor(lens, dtype=torch.int64, device=device),
                T=T, NH=NH, HD=HD, W=W, block_size=block_size, num_blocks=num_blocks,
                scale=1.0 / math.sqrt(HD))


# The five workloads, by what they are.
def tiny_paged_decode(device="cpu"):
    """B=2, Hq=8, Hkv=2, D=64, kv_lens {256, 300}, ps=16; pool of exactly
    the 35 pages needed, placed by a seeded permutation."""
    return paged_decode_case(1001, 2, 8, 2, 64, [256, 300], 16, pool_pages=35, device=device)


def contiguous_decode(device="cpu"):
    """B=16, Hq=32, Hkv=8, D=128, kv_len 2048, bhld."""
    return contig_decode_case(1002, 16, 32, 8, 128, 2048, device=device)


def serving_paged_decode(B=32, device="cpu", fixed_len=None, seed=None):
    """B in {32, 128}, Hq=32, Hkv=8, D=128, ps=16, kv_lens ~ U[512, 4096]
    (or all = fixed_len), pages scattered in a pool 1.5x the pages needed."""
    if seed is None:
        seed = 1003 if B == 32 else 1004
    lens = [fixed_len] * B if fixed_len is not None else (512, 4096)
    return paged_decode_case(seed, B, 32, 8, 128, lens, 16, device=device)


def ragged_prefill(device="cpu", masked=False, seed=1005):
    """8 sequences, prior context ~ U[0, 2048], new rows ~ U[1, 512], Hq=32,
    Hkv=8, D=128, ps=16, causal_offset = prior context; optional 3-D mask
    with 10% of entries dropped."""
    return prefill_case(seed, 8, 32, 8, 128, (0, 2048), (1, 512), 16,
                        mask_frac=0.1 if masked else None, mask_ndim=3, device=device)


def short_q_prefill(device="cpu", seed=1007):
    """Short query runs over long contexts: 16 sequences of 16 new rows after
    16368 cached keys (16384 in all), Hq=32, Hkv=4 (G = 8), D=128, ps=16,
    causal_offset = cached keys."""
    return prefill_case(seed, 16, 32, 4, 128, None, None, 16, device=device,
                        q_lens=[16] * 16, ctx_lens=[16368] * 16)


def swa_fp8(device="cpu", seed=1006):
    """T=64, NH=128 (16-head groups), HD=512, window 128, lens ~ U[1, 128],
    block_size 256, 128 blocks (32768 slots)."""
    return swa_case(seed, 64, 128, 512, 128, 256, 128, len_range=(1, 128), device=device)
