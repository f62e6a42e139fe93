"""Seeded synthetic workloads for paged GDN prefill and decode.

This module only draws inputs and lays out page tables the way a serving
engine would hand them over (CSR page tables: flashinfer.gdn_paged, "Page
table"; FlashInfer CSR paging drill, sections 1-2).  It holds none of the
recurrence's arithmetic, and both the HIP path and the CPU oracle are fed the
same tensors from here.

Page tables and lengths come from a CPU generator; token inputs and pool
rows from a generator on the target device (so CPU and GPU draws differ, and
every test hands the same tensors to both sides).

Token inputs (all shapes row-major):
    q, k  [T, Hqk, K] bf16 -- fp32 N(0,1), L2-normalised over K per (token, head)
                              in fp32, then rounded to bf16
    v     [T, H, V]   bf16 -- N(0,1)
    g     [T, H]      fp32 -- -softplus(N(0,1))   (times ``g_scale``)
    beta  [T, H]      fp32 -- sigmoid(N(0,1))
drawn from one generator in the order q, k, v, g, beta.

Pools are fp32 ``[num_pages, H, V, K]``.  Rows a call reads hold N(0, 1/K)
values; every other row holds the NaN bit pattern 0x7FC00001, so a stray read
turns an output non-finite and a stray write changes bits.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import torch
import torch.nn.functional as F

NAN_BITS = 0x7FC00001
CHUNK = 64


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def token_inputs(T: int, Hqk: int, H: int, K: int, V: int, gen: torch.Generator,
                 device="cpu", g_scale: float = 1.0) -> Dict[str, torch.Tensor]:
    q = torch.randn(T, Hqk, K, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(T, Hqk, K, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(T, H, V, generator=gen, device=device, dtype=torch.float32)
    gx = torch.randn(T, H, generator=gen, device=device, dtype=torch.float32)
    bx = torch.randn(T, H, generator=gen, device=device, dtype=torch.float32)
    q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    return {
        "q": q.contiguous(), "k": k.contiguous(), "v": v.to(torch.bfloat16).contiguous(),
        "g": (-F.softplus(gx) * g_scale).contiguous(),
        "beta": torch.sigmoid(bx).contiguous(),
    }


def csr(ctx_lens: Sequence[int], page_size: int, page_lists: Sequence[Sequence[int]]):
    """Page table tensors (int32) from per-sequence page lists; checks that each
    list has exactly ceil(ctx / page_size) pages."""
    indptr = [0]
    lpl = []
    flat: List[int] = []
    for ctx, pages in zip(ctx_lens, page_lists):
        n = (ctx + page_size - 1) // page_size
        if len(pages) != n:
            raise ValueError(f"ctx {ctx} needs {n} pages, got {len(pages)}")
        flat.extend(int(p) for p in pages)
        indptr.append(len(flat))
        lpl.append(ctx - (n - 1) * page_size)
    i32 = torch.int32
    return (torch.tensor(flat, dtype=i32), torch.tensor(indptr, dtype=i32),
            torch.tensor(lpl, dtype=i32))


def nan_pool(num_rows: int, H: int, V: int, K: int, device="cpu",
             row_stride: Optional[int] = None) -> torch.Tensor:
    """[num_rows, H, V, K] fp32 view full of NaN bits; with ``row_stride`` the
    rows sit ``row_stride`` floats apart in a larger buffer (padded rows)."""
    blk = H * V * K
    rs = blk if row_stride is None else int(row_stride)
    base = torch.empty(num_rows * rs, dtype=torch.float32, device=device)
    base.view(torch.int32).fill_(NAN_BITS)
    return base.as_strided((num_rows, H, V, K), (rs, V * K, K, 1))


def fill_rows(pool: torch.Tensor, rows: Sequence[int], gen: torch.Generator, std: float):
    for r in sorted(set(int(x) for x in rows if int(x) >= 0)):
        pool[r].copy_(torch.randn(pool.shape[1:], generator=gen, device=pool.device) * std)


def _perm(n: int, gen: torch.Generator) -> List[int]:
    return torch.randperm(n, generator=gen).tolist()


def _randint(lo: int, hi: int, gen: torch.Generator) -> int:
    """Uniform integer in [lo, hi]."""
    return int(torch.randint(lo, hi + 1, (1,), generator=gen).item())


def _read_row(pages, prefix, page_size):
    return pages[(prefix - 1) // page_size] if prefix > 0 else -1


def _prefill_batch(prefix: Sequence[int], new: Sequence[int], pages: Sequence[Sequence[int]],
                   page_size: int, Hqk: int, H: int, K: int, V: int, tok_gen, device,
                   g_scale: float = 1.0) -> Dict:
    ctx = [p + n for p, n in zip(prefix, new)]
    idx, ptr, lpl = csr(ctx, page_size, pages)
    cu = [0]
    for n in new:
        cu.append(cu[-1] + n)
    T = cu[-1]
    d = token_inputs(T, Hqk, H, K, V, tok_gen, device=device, g_scale=g_scale)
    d.update(cu_seqlens=torch.tensor(cu, dtype=torch.int32), page_indices=idx,
             page_indptr=ptr, last_page_len=lpl, page_size=page_size,
             prefix=list(prefix), new=list(new), pages=[list(p) for p in pages],
             read_rows=[_read_row(pg, p, page_size) for pg, p in zip(pages, prefix)])
    return d


def _decode_batch(ctx: Sequence[int], pages: Sequence[Sequence[int]], page_size: int,
                  Hqk: int, H: int, K: int, V: int, tok_gen, device, g_scale=1.0) -> Dict:
    idx, ptr, lpl = csr(ctx, page_size, pages)
    d = token_inputs(len(ctx), Hqk, H, K, V, tok_gen, device=device, g_scale=g_scale)
    rd = []
    for c, pg in zip(ctx, pages):
        rd.append(pg[-2] if (c - 1) % page_size == 0 else pg[-1])
    d.update(page_indices=idx, page_indptr=ptr, last_page_len=lpl, page_size=page_size,
             ctx=list(ctx), pages=[list(p) for p in pages], read_rows=rd)
    return d


def config0(device="cpu", seed: int = 0) -> Dict:
    """Tiny paged case: H = Hqk = 2, K = V = 128, page 128, zero pool of 16 pages.

    seq0: prefix 0, 300 new tokens, pages [11, 4, 14]; seq1: prefix 64, 130 new
    tokens, pages [5, 9] (194 tokens fill two pages; page 2 is allocated to it
    but unlisted and must stay untouched).  Then one decode token per sequence.
    """
    gen = generator(seed)  # config 0 is always drawn on the CPU
    H = Hqk = 2
    K = V = 128
    ps = 128
    pool = torch.zeros(16, H, V, K, dtype=torch.float32)
    pre = _prefill_batch([0, 64], [300, 130], [[11, 4, 14], [5, 9]], ps, Hqk, H, K, V, gen, "cpu")
    dec = _decode_batch([301, 195], [[11, 4, 14], [5, 9]], ps, Hqk, H, K, V, gen, "cpu")
    return _to(dict(pool=pool, prefill=pre, decode=dec, H=H, Hqk=Hqk, K=K, V=V,
                    untouched_extra=[2]), device)


def config1(device="cpu", seed: int = 1, heads: int = 16, num_seqs: int = 8,
            max_prefix: int = 8192, max_new: int = 4096, page_size: int = 1024,
            num_pages: int = 512, g_scale: float = 1.0) -> Dict:
    """Paged prefill with shared prefixes.

    B sequences, prefix ~ U[0, max_prefix] redrawn while a multiple of 64, new
    tokens ~ U[1, max_new].  Sequence i >= B/2 shares its first
    min(p_i, p_{i-B/2}) // page_size full pages with sequence i - B/2.  Page ids
    come from a seeded permutation of the pool.
    """
    gen = generator(seed)
    H = Hqk = heads
    K = V = 128
    prefix, new = [], []
    for _ in range(num_seqs):
        p = _randint(0, max_prefix, gen)
        while p % CHUNK == 0:
            p = _randint(0, max_prefix, gen)
        prefix.append(p)
        new.append(_randint(1, max_new, gen))
    perm = iter(_perm(num_pages, gen))
    pages = []
    half = num_seqs // 2
    for i in range(num_seqs):
        n = (prefix[i] + new[i] + page_size - 1) // page_size
        shared = []
        if i >= half:
            j = i - half
            shared = pages[j][:min(prefix[i], prefix[j]) // page_size]
        pages.append(shared + [next(perm) for _ in range(n - len(shared))])
    pre = _prefill_batch(prefix, new, pages, page_size, Hqk, H, K, V, gen_on(seed + 50, device),
                         device, g_scale)
    pool = nan_pool(num_pages, H, V, K, device=device)
    fill_rows(pool, pre["read_rows"], gen_on(seed + 100, device), 1.0 / math.sqrt(K))
    return _to(dict(pool=pool, prefill=pre, H=H, Hqk=Hqk, K=K, V=V), device)


def config2(device="cpu", seed: int = 2, num_seqs: int = 256, qk_heads: int = 16,
            v_heads: int = 32, page_size: int = 1024, num_pages: int = 8192,
            ctx_lo: int = 1024, ctx_hi: int = 32768, new_page_seqs: int = 64,
            g_scale: float = 1.0) -> Dict:
    """Paged decode, T = 1.

    Context (tokens after the call) ~ U[ctx_lo, ctx_hi]; ``new_page_seqs``
    seeded sequences get 1024*m + 1 tokens so that the decoded token opens a
    new page (last_page_len == 1).  Page ids: a seeded permutation.
    """
    gen = generator(seed)
    K = V = 128
    ctx = [_randint(ctx_lo, ctx_hi, gen) for _ in range(num_seqs)]
    forced = _perm(num_seqs, gen)[:new_page_seqs]
    for b in forced:
        m = _randint(max(1, ctx_lo // page_size), max(1, (ctx_hi - 1) // page_size), gen)
        ctx[b] = page_size * m + 1
    perm = iter(_perm(num_pages, gen))
    pages = [[next(perm) for _ in range((c + page_size - 1) // page_size)] for c in ctx]
    dec = _decode_batch(ctx, pages, page_size, qk_heads, v_heads, K, V, gen_on(seed + 50, device),
                        device, g_scale)
    pool = nan_pool(num_pages, v_heads, V, K, device=device)
    fill_rows(pool, dec["read_rows"], gen_on(seed + 100, device), 1.0 / math.sqrt(K))
    return _to(dict(pool=pool, decode=dec, H=v_heads, Hqk=qk_heads, K=K, V=V), device)


def config3(device="cpu", seed: int = 3, heads: int = 32, total: int = 32768,
            splits=(7001, 14500, 20000, 27777), every_n: int = 896,
            num_rows: int = 64, g_scale: float = 1.0, qk_heads: Optional[int] = None) -> Dict:
    """Long chunked prefill with checkpoints, B = 1, fed in len(splits)+1 calls.

    Each call uses the slot-argument form: the request's state lives in slot
    row ``slot`` of a ``num_rows``-row pool (read -1 on the first call, then the
    slot), and checkpoints every ``every_n`` tokens go to a separate NaN-filled
    ``state_checkpoints`` buffer; checkpoint c (position (c+1)*every_n) is
    stored at row c for even c and skipped (-1) for odd c.  ``qk_heads``
    (default ``heads``) q/k heads serve the ``heads`` v-heads.
    """
    gen = generator(seed)
    H = heads
    Hqk = qk_heads or heads
    K = V = 128
    n_ck = total // every_n
    ck_rows = torch.tensor([c if c % 2 == 0 else -1 for c in range(n_ck)], dtype=torch.int32)
    slot = _randint(0, num_rows - 1, gen)
    bounds = [0] + list(splits) + [total]
    tgen = gen_on(seed + 50, device)
    calls = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        d = token_inputs(b - a, Hqk, H, K, V, tgen, device=device, g_scale=g_scale)
        d.update(cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32),
                 prefix_lens=torch.tensor([a], dtype=torch.int32),
                 checkpoint_cu_starts=torch.tensor([a // every_n], dtype=torch.int32),
                 state_indices=torch.tensor([-1 if a == 0 else slot], dtype=torch.int32),
                 output_state_indices=torch.tensor([slot], dtype=torch.int32),
                 start=a, end=b)
        calls.append(d)
    pool = nan_pool(num_rows, H, V, K, device=device)
    ckpt = nan_pool(n_ck, H, V, K, device=device)
    return _to(dict(pool=pool, state_checkpoints=ckpt, checkpoint_state_indices=ck_rows,
                    every_n=every_n, calls=calls, slot=slot, H=H, Hqk=Hqk, K=K, V=V), device)


def config4(device="cpu", seed: int = 4, heads: int = 32, num_prefill: int = 32,
            prefill_pad: int = 4, num_decode: int = 512, decode_pad: int = 16,
            page_size: int = 896, num_pages: int = 16384, new_lo: int = 512,
            new_hi: int = 8192, hit_hi: int = 16384, ctx_lo: int = 2048,
            ctx_hi: int = 65536, layers: Sequence[int] = (0,), g_scale: float = 1.0,
            qk_heads: Optional[int] = None) -> Dict:
    """Mixed hybrid serving step on one pool.

    Prefill: ``num_prefill`` sequences, new tokens ~ U[new_lo, new_hi], prefix
    hit = page_size * floor(U[0, hit_hi] / page_size), plus ``prefill_pad``
    padded sequences (0 new tokens, one scratch page each).  Decode:
    ``num_decode`` sequences with ctx ~ U[ctx_lo, ctx_hi] plus ``decode_pad``
    padded ones (one scratch page, last_page_len 2).  Every page a call reads
    or writes has its own id; page-list entries before the read page (cold
    prefix pages nobody touches) are drawn from a shared cold region.  The page
    tables are drawn once; token inputs are drawn per layer from seed
    ``seed * 1000 + layer``.  ``qk_heads`` (default ``heads``) q/k heads serve
    the ``heads`` v-heads.
    """
    gen = generator(seed)
    H = heads
    Hqk = qk_heads or heads
    K = V = 128
    perm = _perm(num_pages, gen)
    hot = iter(perm)
    pre_prefix, pre_new, pre_pages = [], [], []
    for _ in range(num_prefill):
        L = _randint(new_lo, new_hi, gen)
        p = page_size * (_randint(0, hit_hi, gen) // page_size)
        pre_prefix.append(p)
        pre_new.append(L)
    dec_ctx = [_randint(ctx_lo, ctx_hi, gen) for _ in range(num_decode)]
    # Touched pages first (distinct ids), then the cold region from the rest.
    pre_touched = []
    for p, L in zip(pre_prefix, pre_new):
        n = (p + L + page_size - 1) // page_size
        first = (p - 1) // page_size if p > 0 else 0
        pre_touched.append([next(hot) for _ in range(n - first)])
    pad_pre = [[next(hot)] for _ in range(prefill_pad)]
    dec_touched = []
    for c in dec_ctx:
        n = (c + page_size - 1) // page_size
        dec_touched.append([next(hot) for _ in range(min(2, n))])
    pad_dec = [[next(hot)] for _ in range(decode_pad)]
    cold = list(hot)
    ci = 0

    def cold_pages(m):
        nonlocal ci
        out = []
        for _ in range(m):
            out.append(cold[ci % len(cold)])
            ci += 1
        return out

    for i, (p, L) in enumerate(zip(pre_prefix, pre_new)):
        first = (p - 1) // page_size if p > 0 else 0
        pre_pages.append(cold_pages(first) + pre_touched[i])
    dec_pages = []
    for c, t in zip(dec_ctx, dec_touched):
        n = (c + page_size - 1) // page_size
        dec_pages.append(cold_pages(n - len(t)) + t)
    pre_prefix_all = pre_prefix + [1] * prefill_pad
    pre_new_all = pre_new + [0] * prefill_pad
    pre_pages_all = pre_pages + pad_pre
    dec_ctx_all = dec_ctx + [2] * decode_pad
    dec_pages_all = dec_pages + pad_dec

    out_layers = {}
    for layer in layers:
        tg = gen_on(seed * 1000 + int(layer), device)
        pre = _prefill_batch(pre_prefix_all, pre_new_all, pre_pages_all, page_size, Hqk, H, K,
                             V, tg, device, g_scale)
        dec = _decode_batch(dec_ctx_all, dec_pages_all, page_size, Hqk, H, K, V, tg, device,
                            g_scale)
        out_layers[int(layer)] = dict(prefill=pre, decode=dec)
    first = out_layers[int(layers[0])]
    pool = nan_pool(num_pages, H, V, K, device=device)
    read_rows = [r for r in first["prefill"]["read_rows"][:num_prefill]] + \
                first["decode"]["read_rows"]
    fill_rows(pool, read_rows, gen_on(seed + 100, device), 1.0 / math.sqrt(K))
    return _to(dict(pool=pool, layers=out_layers, H=H, Hqk=Hqk, K=K, V=V,
                    page_size=page_size, num_prefill=num_prefill,
                    num_decode=num_decode), device)


def gen_on(seed: int, device) -> torch.Generator:
    return generator(seed, device if str(device).startswith("cuda") else "cpu")


def _to(obj, device):
    if isinstance(obj, torch.Tensor):
        return obj.to(device) if obj.device != torch.device(device) else obj
    if isinstance(obj, dict):
        return {k: _to(v, device) for k, v in obj.items()}
    if isinstance(obj, list):
        return [_to(v, device) for v in obj]
    return obj
