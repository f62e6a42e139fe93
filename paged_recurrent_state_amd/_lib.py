"""ctypes binding of libgdn_paged.so (include/gdn_paged.h).

Argument marshalling only: every step runs in the HIP library on the tensors'
device, on torch's current stream.  There is no fallback; if the library is
missing the call raises.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import NamedTuple, Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn_paged.so")
_lib = None

GDN_INDEX_INT32 = 0
GDN_INDEX_INT64 = 1
STATUS = {0: "GDN_OK", -1: "GDN_EINVAL", -2: "GDN_EUNSUPPORTED", -3: "GDN_ELAUNCH",
          -4: "GDN_EWORKSPACE"}


class GDNError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class Options(C.Structure):
    """Launch choices of one call (gdn_options_t); every field 0 = the default.

    prefill_split_chunks: 0 the device decides from the lengths, -1 never
    split, m > 0 segments of m chunks.  prefill_tile_waves: 0/8 whole heads,
    4/2/1 V-tiles.  decode_waves: 2/4/8/16 one-pair decode width.
    decode_stream_per_cu: streaming decode workgroups per CU (-1 off).
    decode_stream_grid: streaming decode grid.
    check_error_word / check_num_pages: device address of an int32 and the
    pool's row count; the paged calls then validate their batch first and do
    nothing else when it fails (see ``checked``)."""
    _fields_ = [("prefill_split_chunks", C.c_int32), ("prefill_tile_waves", C.c_int32),
                ("decode_waves", C.c_int32), ("decode_stream_per_cu", C.c_int32),
                ("decode_stream_grid", C.c_int32), ("check_error_word", C.c_void_p),
                ("check_num_pages", C.c_int32)]


class Dims(C.Structure):
    _fields_ = [("num_qk_heads", C.c_int32), ("num_v_heads", C.c_int32),
                ("head_dim_k", C.c_int32), ("head_dim_v", C.c_int32), ("scale", C.c_float),
                ("state_dtype", C.c_int32), ("options", C.POINTER(Options))]


# element types of the state buffers (gdn_dims_t.state_dtype)
STATE_DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class _PrefillSlotsC(C.Structure):
    _fields_ = [("state_indices", C.c_void_p), ("output_state_indices", C.c_void_p),
                ("checkpoint_cu_starts", C.c_void_p), ("prefix_lens", C.c_void_p),
                ("chunk_starts", C.c_void_p)]


class _DecodeSlotsC(C.Structure):
    _fields_ = [("initial_state_indices", C.c_void_p), ("output_state_indices", C.c_void_p)]


class PrefillSlots(NamedTuple):
    """Per-sequence pool rows of a paged prefill batch, all [num_seqs] int32."""
    state_indices: torch.Tensor
    output_state_indices: torch.Tensor
    checkpoint_cu_starts: torch.Tensor
    prefix_lens: torch.Tensor
    chunk_starts: torch.Tensor


class DecodeSlots(NamedTuple):
    """Per-sequence pool rows of a paged decode batch, both [num_seqs] int32."""
    initial_state_indices: torch.Tensor
    output_state_indices: torch.Tensor


CHECK_BITS = {1: "GDN_CHECK_INDPTR", 2: "GDN_CHECK_LAST_PAGE_LEN", 4: "GDN_CHECK_TOKENS",
              8: "GDN_CHECK_PAGE_ID", 16: "GDN_CHECK_SHARED_ROW", 32: "GDN_CHECK_NOT_CHECKED"}


def checked(word: torch.Tensor, num_pages: int, **fields) -> Options:
    """Options that make the paged calls validate their batch into ``word`` (a [1]
    int32 device tensor, kept alive by the caller) against a pool of ``num_pages``
    rows; other fields as in ``Options``."""
    if word.dtype != torch.int32 or word.numel() < 1 or not word.is_cuda:
        raise ValueError("word must be an int32 device tensor")
    return Options(check_error_word=word.data_ptr(), check_num_pages=int(num_pages), **fields)


EXPORTS = ["gdn_check_paged", "gdn_prefill_slots", "gdn_decode_slots", "gdn_prefill_workspace_size",
           "gdn_prefill_paged", "gdn_prefill_paged_noalloc", "gdn_decode_paged", "gdn_prefill", "gdn_decode",
           "gdn_block_table_to_csr", "gdn_csr_to_block_table", "gdn_stream_copy", "gdn_last_error",
           "gdn_version"]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load the library (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m paged_recurrent_state_amd.build`")
    lib = C.CDLL(_LIB_PATH)
    P, I32, I64, SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "gdn_check_paged": (C.c_int, [P, P, P, P, I32, I32, I32, P, P]),
        "gdn_prefill_slots": (C.c_int, [P, P, P, P, I32, I32, C.POINTER(_PrefillSlotsC), P]),
        "gdn_decode_slots": (C.c_int, [P, P, P, I32, C.POINTER(_DecodeSlotsC), P]),
        "gdn_prefill_workspace_size": (SZ, [I64, I32, C.POINTER(Dims)]),
        "gdn_prefill_paged": (C.c_int, [C.POINTER(Dims), P, P, P, P, P, P, I32, I64, P, I64,
                                        P, P, P, I32, C.POINTER(_PrefillSlotsC), P, P, SZ, P]),
        "gdn_prefill_paged_noalloc": (C.c_int, [C.POINTER(Dims), P, P, P, P, P, P, I32, I64, P,
                                                I64, P, P, P, I32, C.POINTER(_PrefillSlotsC),
                                                P, P]),
        "gdn_decode_paged": (C.c_int, [C.POINTER(Dims), P, P, P, P, P, I32, P, I64, P, P, P,
                                       I32, C.POINTER(_DecodeSlotsC), P, P]),
        "gdn_prefill": (C.c_int, [C.POINTER(Dims), P, P, P, P, P, P, I32, I64, P, I64, P, P,
                                  I64, P, I32, P, I64, P, P, P, I32, I32, P, P, SZ, P]),
        "gdn_decode": (C.c_int, [C.POINTER(Dims), P, P, P, P, P, I32, P, I64, P, P, I64, P,
                                 I32, P, P]),
        "gdn_block_table_to_csr": (C.c_int, [P, I64, P, I32, I32, I32, P, P, P, P, P]),
        "gdn_csr_to_block_table": (C.c_int, [P, P, P, I32, I32, I32, P, I64, P, P, P]),
        "gdn_stream_copy": (C.c_int, [P, P, I64, P]),
        "gdn_last_error": (C.c_char_p, []),
        "gdn_version": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GDNError(rc, load().gdn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    if dev.type != "cuda":
        raise ValueError(f"the tensors are on {dev}: the library runs on the GPU only "
                         "(it has no CPU path)")
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, dev, contiguous=True):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _index_dtype(*ts):
    dts = {t.dtype for t in ts if t is not None}
    if not dts:
        return GDN_INDEX_INT32
    if len(dts) > 1:
        raise TypeError("slot index tensors must share one dtype (int32 or int64)")
    dt = dts.pop()
    if dt == torch.int32:
        return GDN_INDEX_INT32
    if dt == torch.int64:
        return GDN_INDEX_INT64
    raise TypeError("slot index tensors must be int32 or int64")


def _state_dtype(dev, *named):
    """The one element type (fp32 or bf16) of a call's state buffers."""
    types = set()
    for t, nm in named:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{nm} must be a tensor")
        if t.dtype not in STATE_DTYPES:
            raise TypeError(f"{nm} must be float32 or bfloat16, got {t.dtype}")
        _need(t, nm, t.dtype, dev, contiguous=False)
        types.add(t.dtype)
    if len(types) > 1:
        raise TypeError("all state buffers of a call must have one dtype")
    return STATE_DTYPES[types.pop()] if types else 0


def _pool_stride(pool: torch.Tensor, name: str, H: int, V: int, K: int) -> int:
    """Row stride (elements) of a [rows, H, V, K] pool whose rows are dense."""
    if pool.dim() != 4 or tuple(pool.shape[1:]) != (H, V, K):
        raise ValueError(f"{name} must be [rows, {H}, {V}, {K}], got {tuple(pool.shape)}")
    if pool.stride()[1:] != (V * K, K, 1):
        raise ValueError(f"every row of {name} must be one dense [H, V, K] block")
    return pool.stride(0) if pool.shape[0] > 1 else H * V * K


def _dims(q, v, scale, state_dtype: int = 0, options: Optional[Options] = None):
    Hqk, K = q.shape[-2], q.shape[-1]
    H, V = v.shape[-2], v.shape[-1]
    if options is not None and not isinstance(options, Options):
        raise TypeError("options must be a paged_recurrent_state_amd.Options")
    # the structure keeps `options` referenced for as long as it lives
    return Dims(Hqk, H, K, V, float(scale) if scale else 0.0, state_dtype,
                C.pointer(options) if options is not None else None)


def _token_checks(q, k, v, g, beta, dev, T):
    _need(q, "q", torch.bfloat16, dev)
    _need(k, "k", torch.bfloat16, dev)
    _need(v, "v", torch.bfloat16, dev)
    _need(g, "g", torch.float32, dev)
    _need(beta, "beta", torch.float32, dev)
    if q.shape != k.shape or q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k must be [T, Hqk, K] and v [T, H, V]")
    if q.shape[0] != T or v.shape[0] != T:
        raise ValueError("q, k, v must have the same number of tokens")
    for t, nm in ((g, "g"), (beta, "beta")):
        if t is not None and tuple(t.shape) != (T, v.shape[1]):
            raise ValueError(f"{nm} must be [T, H]")


def prefill_workspace_size(total_tokens: int, num_seqs: int, num_v_heads: int,
                           num_qk_heads: int, head_dim: int = 128,
                           options: Optional[Options] = None) -> int:
    d = Dims(num_qk_heads, num_v_heads, head_dim, head_dim, 0.0, 0,
             C.pointer(options) if options is not None else None)
    return int(load().gdn_prefill_workspace_size(int(total_tokens), int(num_seqs), C.byref(d)))


def _workspace(ws, nbytes, dev):
    if ws is None:
        # 256-byte aligned: torch's caching allocator returns 512-byte aligned blocks
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    return ws


def prefill_slots(cu_seqlens, page_indices, page_indptr, last_page_len, page_size: int,
                  out: Optional[PrefillSlots] = None) -> PrefillSlots:
    """Rows a paged prefill derives from its page table (one launch, no host sync)."""
    lib = load()
    dev = cu_seqlens.device
    for t, nm in ((cu_seqlens, "cu_seqlens"), (page_indices, "page_indices"),
                  (page_indptr, "page_indptr"), (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    B = last_page_len.shape[0]
    if out is None:
        buf = torch.empty(5, B, dtype=torch.int32, device=dev)
        out = PrefillSlots(*buf.unbind(0))
    sc = _PrefillSlotsC(*[t.data_ptr() for t in out])
    _check(lib.gdn_prefill_slots(_ptr(cu_seqlens), _ptr(page_indices), _ptr(page_indptr),
                                 _ptr(last_page_len), B, int(page_size), C.byref(sc),
                                 _stream(dev)))
    return out


def check_paged(page_indices, page_indptr, last_page_len, page_size: int, num_pages: int,
                cu_seqlens=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Validate a paged batch on the device (prefill when ``cu_seqlens`` is given,
    else decode); returns a [1] int32 device tensor with the GDN_CHECK_* bits
    found (0: none).  No host synchronization."""
    lib = load()
    dev = page_indptr.device
    for t, nm in ((page_indices, "page_indices"), (page_indptr, "page_indptr"),
                  (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    word = out if out is not None else torch.empty(1, dtype=torch.int32, device=dev)
    B = last_page_len.shape[0]
    idx = page_indices if page_indices.numel() else page_indptr
    _check(lib.gdn_check_paged(_ptr(cu_seqlens), _ptr(idx), _ptr(page_indptr),
                               _ptr(last_page_len), B, int(page_size), int(num_pages), _ptr(word),
                               _stream(dev)))
    return word


def stream_copy(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """Copy ``src`` into ``dst`` (contiguous device tensors of equal byte size,
    a multiple of 16) with the library's streaming copy kernel; returns dst."""
    lib = load()
    if not (dst.is_cuda and src.is_cuda and dst.device == src.device):
        raise ValueError("dst and src must be tensors on one GPU")
    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dst and src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("dst and src differ in size")
    _check(lib.gdn_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device)))
    return dst


def decode_slots(page_indices, page_indptr, last_page_len,
                 out: Optional[DecodeSlots] = None) -> DecodeSlots:
    """Rows a paged decode derives from its page table (one launch, no host sync)."""
    lib = load()
    dev = page_indptr.device
    for t, nm in ((page_indices, "page_indices"), (page_indptr, "page_indptr"),
                  (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    B = last_page_len.shape[0]
    if out is None:
        buf = torch.empty(2, B, dtype=torch.int32, device=dev)
        out = DecodeSlots(*buf.unbind(0))
    sc = _DecodeSlotsC(*[t.data_ptr() for t in out])
    _check(lib.gdn_decode_slots(_ptr(page_indices), _ptr(page_indptr), _ptr(last_page_len), B,
                                C.byref(sc), _stream(dev)))
    return out


def block_table_to_csr(block_tables, ctx_lens, page_size: int, bad_rows: Optional[torch.Tensor] = None):
    """Padded block table [B, max_blocks] int32 + ctx_lens [B] int32 -> (page_indptr,
    page_indices, last_page_len), all on the device (two launches, no host sync).

    ``page_indices`` is returned at its capacity, B * max_blocks entries; the
    first ``page_indptr[-1]`` are the pages.  ``bad_rows`` (a [1] int32 device
    tensor), when given, receives the number of rows the CSR form cannot hold.
    """
    lib = load()
    dev = block_tables.device
    if block_tables.dim() != 2 or block_tables.dtype != torch.int32 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be a [B, max_blocks] int32 tensor with unit column stride")
    _need(ctx_lens, "ctx_lens", torch.int32, dev)
    B, mb = block_tables.shape
    if ctx_lens.shape[0] != B:
        raise ValueError("ctx_lens must have one entry per block-table row")
    if bad_rows is not None:
        _need(bad_rows, "bad_rows", torch.int32, dev)
    indptr = torch.empty(B + 1, dtype=torch.int32, device=dev)
    indices = torch.empty(max(B * mb, 1), dtype=torch.int32, device=dev)
    lpl = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    # empty tensors have no storage: stand-ins that are never read
    table = block_tables if block_tables.numel() else indices
    ctx = ctx_lens if B else lpl
    _check(lib.gdn_block_table_to_csr(_ptr(table), max(block_tables.stride(0), mb), _ptr(ctx), B,
                                      mb, int(page_size), _ptr(indptr), _ptr(indices), _ptr(lpl),
                                      _ptr(bad_rows), _stream(dev)))
    lpl = lpl[:B]
    return indptr, indices, lpl


def csr_to_block_table(page_indptr, page_indices, last_page_len, page_size: int, max_blocks: int,
                       bad_rows: Optional[torch.Tensor] = None):
    """CSR page table -> (block_tables [B, max_blocks] int32 padded with 0, ctx_lens [B]
    int32), on the device (no host sync).  ``bad_rows`` as in block_table_to_csr."""
    lib = load()
    dev = page_indptr.device
    for t, nm in ((page_indices, "page_indices"), (page_indptr, "page_indptr"),
                  (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    if bad_rows is not None:
        _need(bad_rows, "bad_rows", torch.int32, dev)
    B = last_page_len.shape[0]
    mb = int(max_blocks)
    table = torch.empty(max(B, 1), max(mb, 1), dtype=torch.int32, device=dev)
    ctx = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    # empty tensors have no storage: stand-ins that are never read
    indices = page_indices if page_indices.numel() else ctx
    lpl = last_page_len if B else ctx
    _check(lib.gdn_csr_to_block_table(_ptr(page_indptr), _ptr(indices), _ptr(lpl), B,
                                      int(page_size), mb, _ptr(table), table.stride(0), _ptr(ctx),
                                      _ptr(bad_rows), _stream(dev)))
    return table[:B, :mb], ctx[:B]


def prefill_paged(q, k, v, g, beta, cu_seqlens, state_pool, page_indices, page_indptr,
                  page_size: int, last_page_len, slots: Optional[PrefillSlots] = None,
                  scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None,
                  options: Optional[Options] = None) -> torch.Tensor:
    """Chunked GDN prefill reading and writing a paged state pool; returns o [T, H, V] bf16."""
    lib = load()
    dev = q.device
    T = q.shape[0]
    _token_checks(q, k, v, g, beta, dev, T)
    for t, nm in ((cu_seqlens, "cu_seqlens"), (page_indices, "page_indices"),
                  (page_indptr, "page_indptr"), (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    d = _dims(q, v, scale, _state_dtype(dev, (state_pool, "state_pool")), options)
    stride = _pool_stride(state_pool, "state_pool", d.num_v_heads, d.head_dim_v, d.head_dim_k)
    B = last_page_len.shape[0]
    o = out if out is not None else torch.empty(T, d.num_v_heads, d.head_dim_v,
                                                dtype=torch.bfloat16, device=dev)
    ws = _workspace(workspace, lib.gdn_prefill_workspace_size(T, B, C.byref(d)), dev)
    sc = None
    if slots is not None:
        for t, nm in zip(slots, PrefillSlots._fields):
            _need(t, nm, torch.int32, dev)
        sc = C.byref(_PrefillSlotsC(*[t.data_ptr() for t in slots]))
    _check(lib.gdn_prefill_paged(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(cu_seqlens), B, T, _ptr(state_pool), stride,
                                 _ptr(page_indices), _ptr(page_indptr), _ptr(last_page_len),
                                 int(page_size), sc, _ptr(o), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(dev)))
    return o


def prefill_paged_noalloc(q, k, v, g, beta, cu_seqlens, state_pool, page_indices, page_indptr,
                          page_size: int, last_page_len, slots: Optional[PrefillSlots] = None,
                          scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                          options: Optional[Options] = None) -> torch.Tensor:
    """prefill_paged with the library's fixed per-device scratch as its workspace (no
    device allocation by the library; pass ``out`` for none at all).  Calls that
    overlap on one device race on that scratch."""
    lib = load()
    dev = q.device
    T = q.shape[0]
    _token_checks(q, k, v, g, beta, dev, T)
    for t, nm in ((cu_seqlens, "cu_seqlens"), (page_indices, "page_indices"),
                  (page_indptr, "page_indptr"), (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    d = _dims(q, v, scale, _state_dtype(dev, (state_pool, "state_pool")), options)
    stride = _pool_stride(state_pool, "state_pool", d.num_v_heads, d.head_dim_v, d.head_dim_k)
    B = last_page_len.shape[0]
    o = out if out is not None else torch.empty(T, d.num_v_heads, d.head_dim_v,
                                                dtype=torch.bfloat16, device=dev)
    sc = None
    if slots is not None:
        for t, nm in zip(slots, PrefillSlots._fields):
            _need(t, nm, torch.int32, dev)
        sc = C.byref(_PrefillSlotsC(*[t.data_ptr() for t in slots]))
    _check(lib.gdn_prefill_paged_noalloc(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(beta), _ptr(cu_seqlens), B, T, _ptr(state_pool),
                                         stride, _ptr(page_indices), _ptr(page_indptr),
                                         _ptr(last_page_len), int(page_size), sc, _ptr(o),
                                         _stream(dev)))
    return o


def decode_paged(q, k, v, g, beta, state_pool, page_indices, page_indptr, page_size: int,
                 last_page_len, slots: Optional[DecodeSlots] = None,
                 scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 options: Optional[Options] = None) -> torch.Tensor:
    """Single-token GDN decode on a paged pool; returns o [B, H, V] bf16."""
    lib = load()
    dev = q.device
    B = q.shape[0]
    _token_checks(q, k, v, g, beta, dev, B)
    for t, nm in ((page_indices, "page_indices"), (page_indptr, "page_indptr"),
                  (last_page_len, "last_page_len")):
        _need(t, nm, torch.int32, dev)
    d = _dims(q, v, scale, _state_dtype(dev, (state_pool, "state_pool")), options)
    stride = _pool_stride(state_pool, "state_pool", d.num_v_heads, d.head_dim_v, d.head_dim_k)
    o = out if out is not None else torch.empty(B, d.num_v_heads, d.head_dim_v,
                                                dtype=torch.bfloat16, device=dev)
    sc = None
    if slots is not None:
        for t, nm in zip(slots, DecodeSlots._fields):
            _need(t, nm, torch.int32, dev)
        sc = C.byref(_DecodeSlotsC(*[t.data_ptr() for t in slots]))
    _check(lib.gdn_decode_paged(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B,
                                _ptr(state_pool), stride, _ptr(page_indices),
                                _ptr(page_indptr), _ptr(last_page_len), int(page_size), sc,
                                _ptr(o), _stream(dev)))
    return o


def prefill(q, k, v, g, beta, cu_seqlens, *, initial_state=None, state_indices=None,
            output_state=None, output_state_indices=None, output_final_state: bool = False,
            state_checkpoints=None, checkpoint_state_indices=None, checkpoint_cu_starts=None,
            prefix_lens=None, checkpoint_every_n_tokens: int = 0,
            scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None,
            options: Optional[Options] = None) -> torch.Tensor:
    """Slot-argument chunked prefill (the general form the paged call wraps)."""
    lib = load()
    dev = q.device
    T = q.shape[0]
    _token_checks(q, k, v, g, beta, dev, T)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    idx = (state_indices, output_state_indices, checkpoint_state_indices,
           checkpoint_cu_starts, prefix_lens)
    idt = _index_dtype(*idx)
    for t, nm in zip(idx, ("state_indices", "output_state_indices",
                           "checkpoint_state_indices", "checkpoint_cu_starts", "prefix_lens")):
        if t is not None:
            _need(t, nm, t.dtype, dev)
    bufs = ((initial_state, "initial_state"), (output_state, "output_state"),
            (state_checkpoints, "state_checkpoints"))
    d = _dims(q, v, scale, _state_dtype(dev, *bufs), options)
    H, V, K = d.num_v_heads, d.head_dim_v, d.head_dim_k
    strides = []
    for t, nm in bufs:
        if t is not None:
            strides.append(_pool_stride(t, nm, H, V, K))
        else:
            strides.append(0)
    B = cu_seqlens.shape[0] - 1
    o = out if out is not None else torch.empty(T, H, V, dtype=torch.bfloat16, device=dev)
    ws = _workspace(workspace, lib.gdn_prefill_workspace_size(T, B, C.byref(d)), dev)
    _check(lib.gdn_prefill(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(cu_seqlens), B, T, _ptr(initial_state), strides[0],
                           _ptr(state_indices), _ptr(output_state), strides[1],
                           _ptr(output_state_indices), int(bool(output_final_state)),
                           _ptr(state_checkpoints), strides[2], _ptr(checkpoint_state_indices),
                           _ptr(checkpoint_cu_starts), _ptr(prefix_lens),
                           int(checkpoint_every_n_tokens), idt, _ptr(o), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(dev)))
    return o


def decode(q, k, v, g, beta, *, initial_state=None, initial_state_indices=None,
           output_state=None, output_state_indices=None, scale: Optional[float] = None,
           out: Optional[torch.Tensor] = None,
           options: Optional[Options] = None) -> torch.Tensor:
    """Single-token step with explicit rows; returns o [B, H, V] bf16."""
    lib = load()
    dev = q.device
    B = q.shape[0]
    _token_checks(q, k, v, g, beta, dev, B)
    idt = _index_dtype(initial_state_indices, output_state_indices)
    for t, nm in ((initial_state_indices, "initial_state_indices"),
                  (output_state_indices, "output_state_indices")):
        if t is not None:
            _need(t, nm, t.dtype, dev)
    d = _dims(q, v, scale, _state_dtype(dev, (initial_state, "initial_state"),
                                        (output_state, "output_state")), options)
    H, V, K = d.num_v_heads, d.head_dim_v, d.head_dim_k
    s_in = s_out = 0
    if initial_state is not None:
        s_in = _pool_stride(initial_state, "initial_state", H, V, K)
    if output_state is not None:
        s_out = _pool_stride(output_state, "output_state", H, V, K)
    o = out if out is not None else torch.empty(B, H, V, dtype=torch.bfloat16, device=dev)
    _check(lib.gdn_decode(C.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), B,
                          _ptr(initial_state), s_in, _ptr(initial_state_indices),
                          _ptr(output_state), s_out, _ptr(output_state_indices), idt, _ptr(o),
                          _stream(dev)))
    return o


def version() -> str:
    return load().gdn_version().decode()
