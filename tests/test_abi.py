"""The C-ABI library loads, exports every symbol include/*.h declares, and
rejects host-checkable bad arguments before any launch (CPU only: these calls
return before touching the HIP runtime)."""

import ctypes as C
import glob
import os
import re

import pytest

from paged_recurrent_state_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[\w\s\*]+?\b(gdn_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.lib_path()):
        pytest.fail("libgdn_paged.so is not built (run python -m paged_recurrent_state_amd.build)")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"gdn_prefill_paged", "gdn_decode_paged", "gdn_prefill_slots", "gdn_decode_slots",
            "gdn_prefill", "gdn_decode"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTS) == names


def test_version(lib):
    assert b"gfx950" in lib.gdn_version()


def dims(H=4, Hqk=2, K=128, V=128, scale=0.0, options=None):
    return _lib.Dims(Hqk, H, K, V, scale, 0, C.pointer(options) if options is not None else None)


def split_opt(m):
    return _lib.Options(prefill_split_chunks=m)


def test_workspace_size(lib):
    d = dims(options=split_opt(-1))  # whole-sequence recurrence
    a = lib.gdn_prefill_workspace_size(0, 1, C.byref(d))
    b = lib.gdn_prefill_workspace_size(64 * 100, 1, C.byref(d))
    c = lib.gdn_prefill_workspace_size(64 * 100, 300, C.byref(d))
    # rows + launch order per sequence, and one 11 KiB intra-chunk record per
    # (chunk slot, v-head) with at most T/64 + 2B + 1 chunk slots
    assert 0 < a < b < c
    assert a % 256 == 0 and b % 256 == 0
    # T record (5 fragments, hi and lo) + scalars per (slot, head), and a
    # 16-byte chunk-table entry per slot (regions rounded up to 256 bytes)
    al = lambda x: (x + 255) // 256 * 256
    assert b - a == 100 * 4 * (10240 + 1024) + al(103 * 16) - al(3 * 16)
    bad = dims(K=64)
    assert lib.gdn_prefill_workspace_size(64, 1, C.byref(bad)) == 0


def test_workspace_size_sequence_parallel(lib):
    """Splitting into segments of m chunks adds the records of both passes, the
    per-sequence scan records, up to 3 segment states per segment, with
    ceil(c / m) <= (T/64 + 2B + 1) / m + B segments in all, and one float per
    (chunk slot, v-head): the bound on each chunk's transition."""
    whole = lib.gdn_prefill_workspace_size(64 * 100, 1, C.byref(dims(options=split_opt(-1))))
    al = lambda x: (x + 255) // 256 * 256
    for m in (4, 7):
        segs = 103 // m + 1
        extra = al(2 * segs * 32) + al(segs * 32) + al(16) + 256 + 3 * segs * 4 * 128 * 128 * 4 \
            + al(103 * 4 * 4)
        d = dims(options=split_opt(m))
        assert lib.gdn_prefill_workspace_size(64 * 100, 1, C.byref(d)) - whole == extra
    # default (the device plans from the lengths): room for the segments of
    # ANY call of at most these sizes, min((T/64 + 2B' + 1)/4 + B', 512/H + B')
    # with B' = min(B, 256/H): min(26, 129) = 26 here
    for d in (dims(), dims(options=split_opt(0))):
        assert lib.gdn_prefill_workspace_size(64 * 100, 1, C.byref(d)) - whole == \
            al(52 * 32) + al(26 * 32) + al(16) + 256 + 78 * 4 * 128 * 128 * 4 + al(103 * 4 * 4)
    # 8 sequences x 32 heads fill 256 units once: min(1017/4 + 8, 16 + 8) = 24
    # segments; 9 sequences do not split themselves, but a smaller batch within
    # the same sizes may, so the room stays (with a 9-entry scan region)
    big0 = dims(H=32, Hqk=32, options=split_opt(-1))
    big = dims(H=32, Hqk=32)
    for B in (8, 9):
        w0 = lib.gdn_prefill_workspace_size(64 * 1000, B, C.byref(big0))
        assert lib.gdn_prefill_workspace_size(64 * 1000, B, C.byref(big)) - w0 == \
            al(48 * 32) + al(24 * 32) + al(B * 16) + 256 + 72 * 32 * 128 * 128 * 4 \
            + al((1000 + 2 * B + 1) * 32 * 4)
    # too few tokens for a 16-chunk sequence: no sequence-parallel room
    assert lib.gdn_prefill_workspace_size(1023, 1, C.byref(dims())) == \
        lib.gdn_prefill_workspace_size(1023, 1, C.byref(dims(options=split_opt(-1))))


@pytest.mark.parametrize("H", [1, 4, 32, 128])
@pytest.mark.parametrize("split", [0, 3])
def test_workspace_size_monotone(lib, H, split):
    """A workspace sized for (T, B) serves every call with fewer tokens or
    sequences: the size never drops as either grows (whether the batch may
    split depends on both)."""
    d = dims(H=H, Hqk=1, options=split_opt(split))
    size = lambda T, B: lib.gdn_prefill_workspace_size(T, B, C.byref(d))  # noqa: E731
    Ts = [0, 1, 63, 64, 65, 640, 1000, 1023, 1024, 4000, 8191, 8192, 30000, 70000, 200000]
    Bs = [1, 2, 3, 7, 8, 9, 16, 64, 65, 256, 257, 300]
    for B in Bs:
        sizes = [size(T, B) for T in Ts]
        assert sizes == sorted(sizes), (H, B, sizes)
    for T in Ts:
        sizes = [size(T, B) for B in Bs]
        assert sizes == sorted(sizes), (H, T, sizes)


@pytest.mark.parametrize("field,value", [("prefill_split_chunks", -2), ("prefill_tile_waves", 3),
                                         ("prefill_tile_waves", 16), ("decode_waves", 1),
                                         ("decode_waves", 32), ("decode_stream_per_cu", -2),
                                         ("decode_stream_grid", -1)])
def test_bad_options(lib, field, value):
    o = _lib.Options()
    setattr(o, field, value)
    d = dims(options=o)
    assert lib.gdn_prefill_workspace_size(64, 1, C.byref(d)) == 0
    assert _prefill_paged(lib, d) == -1
    assert b"options" in lib.gdn_last_error()


def _prefill_paged(lib, d, page_size=128, stride=4 * 128 * 128, ws=1 << 30, pool=1, cu=1,
                   B=1, T=64):
    fake = C.c_void_p(0x1000)  # never dereferenced: the call fails before launching
    return lib.gdn_prefill_paged(C.byref(d), fake, fake, fake, None, None,
                                 fake if cu else None, B, T, fake if pool else None, stride,
                                 fake, fake, fake, page_size, None, fake, fake, ws, None)


@pytest.mark.parametrize("ps", [0, -64, 100, 32])
def test_bad_page_size(lib, ps):
    assert _prefill_paged(lib, dims(), page_size=ps) == -1
    assert b"page_size" in lib.gdn_last_error()


def test_unsupported_head_dim(lib):
    assert _prefill_paged(lib, dims(K=64, V=64)) == -2
    assert _prefill_paged(lib, dims(H=3, Hqk=2)) == -2


def test_null_and_stride_errors(lib):
    assert _prefill_paged(lib, dims(), pool=0) == -1
    assert _prefill_paged(lib, dims(), cu=0) == -1
    assert _prefill_paged(lib, dims(), stride=100) == -1
    assert lib.gdn_prefill_paged(None, None, None, None, None, None, None, 0, 0, None, 0, None,
                                 None, None, 64, None, None, None, 0, None) == -1


def test_workspace_too_small(lib):
    assert _prefill_paged(lib, dims(), ws=1024) == -4
    assert b"workspace" in lib.gdn_last_error()


def test_general_prefill_companion_rules(lib):
    d = dims()
    f = C.c_void_p(0x1000)
    blk = 4 * 128 * 128

    def call(out_state=f, out_idx=None, final=1, ck_idx=None, ck_starts=f, prefix=f, N=64,
             ckpt=f, idx_dtype=0):
        return lib.gdn_prefill(C.byref(d), f, f, f, None, None, f, 1, 64, f, blk, f,
                               out_state, blk, out_idx, final, ckpt, blk, ck_idx, ck_starts,
                               prefix, N, idx_dtype, f, f, 1 << 30, None)

    # output_state_indices needs output_state and output_final_state
    assert call(out_state=None, out_idx=f) == -1
    assert call(out_idx=f, final=0) == -1
    # checkpoint rows need N > 0, prefix_lens, checkpoint_cu_starts, state_checkpoints
    assert call(ck_idx=f, N=0) == -1
    assert call(ck_idx=f, prefix=None) == -1
    assert call(ck_idx=f, ck_starts=None) == -1
    assert call(ck_idx=f, ckpt=None) == -1
    assert call(idx_dtype=7) == -1


def test_slot_calls_reject_bad_args(lib):
    f = C.c_void_p(0x1000)
    out = _lib._PrefillSlotsC(0x1000, 0x1000, 0x1000, 0x1000, None)
    assert lib.gdn_prefill_slots(f, f, f, f, 2, 64, C.byref(out), None) == -1
    out = _lib._PrefillSlotsC(0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert lib.gdn_prefill_slots(f, f, f, f, 2, 96, C.byref(out), None) == -1
    assert lib.gdn_prefill_slots(f, f, f, f, -1, 64, C.byref(out), None) == -1
    dout = _lib._DecodeSlotsC(0x1000, None)
    assert lib.gdn_decode_slots(f, f, f, 2, C.byref(dout), None) == -1


def test_empty_batches_are_no_ops(lib):
    # num_seqs == 0 returns GDN_OK without launching anything
    d = dims()
    assert lib.gdn_prefill_paged(C.byref(d), None, None, None, None, None, C.c_void_p(0x1000),
                                 0, 0, C.c_void_p(0x1000), 4 * 128 * 128, C.c_void_p(0x1000),
                                 C.c_void_p(0x1000), C.c_void_p(0x1000), 64, None, None, None,
                                 0, None) == 0
    assert lib.gdn_last_error() == b""


def test_table_conversions_reject_bad_args(lib):
    f = C.c_void_p(0x1000)
    # block table -> CSR: num_seqs < 0, page_size <= 0, max_blocks > row_stride, NULL outputs
    assert lib.gdn_block_table_to_csr(f, 8, f, -1, 4, 16, f, f, f, None, None) == -1
    assert lib.gdn_block_table_to_csr(f, 8, f, 2, 4, 0, f, f, f, None, None) == -1
    assert lib.gdn_block_table_to_csr(f, 3, f, 2, 4, 16, f, f, f, None, None) == -1
    assert lib.gdn_block_table_to_csr(f, 8, f, 2, -1, 16, f, f, f, None, None) == -1
    assert lib.gdn_block_table_to_csr(f, 8, f, 2, 4, 16, f, None, f, None, None) == -1
    assert b"NULL" in lib.gdn_last_error()
    # CSR -> block table: the same rules
    assert lib.gdn_csr_to_block_table(f, f, f, -1, 16, 4, f, 8, f, None, None) == -1
    assert lib.gdn_csr_to_block_table(f, f, f, 2, -16, 4, f, 8, f, None, None) == -1
    assert lib.gdn_csr_to_block_table(f, f, f, 2, 16, 9, f, 8, f, None, None) == -1
    assert lib.gdn_csr_to_block_table(f, f, None, 2, 16, 4, f, 8, f, None, None) == -1


def test_bad_state_dtype(lib):
    d = dims()
    d.state_dtype = 2
    assert _prefill_paged(lib, d) == -1
    assert b"state_dtype" in lib.gdn_last_error()


def test_check_rejects_bad_args(lib):
    fake = C.c_void_p(0x1000)  # never dereferenced: the call fails before launching
    chk = lambda B=1, ps=64, n=8, word=fake, idx=fake: lib.gdn_check_paged(  # noqa: E731
        None, idx, fake, fake, B, ps, n, word, None)
    assert chk(B=0) == -1
    assert chk(ps=100) == -1
    assert chk(n=0) == -1
    assert chk(word=None) == -1
    assert chk(idx=None) == -1
    # the paged calls' check option needs the pool's row count
    o = _lib.Options(check_error_word=0x1000, check_num_pages=0)
    assert _prefill_paged(lib, dims(options=o)) == -1
    assert b"check_num_pages" in lib.gdn_last_error()


def test_stream_copy_rejects_bad_arguments(lib):
    """Size, null, alignment and overlap are refused on the host; a zero-byte
    copy does nothing (no launch)."""
    EINVAL = -1
    buf = (C.c_uint8 * 4096)()
    base = C.addressof(buf) + (-C.addressof(buf)) % 16
    a, b = C.c_void_p(base), C.c_void_p(base + 1024)
    assert lib.gdn_stream_copy(a, b, 0, None) == 0
    assert lib.gdn_stream_copy(a, b, -16, None) == EINVAL
    assert lib.gdn_stream_copy(a, b, 24, None) == EINVAL
    assert lib.gdn_stream_copy(None, b, 32, None) == EINVAL
    assert lib.gdn_stream_copy(C.c_void_p(base + 8), b, 32, None) == EINVAL
    assert lib.gdn_stream_copy(a, C.c_void_p(base + 512), 1024, None) == EINVAL
    assert b"overlap" in lib.gdn_last_error()


def test_decode_calls_reject_bad_args(lib):
    d = dims()
    f = C.c_void_p(0x1000)  # never dereferenced: every call below fails before launching
    blk = 4 * 128 * 128

    def paged(B=2, pool=f, stride=blk, ps=128, q=f, o=f):
        return lib.gdn_decode_paged(C.byref(d), q, f, f, None, None, B, pool, stride, f, f, f,
                                    ps, None, o, None)

    assert paged(B=-1) == -1
    assert paged(pool=None) == -1
    assert paged(stride=blk - 1) == -1
    assert paged(ps=100) == -1
    assert paged(q=None) == -1
    assert paged(o=None) == -1
    assert paged(B=0) == 0  # an empty batch is a no-op

    def general(B=2, stride=blk, out_state=f, out_idx=f, idx_dtype=0, q=f):
        return lib.gdn_decode(C.byref(d), q, f, f, None, None, B, f, stride, f, out_state, blk,
                              out_idx, idx_dtype, f, None)

    assert general(B=-1) == -1
    assert general(idx_dtype=3) == -1
    assert general(stride=blk - 1) == -1
    assert general(out_state=None) == -1  # output_state_indices needs output_state
    assert general(q=None) == -1


def test_noalloc_refuses_calls_beyond_its_scratch(lib):
    """The fixed-scratch prefill refuses, before touching the device, a call
    whose workspace would exceed the 256 MiB scratch (here a million tokens on
    4 heads: ~690 MB of intra-chunk records)."""
    d = dims()
    f = C.c_void_p(0x1000)
    rc = lib.gdn_prefill_paged_noalloc(C.byref(d), f, f, f, None, None, f, 1, 1_000_000, f,
                                       4 * 128 * 128, f, f, f, 128, None, f, None)
    assert rc == -4
    assert b"fixed scratch" in lib.gdn_last_error()
