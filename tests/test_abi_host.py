"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects out-of-contract arguments before launching anything.

No GPU is touched: every call here fails validation (or is a pure host query),
so the pointers passed are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import sparse_attention_fp8_amd as dsa
from sparse_attention_fp8_amd.binding import _Batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, ERR_NULL, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE = 0, -1, -2, -3, -4
FAKE = 0x10000  # a 256-byte aligned non-NULL address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int32_t|size_t|int)\s+(dsa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def batch(**kw):
    f = dict(num_seqs=2, num_rows=3, max_seq_len=5000, max_q_len=2, bt_stride=79, num_pages=200,
             seq_lens=FAKE, query_start=FAKE, block_table=FAKE)
    f.update(kw)
    return _Batch(**f)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"dsa_indexer_logits_paged", "dsa_indexer_logits_prefill", "dsa_topk",
            "dsa_sparse_mla_decode", "dsa_indexer_q_quant_fp8", "dsa_indexer_k_quant_and_cache",
            "dsa_latent_cache_write", "dsa_sparse_mla_decode_fp8", "dsa_latent_cache_write_fp8"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.dsa_version()
    for st in (OK, ERR_NULL, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, -5):
        assert lib.dsa_status_string(st)
    assert lib.dsa_status_string(42) == b"unknown dsa_status"


def idx_call(lib, fn, b, **kw):
    a = dict(q=FAKE, w=FAKE, cache=FAKE, page_stride=8448, logits=FAKE, logits_stride=5000, clean=1)
    a.update(kw)
    f = getattr(lib, fn)
    bp = None if b is None else ctypes.byref(b)
    return f(bp, a["q"], a["w"], a["cache"], a["page_stride"], a["logits"], a["logits_stride"], a["clean"], None)


@pytest.mark.parametrize("fn", ["dsa_indexer_logits_paged", "dsa_indexer_logits_prefill"])
def test_indexer_argument_checks(lib, fn):
    assert idx_call(lib, fn, None) == ERR_NULL
    assert idx_call(lib, fn, batch(num_seqs=-1)) == ERR_UNSUPPORTED
    assert idx_call(lib, fn, batch(num_seqs=4097)) == ERR_UNSUPPORTED
    assert idx_call(lib, fn, batch(num_rows=-2)) == ERR_INVALID
    assert idx_call(lib, fn, batch(bt_stride=78)) == ERR_INVALID          # < ceil(5000/64) = 79
    assert idx_call(lib, fn, batch(seq_lens=None)) == ERR_NULL
    assert idx_call(lib, fn, batch(block_table=None)) == ERR_NULL
    assert idx_call(lib, fn, batch(), page_stride=8447) == ERR_INVALID
    assert idx_call(lib, fn, batch(), page_stride=8456) == ERR_INVALID     # not a multiple of 16
    assert idx_call(lib, fn, batch(), logits_stride=4999) == ERR_INVALID   # < max_seq_len
    assert idx_call(lib, fn, batch(), logits_stride=5002) == ERR_INVALID   # not a multiple of 4
    assert idx_call(lib, fn, batch(), clean=2) == ERR_INVALID
    assert idx_call(lib, fn, batch(), q=None) == ERR_NULL
    assert idx_call(lib, fn, batch(), logits=FAKE + 4) == ERR_INVALID      # misaligned
    assert idx_call(lib, fn, batch(), cache=None) == ERR_NULL
    idx_call(lib, fn, batch(), page_stride=100)
    assert b"idx_page_stride" in lib.dsa_last_error_message()
    # nothing to do is a success that launches nothing
    assert idx_call(lib, fn, batch(num_rows=0)) == OK


def topk_call(lib, b, k=2048, ws=FAKE, ws_bytes=1 << 40, **kw):
    a = dict(logits=FAKE, stride=5000, indices=FAKE)
    a.update(kw)
    return lib.dsa_topk(None if b is None else ctypes.byref(b), a["logits"], a["stride"], k, a["indices"],
                        ws, ws_bytes, None)


def test_topk_argument_checks(lib):
    assert topk_call(lib, None) == ERR_NULL
    assert topk_call(lib, batch(), k=0) == ERR_UNSUPPORTED
    assert topk_call(lib, batch(), k=2049) == ERR_UNSUPPORTED
    assert topk_call(lib, batch(), stride=4000) == ERR_INVALID
    assert topk_call(lib, batch(), logits=None) == ERR_NULL
    assert topk_call(lib, batch(), indices=None) == ERR_NULL
    assert topk_call(lib, batch(), logits=FAKE + 8) == ERR_INVALID
    long = batch(max_seq_len=131072, bt_stride=2048)
    need = lib.dsa_topk_workspace_bytes(ctypes.byref(long), 2048)
    assert need > 0
    assert topk_call(lib, long, stride=131072, ws=None) == ERR_WORKSPACE
    assert topk_call(lib, long, stride=131072, ws_bytes=need - 1) == ERR_WORKSPACE
    assert topk_call(lib, long, stride=131072, ws=FAKE + 16) == ERR_INVALID
    assert b"workspace" in lib.dsa_last_error_message()


def test_topk_workspace_sizes(lib):
    # rows of up to 65536 keys are selected by one workgroup: no workspace
    assert lib.dsa_topk_workspace_bytes(ctypes.byref(batch(max_seq_len=32768, bt_stride=512)), 2048) == 0
    assert lib.dsa_topk_workspace_bytes(ctypes.byref(batch(max_seq_len=65536, bt_stride=1024)), 2048) == 0
    b = batch(max_seq_len=65537, bt_stride=1025, num_rows=4096)
    need = lib.dsa_topk_workspace_bytes(ctypes.byref(b), 2048)
    assert need >= 4096 * 3 * 2048 * 8 and need % 256 == 0      # longer: three 32768-key chunks per row
    assert lib.dsa_topk_workspace_bytes(None, 2048) == 0
    # past four chunks the merge adds a level: groups of four chunks keep k each
    one_m = batch(max_seq_len=1 << 20, bt_stride=1 << 14, num_rows=2)
    need = lib.dsa_topk_workspace_bytes(ctypes.byref(one_m), 2048)
    assert need >= 2 * 32 * 2048 * 8 + 2 * 8 * 2048 * 8 and need % 256 == 0


def test_topk_longest_row(lib):
    ok_len, too_long = 4 * 1024 * 1024, 4 * 1024 * 1024 + 1
    b = batch(max_seq_len=ok_len, bt_stride=ok_len // 64)
    assert lib.dsa_topk_workspace_bytes(ctypes.byref(b), 2048) > 0
    assert topk_call(lib, batch(max_seq_len=too_long, bt_stride=too_long // 64 + 1), stride=too_long + 3) \
        == ERR_UNSUPPORTED
    assert b"max_seq_len" in lib.dsa_last_error_message()


def mla_call(lib, b, H=16, k=2048, splits=0, ws=FAKE, ws_bytes=1 << 40, **kw):
    a = dict(q=FAKE, kv=FAKE, kv_stride=64 * 576, indices=FAKE, scale=0.07, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.dsa_sparse_mla_decode(None if b is None else ctypes.byref(b), a["q"], H, a["kv"], a["kv_stride"],
                                     a["indices"], k, a["scale"], splits, a["out"], a["lse"], ws, ws_bytes, None)


def test_sparse_mla_argument_checks(lib):
    assert mla_call(lib, None) == ERR_NULL
    for H in (0, 8, 24, 100, 1040, -16):
        assert mla_call(lib, batch(), H=H) == ERR_UNSUPPORTED, H
    # every multiple of 16 up to 128 (one GPU's share of the heads) is accepted;
    # with no rows nothing is launched
    for H in range(16, 129, 16):
        assert mla_call(lib, batch(num_rows=0), H=H) == OK, H
        assert lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(batch(num_rows=1)), H, 2048, 0) > 0, H
    assert mla_call(lib, batch(), k=0) == ERR_UNSUPPORTED
    assert mla_call(lib, batch(), k=4096) == ERR_UNSUPPORTED
    assert mla_call(lib, batch(), kv_stride=64 * 576 - 8) == ERR_INVALID
    assert mla_call(lib, batch(), kv_stride=64 * 576 + 4) == ERR_INVALID
    assert mla_call(lib, batch(), scale=float("inf")) == ERR_INVALID
    assert mla_call(lib, batch(), splits=-1) == ERR_INVALID
    assert mla_call(lib, batch(), out=None) == ERR_NULL
    assert mla_call(lib, batch(), lse=None) == ERR_NULL
    assert mla_call(lib, batch(), q=FAKE + 2) == ERR_INVALID
    assert mla_call(lib, batch(), kv=None) == ERR_NULL
    b = batch(num_rows=1)
    need = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(b), 16, 2048, 0)
    assert need > 0
    assert mla_call(lib, b, ws=None) == ERR_WORKSPACE
    assert mla_call(lib, b, ws_bytes=need - 1) == ERR_WORKSPACE


def test_sparse_mla_noalloc_argument_checks(lib):
    """The no-allocation variant takes the same checks; a forced split count
    whose partials exceed its 32 MiB device array is rejected before any
    device call (so this runs without a GPU)."""
    f = lib.dsa_sparse_mla_decode_noalloc

    def call(b, H=16, splits=0, **kw):
        a = dict(q=FAKE, kv=FAKE, kv_stride=64 * 576, indices=FAKE, scale=0.07, out=FAKE, lse=FAKE)
        a.update(kw)
        return f(None if b is None else ctypes.byref(b), a["q"], H, a["kv"], a["kv_stride"], a["indices"], 2048,
                 a["scale"], splits, a["out"], a["lse"], None)
    assert call(None) == ERR_NULL
    assert call(batch(), H=24) == ERR_UNSUPPORTED
    assert call(batch(), kv_stride=64 * 576 + 4) == ERR_INVALID
    assert call(batch(), lse=None) == ERR_NULL
    assert call(batch(num_rows=0)) == OK
    # 32 splits x 4096 rows x 128 heads of partials: far above 32 MiB
    big = batch(num_rows=4096, max_seq_len=65536, bt_stride=1024)
    assert call(big, H=128, splits=32) == ERR_UNSUPPORTED
    msg = lib.dsa_last_error_message()
    assert b"scratch" in msg and b"33554432" in msg


def test_split_heuristic_and_workspace(lib):
    def splits(R, L, H):
        return lib.dsa_sparse_mla_pick_splits(ctypes.byref(batch(num_rows=R, max_seq_len=L, bt_stride=(L + 63) // 64)), H, 2048)
    assert splits(1, 131072, 16) >= 16          # single long row: many splits
    assert splits(1, 4096, 16) >= 16
    assert splits(4096, 65536, 16) == 1         # prefill-sized batch: single pass
    assert splits(1, 100, 16) == 2              # never more splits than tiles holding keys
    assert 1 <= splits(128, 65536, 128) <= 4
    # a last 64-head block of H % 64 heads counts as a block of its own
    assert splits(1, 4096, 112) == splits(1, 4096, 128) and splits(1, 4096, 80) == splits(1, 4096, 128)
    # one split needs no workspace
    b = batch(num_rows=4096, max_seq_len=65536, bt_stride=1024)
    assert lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(b), 16, 2048, 1) == 0
    b = batch(num_rows=2, max_seq_len=5000, bt_stride=79)
    ws = lib.dsa_sparse_mla_workspace_bytes(ctypes.byref(b), 32, 2048, 4)
    assert ws >= 4 * 2 * 32 * (512 * 4 + 8)


def test_binding_rejects_host_tensors():
    import torch
    b = dsa.Batch(seq_lens=torch.zeros(1, dtype=torch.int32), query_start=torch.zeros(2, dtype=torch.int32),
                  block_table=torch.zeros(1, 1, dtype=torch.int32), num_rows=0, max_seq_len=0, max_q_len=0,
                  num_pages=1)
    with pytest.raises(ValueError):
        b.c_struct()


# --------------------------------------------------------------------------
# quantiser and cache writers

def test_q_quant_rejects_bad_arguments(lib):
    f = lib.dsa_indexer_q_quant_fp8
    assert f(0, None, None, None, None, None) == OK                  # nothing to do
    assert f(-1, FAKE, FAKE, FAKE, FAKE, None) == ERR_UNSUPPORTED
    assert f((1 << 24) + 1, FAKE, FAKE, FAKE, FAKE, None) == ERR_UNSUPPORTED
    assert f(4, FAKE, None, FAKE, FAKE, None) == ERR_NULL
    assert f(4, FAKE + 8, FAKE, FAKE, FAKE, None) == ERR_INVALID      # q not 16-byte aligned
    assert b"q must be 16-byte aligned" in lib.dsa_last_error_message()
    assert f(4, FAKE, FAKE, FAKE + 4, FAKE, None) == ERR_INVALID      # codes not 8-byte aligned
    assert f(4, FAKE, FAKE + 2, FAKE, FAKE, None) == ERR_INVALID


def k_write(lib, **kw):
    a = dict(T=10, k=FAKE, k_stride=128, slots=FAKE, cache=FAKE, stride=8448, pages=4)
    a.update(kw)
    return lib.dsa_indexer_k_quant_and_cache(a["T"], a["k"], a["k_stride"], a["slots"], a["cache"], a["stride"],
                                             a["pages"], None)


def test_k_writer_rejects_bad_arguments(lib):
    assert k_write(lib, T=0, k=None, slots=None, cache=None) == OK
    assert k_write(lib, pages=0, cache=None) == OK                    # no page to write
    assert k_write(lib, T=-3) == ERR_UNSUPPORTED
    assert k_write(lib, pages=-1) == ERR_INVALID
    assert k_write(lib, k_stride=120) == ERR_INVALID
    assert k_write(lib, k_stride=132) == ERR_INVALID                  # not a multiple of 8
    assert k_write(lib, stride=8440) == ERR_INVALID
    assert b"idx_page_stride" in lib.dsa_last_error_message()
    assert k_write(lib, stride=8456) == ERR_INVALID                   # not a multiple of 16
    assert k_write(lib, slots=None) == ERR_NULL
    assert k_write(lib, k=FAKE + 8) == ERR_INVALID
    assert k_write(lib, slots=FAKE + 4) == ERR_INVALID


def latent_write(lib, **kw):
    a = dict(T=10, lat=FAKE, lat_stride=512, rope=FAKE, rope_stride=64, slots=FAKE, cache=FAKE, stride=36864,
             pages=4)
    a.update(kw)
    return lib.dsa_latent_cache_write(a["T"], a["lat"], a["lat_stride"], a["rope"], a["rope_stride"], a["slots"],
                                      a["cache"], a["stride"], a["pages"], None)


def test_latent_writer_rejects_bad_arguments(lib):
    assert latent_write(lib, T=0, lat=None, rope=None, slots=None, cache=None) == OK
    assert latent_write(lib, T=(1 << 24) + 1) == ERR_UNSUPPORTED
    assert latent_write(lib, lat_stride=504) == ERR_INVALID
    assert latent_write(lib, rope_stride=60) == ERR_INVALID
    assert latent_write(lib, stride=36864 - 8) == ERR_INVALID
    assert b"kv_page_stride" in lib.dsa_last_error_message()
    assert latent_write(lib, rope=None) == ERR_NULL
    assert latent_write(lib, cache=FAKE + 8) == ERR_INVALID


def test_fp8_latent_entries_reject_bad_arguments(lib):
    b = batch()
    f = lib.dsa_sparse_mla_decode_fp8
    args = lambda **kw: dict(dict(q=FAKE, H=16, kv=FAKE, stride=41984, idx=FAKE, k=2048, sc=0.07, sp=1,
                                  out=FAKE, lse=FAKE, ws=None, wsb=0), **kw)
    call = lambda a: f(ctypes.byref(b), a["q"], a["H"], a["kv"], a["stride"], a["idx"], a["k"], a["sc"], a["sp"],
                       a["out"], a["lse"], a["ws"], a["wsb"], None)
    assert call(args(stride=41968)) == ERR_INVALID
    assert b"kv_page_stride_bytes" in lib.dsa_last_error_message()
    assert call(args(stride=41984 + 8)) == ERR_INVALID
    assert call(args(H=24)) == ERR_UNSUPPORTED
    assert call(args(kv=None)) == ERR_NULL
    assert call(args(kv=FAKE + 8)) == ERR_INVALID
    assert call(args(sp=4)) == ERR_WORKSPACE                   # split partials need a workspace
    w = lib.dsa_latent_cache_write_fp8
    assert w(0, None, 512, None, 64, None, None, 41984, 4, None) == OK
    assert w(10, FAKE, 512, FAKE, 64, FAKE, FAKE, 8448, 4, None) == ERR_INVALID
    assert w(10, FAKE, 500, FAKE, 64, FAKE, FAKE, 41984, 4, None) == ERR_INVALID
    assert w(10, FAKE, 512, None, 64, FAKE, FAKE, 41984, 4, None) == ERR_NULL
    assert w(-1, FAKE, 512, FAKE, 64, FAKE, FAKE, 41984, 4, None) == ERR_UNSUPPORTED
