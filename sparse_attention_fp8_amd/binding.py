"""ctypes binding of libdsa (include/dsa.h).

Argument marshalling only: shape, dtype and device checks on the torch
tensors, then a call into the C ABI with raw device pointers and the current
HIP stream.  Every step of the computation runs in libdsa's HIP kernels; there
is no Python or CPU fallback, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

DSA_OK = 0
PAGE = 64
IDX_HEADS = 64
IDX_DIM = 128
IDX_PAGE_BYTES = 8448
KV_DIM = 576
V_DIM = 512
MAX_TOPK = 2048
KV8_PAGE_BYTES = 41984    # fp8 latent page: 64 x (512 e4m3 + 64 bf16) rows, then 64 x 4 fp32 scales


class DSAError(RuntimeError):
    """A non-OK status from libdsa (the message carries the library's detail)."""

    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed with status {status}: {detail}")
        self.status = status


class _Batch(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32), ("bt_stride", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p), ("query_start", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
    ]


def library_path() -> str:
    return os.environ.get("LIBDSA_PATH", os.path.join(_HERE, "libdsa.so"))


def load():
    """Load libdsa.so (built in-tree by ``__graft_entry__.build()``); raises if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"libdsa not built: {path} is missing (run `python __graft_entry__.py build` "
                          f"or `python -m sparse_attention_fp8_amd.build`)")
    lib = ctypes.CDLL(path)
    B = ctypes.POINTER(_Batch)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dsa_indexer_logits_paged": (ctypes.c_int, [B, vp, vp, vp, i64, vp, i64, ctypes.c_int, vp]),
        "dsa_indexer_logits_prefill": (ctypes.c_int, [B, vp, vp, vp, i64, vp, i64, ctypes.c_int, vp]),
        "dsa_topk": (ctypes.c_int, [B, vp, i64, i32, vp, vp, sz, vp]),
        "dsa_sparse_mla_decode": (ctypes.c_int, [B, vp, i32, vp, i64, vp, i32, f32, i32, vp, vp, vp, sz, vp]),
        "dsa_sparse_mla_decode_fp8": (ctypes.c_int, [B, vp, i32, vp, i64, vp, i32, f32, i32, vp, vp, vp, sz, vp]),
        "dsa_sparse_mla_decode_noalloc": (ctypes.c_int, [B, vp, i32, vp, i64, vp, i32, f32, i32, vp, vp, vp]),
        "dsa_latent_cache_write_fp8": (ctypes.c_int, [i32, vp, i64, vp, i64, vp, vp, i64, i32, vp]),
        "dsa_indexer_q_quant_fp8": (ctypes.c_int, [i32, vp, vp, vp, vp, vp]),
        "dsa_indexer_k_quant_and_cache": (ctypes.c_int, [i32, vp, i64, vp, vp, i64, i32, vp]),
        "dsa_latent_cache_write": (ctypes.c_int, [i32, vp, i64, vp, i64, vp, vp, i64, i32, vp]),
        "dsa_topk_workspace_bytes": (sz, [B, i32]),
        "dsa_sparse_mla_workspace_bytes": (sz, [B, i32, i32, i32]),
        "dsa_sparse_mla_pick_splits": (i32, [B, i32, i32]),
        "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "dsa_last_error_message": (ctypes.c_char_p, []),
        "dsa_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int, func: str):
    if status != DSA_OK:
        lib = load()
        raise DSAError(status, func, lib.dsa_last_error_message().decode() or lib.dsa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None:
        for i, (got, want) in enumerate(zip(t.shape, shape)):
            if want is not None and got != want:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
        if len(t.shape) != len(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def _need_rows(t: torch.Tensor, name: str, dtype, rows: int, min_cols: int, device=None):
    """A 2-D tensor whose rows may be strided (a slice of a wider buffer) but
    whose elements inside a row are contiguous."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < min_cols:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected ({rows}, >= {min_cols})")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride inside a row")


@dataclass
class Batch:
    """Device-side batch description plus its host hints (dsa_batch_t)."""
    seq_lens: torch.Tensor      # [B] int32
    query_start: torch.Tensor   # [B+1] int32
    block_table: torch.Tensor   # [B, bt_stride] int32
    num_rows: int
    max_seq_len: int
    max_q_len: int
    num_pages: int

    @classmethod
    def from_host(cls, seq_lens, query_start, block_table, num_pages, device="cuda"):
        """Build from host tensors, computing the host hints from them."""
        seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32)
        query_start = torch.as_tensor(query_start, dtype=torch.int32)
        block_table = torch.as_tensor(block_table, dtype=torch.int32)
        q = query_start[1:] - query_start[:-1]
        return cls(seq_lens=seq_lens.to(device).contiguous(), query_start=query_start.to(device).contiguous(),
                   block_table=block_table.to(device).contiguous(), num_rows=int(query_start[-1]),
                   max_seq_len=int(seq_lens.max()) if seq_lens.numel() else 0,
                   max_q_len=int(q.max()) if q.numel() else 0, num_pages=int(num_pages))

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def device(self):
        return self.seq_lens.device

    def c_struct(self) -> _Batch:
        _need(self.seq_lens, "seq_lens", torch.int32, (None,))
        _need(self.query_start, "query_start", torch.int32, (self.num_seqs + 1,), self.device)
        _need(self.block_table, "block_table", torch.int32, (self.num_seqs, None), self.device)
        return _Batch(self.num_seqs, self.num_rows, self.max_seq_len, self.max_q_len,
                      int(self.block_table.shape[1]), self.num_pages,
                      _ptr(self.seq_lens), _ptr(self.query_start), _ptr(self.block_table))


def _indexer(fn_name, batch: Batch, q_fp8, weights, idx_cache, logits, clean_logits=True):
    lib = load()
    dev = batch.device
    R = batch.num_rows
    _need(q_fp8, "q_fp8", torch.uint8, (R, IDX_HEADS, IDX_DIM), dev)
    _need(weights, "weights", torch.float32, (R, IDX_HEADS), dev)
    _need(idx_cache, "idx_cache", torch.uint8, (batch.num_pages, None), dev)
    _need(logits, "logits", torch.float32, (R, None), dev)
    st = getattr(lib, fn_name)(ctypes.byref(batch.c_struct()), _ptr(q_fp8), _ptr(weights), _ptr(idx_cache),
                               int(idx_cache.shape[1]), _ptr(logits), int(logits.shape[1]),
                               1 if clean_logits else 0, _stream(dev))
    _check(st, fn_name)
    return logits


def indexer_logits_paged(batch, q_fp8, weights, idx_cache, logits, clean_logits=True):
    """dsa_indexer_logits_paged into ``logits`` [R, stride] (returned)."""
    return _indexer("dsa_indexer_logits_paged", batch, q_fp8, weights, idx_cache, logits, clean_logits)


def indexer_logits_prefill(batch, q_fp8, weights, idx_cache, logits, clean_logits=True):
    """dsa_indexer_logits_prefill into ``logits`` [R, stride] (returned)."""
    return _indexer("dsa_indexer_logits_prefill", batch, q_fp8, weights, idx_cache, logits, clean_logits)


def topk_workspace_bytes(batch: Batch, k: int = MAX_TOPK) -> int:
    return int(load().dsa_topk_workspace_bytes(ctypes.byref(batch.c_struct()), int(k)))


def topk(batch: Batch, logits, indices, k: int = MAX_TOPK, workspace=None):
    """dsa_topk into ``indices`` [R, k] int32 (returned)."""
    lib = load()
    dev = batch.device
    R = batch.num_rows
    _need(logits, "logits", torch.float32, (R, None), dev)
    _need(indices, "indices", torch.int32, (R, k), dev)
    need = topk_workspace_bytes(batch, k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.dsa_topk(ctypes.byref(batch.c_struct()), _ptr(logits), int(logits.shape[1]), int(k), _ptr(indices),
                      _ptr(workspace), wbytes, _stream(dev))
    _check(st, "dsa_topk")
    return indices


def sparse_mla_workspace_bytes(batch: Batch, num_heads: int, k: int = MAX_TOPK, num_splits: int = 0) -> int:
    return int(load().dsa_sparse_mla_workspace_bytes(ctypes.byref(batch.c_struct()), int(num_heads), int(k),
                                                     int(num_splits)))


def sparse_mla_pick_splits(batch: Batch, num_heads: int, k: int = MAX_TOPK) -> int:
    return int(load().dsa_sparse_mla_pick_splits(ctypes.byref(batch.c_struct()), int(num_heads), int(k)))


def sparse_mla_decode(batch: Batch, q, kv_cache, indices, softmax_scale, out, lse, num_splits=0, workspace=None):
    """dsa_sparse_mla_decode into ``out`` [R, H, 512] bf16 and ``lse`` [R, H] fp32 (returned)."""
    lib = load()
    dev = batch.device
    R = batch.num_rows
    _need(q, "q", torch.bfloat16, (R, None, KV_DIM), dev)
    H = int(q.shape[1])
    _need(kv_cache, "kv_cache", torch.bfloat16, (batch.num_pages, None), dev)
    _need(indices, "indices", torch.int32, (R, None), dev)
    k = int(indices.shape[1])
    _need(out, "out", torch.bfloat16, (R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (R, H), dev)
    need = sparse_mla_workspace_bytes(batch, H, k, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.dsa_sparse_mla_decode(ctypes.byref(batch.c_struct()), _ptr(q), H, _ptr(kv_cache),
                                   int(kv_cache.shape[1]), _ptr(indices), k, float(softmax_scale),
                                   int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(dev))
    _check(st, "dsa_sparse_mla_decode")
    return out, lse


NOALLOC_SCRATCH_BYTES = 32 << 20   # the library's device array behind sparse_mla_decode_noalloc


def sparse_mla_decode_noalloc(batch: Batch, q, kv_cache, indices, softmax_scale, out, lse, num_splits=0):
    """dsa_sparse_mla_decode_noalloc: dsa_sparse_mla_decode with the split
    partials in the library's own device array (nothing is allocated, here or
    in the library).  Calls that overlap in time on one device race."""
    lib = load()
    dev = batch.device
    R = batch.num_rows
    _need(q, "q", torch.bfloat16, (R, None, KV_DIM), dev)
    H = int(q.shape[1])
    _need(kv_cache, "kv_cache", torch.bfloat16, (batch.num_pages, None), dev)
    _need(indices, "indices", torch.int32, (R, None), dev)
    k = int(indices.shape[1])
    _need(out, "out", torch.bfloat16, (R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (R, H), dev)
    st = lib.dsa_sparse_mla_decode_noalloc(ctypes.byref(batch.c_struct()), _ptr(q), H, _ptr(kv_cache),
                                           int(kv_cache.shape[1]), _ptr(indices), k, float(softmax_scale),
                                           int(num_splits), _ptr(out), _ptr(lse), _stream(dev))
    _check(st, "dsa_sparse_mla_decode_noalloc")
    return out, lse


def indexer_q_quant_fp8(q, weights, q_fp8=None, weights_out=None):
    """dsa_indexer_q_quant_fp8: q [R, 64, 128] bf16 and weights [R, 64] fp32 ->
    (q_fp8 [R, 64, 128] uint8 e4m3fn codes, weights_out [R, 64] fp32 with the
    per-(row, head) scale folded in).  ``weights_out`` may be ``weights``."""
    lib = load()
    dev = q.device
    R = int(q.shape[0])
    _need(q, "q", torch.bfloat16, (R, IDX_HEADS, IDX_DIM), dev)
    _need(weights, "weights", torch.float32, (R, IDX_HEADS), dev)
    if q_fp8 is None:
        q_fp8 = torch.empty(R, IDX_HEADS, IDX_DIM, dtype=torch.uint8, device=dev)
    if weights_out is None:
        weights_out = torch.empty(R, IDX_HEADS, dtype=torch.float32, device=dev)
    _need(q_fp8, "q_fp8", torch.uint8, (R, IDX_HEADS, IDX_DIM), dev)
    _need(weights_out, "weights_out", torch.float32, (R, IDX_HEADS), dev)
    st = lib.dsa_indexer_q_quant_fp8(R, _ptr(q), _ptr(weights), _ptr(q_fp8), _ptr(weights_out), _stream(dev))
    _check(st, "dsa_indexer_q_quant_fp8")
    return q_fp8, weights_out


def indexer_k_quant_and_cache(k, slot_mapping, idx_cache):
    """dsa_indexer_k_quant_and_cache: quantise k [T, >=128] bf16 (rows may be
    strided) and write it into idx_cache [num_pages, page_stride] uint8 at the
    slots of slot_mapping [T] int64.  Returns idx_cache."""
    lib = load()
    dev = k.device
    T = int(k.shape[0])
    _need_rows(k, "k", torch.bfloat16, T, IDX_DIM, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    _need(idx_cache, "idx_cache", torch.uint8, (None, None), dev)
    st = lib.dsa_indexer_k_quant_and_cache(T, _ptr(k), int(k.stride(0)), _ptr(slot_mapping), _ptr(idx_cache),
                                           int(idx_cache.shape[1]), int(idx_cache.shape[0]), _stream(dev))
    _check(st, "dsa_indexer_k_quant_and_cache")
    return idx_cache


def latent_cache_write(latent, rope, slot_mapping, kv_cache):
    """dsa_latent_cache_write: latent [T, >=512] and rope [T, >=64] bf16 (rows
    may be strided) into kv_cache [num_pages, page_stride] bf16 at the slots of
    slot_mapping [T] int64.  Returns kv_cache."""
    lib = load()
    dev = latent.device
    T = int(latent.shape[0])
    _need_rows(latent, "latent", torch.bfloat16, T, V_DIM, dev)
    _need_rows(rope, "rope", torch.bfloat16, T, KV_DIM - V_DIM, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    _need(kv_cache, "kv_cache", torch.bfloat16, (None, None), dev)
    st = lib.dsa_latent_cache_write(T, _ptr(latent), int(latent.stride(0)), _ptr(rope), int(rope.stride(0)),
                                    _ptr(slot_mapping), _ptr(kv_cache), int(kv_cache.shape[1]),
                                    int(kv_cache.shape[0]), _stream(dev))
    _check(st, "dsa_latent_cache_write")
    return kv_cache


def sparse_mla_decode_fp8(batch: Batch, q, kv_cache_fp8, indices, softmax_scale, out, lse, num_splits=0,
                          workspace=None):
    """dsa_sparse_mla_decode_fp8 over an fp8 latent cache [num_pages, page_stride_bytes] uint8 into ``out``
    [R, H, 512] bf16 and ``lse`` [R, H] fp32 (returned)."""
    lib = load()
    dev = batch.device
    R = batch.num_rows
    _need(q, "q", torch.bfloat16, (R, None, KV_DIM), dev)
    H = int(q.shape[1])
    _need(kv_cache_fp8, "kv_cache_fp8", torch.uint8, (batch.num_pages, None), dev)
    _need(indices, "indices", torch.int32, (R, None), dev)
    k = int(indices.shape[1])
    _need(out, "out", torch.bfloat16, (R, H, V_DIM), dev)
    _need(lse, "lse", torch.float32, (R, H), dev)
    need = sparse_mla_workspace_bytes(batch, H, k, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.dsa_sparse_mla_decode_fp8(ctypes.byref(batch.c_struct()), _ptr(q), H, _ptr(kv_cache_fp8),
                                       int(kv_cache_fp8.shape[1]), _ptr(indices), k, float(softmax_scale),
                                       int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), wbytes, _stream(dev))
    _check(st, "dsa_sparse_mla_decode_fp8")
    return out, lse


def latent_cache_write_fp8(latent, rope, slot_mapping, kv_cache_fp8):
    """dsa_latent_cache_write_fp8: quantise latent [T, >=512] (4 groups of 128) and copy rope [T, >=64]
    (bf16, rows may be strided) into kv_cache_fp8 [num_pages, page_stride_bytes] uint8 at the slots of
    slot_mapping [T] int64.  Returns kv_cache_fp8."""
    lib = load()
    dev = latent.device
    T = int(latent.shape[0])
    _need_rows(latent, "latent", torch.bfloat16, T, V_DIM, dev)
    _need_rows(rope, "rope", torch.bfloat16, T, KV_DIM - V_DIM, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, (T,), dev)
    _need(kv_cache_fp8, "kv_cache_fp8", torch.uint8, (None, None), dev)
    st = lib.dsa_latent_cache_write_fp8(T, _ptr(latent), int(latent.stride(0)), _ptr(rope), int(rope.stride(0)),
                                        _ptr(slot_mapping), _ptr(kv_cache_fp8), int(kv_cache_fp8.shape[1]),
                                        int(kv_cache_fp8.shape[0]), _stream(dev))
    _check(st, "dsa_latent_cache_write_fp8")
    return kv_cache_fp8
