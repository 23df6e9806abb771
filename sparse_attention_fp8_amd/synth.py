"""Seeded synthetic DSA workloads: the inputs of one DSA layer step, nothing else.

This module only draws random inputs and lays them out in the cache formats the
library reads.  It holds none of the attention arithmetic: the oracle (under
``oracle/``) and the HIP library both consume the bytes produced here.

Workload shapes follow the decode setting of the vLLM PR "[Feature]
TRITON_MLA_SPARSE backend for SM8x/11x/12x DSA Sparse MLA Support" (sections
Changes and Benchmarks): an FP8 indexer-K cache of 132 bytes per token (128
e4m3 values plus one fp32 scale), a bf16 latent cache of 576 values per token
(512 latent + 64 rope), block size 64, top-k 2048, and the vllm-dsa-mtp-sm80
README's note that indexer pages are addressed by their page stride (so padded
pages are allowed).

Value distributions: indexer q is bf16(N(0,1)) quantised per (token, head)
group of 128 to e4m3 with scale amax/448, the scale being folded into the head
weight (w' = w * s_q, w ~ N(0, 1/64)); indexer K is N(0,1) per token quantised
to e4m3 with scale amax/448; MLA q and the latent cache are bf16(N(0,1)).
Physical pages are a random permutation, so logical neighbours are never
physical neighbours.

The fp8 rounding is done with torch's float8_e4m3fn cast after clamping to
+-448 (round to nearest even, saturating).  It is input preparation: the
library never quantises, it reads the codes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 64                 # tokens per cache block
IDX_HEADS = 64            # indexer heads
IDX_DIM = 128             # indexer head dim (bytes per token of fp8 K)
IDX_SCALE_OFFSET = PAGE * IDX_DIM          # 8192: fp32 scales follow the codes
IDX_PAGE_BYTES = IDX_SCALE_OFFSET + 4 * PAGE   # 8448 bytes per indexer page
KV_DIM = 576              # latent 512 + rope 64
V_DIM = 512
TOPK = 2048
E4M3_MAX = 448.0

FP8_NAN = 0x7F            # e4m3fn NaN code, used to poison unreferenced slots
BF16_NAN = 0x7FC0


@dataclass
class Workload:
    """Host tensors of one synthetic DSA step (all on CPU)."""
    name: str
    seq_lens: torch.Tensor        # [B] int32, cached tokens incl. this step's queries
    query_start: torch.Tensor     # [B+1] int32
    block_table: torch.Tensor     # [B, bt_stride] int32, logical block -> physical page
    num_pages: int                # physical pages in each cache
    q_fp8: torch.Tensor           # [R, 64, 128] uint8 e4m3fn codes
    weights: torch.Tensor         # [R, 64] float32, q scale folded in
    idx_cache: torch.Tensor       # [num_pages, idx_page_stride] uint8
    q_mla: torch.Tensor           # [R, H, 576] bfloat16
    kv_cache: torch.Tensor        # [num_pages, kv_page_stride] bfloat16 (page = [64][576] first)
    num_heads: int
    softmax_scale: float
    topk: int = TOPK
    extras: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.numel())

    @property
    def num_rows(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.numel() else 0

    @property
    def max_q_len(self) -> int:
        qs = self.query_start
        return int((qs[1:] - qs[:-1]).max()) if qs.numel() > 1 else 0

    @property
    def idx_page_stride(self) -> int:
        return int(self.idx_cache.shape[1])

    @property
    def kv_page_stride(self) -> int:
        return int(self.kv_cache.shape[1])

    def row_extents(self) -> np.ndarray:
        """e_r for each row: row i of a sequence with q_len queries and L cached
        tokens sees keys [0, L - q_len + i + 1)."""
        out = np.zeros(self.num_rows, dtype=np.int64)
        qs = self.query_start.numpy()
        for b, L in enumerate(self.seq_lens.numpy()):
            q = qs[b + 1] - qs[b]
            for i in range(q):
                out[qs[b] + i] = max(0, int(L) - q + i + 1)
        return out


def _quantize_rows_e4m3(x: torch.Tensor):
    """Per-row (last dim) e4m3 codes and fp32 scales with scale = amax / 448."""
    x = x.float()
    amax = x.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (x / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.squeeze(-1)


def make_workload(seq_lens, q_lens, num_heads, seed, *, name="custom", spare_pages=64,
                  idx_page_pad=0, kv_page_pad=0, poison=False, topk=TOPK,
                  softmax_scale=1.0 / math.sqrt(192.0), gen_chunk_pages=2048):
    """Build a seeded workload.

    Draw order (fixed): block-table permutation, indexer q, indexer K, head
    weights, MLA q, latent cache.  ``poison`` fills spare pages, the slots past
    each sequence's end in its last page, and the page padding with NaN codes,
    so any read of an unreferenced slot shows up as NaN downstream.
    """
    seq_lens = [int(x) for x in seq_lens]
    q_lens = [int(x) for x in q_lens]
    assert len(seq_lens) == len(q_lens) and spare_pages >= 1
    g = torch.Generator().manual_seed(int(seed))
    B = len(seq_lens)
    pages_per_seq = [(L + PAGE - 1) // PAGE for L in seq_lens]
    live_pages = sum(pages_per_seq)
    num_pages = live_pages + spare_pages
    perm = torch.randperm(num_pages, generator=g).to(torch.int32)
    bt_stride = max(1, max(pages_per_seq) if pages_per_seq else 1)
    spare = perm[live_pages:]
    block_table = spare[0].repeat(B, bt_stride).clone()   # unused entries -> a spare page
    cur = 0
    for b, n in enumerate(pages_per_seq):
        block_table[b, :n] = perm[cur:cur + n]
        cur += n
    query_start = torch.zeros(B + 1, dtype=torch.int32)
    query_start[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    R = int(query_start[-1])

    # indexer q: bf16(N(0,1)) -> per (row, head) e4m3 with amax/448 scale
    q_idx = torch.randn(R, IDX_HEADS, IDX_DIM, generator=g).to(torch.bfloat16)
    q_fp8, s_q = _quantize_rows_e4m3(q_idx)

    # indexer K cache: N(0,1) per token, e4m3 with per-token fp32 scale
    idx_stride = IDX_PAGE_BYTES + int(idx_page_pad)
    idx_cache = torch.zeros(num_pages, idx_stride, dtype=torch.uint8)
    for p0 in range(0, num_pages, gen_chunk_pages):
        p1 = min(num_pages, p0 + gen_chunk_pages)
        k = torch.randn(p1 - p0, PAGE, IDX_DIM, generator=g)
        codes, scales = _quantize_rows_e4m3(k)
        idx_cache[p0:p1, :IDX_SCALE_OFFSET] = codes.reshape(p1 - p0, -1)
        idx_cache[p0:p1, IDX_SCALE_OFFSET:IDX_PAGE_BYTES] = scales.contiguous().view(torch.uint8).reshape(p1 - p0, -1)

    w = torch.randn(R, IDX_HEADS, generator=g) * (1.0 / 8.0)
    weights = (w * s_q).float().contiguous()

    q_mla = torch.randn(R, num_heads, KV_DIM, generator=g).to(torch.bfloat16)
    kv_stride = PAGE * KV_DIM + int(kv_page_pad)
    kv_cache = torch.zeros(num_pages, kv_stride, dtype=torch.bfloat16)
    for p0 in range(0, num_pages, gen_chunk_pages):
        p1 = min(num_pages, p0 + gen_chunk_pages)
        kv_cache[p0:p1, :PAGE * KV_DIM] = torch.randn(p1 - p0, PAGE * KV_DIM, generator=g).to(torch.bfloat16)

    if poison:
        _poison(idx_cache, kv_cache, block_table, seq_lens, pages_per_seq, spare)

    return Workload(name=name, seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                    query_start=query_start, block_table=block_table.contiguous(),
                    num_pages=num_pages, q_fp8=q_fp8.contiguous(), weights=weights,
                    idx_cache=idx_cache, q_mla=q_mla.contiguous(), kv_cache=kv_cache,
                    num_heads=int(num_heads), softmax_scale=float(softmax_scale), topk=int(topk))


def _poison(idx_cache, kv_cache, block_table, seq_lens, pages_per_seq, spare):
    nan_f32 = torch.tensor([float("nan")], dtype=torch.float32).view(torch.uint8)
    kv_u16 = kv_cache.view(torch.int16)
    for p in spare.tolist():
        idx_cache[p, :] = FP8_NAN
        idx_cache[p, IDX_SCALE_OFFSET:IDX_PAGE_BYTES] = nan_f32.repeat(PAGE)
        kv_u16[p, :] = BF16_NAN
    # page padding bytes / elements of live pages
    if idx_cache.shape[1] > IDX_PAGE_BYTES:
        idx_cache[:, IDX_PAGE_BYTES:] = FP8_NAN
    if kv_cache.shape[1] > PAGE * KV_DIM:
        kv_u16[:, PAGE * KV_DIM:] = BF16_NAN
    for b, L in enumerate(seq_lens):
        n = pages_per_seq[b]
        if n == 0 or L % PAGE == 0:
            continue
        p = int(block_table[b, n - 1])
        for slot in range(L % PAGE, PAGE):
            idx_cache[p, slot * IDX_DIM:(slot + 1) * IDX_DIM] = FP8_NAN
            idx_cache[p, IDX_SCALE_OFFSET + 4 * slot:IDX_SCALE_OFFSET + 4 * slot + 4] = nan_f32
            kv_u16[p, slot * KV_DIM:(slot + 1) * KV_DIM] = BF16_NAN


# ----------------------------------------------------------------------------
# The five workloads the library is measured on.

CONFIGS = {
    "c1": "decode, batch 1, context 4096, 16 MLA heads",
    "c2": "decode, batch 32, contexts uniform in [512, 32768], 16 MLA heads",
    "c3": "long-context decode, batch 1, context 131072, 16 MLA heads",
    "c4": "chunked prefill, 4096 queries appended to a 61440-token prefix, 16 MLA heads",
    "c5": "MTP decode, batch 64, 2 queries per sequence, contexts log-uniform in [1024, 65536], 128 MLA heads",
    # beyond the five: the longest row one top-k call takes (32 chunks of 32768 keys merged)
    "x1m": "long-context decode, batch 1, context 1048576, 16 MLA heads",
}

DEFAULT_SEEDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5, "x1m": 6}


def config_shape(name: str, seed: int):
    """(seq_lens, q_lens, num_heads) of a named workload; contexts drawn from ``seed``."""
    rng = np.random.default_rng(int(seed))
    if name == "c1":
        return [4096], [1], 16
    if name == "c2":
        return rng.integers(512, 32768, size=32, endpoint=True).tolist(), [1] * 32, 16
    if name == "c3":
        return [131072], [1], 16
    if name == "c4":
        return [65536], [4096], 16
    if name == "c5":
        lo, hi = math.log(1024.0), math.log(65536.0)
        L = np.floor(np.exp(rng.uniform(lo, hi, size=64))).astype(np.int64)
        return np.clip(L, 1024, 65536).tolist(), [2] * 64, 128
    if name == "x1m":
        return [1 << 20], [1], 16
    raise KeyError(name)


def make_config(name: str, seed: int | None = None, **kw) -> Workload:
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    seq_lens, q_lens, heads = config_shape(name, seed)
    return make_workload(seq_lens, q_lens, heads, seed, name=name, **kw)
