"""Batch invariance and run-to-run determinism of the whole step.

With num_splits = 1 (the single-pass sparse MLA), every output of a query row
-- its logits over [0, e_r), its top-k indices, its attention output and lse --
must be bit-identical whatever else shares the batch: the row alone, the row
among other decode rows, among draft+verify (two-row) sequences, in another
order, with other page ids.  Each row's arithmetic is a fixed sequence of
operations that depends only on the row's own inputs.  The automatic split
choice depends on the batch (it changes the summation order), so invariance is
promised for num_splits = 1 only; every mode is still deterministic from run to
run, which the last test checks.  The batch results are also checked against
the oracle, so an invariant-but-wrong path cannot pass.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_fp8_amd as dsa
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, check_mla, mla_oracle, oracle_indexer

pytestmark = pytest.mark.gpu


def kv8_cache(wl):
    """The fp8 latent cache of every slot of wl's bf16 cache, written on the GPU."""
    slots = wl.num_pages * 64
    rows = wl.kv_cache[:, :64 * 576].reshape(slots, 576).to(DEV)
    kv8 = torch.zeros(wl.num_pages, dsa.binding.KV8_PAGE_BYTES, dtype=torch.uint8, device=DEV)
    dsa.latent_cache_write_fp8(rows[:, :512], rows[:, 512:], torch.arange(slots, dtype=torch.int64, device=DEV), kv8)
    torch.cuda.synchronize()
    return kv8.cpu()


def sub_workload(wl, seqs, perm_seed=None, kv8=None):
    """The sequences `seqs` of `wl` (in that order) as a workload of their own,
    sharing wl's caches; with perm_seed the physical pages are renumbered by a
    random permutation (caches permuted to match)."""
    qs = wl.query_start.numpy()
    rows = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in seqs]).astype(np.int64)
    q_lens = [int(qs[b + 1] - qs[b]) for b in seqs]
    query_start = np.zeros(len(seqs) + 1, np.int32)
    query_start[1:] = np.cumsum(q_lens)
    bt = wl.block_table.numpy()[seqs]
    idx_cache, kv_cache = wl.idx_cache, wl.kv_cache
    if perm_seed is not None:
        perm = np.random.default_rng(perm_seed).permutation(wl.num_pages)   # old id -> new id
        inv = np.argsort(perm)
        bt = perm[bt]
        idx_cache = idx_cache[torch.from_numpy(inv)]
        kv_cache = kv_cache[torch.from_numpy(inv)]
        if kv8 is not None:
            kv8 = kv8[torch.from_numpy(inv)]
    sl = wl.seq_lens.numpy()[seqs]
    batch = dsa.Batch.from_host(torch.from_numpy(sl.copy()), torch.from_numpy(query_start),
                                torch.from_numpy(np.ascontiguousarray(bt)), wl.num_pages, device=DEV)
    t = {"q_fp8": wl.q_fp8[rows].to(DEV), "weights": wl.weights[rows].to(DEV), "q_mla": wl.q_mla[rows].to(DEV),
         "idx_cache": idx_cache.to(DEV), "kv_cache": kv_cache.to(DEV)}
    if kv8 is not None:
        t["kv8"] = kv8.to(DEV)
    return batch, t, rows


def run(batch, t, wl, prefill, splits):
    R, H, k = batch.num_rows, wl.num_heads, wl.topk
    stride = (batch.max_seq_len + 3) // 4 * 4 + 12
    logits = torch.full((R, stride), float("nan"), dtype=torch.float32, device=DEV)
    indices = torch.empty(R, k, dtype=torch.int32, device=DEV)
    out = torch.empty(R, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(R, H, dtype=torch.float32, device=DEV)
    fn = dsa.indexer_logits_prefill if prefill else dsa.indexer_logits_paged
    fn(batch, t["q_fp8"], t["weights"], t["idx_cache"], logits, clean_logits=True)
    dsa.topk(batch, logits, indices, k=k)
    if "kv8" in t:
        dsa.sparse_mla_decode_fp8(batch, t["q_mla"], t["kv8"], indices, wl.softmax_scale, out, lse,
                                  num_splits=splits)
    else:
        dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], indices, wl.softmax_scale, out, lse,
                              num_splits=splits)
    torch.cuda.synchronize()
    return (logits.cpu().numpy(), indices.cpu().numpy(), out.view(torch.int16).cpu().numpy(),
            lse.cpu().numpy())


def extents(wl):
    return wl.row_extents()


CASES = {
    # decode rows, two-row (draft + verify) sequences, contexts around k and far above it
    "decode_mtp": dict(seq_lens=[5000, 700, 2048, 9000, 64, 3000], q_lens=[1, 2, 1, 2, 1, 1], H=16, prefill=False),
    "heads128": dict(seq_lens=[4100, 2500, 300], q_lens=[2, 1, 2], H=128, prefill=False),
    "prefill": dict(seq_lens=[3000, 2200], q_lens=[40, 17], H=16, prefill=True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_rows_are_batch_invariant_with_one_split(case):
    c = CASES[case]
    wl = synth.make_workload(c["seq_lens"], c["q_lens"], c["H"], seed=31, spare_pages=5)
    ext = extents(wl)
    B = len(c["seq_lens"])
    full_batch, full_t, _ = sub_workload(wl, list(range(B)))
    full = run(full_batch, full_t, wl, c["prefill"], 1)

    # the whole batch is right (against the oracle) before its invariance means anything
    stride = full[0].shape[1]
    ref, mag, _ = oracle_indexer(wl, stride)
    check_logits(full[0], ref, mag, f"{case} batch logits")
    o_ref, l_ref = mla_oracle(wl, full[1])
    check_mla(torch.from_numpy(full[2]).view(torch.bfloat16), torch.from_numpy(full[3]), o_ref, l_ref,
              f"{case} batch sparse MLA")

    layouts = [[b] for b in range(B)] + [list(reversed(range(B))), [B - 1, 0] if B > 1 else [0]]
    for li, seqs in enumerate(layouts):
        batch, t, rows = sub_workload(wl, seqs, perm_seed=100 + li)
        got = run(batch, t, wl, c["prefill"], 1)
        for o, r in enumerate(rows):
            e = int(ext[r])
            what = f"{case}: row {r} with sequences {seqs}"
            assert np.array_equal(got[0][o, :e].view(np.uint32), full[0][r, :e].view(np.uint32)), f"{what}: logits"
            assert np.array_equal(got[1][o], full[1][r]), f"{what}: top-k"
            assert np.array_equal(got[2][o], full[2][r]), f"{what}: out"
            assert np.array_equal(got[3][o].view(np.uint32), full[3][r].view(np.uint32)), f"{what}: lse"


@pytest.mark.parametrize("splits", [0, 1, 4])
def test_step_is_deterministic_run_to_run(splits):
    wl = synth.make_workload([40000, 2500, 130, 7000], [1, 2, 1, 1], 16, seed=12, spare_pages=4)
    batch, t, _ = sub_workload(wl, [0, 1, 2, 3])
    first = run(batch, t, wl, False, splits)
    for _ in range(3):
        again = run(batch, t, wl, False, splits)
        for a, b in zip(first, again):
            assert np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("H", [16, 128])
def test_fp8_latent_rows_are_batch_invariant_with_one_split(H):
    """The same invariance over the fp8 latent cache (written on the GPU from
    the bf16 rows), checked against the oracle over the dequantised rows."""
    wl = synth.make_workload([5000, 700, 2048, 9000, 64], [1, 2, 1, 2, 1], H, seed=33, spare_pages=5)
    kv8 = kv8_cache(wl)
    B = wl.num_seqs
    full_batch, full_t, _ = sub_workload(wl, list(range(B)), kv8=kv8)
    full = run(full_batch, full_t, wl, False, 1)
    o_ref, l_ref = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), kv8.numpy(), wl.block_table.numpy(),
                                  wl.seq_lens.numpy(), wl.query_start.numpy(), full[1], wl.softmax_scale,
                                  num_pages=wl.num_pages, kv_format="fp8")
    check_mla(torch.from_numpy(full[2]).view(torch.bfloat16), torch.from_numpy(full[3]), o_ref, l_ref,
              f"fp8 H={H} batch sparse MLA")
    for li, seqs in enumerate([[b] for b in range(B)] + [list(reversed(range(B)))]):
        batch, t, rows = sub_workload(wl, seqs, perm_seed=200 + li, kv8=kv8)
        got = run(batch, t, wl, False, 1)
        for o, r in enumerate(rows):
            what = f"fp8 H={H}: row {r} with sequences {seqs}"
            assert np.array_equal(got[1][o], full[1][r]), f"{what}: top-k"
            assert np.array_equal(got[2][o], full[2][r]), f"{what}: out"
            assert np.array_equal(got[3][o].view(np.uint32), full[3][r].view(np.uint32)), f"{what}: lse"
