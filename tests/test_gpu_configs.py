"""Full-size workloads c1..c5 (and x1m, one 1,048,576-token decode row: the
longest row one top-k call takes, 32 chunks merged) in the launch
configuration bench.py times.

Each test runs one whole step on the GPU (indexer -- the prefill entry for the
chunked-prefill workload --, top-k with its workspace, sparse MLA with the
automatic split choice, dirty logits) and checks it against the oracle:
  top-k           bit-exact on EVERY row, against the oracle's selection over
                  the GPU's own logits row
  indexer logits  |gpu - oracle| <= 1e-3 * sum_h |w_h| relu(dot_h) kscale over
                  [0, e_r), plus the plain relative check of check_logits
  sparse MLA      max-abs <= 2e-2, mean-abs <= 2e-3 vs the oracle (float64) over
                  the GPU's indices, lse <= 1e-3
Logits and sparse MLA are checked on every row of the decode workloads (1, 32,
1, 128 and 1 rows) and on every 32nd row of the 4096-row chunked prefill (128
rows, the first at the shortest causal extent) plus its last row.
"""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, check_mla, to_dev

pytestmark = pytest.mark.gpu

PREFILL_ROW_STRIDE = 32


def checked_rows(wl):
    R = wl.num_rows
    if wl.max_q_len > 2:
        return sorted(set(range(0, R, PREFILL_ROW_STRIDE)) | {R - 1})
    return list(range(R))


def run_step(dsa, wl):
    batch, t = to_dev(wl)
    R, H, k = wl.num_rows, wl.num_heads, wl.topk
    stride = (wl.max_seq_len + 3) // 4 * 4
    logits = torch.empty(R, stride, dtype=torch.float32, device=DEV)
    indices = torch.empty(R, k, dtype=torch.int32, device=DEV)
    out = torch.empty(R, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(R, H, dtype=torch.float32, device=DEV)
    ws_topk = torch.empty(max(dsa.topk_workspace_bytes(batch, k), 1), dtype=torch.uint8, device=DEV)
    ws_mla = torch.empty(max(dsa.sparse_mla_workspace_bytes(batch, H, k, 0), 1), dtype=torch.uint8, device=DEV)
    indexer = dsa.indexer_logits_prefill if wl.max_q_len > 2 else dsa.indexer_logits_paged
    indexer(batch, t["q_fp8"], t["weights"], t["idx_cache"], logits, clean_logits=False)
    dsa.topk(batch, logits, indices, k=k, workspace=ws_topk)
    dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], indices, wl.softmax_scale, out, lse,
                          num_splits=0, workspace=ws_mla)
    torch.cuda.synchronize()
    return stride, logits, indices, out, lse


def check_topk_every_row(wl, logits_host, got_idx, name):
    """Bit-exact top-k of every row against the oracle's selection over the
    GPU's own logits (rows checked in parallel on the host)."""
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())

    def one(r):
        want = oracle.topk_row(logits_host[r], int(ext[r]), wl.topk)
        return r if not np.array_equal(got_idx[r], want) else None

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        bad = [r for r in ex.map(one, range(wl.num_rows)) if r is not None]
    assert not bad, f"{name}: top-k differs on {len(bad)} of {wl.num_rows} rows, first {bad[:5]}"


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "x1m"])
def test_config_full_step(dsa, name):
    wl = synth.make_config(name)
    stride, logits, indices, out, lse = run_step(dsa, wl)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    logits_host = logits.cpu().numpy()
    got_idx = indices.cpu().numpy()
    check_topk_every_row(wl, logits_host, got_idx, name)

    rows = checked_rows(wl)
    ref, mag, _ = oracle.indexer_logits(wl.q_fp8.numpy(), wl.weights.numpy(), wl.idx_cache.numpy(),
                                        wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                        stride, clean=True, rows=rows)
    # all checked rows at once (each compared over its own extent; the rest is -inf in both)
    got_l = logits_host[rows].astype(np.float64)
    for o, r in enumerate(rows):
        got_l[o, int(ext[r]):] = -np.inf
    check_logits(got_l, ref, mag, f"{name} logits, {len(rows)} rows")
    del got_l, ref, mag

    # sparse MLA over the GPU's indices
    o_ref, l_ref = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                     wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                     got_idx[rows], wl.softmax_scale, num_pages=wl.num_pages, rows=rows)
    check_mla(out[rows], lse[rows], o_ref, l_ref, f"{name} sparse MLA, {len(rows)} rows")
