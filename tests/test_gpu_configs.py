"""Full-size workloads c1..c5 (and x1m, one 1,048,576-token decode row: the
longest row one top-k call takes, 32 chunks merged) in the launch
configuration bench.py times.

Each test runs one whole step on the GPU (indexer -- the prefill entry for the
chunked-prefill workload --, top-k with its workspace, sparse MLA with the
automatic split choice, dirty logits) and checks sampled rows the oracle can
compute one by one:
  indexer logits  |gpu - oracle| <= 1e-3 * sum_h |w_h| relu(dot_h) kscale over [0, e_r)
  top-k           bit-exact vs the oracle's selection over the GPU's own logits row
  sparse MLA      max-abs <= 2e-2, mean-abs <= 2e-3 vs the oracle (float64), lse <= 1e-3
Sampled rows cover the first, last and middle rows and the longest and shortest
contexts of each workload.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, check_mla, to_dev

pytestmark = pytest.mark.gpu


def sample_rows(wl):
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    R = len(ext)
    rows = {0, R - 1, R // 2, int(np.argmax(ext)), int(np.argmin(ext))}
    return sorted(rows)


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


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "x1m"])
def test_config_sampled_rows(dsa, name):
    wl = synth.make_config(name)
    stride, logits, indices, out, lse = run_step(dsa, wl)
    rows = sample_rows(wl)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    got_l = logits[rows].cpu().numpy().astype(np.float64)
    ref, mag, _ = oracle.indexer_logits(wl.q_fp8.numpy(), wl.weights.numpy(), wl.idx_cache.numpy(),
                                        wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                        stride, clean=True, rows=rows)
    for o, r in enumerate(rows):
        e = int(ext[r])
        check_logits(got_l[o:o + 1, :e], ref[o:o + 1, :e], mag[o:o + 1, :e], f"{name} row {r} logits")
    # top-k: bit-exact against the selection over the GPU's own logits rows
    want_idx = oracle.topk(got_l, wl.seq_lens.numpy(), wl.query_start.numpy(), wl.topk, rows=rows)
    got_idx = indices[rows].cpu().numpy()
    assert np.array_equal(got_idx, want_idx), f"{name}: top-k differs on sampled rows"
    # sparse MLA over the GPU's indices
    o_ref, l_ref = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                     wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                     got_idx, wl.softmax_scale, num_pages=wl.num_pages, rows=rows)
    check_mla(out[rows], lse[rows], o_ref, l_ref, f"{name} sparse MLA")
