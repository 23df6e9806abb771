"""Whole-step HIP graph capture: indexer -> top-k -> sparse MLA recorded once
and replayed several times, with eager work and synchronisations between the
replays.  Every replay must reproduce the eager step bit for bit (the step is
deterministic: fixed reduction orders, ties to the lower index), and the eager
step itself is checked against the oracle.  The library records no memset
nodes (clean logits and split partials are written by kernels)."""
import numpy as np
import pytest
import torch

from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, check_mla, mla_oracle, oracle_indexer, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode,splits", [("paged", 0), ("paged", 1), ("paged", 3), ("prefill", 0), ("prefill", 2),
                                        ("noalloc", 0), ("noalloc", 3)])
def test_step_graph_replays_match_eager(dsa, mode, splits):
    """mode: paged -- the decode step; prefill -- a chunked-prefill step (the
    prefill indexer with clean logits, rows over two 8192-key chunks); noalloc
    -- the decode step with the sparse MLA call that keeps its partials in the
    library's static device array (the entry point for callers under capture)."""
    if mode == "prefill":
        wl = synth.make_workload([3000, 300, 9000], [150, 40, 20], 16, seed=13, spare_pages=4, poison=True)
    else:
        wl = synth.make_workload([2500, 130, 7000, 40000], [2, 1, 1, 1], 16, seed=11, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    R, H, k = wl.num_rows, wl.num_heads, wl.topk
    stride = (wl.max_seq_len + 3) // 4 * 4
    logits = torch.empty(R, stride, dtype=torch.float32, device=DEV)
    indices = torch.empty(R, k, dtype=torch.int32, device=DEV)
    out = torch.empty(R, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(R, H, dtype=torch.float32, device=DEV)
    ws_topk = torch.empty(max(dsa.topk_workspace_bytes(batch, k), 1), dtype=torch.uint8, device=DEV)
    ws_mla = torch.empty(max(dsa.sparse_mla_workspace_bytes(batch, H, k, splits), 1), dtype=torch.uint8,
                         device=DEV)

    indexer = dsa.indexer_logits_prefill if mode == "prefill" else dsa.indexer_logits_paged

    def step():
        indexer(batch, t["q_fp8"], t["weights"], t["idx_cache"], logits, clean_logits=True)
        dsa.topk(batch, logits, indices, k=k, workspace=ws_topk)
        if mode == "noalloc":
            dsa.sparse_mla_decode_noalloc(batch, t["q_mla"], t["kv_cache"], indices, wl.softmax_scale, out, lse,
                                          num_splits=splits)
        else:
            dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], indices, wl.softmax_scale, out, lse,
                                  num_splits=splits, workspace=ws_mla)

    step()
    torch.cuda.synchronize()
    eager = [x.clone() for x in (logits, indices, out, lse)]
    ref, mag, _ = oracle_indexer(wl, stride)
    check_logits(eager[0].cpu().numpy(), ref, mag, "eager step")
    o_ref, l_ref = mla_oracle(wl, eager[1].cpu().numpy())
    check_mla(eager[2], eager[3], o_ref, l_ref, "eager step")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        # scribble over every output between replays, eagerly
        logits.fill_(float("nan"))
        indices.fill_(-7)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("logits", "indices", "out", "lse"), (logits, indices, out, lse), eager):
            a = got.view(torch.int32) if got.dtype == torch.float32 else got
            b = want.view(torch.int32) if want.dtype == torch.float32 else want
            if got.dtype == torch.bfloat16:
                a, b = got.view(torch.int16), want.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
