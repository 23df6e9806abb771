"""dsa_sparse_mla_decode_noalloc against dsa_sparse_mla_decode.

The no-allocation entry point runs the same kernels with the split partials in
the library's device array instead of a workspace.  Two calls in a row, the
second on a smaller input (so the array holds the first call's partials when
the second starts): each must equal the workspace entry point bit for bit at
the same split count, and meet the oracle's tolerances (out max-abs 2e-2,
mean-abs 2e-3, lse 1e-3) with the automatic split count.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_mla, mla_oracle, to_dev

pytestmark = pytest.mark.gpu


def _inputs(seq_lens, q_lens, H, seed):
    wl = synth.make_workload(seq_lens, q_lens, H, seed=seed, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    rng = np.random.default_rng(seed)
    idx = np.stack([oracle.topk_row(rng.normal(size=max(int(e), 1)), int(e), 2048) for e in ext]).astype(np.int32)
    return wl, batch, t, idx


def _run(fn, wl, batch, t, idx, splits, **kw):
    R, H = wl.num_rows, wl.num_heads
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    fn(batch, t["q_mla"], t["kv_cache"], torch.from_numpy(idx).to(DEV), wl.softmax_scale, out, lse,
       num_splits=splits, **kw)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_equals_workspace_entry_two_calls(dsa):
    big = _inputs([9000, 30000, 2500, 700] * 8, [1, 1, 2, 1] * 8, 16, seed=51)      # 40 rows
    small = _inputs([5000, 130], [1, 2], 32, seed=52)                                 # 3 rows
    for wl, batch, t, idx in (big, small):
        auto = dsa.sparse_mla_pick_splits(batch, wl.num_heads, 2048)
        assert auto > 1                      # the partials go through the device array
        for splits in (0, auto, 3):
            s = splits or auto
            got = _run(dsa.sparse_mla_decode_noalloc, wl, batch, t, idx, splits)
            ws = torch.empty(dsa.sparse_mla_workspace_bytes(batch, wl.num_heads, 2048, s), dtype=torch.uint8,
                             device=DEV)
            want = _run(dsa.sparse_mla_decode, wl, batch, t, idx, s, workspace=ws)
            assert torch.equal(got[0].view(torch.int16), want[0].view(torch.int16)), (wl.num_rows, splits)
            assert torch.equal(got[1].view(torch.int32), want[1].view(torch.int32)), (wl.num_rows, splits)
        o_ref, l_ref = mla_oracle(wl, idx)
        out, lse = _run(dsa.sparse_mla_decode_noalloc, wl, batch, t, idx, 0)
        check_mla(out, lse, o_ref, l_ref, f"noalloc, {wl.num_rows} rows")


def test_noalloc_rejects_partials_beyond_its_array(dsa):
    wl, batch, t, idx = _inputs([3000] * 2, [1] * 2, 16, seed=53)
    # 2 rows x 16 heads x 2056 B per split: no split count of k = 2048 overflows
    # 32 MiB here, so fake a batch whose forced partials would
    import sparse_attention_fp8_amd as lib
    b = lib.Batch(seq_lens=batch.seq_lens, query_start=batch.query_start, block_table=batch.block_table,
                  num_rows=2, max_seq_len=batch.max_seq_len, max_q_len=1, num_pages=batch.num_pages)
    out = torch.empty(2, 1024, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(2, 1024, dtype=torch.float32, device=DEV)
    q = torch.zeros(2, 1024, 576, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lib.DSAError) as ei:
        lib.sparse_mla_decode_noalloc(b, q, t["kv_cache"], torch.from_numpy(idx).to(DEV), wl.softmax_scale, out,
                                      lse, num_splits=32)
    assert ei.value.status == -3 and "scratch" in str(ei.value)
