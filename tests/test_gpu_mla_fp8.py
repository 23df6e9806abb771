"""GPU parity of the fp8 latent cache: its writer (bit-exact against the
oracle) and sparse MLA over it (against the oracle's attention over the
dequantised rows, with the bf16 path's tolerances: out max-abs 2e-2, mean-abs
2e-3, lse 1e-3).  Every unreferenced slot of the fp8 cache is poisoned (NaN
codes, NaN scales, NaN rope), so a read outside the selected rows shows up."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, check_mla, oracle_indexer, rising_scores, run_indexer, run_topk, to_dev
from test_gpu_quant import slots_for

pytestmark = pytest.mark.gpu

NAN_F32 = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)


def poisoned_kv8(num_pages, stride=oracle.KV8_PAGE_BYTES):
    c = np.full((num_pages, stride), 0x7F, np.uint8)                     # e4m3 NaN codes
    rope = c[:, :oracle.KV8_SCALE_OFFSET].reshape(num_pages, 64, 640)[:, :, 512:]
    rope[:] = np.tile(np.frombuffer(np.uint16(synth.BF16_NAN).tobytes(), np.uint8), 64)[None, None, :]
    c[:, oracle.KV8_SCALE_OFFSET:oracle.KV8_PAGE_BYTES] = np.tile(NAN_F32, 256)[None, :]
    return c


def live_slots(wl):
    bt = wl.block_table.numpy()
    return np.concatenate([bt[b, np.arange(n) // 64].astype(np.int64) * 64 + np.arange(n) % 64
                           for b, n in enumerate(wl.seq_lens.numpy())])


def kv8_of(wl, stride=oracle.KV8_PAGE_BYTES):
    """The fp8 latent cache holding the workload's live tokens (oracle writer),
    everything else poisoned."""
    slots = live_slots(wl)
    rows = wl.kv_cache.view(torch.int16).numpy().view(np.uint16)[:, :64 * 576].reshape(-1, 576)
    r = rows[slots // 64 * 64 + slots % 64]
    return oracle.latent_cache_write_fp8(r[:, :512], r[:, 512:], slots, poisoned_kv8(wl.num_pages, stride))


def mla8_inputs(seq_lens, q_lens, H, seed, stride=oracle.KV8_PAGE_BYTES, k=2048):
    wl = synth.make_workload(seq_lens, q_lens, H, seed=seed, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    kv8 = kv8_of(wl, stride)
    t["kv8"] = torch.from_numpy(kv8).to(DEV)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    rng = np.random.default_rng(seed)
    idx = np.stack([oracle.topk_row(rng.normal(size=max(int(e), 1)), int(e), k) for e in ext])
    return wl, batch, t, kv8, idx


def run_mla8(dsa, wl, batch, t, idx, splits, workspace=None):
    R, H = wl.num_rows, wl.num_heads
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_decode_fp8(batch, t["q_mla"], t["kv8"], torch.from_numpy(idx.astype(np.int32)).to(DEV),
                              wl.softmax_scale, out, lse, num_splits=splits, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse


def mla8_oracle(wl, kv8, idx, rows=None):
    return oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), kv8, wl.block_table.numpy(),
                             wl.seq_lens.numpy(), wl.query_start.numpy(), idx, wl.softmax_scale,
                             num_pages=wl.num_pages, rows=rows, kv_format="fp8")


@pytest.mark.parametrize("T,num_pages,lat_stride,rope_stride,page_pad", [(1, 2, 512, 64, 0), (100, 3, 576, 64, 16),
                                                                         (3000, 60, 1024, 72, 0)])
def test_latent_cache_write_fp8_bit_exact(dsa, T, num_pages, lat_stride, rope_stride, page_pad):
    rng = np.random.default_rng(T + 2)
    stride = oracle.KV8_PAGE_BYTES + page_pad
    cache0 = rng.integers(0, 256, (num_pages, stride), dtype=np.uint8)
    x = rng.standard_normal((T, lat_stride)) * np.exp2(rng.integers(-6, 7, (T, 1)))
    x[0, :128] = 0.0                                   # an all-zero group
    lat = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    rope = torch.randn(T, rope_stride, generator=torch.Generator().manual_seed(T)).to(torch.bfloat16)
    slots = slots_for(num_pages, T, rng)
    cache = torch.from_numpy(cache0.copy()).to(DEV)
    dsa.latent_cache_write_fp8(lat.to(DEV)[:, :512], rope.to(DEV)[:, :64], torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    bits = lambda a: a.view(torch.int16).numpy().view(np.uint16)
    want = oracle.latent_cache_write_fp8(bits(lat)[:, :512], bits(rope)[:, :64], slots, cache0)
    got = cache.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, f"{bad.shape[0]} bytes differ, first at page/byte {tuple(bad[0])}"


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 12, 16, 32])
@pytest.mark.parametrize("H", [16, 32, 48, 64, 80, 96, 112, 128])
def test_sparse_mla_fp8_parity(dsa, H, splits):
    wl, batch, t, kv8, idx = mla8_inputs([3000, 700, 130, 2049], [1, 2, 1, 1], H, seed=H + splits)
    out, lse = run_mla8(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla8_oracle(wl, kv8, idx)
    check_mla(out, lse, o_ref, l_ref, f"fp8 H={H} splits={splits}")


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 16])
@pytest.mark.parametrize("k", [1, 100, 2047])
@pytest.mark.parametrize("H", [16, 64, 128])
def test_sparse_mla_fp8_parity_other_k(dsa, H, k, splits):
    """k below the 2048 maximum over the fp8 latent cache: a partial last
    tile, fewer tiles per split, rows with fewer keys than k."""
    wl, batch, t, kv8, idx = mla8_inputs([3000, 700, 130, 2049, 40], [1, 2, 1, 1, 1], H,
                                         seed=7 * k + H + splits, k=k)
    out, lse = run_mla8(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla8_oracle(wl, kv8, idx)
    check_mla(out, lse, o_ref, l_ref, f"fp8 H={H} k={k} splits={splits}")


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("H", [16, 64, 128])
def test_sparse_mla_fp8_rising_scores_rescale(dsa, H, splits):
    """Scores that climb tile by tile (the rope keys grow with the selection
    position), so the accumulators are rescaled in the middle of a split."""
    wl = synth.make_workload([5000, 3000], [1, 2], H, seed=91 + H, spare_pages=4, poison=True)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    rng = np.random.default_rng(H + 1)
    idx = np.stack([oracle.topk_row(rng.normal(size=max(int(e), 1)), int(e), 2048) for e in ext])
    rising_scores(wl, idx)
    batch, t = to_dev(wl)
    kv8 = kv8_of(wl)
    t["kv8"] = torch.from_numpy(kv8).to(DEV)
    out, lse = run_mla8(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla8_oracle(wl, kv8, idx)
    assert l_ref[0].min() > 60.0
    check_mla(out, lse, o_ref, l_ref, f"H={H} splits={splits}")


def test_sparse_mla_fp8_padded_pages_masked_and_empty_rows(dsa):
    wl, batch, t, kv8, idx = mla8_inputs([5000, 600, 64], [1, 2, 1], 16, seed=78,
                                         stride=oracle.KV8_PAGE_BYTES + 128)
    idx = idx.copy()
    idx[0, 10:20] = idx[0, 0]            # duplicates count as listed
    idx[0, 100:400] = -1                 # masked stretch
    idx[1, 5] = 599                      # row 1 sees [0, 599): 599 is out of range
    idx[2, 7] = 10 ** 6
    idx[3, :] = -1                       # nothing valid: out 0, lse -inf
    for splits in (1, 0, 7):
        out, lse = run_mla8(dsa, wl, batch, t, idx, splits)
        assert torch.all(out[3] == 0) and torch.all(torch.isneginf(lse[3]))
        o_ref, l_ref = mla8_oracle(wl, kv8, idx)
        check_mla(out, lse, o_ref, l_ref, f"fp8 splits={splits}")


def test_fp8_cache_written_on_gpu_feeds_the_step(dsa):
    """bf16 latent rows -> dsa_latent_cache_write_fp8 -> (indexer, top-k) ->
    dsa_sparse_mla_decode_fp8: the written cache equals the oracle's byte for
    byte and the attention matches the oracle over it."""
    wl = synth.make_workload([2500, 130, 7000], [2, 1, 1], 32, seed=17, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    slots = live_slots(wl)
    rows = wl.kv_cache[:, :64 * 576].reshape(-1, 576)[torch.from_numpy(slots // 64 * 64 + slots % 64)]
    cache0 = poisoned_kv8(wl.num_pages)
    kv8 = torch.from_numpy(cache0.copy()).to(DEV)
    rd = rows.to(DEV)
    dsa.latent_cache_write_fp8(rd[:, :512], rd[:, 512:], torch.from_numpy(slots).to(DEV), kv8)
    stride = 7000
    logits = run_indexer(dsa, wl, batch, t, stride)
    ref, mag, _ = oracle_indexer(wl, stride)
    check_logits(logits.cpu().numpy(), ref, mag, "fp8 step")
    idx = run_topk(dsa, batch, logits)
    t["kv8"] = kv8
    out, lse = run_mla8(dsa, wl, batch, t, idx, 0)
    bits = rows.view(torch.int16).numpy().view(np.uint16)
    want_cache = oracle.latent_cache_write_fp8(bits[:, :512], bits[:, 512:], slots, cache0)
    assert np.array_equal(kv8.cpu().numpy(), want_cache)
    o_ref, l_ref = mla8_oracle(wl, want_cache, idx)
    check_mla(out, lse, o_ref, l_ref, "fp8 step")
