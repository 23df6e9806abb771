"""GPU parity of every libdsa entry point against the float64 oracle.

Sizes are small enough for the oracle to finish in seconds but span several
tiles, ragged page tails, multi-chunk top-k rows and every split mode.  Caches
are poisoned (NaN codes / scales / bf16) outside the live tokens, so any read
of an unreferenced slot shows up.  Tolerances:
  indexer logits   |gpu - oracle| <= 1e-3 * sum_h |w_h| relu(dot_h) kscale   (the
                   magnitude the signed 64-head sum is made of; -inf masks equal),
                   and the plain |gpu - oracle| <= 1e-3 * |oracle| wherever the
                   head sum keeps at least a tenth of its magnitude (|oracle| >=
                   0.1 * magnitude); the plain relative error over |oracle| >
                   1e-3 * magnitude is printed.  The fp8 MFMA adds each aligned
                   group of 8 products in a narrow adder (a product 2^14 or more
                   below the group's largest is dropped:
                   test_indexer_fp8_mfma_group_sum pins the part the tolerance
                   relies on), which leaves errors near 3e-5 of the magnitude;
                   where the 64 heads cancel to below a tenth of it, no fp8-MFMA
                   sum meets a plain 1e-3 relative bound.
  top-k            bit-exact vs a CPU selection over the GPU's own logits
  sparse MLA out   max-abs <= 2e-2, mean-abs <= 2e-3 vs the oracle's float64
                   (pre-rounding) value; lse abs <= 1e-3
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
LOGIT_TOL = 1e-3
PLAIN_REL_FLOOR = 0.1      # plain relative check where |oracle| >= this fraction of the magnitude
OUT_MAX, OUT_MEAN, LSE_TOL = 2e-2, 2e-3, 1e-3


def to_dev(wl):
    import sparse_attention_fp8_amd as dsa
    batch = dsa.Batch.from_host(wl.seq_lens, wl.query_start, wl.block_table, wl.num_pages, device=DEV)
    return batch, {"q_fp8": wl.q_fp8.to(DEV), "weights": wl.weights.to(DEV), "idx_cache": wl.idx_cache.to(DEV),
                   "q_mla": wl.q_mla.to(DEV), "kv_cache": wl.kv_cache.to(DEV)}


def run_indexer(dsa, wl, batch, t, stride, clean=True, prefill=False, fill=float("nan")):
    logits = torch.full((wl.num_rows, stride), fill, dtype=torch.float32, device=DEV)
    fn = dsa.indexer_logits_prefill if prefill else dsa.indexer_logits_paged
    fn(batch, t["q_fp8"], t["weights"], t["idx_cache"], logits, clean_logits=clean)
    torch.cuda.synchronize()
    return logits


def oracle_indexer(wl, stride, clean=True, rows=None):
    return oracle.indexer_logits(wl.q_fp8.numpy(), wl.weights.numpy(), wl.idx_cache.numpy(),
                                 wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                 stride, clean=clean, rows=rows)


def check_logits(got, ref, mag, what=""):
    """Asserts both logits tolerances; returns (and prints) the error figures."""
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    assert np.isfinite(got[fin]).all(), f"{what}: non-finite logits where the oracle is finite"
    o, m = ref[fin], mag[fin]
    err = np.abs(got[fin] - o)
    bound = LOGIT_TOL * m
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} logits out of tolerance, worst ratio {(err / np.maximum(bound, 1e-300)).max():.3g}"
    stats = {"n": int(o.size), "err_over_mag": float((err / np.maximum(m, 1e-300)).max()) if o.size else 0.0}
    wide = np.abs(o) > LOGIT_TOL * m
    if wide.any():
        rel = err[wide] / np.abs(o[wide])
        stats.update(plain_rel_max=float(rel.max()), plain_rel_over_1e3=int((rel > LOGIT_TOL).sum()),
                     plain_rel_n=int(wide.sum()))
    kept = np.abs(o) >= PLAIN_REL_FLOOR * m
    kept &= o != 0
    if kept.any():
        rel = err[kept] / np.abs(o[kept])
        worst = int(np.argmax(rel))
        assert rel[worst] <= LOGIT_TOL, (f"{what}: plain relative error {rel[worst]:.3g} > {LOGIT_TOL} at a logit "
                                         f"holding {np.abs(o[kept][worst]) / m[kept][worst]:.3g} of its magnitude")
        stats["plain_rel_max_kept"] = float(rel.max())
        stats["kept_frac"] = float(kept.sum() / max(o.size, 1))
    print(f"[logits] {what}: " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in stats.items()))
    return stats


def mla_oracle(wl, idx, rows=None):
    return oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                             wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(), idx,
                             wl.softmax_scale, num_pages=wl.num_pages, rows=rows)


def check_mla(out, lse, o_ref, l_ref, what=""):
    o = out.float().cpu().numpy().astype(np.float64)
    ls = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    d = np.abs(o - o_ref)
    assert d.max() <= OUT_MAX and d.mean() <= OUT_MEAN, f"{what}: out max {d.max():.3g} mean {d.mean():.3g}"
    assert np.array_equal(np.isneginf(ls), np.isneginf(l_ref)), f"{what}: -inf lse pattern differs"
    fin = np.isfinite(l_ref)
    if fin.any():
        assert np.abs(ls[fin] - l_ref[fin]).max() <= LSE_TOL, f"{what}: lse err {np.abs(ls[fin] - l_ref[fin]).max():.3g}"


# --------------------------------------------------------------------------
# indexer logits

INDEXER_CASES = {
    "decode_edges": ([1, 63, 64, 65, 130, 2047, 2048, 2049], [1] * 8, {}),
    "mtp_pairs": ([3000, 700, 64, 2], [2, 2, 2, 2], {}),
    "qlen_ge_len": ([5, 300, 3], [5, 3, 7], {}),
    "padded_pages": ([1000, 333], [1, 3], {"idx_page_pad": 512}),
    "prefill_rows": ([2600], [200], {}),
    "prefill_chunks": ([9000, 5000, 64], [300, 17, 9], {}),
    "many_seqs": (list(range(1, 400, 7)), [1] * 57, {}),
    # more than 64 sequences: the paged kernel's workgroup-wide page prefix
    "over_64_seqs": ([(37 * i) % 700 + 1 for i in range(100)], [1 + (i % 3 == 0) for i in range(100)], {}),
}


@pytest.mark.parametrize("prefill", [False, True], ids=["paged", "prefill"])
@pytest.mark.parametrize("case", list(INDEXER_CASES))
def test_indexer_parity(dsa, case, prefill):
    seq_lens, q_lens, kw = INDEXER_CASES[case]
    wl = synth.make_workload(seq_lens, q_lens, 16, seed=101, spare_pages=5, poison=True, **kw)
    batch, t = to_dev(wl)
    stride = (wl.max_seq_len + 3) // 4 * 4 + 8
    got = run_indexer(dsa, wl, batch, t, stride, clean=True, prefill=prefill).cpu().numpy()
    ref, mag, _ = oracle_indexer(wl, stride, clean=True)
    check_logits(got, ref, mag, f"{case}/{'prefill' if prefill else 'paged'}")


@pytest.mark.parametrize("prefill", [False, True], ids=["paged", "prefill"])
def test_indexer_dirty_leaves_tail(dsa, prefill):
    wl = synth.make_workload([777, 64, 1], [2, 1, 1], 16, seed=5, spare_pages=2, poison=True)
    batch, t = to_dev(wl)
    stride = 1024
    got = run_indexer(dsa, wl, batch, t, stride, clean=False, prefill=prefill, fill=12345.0).cpu().numpy()
    ref, mag, ext = oracle_indexer(wl, stride, clean=False)
    for r, e in enumerate(ext):
        assert np.all(got[r, e:] == 12345.0), f"row {r}: dirty tail was written"
    check_logits(got[:, :max(ext)], ref[:, :max(ext)], mag[:, :max(ext)], "dirty")


@pytest.mark.parametrize("prefill", [False, True], ids=["paged", "prefill"])
def test_indexer_clean_short_prefix_wide_stride(dsa, prefill):
    """clean_logits where most of each row lies past its causal extent: a
    300-row prefill of a 300-token sequence (extents 1..300), 40 rows at the
    end of 2100 tokens, 50 rows of a 20-token sequence (30 rows see nothing),
    and a logits stride of three 4096-key chunks plus a ragged 132: whole
    chunks, whole stages and stage tails past every extent must read -inf,
    and every column must be written (the buffer starts as NaN)."""
    wl = synth.make_workload([300, 2100, 20], [300, 40, 50], 16, seed=77, spare_pages=3, poison=True)
    batch, t = to_dev(wl)
    stride = 3 * 4096 + 132
    got = run_indexer(dsa, wl, batch, t, stride, clean=True, prefill=prefill).cpu().numpy()
    assert not np.isnan(got).any(), "unwritten logits columns"
    ref, mag, ext = oracle_indexer(wl, stride, clean=True)
    for r, e in enumerate(ext):
        assert np.isneginf(got[r, e:]).all(), f"row {r}: columns past e_r={e} are not -inf"
    check_logits(got, ref, mag, f"clean_wide/{'prefill' if prefill else 'paged'}")


@pytest.mark.parametrize("prefill", [False, True], ids=["paged", "prefill"])
def test_indexer_fp8_mfma_group_sum(dsa, prefill):
    """The arithmetic fact the logits tolerance rests on, pinned through the
    public API: one head (w = 1) whose dot has two non-zero products, a large
    one (16 * 16 = 256) and a small one (256 * 2^-j).  Products at least 8
    dimensions apart (in different aligned groups of 8) are summed in fp32:
    exact for every j here.  Products inside one group are summed exactly for
    j <= 13; for larger j the GPU may drop the small one, but never gives
    anything other than the exact sum or the large product alone."""
    L = 64
    wl = synth.make_workload([L], [1], 16, seed=3, spare_pages=1)
    page = int(wl.block_table[0, 0])
    cache = wl.idx_cache.numpy().copy()
    enc = lambda v: int(oracle.e4m3fn_encode(np.array([v]))[0])
    small = [2.0 ** -j for j in range(10)]          # times k = 1 and q = 1: 2^0 .. 2^-9
    for d1, d2 in ((0, 1), (0, 7), (8, 15), (40, 47), (0, 8), (0, 63), (0, 64), (5, 100), (120, 127)):
        c = cache.copy()
        c[page, :8192] = 0
        c[page, 8192:8448] = np.ones(64, np.float32).view(np.uint8)
        for s, v in enumerate(small):
            c[page, s * 128 + d1] = enc(16.0)
            c[page, s * 128 + d2] = enc(v)
        q = np.zeros((1, 64, 128), np.uint8)
        w = np.zeros((1, 64), np.float32)
        q[0, 0, d1], q[0, 0, d2], w[0, 0] = enc(16.0), enc(1.0), 1.0
        wl.idx_cache, wl.q_fp8, wl.weights = torch.from_numpy(c), torch.from_numpy(q), torch.from_numpy(w)
        batch, t = to_dev(wl)
        got = run_indexer(dsa, wl, batch, t, L, prefill=prefill).cpu().numpy().astype(np.float64)
        for s, v in enumerate(small):
            exact = 256.0 + v
            ratio_log2 = 8 + s
            if d1 // 8 != d2 // 8 or ratio_log2 <= 13:
                assert got[0, s] == exact, (d1, d2, ratio_log2, got[0, s])
            else:
                assert got[0, s] in (exact, 256.0), (d1, d2, ratio_log2, got[0, s])
        assert np.all(got[0, len(small):] == 0.0)                 # all-zero keys


def test_indexer_all_fp8_codes_decode_exactly(dsa):
    """Two heads with weights +1/-1 and q = +e_d / -e_d give logit = k_d * scale
    exactly, so every finite e4m3 byte is checked through the MFMA decode."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    L = 256
    wl = synth.make_workload([L], [1], 16, seed=3, spare_pages=1)
    rng = np.random.default_rng(0)
    cache = wl.idx_cache.numpy().copy()
    bt = wl.block_table.numpy()
    codes = np.zeros((L, 128), np.uint8)
    for d in range(128):
        codes[:, d] = np.concatenate([rng.permutation(finite), finite[:2]])
    scales = rng.uniform(0.25, 4.0, size=L).astype(np.float32)
    for s in range(L):
        p, slot = bt[0, s // 64], s % 64
        cache[p, slot * 128:(slot + 1) * 128] = codes[s]
        cache[p, 8192 + 4 * slot:8192 + 4 * slot + 4] = scales[s:s + 1].view(np.uint8)
    wl.idx_cache = torch.from_numpy(cache)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for d in (0, 1, 31, 64, 127):
        q = np.zeros((1, 64, 128), np.uint8)
        w = np.zeros((1, 64), np.float32)
        q[0, 3, d], w[0, 3] = 0x38, 1.0
        q[0, 40, d], w[0, 40] = 0xB8, -1.0
        wl.q_fp8, wl.weights = torch.from_numpy(q), torch.from_numpy(w)
        batch, t = to_dev(wl)
        got = run_indexer(dsa, wl, batch, t, L).cpu().numpy()[0]
        want = (dec[:, d] * scales.astype(np.float64)).astype(np.float32)
        assert np.array_equal(got, want), f"dim {d}: {np.nonzero(got != want)[0][:8]}"


def test_indexer_out_of_range_pages_are_masked(dsa):
    wl = synth.make_workload([300, 200], [1, 1], 16, seed=9, spare_pages=2)
    bt = wl.block_table.clone()
    bt[0, 1] = wl.num_pages + 5     # a bad id inside sequence 0
    bt[1, 0] = -3
    wl.block_table = bt
    batch, t = to_dev(wl)
    got = run_indexer(dsa, wl, batch, t, 304).cpu().numpy()
    ref, mag, _ = oracle_indexer(wl, 304)
    check_logits(got, ref, mag, "bad pages")
    assert np.all(np.isneginf(got[0, 64:128])) and np.all(np.isneginf(got[1, :64]))


# --------------------------------------------------------------------------
# top-k

def run_topk(dsa, batch, logits, k=2048):
    idx = torch.full((logits.shape[0], k), -7, dtype=torch.int32, device=DEV)
    dsa.topk(batch, logits, idx, k=k)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def check_topk(got, logits_np, wl, k):
    ref = oracle.topk(logits_np, wl.seq_lens.numpy(), wl.query_start.numpy(), k)
    for r in range(ref.shape[0]):
        assert np.array_equal(got[r], ref[r]), f"row {r}: first diff at {np.nonzero(got[r] != ref[r])[0][:5]}"


@pytest.mark.parametrize("k", [2048, 1, 100, 2047])
def test_topk_on_indexer_logits(dsa, k):
    wl = synth.make_workload([1, 2047, 2048, 2049, 5000, 16384, 16385, 40000], [1] * 8, 16, seed=17, spare_pages=3)
    batch, t = to_dev(wl)
    stride = 40000
    logits = run_indexer(dsa, wl, batch, t, stride)
    got = run_topk(dsa, batch, logits, k)
    check_topk(got, logits.cpu().numpy(), wl, k)


@pytest.mark.parametrize("pool", ["small_set", "signed_zero", "constant"])
def test_topk_forced_ties(dsa, pool):
    """Logits drawn from a tiny value set: most of the selection is decided by the
    lower-index tie rule; rows span one and several chunks."""
    lens = [10, 2048, 3000, 16384, 17000, 50000]
    wl = synth.make_workload(lens, [1] * len(lens), 16, seed=23, spare_pages=2)
    batch, _ = to_dev(wl)
    rng = np.random.default_rng(1)
    vals = {"small_set": np.array([-1.0, 0.0, 1.0, 2.0, 2.5], np.float32),
            "signed_zero": np.array([-0.0, 0.0, -1.0], np.float32),
            "constant": np.array([3.25], np.float32)}[pool]
    host = rng.choice(vals, size=(len(lens), 50000)).astype(np.float32)
    logits = torch.from_numpy(host).to(DEV)
    got = run_topk(dsa, batch, logits)
    check_topk(got, host, wl, 2048)


@pytest.mark.parametrize("L", [4_194_304, 2_000_000, 600_000, 140_000])
def test_topk_long_rows_merge(dsa, L):
    """Rows far past one 32768-key chunk: many chunks feed the candidate merge,
    through a group level past four chunks (2M keys: 62 chunks, 16 groups;
    the 4,194,304-key maximum: 128 chunks, 32 groups, 65536 candidates in the
    final merge, which reads them without LDS staging); values repeat heavily,
    so ties decide much of the selection."""
    import sparse_attention_fp8_amd as lib
    lens = [L, L - 1000, 5000]
    qs = [0, 1, 2, 3]
    batch = lib.Batch.from_host(lens, qs, np.zeros((3, (L + 63) // 64), np.int32), 1, device=DEV)
    rng = np.random.default_rng(L)
    host = np.round(rng.normal(size=(3, L)) * 4.0).astype(np.float32)   # ~30 distinct values
    host[1, ::7] = host[1, 0]
    logits = torch.from_numpy(host).to(DEV)
    got = run_topk(dsa, batch, logits)
    ref = oracle.topk(host, np.array(lens), np.array(qs), 2048)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dist", ["grid", "narrow"])
@pytest.mark.parametrize("k", [2048, 700])
def test_topk_small_bin_ties(dsa, dist, k):
    """After two 11-bit digits the threshold bin usually holds a few keys (at
    most 64), which are ranked in one wave instead of a third digit pass.
    Every third key copies its left neighbour, so the tie rule decides inside
    that bin: with logits on a 2^-10 grid each bin holds copies of one value;
    with a narrow continuous distribution (1.5 + 0.05 N(0,1)) a bin holds a
    few distinct values and their copies."""
    lens = [2049, 3000, 9000, 16384, 24000, 32768]
    wl = synth.make_workload(lens, [1] * len(lens), 16, seed=31, spare_pages=2)
    batch, _ = to_dev(wl)
    rng = np.random.default_rng(k + (1 if dist == "grid" else 2))
    x = rng.normal(size=(len(lens), 32768))
    host = (np.round(x * 1024.0) / 1024.0 if dist == "grid" else 1.5 + 0.05 * x).astype(np.float32)
    host[:, 1::3] = host[:, 0:-1:3]
    logits = torch.from_numpy(host).to(DEV)
    got = run_topk(dsa, batch, logits, k)
    check_topk(got, host, wl, k)


def test_topk_nan_logits_stay_in_range(dsa):
    """NaN logits give an unspecified selection, but every entry must still be
    -1 or an index in [0, e_r), ascending and distinct before the -1 padding.
    The all-ones NaN maps to the excluded key, so the third row has fewer than
    k orderable keys: exactly those are returned, then -1."""
    lens = [5000, 40000, 3000]
    wl = synth.make_workload(lens, [1] * len(lens), 16, seed=37, spare_pages=2)
    batch, _ = to_dev(wl)
    rng = np.random.default_rng(5)
    host = rng.normal(size=(3, 40000)).astype(np.float32)
    bits = host.view(np.uint32)
    for pattern, frac in ((0xFFFFFFFF, 0.2), (0x7FC00000, 0.05), (0xFFC00000, 0.05)):
        mask = rng.random(size=bits.shape) < frac
        bits[mask] = pattern
    bits[2, :2000] = 0xFFFFFFFF                       # row 2: 1000 orderable keys at most
    logits = torch.from_numpy(host).to(DEV)
    got = run_topk(dsa, batch, logits)
    for r, e in enumerate(lens):
        row = got[r]
        valid = row[row >= 0]
        assert np.all(row[len(valid):] == -1), f"row {r}: -1 padding is not a suffix"
        assert np.all(valid < e) and np.all(np.diff(valid) > 0), f"row {r}: out of range or not ascending"
    orderable = np.nonzero(bits[2, :3000] != 0xFFFFFFFF)[0]
    assert np.array_equal(got[2, :len(orderable)], orderable) and np.all(got[2, len(orderable):] == -1)


@pytest.mark.parametrize("payload", [0xFFFFFFFE, 0xFFE00000, 0xFFFFFFFF])
def test_topk_negative_nan_payloads_not_taken(dsa, payload):
    """Negative NaNs with bits at or above 0xFFE00000 are never taken.  Rows
    hold exactly k orderable keys besides them (one row in one chunk, one
    across two chunks), or k orderable keys with one such NaN among the first
    k positions: the orderable keys are returned, then -1 where they run out."""
    k = 2048
    lens = [5000, 40000, 3000]
    wl = synth.make_workload(lens, [1] * len(lens), 16, seed=41, spare_pages=2)
    batch, _ = to_dev(wl)
    rng = np.random.default_rng(payload & 0xFFFF)
    host = rng.normal(size=(3, 40000)).astype(np.float32)
    bits = host.view(np.uint32)
    keep = {0: rng.choice(5000, k, replace=False), 1: rng.choice(40000, k, replace=False)}
    for r, idx in keep.items():
        nan = np.ones(lens[r], bool)
        nan[idx] = False
        bits[r, :lens[r]][nan] = payload
    bits[2, :] = 0xFFFFFFFF
    bits[2, :k] = rng.normal(size=k).astype(np.float32).view(np.uint32)
    bits[2, 100] = payload                         # k orderable keys minus one
    logits = torch.from_numpy(host).to(DEV)
    got = run_topk(dsa, batch, logits, k)
    for r in (0, 1):
        assert np.array_equal(got[r], np.sort(keep[r])), f"row {r}"
    want2 = np.array([i for i in range(k) if i != 100] + [-1])
    assert np.array_equal(got[2], want2)


def test_topk_ties_from_duplicated_pages(dsa):
    """Every logical block of a sequence maps to the same physical page, so the
    logits repeat every 64 keys: ties broken only by index."""
    wl = synth.make_workload([20000, 3000], [1, 1], 16, seed=29, spare_pages=2)
    bt = wl.block_table.clone()
    bt[0, :] = bt[0, 0]
    bt[1, :] = bt[1, 3]
    wl.block_table = bt
    batch, t = to_dev(wl)
    logits = run_indexer(dsa, wl, batch, t, 20000)
    h = logits.cpu().numpy()
    assert np.array_equal(h[0, :64], h[0, 64:128])
    got = run_topk(dsa, batch, logits)
    check_topk(got, h, wl, 2048)


# --------------------------------------------------------------------------
# sparse MLA

def mla_inputs(dsa, seq_lens, q_lens, H, seed, k=2048):
    wl = synth.make_workload(seq_lens, q_lens, H, seed=seed, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    seq, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    rng = np.random.default_rng(seed)
    idx = np.stack([oracle.topk_row(rng.normal(size=max(int(e), 1)), int(e), k) for e in ext])
    return wl, batch, t, idx


def run_mla(dsa, wl, batch, t, idx, splits):
    R, H = wl.num_rows, wl.num_heads
    out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], torch.from_numpy(idx.astype(np.int32)).to(DEV),
                          wl.softmax_scale, out, lse, num_splits=splits)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 12, 16, 32])
@pytest.mark.parametrize("H", [16, 32, 48, 64, 80, 96, 112, 128])
def test_sparse_mla_parity(dsa, H, splits):
    wl, batch, t, idx = mla_inputs(dsa, [3000, 700, 130, 2049], [1, 2, 1, 1], H, seed=H + splits)
    out, lse = run_mla(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla_oracle(wl, idx)
    check_mla(out, lse, o_ref, l_ref, f"H={H} splits={splits}")


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 16])
@pytest.mark.parametrize("k", [1, 100, 2047])
@pytest.mark.parametrize("H", [16, 64, 128])
def test_sparse_mla_parity_other_k(dsa, H, k, splits):
    """k below the 2048 maximum: a partial last tile (k % 64 != 0), a split
    width cut from fewer tiles, and rows with fewer keys than k (a -1 tail)."""
    wl, batch, t, idx = mla_inputs(dsa, [3000, 700, 130, 2049, 40], [1, 2, 1, 1, 1], H,
                                   seed=7 * k + H + splits, k=k)
    out, lse = run_mla(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla_oracle(wl, idx)
    check_mla(out, lse, o_ref, l_ref, f"H={H} k={k} splits={splits}")


def rising_scores(wl, idx, row=0):
    """Make row `row`'s scores climb with the selection position: every head's
    rope q becomes 0.5 and the rope part of the key at position p of the row's
    list becomes p // 64, so each 64-key tile adds about 2.3 to the scores
    (scale 1/sqrt(192)).  The running maximum then passes its lazy-rescale
    margin every few tiles.  The latent (value) part is left as it is."""
    wl.q_mla[row, :, 512:] = 0.5
    b = int(np.searchsorted(wl.query_start.numpy(), row, side="right")) - 1
    toks = idx[row][idx[row] >= 0].astype(np.int64)
    pos = np.nonzero(idx[row] >= 0)[0]
    pages = wl.block_table[b].numpy().astype(np.int64)[toks // 64]
    kv = wl.kv_cache.view(-1)
    base = torch.from_numpy(pages * wl.kv_cache.shape[1] + (toks % 64) * 576 + 512)
    cols = base[:, None] + torch.arange(64)[None, :]
    kv[cols.reshape(-1)] = torch.from_numpy(np.repeat((pos // 64).astype(np.float32), 64)).to(torch.bfloat16)


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("H", [16, 32, 48, 64, 128])
def test_sparse_mla_rising_scores_rescale(dsa, H, splits):
    """Scores that climb tile by tile, so the accumulators are rescaled in the
    middle of a split (random scores almost never move the maximum that far)."""
    wl = synth.make_workload([5000, 3000], [1, 2], H, seed=90 + H, spare_pages=4, poison=True)
    _, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    rng = np.random.default_rng(H)
    idx = np.stack([oracle.topk_row(rng.normal(size=max(int(e), 1)), int(e), 2048) for e in ext])
    rising_scores(wl, idx)
    batch, t = to_dev(wl)
    out, lse = run_mla(dsa, wl, batch, t, idx, splits)
    o_ref, l_ref = mla_oracle(wl, idx)
    assert l_ref[0].min() > 60.0        # the climb happened (the last tile scores about 70)
    check_mla(out, lse, o_ref, l_ref, f"H={H} splits={splits}")


def test_sparse_mla_masked_duplicate_and_invalid_entries(dsa):
    wl, batch, t, idx = mla_inputs(dsa, [5000, 600], [1, 2], 16, seed=77)
    idx = idx.copy()
    idx[0, 10:20] = idx[0, 0]            # duplicates count as listed
    idx[0, 100:400] = -1                 # masked stretch
    idx[1, 5] = 599                      # row 1 sees [0, 599): 599 is out of range
    idx[2, 7] = 10 ** 6
    idx[2, 8] = -42
    for splits in (1, 0, 7):
        out, lse = run_mla(dsa, wl, batch, t, idx, splits)
        o_ref, l_ref = mla_oracle(wl, idx)
        check_mla(out, lse, o_ref, l_ref, f"splits={splits}")


def test_sparse_mla_empty_rows(dsa):
    wl, batch, t, idx = mla_inputs(dsa, [300, 2000], [1, 1], 32, seed=5)
    idx = idx.copy()
    idx[0, :] = -1
    for splits in (1, 4):
        out, lse = run_mla(dsa, wl, batch, t, idx, splits)
        assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
        o_ref, l_ref = mla_oracle(wl, idx)
        check_mla(out, lse, o_ref, l_ref, f"splits={splits}")


def test_sparse_mla_split_matches_single_pass(dsa):
    wl, batch, t, idx = mla_inputs(dsa, [9000, 4000, 2500], [1, 1, 2], 64, seed=8)
    o1, l1 = run_mla(dsa, wl, batch, t, idx, 1)
    for s in (2, 5, 32):
        o2, l2 = run_mla(dsa, wl, batch, t, idx, s)
        d = (o1.float() - o2.float()).abs()
        assert d.max().item() <= 1.6e-2 and d.mean().item() <= 1e-3, s
        assert (l1 - l2).abs().max().item() <= 1e-4, s


def test_page_permutation_invariance_gpu(dsa):
    """Moving every physical page and rewriting the block table leaves all three
    stages bit-identical."""
    wl = synth.make_workload([4000, 2100, 90], [1, 2, 1], 16, seed=31, spare_pages=6)
    perm = torch.randperm(wl.num_pages, generator=torch.Generator().manual_seed(3))
    wl2 = synth.make_workload([4000, 2100, 90], [1, 2, 1], 16, seed=31, spare_pages=6)
    wl2.idx_cache = torch.empty_like(wl.idx_cache)
    wl2.idx_cache[perm] = wl.idx_cache
    wl2.kv_cache = torch.empty_like(wl.kv_cache)
    wl2.kv_cache[perm] = wl.kv_cache
    wl2.block_table = perm[wl.block_table.long()].to(torch.int32)
    res = []
    for w in (wl, wl2):
        batch, t = to_dev(w)
        logits = run_indexer(dsa, w, batch, t, 4000)
        idx = torch.from_numpy(run_topk(dsa, batch, logits)).to(DEV)
        out = torch.empty(w.num_rows, 16, 512, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(w.num_rows, 16, device=DEV)
        dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], idx, w.softmax_scale, out, lse)
        torch.cuda.synchronize()
        res.append((logits.cpu(), idx.cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                           b.view(torch.uint8) if b.dtype != torch.int32 else b)


def test_full_step_small(dsa):
    """indexer -> top-k -> sparse MLA chained on the GPU, each checked."""
    wl = synth.make_workload([2500, 130, 7000], [2, 1, 1], 16, seed=7, spare_pages=4, poison=True)
    batch, t = to_dev(wl)
    stride = 7000
    logits = run_indexer(dsa, wl, batch, t, stride)
    ref, mag, _ = oracle_indexer(wl, stride)
    check_logits(logits.cpu().numpy(), ref, mag, "step")
    idx = run_topk(dsa, batch, logits)
    check_topk(idx, logits.cpu().numpy(), wl, 2048)
    out, lse = run_mla(dsa, wl, batch, t, idx, 0)
    o_ref, l_ref = mla_oracle(wl, idx)
    check_mla(out, lse, o_ref, l_ref, "step")


def test_sparse_mla_workspace_reused_across_calls(dsa):
    """One workspace, never initialised (random bytes), serves consecutive split
    calls of different shapes: every call writes each partial it merges, so
    nothing left by an earlier call (or the random fill) reaches the output."""
    wa = synth.make_workload([5000, 3000, 130], [1, 1, 2], 32, seed=21, spare_pages=3, poison=True)
    wb = synth.make_workload([9000], [1], 32, seed=22, spare_pages=3, poison=True)
    ia = np.stack([np.sort(np.random.default_rng(r).choice(max(e, 1), size=2048, replace=e < 2048))
                   for r, e in enumerate(oracle.row_extents(wa.seq_lens.numpy(), wa.query_start.numpy())[1])]).astype(np.int32)
    ib = np.sort(np.random.default_rng(9).choice(9000, size=2048, replace=False))[None].astype(np.int32)
    ba, ta = to_dev(wa)
    bb, tb = to_dev(wb)
    need = max(dsa.sparse_mla_workspace_bytes(ba, 32, 2048, 8), dsa.sparse_mla_workspace_bytes(bb, 32, 2048, 3))
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, generator=torch.Generator().manual_seed(5)).to(DEV)
    for wl, batch, t, idx, splits in ((wa, ba, ta, ia, 8), (wb, bb, tb, ib, 3), (wa, ba, ta, ia, 8), (wb, bb, tb, ib, 32)):
        R, H = wl.num_rows, wl.num_heads
        out = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
        dsa.sparse_mla_decode(batch, t["q_mla"], t["kv_cache"], torch.from_numpy(idx).to(DEV), wl.softmax_scale,
                              out, lse, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        o_ref, l_ref = mla_oracle(wl, idx)
        check_mla(out, lse, o_ref, l_ref, f"reused workspace, splits={splits}")
