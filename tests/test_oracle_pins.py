"""Pins of the float64 oracle against things other than itself.

Each test checks the oracle against a library routine, a closed form, a
hand-worked value, an invariant or a brute-force computation written
independently (pure Python loops), chosen so that a dropped term, a wrong sign,
an off-by-one in the causal bound or a transposed operand fails one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

HERE = os.path.dirname(__file__)
GOLD = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))


# --------------------------------------------------------------------------
# helpers that lay explicit values out in the cache formats (no arithmetic)

def build_idx_cache(tokens_codes, tokens_scales, page_ids, num_pages, stride=synth.IDX_PAGE_BYTES):
    """tokens_codes [L,128] u8, scales [L] f32; logical block j lives in page page_ids[j]."""
    cache = np.zeros((num_pages, stride), dtype=np.uint8)
    for s in range(len(tokens_scales)):
        p, slot = page_ids[s // 64], s % 64
        cache[p, slot * 128:(slot + 1) * 128] = tokens_codes[s]
        cache[p, 8192 + 4 * slot:8192 + 4 * slot + 4] = np.array([tokens_scales[s]], np.float32).view(np.uint8)
    return cache


def build_kv_cache(rows_u16, page_ids, num_pages, stride=64 * 576):
    cache = np.zeros((num_pages, stride), dtype=np.uint16)
    for s in range(rows_u16.shape[0]):
        p, slot = page_ids[s // 64], s % 64
        cache[p, slot * 576:(slot + 1) * 576] = rows_u16[s]
    return cache


def to_bf16_bits(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_lib(codes):
    """torch's own e4m3fn -> float64 conversion (the library routine)."""
    t = torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# O1: fp8 decode

def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(codes)
    ref = fp8_lib(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_hand_values():
    for code, val in GOLD["e4m3_codes"].items():
        if code == "about":
            continue
        assert oracle.e4m3fn_decode(np.array([int(code, 16)], np.uint8))[0] == val, code
    assert oracle.e4m3fn_decode(np.array([0x7E], np.uint8))[0] == 448.0
    assert np.signbit(oracle.e4m3fn_decode(np.array([0x80], np.uint8))[0])


def test_bf16_decode_matches_torch():
    x = torch.randn(10000, dtype=torch.float32).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_decode(bits), x.to(torch.float64).numpy())


# --------------------------------------------------------------------------
# geometry

def test_row_extents_causal_bound():
    # two sequences: L=5, q_len=2 -> rows see 4 and 5 keys; L=3, q_len=3 -> 1, 2, 3
    seq, ext = oracle.row_extents([5, 3], [0, 2, 5])
    assert seq.tolist() == [0, 0, 1, 1, 1]
    assert ext.tolist() == [4, 5, 1, 2, 3]
    # q_len > L floors at 0
    _, ext = oracle.row_extents([1], [0, 3])
    assert ext.tolist() == [0, 0, 1]


# --------------------------------------------------------------------------
# O3: indexer logits

def _gold_indexer_inputs(stride=synth.IDX_PAGE_BYTES):
    g = GOLD["indexer"]
    q = np.zeros((2, 64, 128), np.uint8)
    w = np.zeros((2, 64), np.float32)
    for r, heads in g["q_codes"].items():
        for h, dims in heads.items():
            for d, c in dims.items():
                q[int(r), int(h), int(d)] = int(c, 16)
    for r, heads in g["weights"].items():
        for h, v in heads.items():
            w[int(r), int(h)] = v
    L = g["seq_len"]
    codes = np.zeros((L, 128), np.uint8)
    for s, dims in g["k_codes"].items():
        for d, c in dims.items():
            codes[int(s), int(d)] = int(c, 16)
    scales = np.array([g["k_scales"][str(s)] for s in range(L)], np.float32)
    cache = build_idx_cache(codes, scales, [1], 2, stride)
    return q, w, cache, np.array([[1]], np.int32), [L], [0, 2]


@pytest.mark.parametrize("stride", [synth.IDX_PAGE_BYTES, synth.IDX_PAGE_BYTES + 512])
def test_indexer_hand_worked(stride):
    q, w, cache, bt, sl, qs = _gold_indexer_inputs(stride)
    logits, mag, ext = oracle.indexer_logits(q, w, cache, bt, sl, qs, logits_stride=4, clean=True)
    exp = GOLD["indexer"]["expected_logits"]
    exp_mag = GOLD["indexer"]["expected_magnitudes"]
    for r in range(2):
        want = [float(v) for v in exp[str(r)]]
        got = logits[r, :3].tolist()
        assert got == want, (r, got, want)
        assert logits[r, 3] == -np.inf
        want_mag = [float(v) for v in exp_mag[str(r)]]
        assert mag[r, :len(want_mag)].tolist() == want_mag, (r, mag[r, :3], want_mag)
    assert ext.tolist() == [2, 3]


def test_indexer_dirty_leaves_tail_unwritten():
    q, w, cache, bt, sl, qs = _gold_indexer_inputs()
    logits, _, _ = oracle.indexer_logits(q, w, cache, bt, sl, qs, logits_stride=4, clean=False)
    assert np.isnan(logits[0, 2:]).all() and np.isnan(logits[1, 3:]).all()


def _brute_logit(q_codes, w, k_codes, k_scale):
    """Pure-Python loops over heads and dims; values from torch's fp8 conversion.
    Returns (logit, magnitude): the head sum with w_h, and the same sum with
    |w_h| (the scale of the logits tolerance), each times the K scale."""
    qv = fp8_lib(q_codes)
    kv = fp8_lib(k_codes)
    total = 0.0
    size = 0.0
    for h in range(64):
        dot = 0.0
        for d in range(128):
            dot += float(qv[h, d]) * float(kv[d])
        relu = dot if dot > 0.0 else 0.0
        total += float(w[h]) * relu
        size += abs(float(w[h])) * relu
    return total * float(k_scale), size * float(k_scale)


def test_indexer_matches_brute_force_loops():
    wl = synth.make_workload([70, 5], [2, 1], 16, seed=11, spare_pages=3, poison=True)
    logits, mag, ext = oracle.indexer_logits(wl.q_fp8.numpy(), wl.weights.numpy(), wl.idx_cache.numpy(),
                                             wl.block_table.numpy(), wl.seq_lens.numpy(),
                                             wl.query_start.numpy(), logits_stride=80)
    bt = wl.block_table.numpy()
    cache = wl.idx_cache.numpy()
    rng = np.random.default_rng(0)
    seq, _ = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    for r in range(3):
        for s in sorted(set(rng.integers(0, ext[r], size=6).tolist()) | {0, ext[r] - 1}):
            p, slot = bt[seq[r], s // 64], s % 64
            kc = cache[p, slot * 128:(slot + 1) * 128]
            ks = cache[p, 8192 + 4 * slot:8192 + 4 * slot + 4].view(np.float32)[0]
            want, want_mag = _brute_logit(wl.q_fp8.numpy()[r], wl.weights.numpy()[r], kc, ks)
            # both tolerances scale with the loops' own magnitude, not the oracle's
            assert abs(logits[r, s] - want) <= 1e-12 * max(1.0, want_mag), (r, s)
            assert abs(mag[r, s] - want_mag) <= 1e-12 * max(1.0, want_mag), (r, s)
            assert want_mag >= abs(want)
        assert np.all(np.isneginf(logits[r, ext[r]:]))
    assert np.isfinite(logits[0, :ext[0]]).all()


def test_indexer_one_hot_and_signed_pair_give_k_times_scale():
    """One head with w=1 and q = e_d gives relu(k_d)*scale; adding w=-1 with
    q = -e_d gives exactly k_d*scale.  Covers every finite code at every dim."""
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    L = 254
    rng = np.random.default_rng(5)
    codes = np.zeros((L, 128), np.uint8)
    for d in range(128):
        codes[:, d] = rng.permutation(finite)
    scales = rng.uniform(0.5, 2.0, size=L).astype(np.float32)
    cache = build_idx_cache(codes, scales, [2, 0, 3, 1], 4)
    bt = np.array([[2, 0, 3, 1]], np.int32)
    for d in (0, 17, 127):
        q = np.zeros((1, 64, 128), np.uint8)
        w = np.zeros((1, 64), np.float32)
        q[0, 5, d], w[0, 5] = 0x38, 1.0            # +1.0
        lg1, mag1, _ = oracle.indexer_logits(q, w, cache, bt, [L], [0, 1], L)
        kd = fp8_lib(codes[:, d]) * scales.astype(np.float64)
        assert np.array_equal(lg1[0], np.maximum(kd, 0.0))
        assert np.array_equal(mag1[0], np.maximum(kd, 0.0))      # w = +1: magnitude = logit
        q[0, 9, d], w[0, 9] = 0xB8, -1.0           # -1.0
        lg2, mag2, _ = oracle.indexer_logits(q, w, cache, bt, [L], [0, 1], L)
        assert np.array_equal(lg2[0], kd)
        # relu(k_d) from the +1 head and relu(-k_d) from the -1 head add up to |k_d|
        assert np.array_equal(mag2[0], np.abs(kd))
        w[0, 9] = -3.0                             # |w| scales its head's share
        _, mag3, _ = oracle.indexer_logits(q, w, cache, bt, [L], [0, 1], L)
        assert np.array_equal(mag3[0], np.maximum(kd, 0.0) + 3.0 * np.maximum(-kd, 0.0))


def test_indexer_all_negative_dots_give_zero():
    L = 10
    codes = np.full((L, 128), 0x38, np.uint8)      # k = +1 everywhere
    cache = build_idx_cache(codes, np.ones(L, np.float32), [0], 1)
    q = np.full((1, 64, 128), 0xB8, np.uint8)      # q = -1 everywhere
    w = np.random.default_rng(1).normal(size=(1, 64)).astype(np.float32)
    lg, mag, _ = oracle.indexer_logits(q, w, cache, np.array([[0]]), [L], [0, 1], L)
    assert np.array_equal(lg[0], np.zeros(L)) and np.array_equal(mag[0], np.zeros(L))


def test_indexer_magnitude_bounds_and_same_sign_weights():
    """magnitude >= |logit| everywhere; with every weight >= 0 it equals the
    logit, with every weight <= 0 it equals -logit (closed forms of |w|)."""
    wl = synth.make_workload([300, 70], [2, 1], 16, seed=13, spare_pages=2)
    q8, w = wl.q_fp8.numpy(), wl.weights.numpy()
    rest = (wl.idx_cache.numpy(), wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(), 304)
    lg, mag, _ = oracle.indexer_logits(q8, w, *rest)
    fin = np.isfinite(lg)
    assert np.all(mag[fin] >= np.abs(lg[fin]))
    assert np.any(mag[fin] > np.abs(lg[fin]) * (1 + 1e-6))   # mixed-sign weights cancel somewhere
    for sign in (1.0, -1.0):
        ws = (sign * np.abs(w)).astype(np.float32)
        lg_s, mag_s, _ = oracle.indexer_logits(q8, ws, *rest)
        assert np.allclose(sign * lg_s[fin], mag_s[fin], rtol=1e-15, atol=0)
        assert np.array_equal(mag_s[fin], mag[fin])      # magnitude ignores the weights' signs


def test_indexer_page_permutation_invariance():
    wl = synth.make_workload([200, 64, 1], [1, 2, 1], 16, seed=3, spare_pages=4)
    args = (wl.q_fp8.numpy(), wl.weights.numpy())
    base, _, _ = oracle.indexer_logits(*args, wl.idx_cache.numpy(), wl.block_table.numpy(),
                                       wl.seq_lens.numpy(), wl.query_start.numpy(), 256)
    perm = np.random.default_rng(7).permutation(wl.num_pages)
    cache2 = np.zeros_like(wl.idx_cache.numpy())
    cache2[perm] = wl.idx_cache.numpy()
    bt2 = perm[wl.block_table.numpy()]
    moved, _, _ = oracle.indexer_logits(*args, cache2, bt2, wl.seq_lens.numpy(), wl.query_start.numpy(), 256)
    assert np.array_equal(base, moved)


def test_indexer_out_of_range_page_is_masked():
    q, w, cache, bt, sl, qs = _gold_indexer_inputs()
    lg, _, _ = oracle.indexer_logits(q, w, cache, np.array([[7]]), sl, qs, 4)
    assert np.all(np.isneginf(lg))


# --------------------------------------------------------------------------
# O4: top-k

def _brute_topk(vals, e, k):
    """Repeatedly take the largest remaining value, lowest index first."""
    remaining = list(range(e))
    chosen = []
    for _ in range(min(k, e)):
        best = remaining[0]
        for s in remaining[1:]:
            if vals[s] > vals[best]:
                best = s
        chosen.append(best)
        remaining.remove(best)
    return sorted(chosen) + [-1] * (k - len(chosen))


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(0)
    pool = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, -np.inf, 3.5])
    for trial in range(300):
        e = int(rng.integers(0, 40))
        k = int(rng.integers(1, 45))
        vals = rng.choice(pool, size=max(e, 1) + 3)
        got = oracle.topk_row(vals, e, k).tolist()
        assert got == _brute_topk(vals.tolist(), e, k), (trial, e, k)


def test_topk_signed_zero_ties_go_to_lower_index():
    vals = np.array([0.0, -0.0, 0.0, -0.0, 1.0])
    assert oracle.topk_row(vals, 5, 3).tolist() == [0, 1, 4]
    vals = np.array([-0.0, 0.0, 5.0])
    assert oracle.topk_row(vals, 3, 2).tolist() == [0, 2]


def test_topk_short_row_is_identity():
    vals = np.random.default_rng(2).normal(size=3000)
    for e in (0, 1, 63, 2047, 2048):
        got = oracle.topk_row(vals, e, 2048)
        assert got[:e].tolist() == list(range(e)) and np.all(got[e:] == -1)


def test_topk_hand_worked():
    g = GOLD["indexer"]
    q, w, cache, bt, sl, qs = _gold_indexer_inputs()
    lg, _, _ = oracle.indexer_logits(q, w, cache, bt, sl, qs, 4)
    for key, rows in g["expected_topk"].items():
        k = int(key[1:])
        got = oracle.topk(lg, sl, qs, k)
        for r, want in rows.items():
            assert got[int(r)].tolist() == want, (key, r)


def test_topk_full_sort_reference():
    """Against a full descending sort (stable on index) of random rows."""
    rng = np.random.default_rng(9)
    for _ in range(20):
        e = int(rng.integers(2049, 6000))
        vals = rng.normal(size=e).astype(np.float32)
        vals[rng.integers(0, e, size=200)] = vals[0]             # plant ties
        order = sorted(range(e), key=lambda s: (-float(vals[s]), s))
        assert oracle.topk_row(vals, e, 2048).tolist() == sorted(order[:2048])


# --------------------------------------------------------------------------
# O5/O6: sparse MLA

def _gold_mla_inputs():
    g = GOLD["sparse_mla"]
    rows = np.zeros((g["seq_len"], 576), np.float32)
    for s, dims in g["rows"].items():
        for d, v in dims.items():
            rows[int(s), int(d)] = v
    kv = build_kv_cache(to_bf16_bits(rows), [0], 2)
    q = np.zeros((1, 1, 576), np.float32)
    for d, v in g["q"].items():
        q[0, 0, int(d)] = v
    return to_bf16_bits(q), kv, np.array([[0]], np.int32), [g["seq_len"]], [0, 1], g["scale"]


def test_sparse_mla_hand_worked():
    q, kv, bt, sl, qs, scale = _gold_mla_inputs()
    for case in GOLD["sparse_mla"]["cases"]:
        idx = np.array([case["indices"]])
        for fn in (lambda: oracle.sparse_mla(q, kv, bt, sl, qs, idx, scale),
                   lambda: oracle.sparse_mla_split(q, kv, bt, sl, qs, idx, scale, 2)):
            out, lse = fn()
            want = np.zeros(512)
            env = {"e": math.e, "log": math.log, "inf": math.inf}
            for d, expr in case["expected"]["out"].items():
                want[int(d)] = eval(expr, env)
            lse_want = eval(case["expected"]["lse"], env)
            assert np.allclose(out[0, 0], want, rtol=0, atol=1e-14), case["indices"]
            if np.isinf(lse_want):
                assert lse[0, 0] == lse_want
            else:
                assert abs(lse[0, 0] - lse_want) < 1e-14


def _mla_workload(seq_lens, q_lens, H, seed, **kw):
    return synth.make_workload(seq_lens, q_lens, H, seed, spare_pages=3, poison=True, **kw)


def test_sparse_mla_short_context_equals_dense_attention():
    """e_r <= k: the identity index list makes sparse MLA dense causal attention
    (torch scaled_dot_product_attention in float64 on the gathered rows)."""
    wl = _mla_workload([300, 77], [2, 1], 16, seed=4)
    seq, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    idx = np.stack([oracle.topk_row(np.zeros(400), int(e), 2048) for e in ext])
    out, lse = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                 wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                 idx, wl.softmax_scale)
    kv = wl.kv_cache.to(torch.float64)
    for r in range(wl.num_rows):
        b, e = seq[r], int(ext[r])
        pages = wl.block_table[b, :(e + 63) // 64].long()
        C = kv[pages, :64 * 576].reshape(-1, 576)[:e]
        qh = wl.q_mla[r].to(torch.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qh[None, :, None, :], C[None, None, :, :].expand(1, 16, e, 576),
            C[None, None, :, :512].expand(1, 16, e, 512), scale=wl.softmax_scale)[0, :, 0, :]
        assert np.allclose(out[r], ref.numpy(), rtol=0, atol=1e-12)
        z = wl.softmax_scale * (qh @ C.T)
        assert np.allclose(lse[r], torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)


def test_sparse_mla_special_cases():
    wl = _mla_workload([50], [1], 16, seed=8)
    qb = wl.q_mla.view(torch.int16).numpy().copy()
    kvb = wl.kv_cache.view(torch.int16).numpy()
    args = (kvb, wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy())
    kv = wl.kv_cache.to(torch.float64)
    page = int(wl.block_table[0, 0])
    rows = kv[page, :64 * 576].reshape(64, 576)
    # one valid index: out = v, lse = z
    idx = np.array([[-1, 7, 99, -1]])
    out, lse = oracle.sparse_mla(qb, *args, idx, wl.softmax_scale)
    assert np.allclose(out[0], rows[7, :512].numpy()[None, :].repeat(16, 0), atol=0)
    z = wl.softmax_scale * (wl.q_mla[0].to(torch.float64) @ rows[7])
    assert np.allclose(lse[0], z.numpy(), atol=1e-12)
    # q = 0: uniform weights -> mean of V, lse = ln n
    q0 = np.zeros_like(qb)
    sel = [3, 9, 10, 49]
    out, lse = oracle.sparse_mla(q0, *args, np.array([sel]), wl.softmax_scale)
    assert np.allclose(out[0], rows[sel, :512].mean(0).numpy()[None, :], atol=1e-14)
    assert np.allclose(lse[0], math.log(4), atol=1e-14)


def test_sparse_mla_brute_force_loops():
    wl = _mla_workload([130], [2], 16, seed=12)
    rng = np.random.default_rng(3)
    seq, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    idx = rng.integers(-3, 135, size=(2, 24))
    idx[0, :3] = [5, 5, 129]          # a duplicate, and key 129 = just past row 0's bound (e = 129)
    idx[1, :2] = [129, 0]             # key 129 is row 1's last key (e = 130)
    out, lse = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                 wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                 idx, wl.softmax_scale)
    kvf = wl.kv_cache.float().numpy()
    qf = wl.q_mla.float().numpy()
    bt = wl.block_table.numpy()
    for r in range(2):
        valid = [int(s) for s in idx[r] if 0 <= s < ext[r]]
        for h in (0, 7, 15):
            zs, vs = [], []
            for s in valid:
                row = kvf[bt[0, s // 64], (s % 64) * 576:(s % 64 + 1) * 576]
                zs.append(wl.softmax_scale * sum(float(qf[r, h, d]) * float(row[d]) for d in range(576)))
                vs.append(row[:512])
            M = max(zs)
            ws = [math.exp(z - M) for z in zs]
            Ls = sum(ws)
            ref = sum(w * v.astype(np.float64) for w, v in zip(ws, vs)) / Ls
            assert np.allclose(out[r, h], ref, atol=1e-12)
            assert abs(lse[r, h] - (M + math.log(Ls))) < 1e-12


@pytest.mark.parametrize("splits", [1, 2, 3, 16, 32])
def test_sparse_mla_split_equals_single_pass(splits):
    wl = _mla_workload([3000, 700, 64], [1, 2, 1], 32, seed=21)
    rng = np.random.default_rng(splits)
    seq, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    idx = np.stack([oracle.topk_row(rng.normal(size=4000), int(e), 2048) for e in ext])
    idx[1, 5:400] = -1                                   # a masked stretch
    a = (wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(), wl.block_table.numpy(),
         wl.seq_lens.numpy(), wl.query_start.numpy(), idx, wl.softmax_scale)
    o1, l1 = oracle.sparse_mla(*a)
    o2, l2 = oracle.sparse_mla_split(*a, splits)
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_sparse_mla_page_permutation_invariance():
    wl = _mla_workload([500, 90], [1, 1], 16, seed=5)
    seq, ext = oracle.row_extents(wl.seq_lens.numpy(), wl.query_start.numpy())
    idx = np.stack([oracle.topk_row(np.arange(600.0)[::-1], int(e), 256) for e in ext])
    q = wl.q_mla.view(torch.int16).numpy()
    kv = wl.kv_cache.view(torch.int16).numpy()
    base = oracle.sparse_mla(q, kv, wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                             idx, wl.softmax_scale)
    perm = np.random.default_rng(1).permutation(wl.num_pages)
    kv2 = np.zeros_like(kv)
    kv2[perm] = kv
    moved = oracle.sparse_mla(q, kv2, perm[wl.block_table.numpy()], wl.seq_lens.numpy(),
                              wl.query_start.numpy(), idx, wl.softmax_scale)
    assert np.array_equal(base[0], moved[0]) and np.array_equal(base[1], moved[1])


def test_sparse_mla_empty_row():
    wl = _mla_workload([10], [1], 16, seed=2)
    out, lse = oracle.sparse_mla(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                 wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                 np.full((1, 8), -1), wl.softmax_scale)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    out, lse = oracle.sparse_mla_split(wl.q_mla.view(torch.int16).numpy(), wl.kv_cache.view(torch.int16).numpy(),
                                       wl.block_table.numpy(), wl.seq_lens.numpy(), wl.query_start.numpy(),
                                       np.full((1, 8), -1), wl.softmax_scale, 4)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
