"""Pins of the oracle's quantiser and cache writers against things other than
themselves: torch's own float8_e4m3fn cast, a brute-force nearest-code search,
values worked by hand from the OCP E4M3 definition, the reconstruction bound
of a 3-bit mantissa, and the cache layouts written out by explicit loops.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_oracle_pins import build_idx_cache, build_kv_cache, to_bf16_bits


def torch_e4m3(y):
    """torch's float32 -> e4m3fn conversion (the library routine), as bytes."""
    t = torch.tensor(np.asarray(y, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def grid():
    return oracle.e4m3fn_decode(np.arange(127, dtype=np.uint8))


# --------------------------------------------------------------------------
# e4m3fn encode

def test_encode_matches_torch_on_codes_midpoints_and_neighbours():
    g = grid()
    mids = (g[:-1] + g[1:]) / 2                       # every tie, exact in fp32
    vals = np.concatenate([g, mids]).astype(np.float32)
    up = np.nextafter(vals, np.float32(np.inf))
    dn = np.nextafter(vals, np.float32(-np.inf))
    rng = np.random.default_rng(5)
    rand = (rng.choice([-1, 1], 20000) * np.exp2(rng.uniform(-13, np.log2(448), 20000))).astype(np.float32)
    y = np.concatenate([vals, up, dn, -vals, -up, -dn, rand, np.float32([0.0, -0.0])])
    y = y[np.abs(y) <= 448]
    assert np.array_equal(oracle.e4m3fn_encode(y), torch_e4m3(y))


def test_encode_brute_force_nearest_code():
    """Nearest of all finite codes by exhaustive search, ties to the even code."""
    rng = np.random.default_rng(9)
    y = (rng.standard_normal(3000) * 40).astype(np.float32)
    y = np.concatenate([y, ((np.arange(-40, 41) + 0.5) * 2.0 ** -9).astype(np.float32)])
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = {c: float(oracle.e4m3fn_decode(np.uint8(c))) for c in finite}
    for v in y.astype(np.float64):
        best = None
        for c in finite:
            if (c >> 7) != int(np.signbit(v)):      # sign kept, zero included
                continue
            d = abs(vals[c] - v)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
                best = (d, c)
        assert oracle.e4m3fn_encode(v) == best[1], v


def test_encode_saturates_and_keeps_sign():
    big = np.float32([448.0, 449.0, 464.0, 479.99, 480.0, 1.0e6, 3.0e38])
    assert set(oracle.e4m3fn_encode(big).tolist()) == {0x7E}
    assert set(oracle.e4m3fn_encode(-big).tolist()) == {0xFE}
    assert oracle.e4m3fn_encode(np.float32(-0.0)) == 0x80
    assert oracle.e4m3fn_encode(np.float32(-2.0 ** -11)) == 0x80     # rounds to -0
    assert oracle.e4m3fn_encode(np.float32(np.nan)) == 0x7F


# --------------------------------------------------------------------------
# per-group quantiser

def test_quantize_hand_worked_group():
    """amax 56 gives the exact scale 56 / 448 = 0.125, so y = 8x exactly.
    Codes from the format: 448 = 1.75 * 2^8 -> e 15, m 6 -> 0x7E; 8 = 2^3 ->
    e 10, m 0 -> 0x50; y 8.5 ties 8 (0x50) / 9 (0x51) -> even 0x50; y 9.5 ties
    9 / 10 -> 0x52; y 17 ties 16 (0x58) / 18 (0x59) -> 0x58; y 0.5 -> e 6 ->
    0x30; y 2^-9 is the least subnormal 0x01; y 2^-10 ties 0 / 2^-9 -> 0x00;
    y 1.5 * 2^-9 ties codes 1 / 2 -> 0x02; y -112 = -1.75 * 2^6 -> 0xEE."""
    x = [56.0, 1.0, 1.0625, 1.1875, 2.125, 0.0625, 2.0 ** -12, 2.0 ** -13, 3 * 2.0 ** -13, -14.0, -56.0]
    want = [0x7E, 0x50, 0x50, 0x52, 0x58, 0x30, 0x01, 0x00, 0x02, 0xEE, 0xFE]
    grp = np.zeros(128, np.float32)
    grp[:len(x)] = x
    codes, scale = oracle.quantize_groups_fp8(to_bf16_bits(grp)[None])
    assert scale[0] == np.float32(0.125)
    assert codes[0, :len(x)].tolist() == want
    assert not codes[0, len(x):].any()


def test_quantize_zero_group_takes_unit_scale():
    z = np.zeros((2, 128), np.float32)
    z[1] = -0.0
    codes, scale = oracle.quantize_groups_fp8(to_bf16_bits(z))
    assert scale.tolist() == [1.0, 1.0]
    assert not codes[0].any() and (codes[1] == 0x80).all()


@pytest.mark.parametrize("spread", [1.0, 12.0])
def test_quantize_reconstruction_bound_and_full_range(spread):
    """Each nonzero group uses the top code 448, and dec(code) * scale is within
    half a unit in the last place of x: 2^-4 |x| for normals (3-bit mantissa),
    2^-10 * scale in the subnormal range (plus fp32 slack)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 128)) * np.exp2(rng.uniform(-spread, spread, (200, 128)))
    bits = to_bf16_bits(x)
    xe = oracle.bf16_decode(bits)
    codes, scale = oracle.quantize_groups_fp8(bits)
    rec = oracle.e4m3fn_decode(codes) * scale[:, None].astype(np.float64)
    assert (np.abs(oracle.e4m3fn_decode(codes)).max(axis=1) == 448.0).all()
    bound = np.maximum(2.0 ** -4 * np.abs(xe), 2.0 ** -10 * scale[:, None]) * (1 + 2.0 ** -18)
    assert (np.abs(rec - xe) <= bound).all()


def test_quantize_equals_torch_cast_path():
    """The same groups through torch's fp32 arithmetic and its e4m3fn cast."""
    g = torch.Generator().manual_seed(2)
    x = torch.randn(64, 128, generator=g).to(torch.bfloat16)
    x[3] = 0
    xf = x.float()
    amax = xf.abs().amax(dim=-1, keepdim=True)
    sc = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    want = (xf / sc).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes, scale = oracle.quantize_groups_fp8(x.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(codes, want)
    assert np.array_equal(scale, sc.squeeze(-1).numpy())


def test_q_quant_weight_fold_preserves_logits():
    """Folding s_q into w keeps sum_h w relu(q . k) within the quantisation
    bound; folding 1/s_q, or not folding, would be off by orders of magnitude."""
    rng = np.random.default_rng(4)
    R, n = 3, 50
    q = to_bf16_bits(rng.standard_normal((R, 64, 128)))
    w = (rng.standard_normal((R, 64)) / 8).astype(np.float32)
    k = rng.standard_normal((n, 128))
    codes, w2 = oracle.indexer_q_quant(q, w)
    _, s = oracle.quantize_groups_fp8(q)
    assert np.array_equal(w2, (w * s).astype(np.float32))
    Q = oracle.bf16_decode(q)
    Q8 = oracle.e4m3fn_decode(codes)
    for r in range(R):
        exact = w[r].astype(np.float64) @ np.maximum(Q[r] @ k.T, 0)
        quant = w2[r].astype(np.float64) @ np.maximum(Q8[r] @ k.T, 0)
        err_dot = (2.0 ** -4 * np.abs(Q[r]) + 2.0 ** -10 * s[r][:, None]) @ np.abs(k.T)
        bound = np.abs(w[r]).astype(np.float64) @ err_dot * 1.01 + 1e-9
        assert (np.abs(quant - exact) <= bound).all()
        assert np.abs(quant - exact).max() < 0.1 * np.abs(exact).max()


# --------------------------------------------------------------------------
# cache writers

def slot_case(num_pages, T, rng):
    """Distinct slots on random pages, two padding tokens (-1) and one slot past
    the last page."""
    slots = rng.choice(num_pages * 64, size=T, replace=False).astype(np.int64)
    slots[1] = -1
    slots[T // 2] = -1
    slots[-1] = num_pages * 64 + 5
    return slots


def test_k_writer_matches_explicit_layout():
    rng = np.random.default_rng(6)
    num_pages, T, stride = 5, 70, synth.IDX_PAGE_BYTES + 48
    cache0 = rng.integers(0, 256, (num_pages, stride), dtype=np.uint8)
    k = to_bf16_bits(rng.standard_normal((T, 128)))
    slots = slot_case(num_pages, T, rng)
    got = oracle.indexer_k_quant_and_cache(k, slots, cache0)
    codes, scale = oracle.quantize_groups_fp8(k)
    want = cache0.copy()
    for t in range(T):
        s = int(slots[t])
        if s < 0 or s >= num_pages * 64:
            continue
        page_ids = list(range(num_pages))
        one = build_idx_cache(codes[t:t + 1], scale[t:t + 1], page_ids, num_pages, stride)
        p, sl = s // 64, s % 64
        want[p, sl * 128:(sl + 1) * 128] = one[0, :128]
        want[p, 8192 + 4 * sl:8192 + 4 * sl + 4] = one[0, 8192:8196]
    assert np.array_equal(got, want)


def test_k_writer_round_trips_through_the_reader():
    """Write a whole sequence through a permuted block table, read it back with
    the indexer's own key reader: the codes and scales of the quantiser."""
    rng = np.random.default_rng(8)
    L, num_pages = 150, 6
    bt = rng.permutation(num_pages)[:3]
    k = to_bf16_bits(rng.standard_normal((L, 128)) * 3)
    s = np.arange(L)
    slots = bt[s // 64] * 64 + s % 64
    cache = oracle.indexer_k_quant_and_cache(k, slots, np.zeros((num_pages, synth.IDX_PAGE_BYTES), np.uint8))
    codes, scales = oracle.indexer_keys(cache, bt, s)
    want_c, want_s = oracle.quantize_groups_fp8(k)
    assert np.array_equal(codes, want_c) and np.array_equal(scales, want_s.astype(np.float64))


def test_latent_writer_matches_explicit_layout():
    rng = np.random.default_rng(7)
    num_pages, T, stride = 4, 90, 64 * 576 + 8
    cache0 = rng.integers(0, 65536, (num_pages, stride), dtype=np.uint16)
    lat = rng.integers(0, 65536, (T, 512), dtype=np.uint16)
    rope = rng.integers(0, 65536, (T, 64), dtype=np.uint16)
    slots = slot_case(num_pages, T, rng)
    got = oracle.latent_cache_write(lat, rope, slots, cache0)
    want = cache0.copy()
    for t in range(T):
        s = int(slots[t])
        if 0 <= s < num_pages * 64:
            row = np.concatenate([lat[t], rope[t]])
            one = build_kv_cache(row[None], [0], 1, stride)
            want[s // 64, (s % 64) * 576:(s % 64 + 1) * 576] = one[0, :576]
    assert np.array_equal(got, want)


# --------------------------------------------------------------------------
# fp8 latent cache

def test_fp8_latent_writer_matches_explicit_layout_and_round_trips():
    rng = np.random.default_rng(11)
    num_pages, T, stride = 3, 70, oracle.KV8_PAGE_BYTES + 64
    cache0 = rng.integers(0, 256, (num_pages, stride), dtype=np.uint8)
    lat_f = rng.standard_normal((T, 512)) * np.exp2(rng.integers(-4, 5, (T, 4))).repeat(128, axis=1)
    lat = to_bf16_bits(lat_f)
    rope = to_bf16_bits(rng.standard_normal((T, 64)))
    slots = slot_case(num_pages, T, rng)
    got = oracle.latent_cache_write_fp8(lat, rope, slots, cache0)
    want = cache0.copy()
    for t in range(T):
        s = int(slots[t])
        if not 0 <= s < num_pages * 64:
            continue
        p, sl = s // 64, s % 64
        for g in range(4):
            codes, scale = oracle.quantize_groups_fp8(lat[t, 128 * g:128 * (g + 1)][None])
            want[p, sl * 640 + 128 * g:sl * 640 + 128 * (g + 1)] = codes[0]
            want[p, 40960 + 16 * sl + 4 * g:40960 + 16 * sl + 4 * g + 4] = np.float32(scale[0]).reshape(1).view(np.uint8)
        want[p, sl * 640 + 512:sl * 640 + 640] = rope[t].view(np.uint8)
    assert np.array_equal(got, want)
    ok = (slots >= 0) & (slots < num_pages * 64)
    rows = oracle.kv8_rows(got, slots[ok] // 64, slots[ok] % 64)
    x = oracle.bf16_decode(lat[ok])
    sc = np.abs(x).reshape(-1, 4, 128).max(axis=2).repeat(128, axis=1) / 448
    assert (np.abs(rows[:, :512] - x) <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sc) * 1.0001).all()
    assert np.array_equal(rows[:, 512:], oracle.bf16_decode(rope[ok]))


def exact_fp8_latent(rng, T):
    """Latent rows whose every group is an e4m3 value times a power of two, with
    one element on the top code: the quantiser reproduces them exactly."""
    codes = rng.integers(0, 0x7F, (T, 4, 128)).astype(np.uint8) | (rng.integers(0, 2, (T, 4, 128)) << 7).astype(np.uint8)
    codes[:, :, 0] = 0x7E
    e = rng.integers(-8, 4, (T, 4, 1))
    return (oracle.e4m3fn_decode(codes) * np.exp2(e)).reshape(T, 512)


def test_fp8_cache_mla_equals_bf16_cache_mla_on_exactly_representable_rows():
    """Rows the fp8 format holds exactly (and bf16 too): sparse MLA over the fp8
    cache must equal sparse MLA over a bf16 cache of the same values."""
    rng = np.random.default_rng(12)
    seq_lens, q_lens, H = [300, 2200], [1, 2], 16
    wl = synth.make_workload(seq_lens, q_lens, H, seed=3, spare_pages=2)
    L = sum(seq_lens)
    lat = exact_fp8_latent(rng, L)
    rope = rng.standard_normal((L, 64))
    bt = wl.block_table.numpy()
    slots = np.concatenate([bt[b, np.arange(n) // 64].astype(np.int64) * 64 + np.arange(n) % 64
                            for b, n in enumerate(seq_lens)])
    kv8 = oracle.latent_cache_write_fp8(to_bf16_bits(lat), to_bf16_bits(rope), slots,
                                        np.zeros((wl.num_pages, oracle.KV8_PAGE_BYTES), np.uint8))
    kv16 = oracle.latent_cache_write(to_bf16_bits(lat), to_bf16_bits(rope), slots,
                                     np.zeros((wl.num_pages, 64 * 576), np.uint16))
    assert np.array_equal(oracle.kv8_rows(kv8, slots // 64, slots % 64),
                          oracle.bf16_decode(kv16.reshape(-1, 576)[slots // 64 * 64 + slots % 64]))
    idx = np.stack([np.sort(rng.choice(int(e), size=min(2048, int(e)), replace=False).tolist() +
                            [-1] * (2048 - min(2048, int(e)))) for e in wl.row_extents()])
    idx = np.where(idx < 0, -1, idx)
    q = wl.q_mla.view(torch.int16).numpy()
    args = (bt, wl.seq_lens.numpy(), wl.query_start.numpy(), idx, wl.softmax_scale)
    o8, l8 = oracle.sparse_mla(q, kv8, *args, kv_format="fp8")
    o16, l16 = oracle.sparse_mla(q, kv16, *args)
    assert np.array_equal(o8, o16) and np.array_equal(l8, l16)
    o8s, l8s = oracle.sparse_mla_split(q, kv8, *args, 5, kv_format="fp8")
    assert np.allclose(o8s, o8, atol=1e-12) and np.allclose(l8s, l8, atol=1e-12)
