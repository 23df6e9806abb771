"""GPU parity of the quantiser and the cache writers against the oracle.

Bar: bit-exact.  The codes are integers decided in IEEE fp32 on both sides
(amax, scale = amax / 448, x / scale, round to nearest even), the folded
weight is one fp32 multiply and the writers copy bytes, so every output byte
must match.  Inputs cover exact rounding ties (power-of-two scales with values
on e4m3 midpoints), e4m3 subnormals and underflow to zero, all-zero and -0
groups, strided source rows, padding slots (-1) and slots past the cache, on
caches filled with random bytes so a stray or missing write shows up.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_fp8_amd import synth

from test_gpu_parity import DEV, check_logits, to_dev

pytestmark = pytest.mark.gpu


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).numpy().view(np.uint16)


def tricky_groups(n, seed):
    """[n, 128] bf16 groups: random normals, plus groups built on a power-of-two
    scale whose values sit on e4m3 codes and midpoints (exact ties), tiny
    values (subnormal codes, underflow), an all-zero and an all -0 group."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 128, generator=g) * torch.exp2(torch.randint(-6, 7, (n, 1), generator=g).float())
    grid = oracle.e4m3fn_decode(np.arange(127, dtype=np.uint8))
    mids = np.concatenate([grid, (grid[:-1] + grid[1:]) / 2])
    rng = np.random.default_rng(seed)
    for i in range(0, n, 3):
        e = int(rng.integers(-24, 12))
        y = rng.choice(mids, 128) * rng.choice([-1.0, 1.0], 128)
        y[int(rng.integers(128))] = 448.0          # amax = 448 * 2^e -> scale 2^e exactly
        x[i] = torch.tensor(y * 2.0 ** e, dtype=torch.float32)
    if n > 2:
        x[1] = 0.0
        x[2] = -0.0
    if n > 4:
        x[4, 1:] *= 1e-4                            # large dynamic range: subnormals, zeros
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("R", [1, 5, 37, 300])
def test_q_quant_bit_exact(dsa, R):
    q = tricky_groups(R * 64, seed=R).reshape(R, 64, 128)
    w = torch.randn(R, 64, generator=torch.Generator().manual_seed(R + 1)) / 8
    codes, w2 = dsa.indexer_q_quant_fp8(q.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    want_c, want_w = oracle.indexer_q_quant(bf16_bits(q), w.numpy())
    got_c = codes.cpu().numpy()
    bad = np.nonzero(got_c != want_c)
    assert bad[0].size == 0, (f"{bad[0].size} codes differ, first at {tuple(int(b[0]) for b in bad)}: "
                              f"gpu {got_c[bad][0]:#04x} oracle {want_c[bad][0]:#04x}")
    assert np.array_equal(w2.cpu().numpy().view(np.uint32), want_w.view(np.uint32))


def test_q_quant_in_place_weights(dsa):
    R = 9
    q = tricky_groups(R * 64, seed=99).reshape(R, 64, 128)
    w = torch.randn(R, 64, generator=torch.Generator().manual_seed(3)) / 8
    wd = w.to(DEV)
    codes, w2 = dsa.indexer_q_quant_fp8(q.to(DEV), wd, weights_out=wd)
    torch.cuda.synchronize()
    assert w2.data_ptr() == wd.data_ptr()
    want_c, want_w = oracle.indexer_q_quant(bf16_bits(q), w.numpy())
    assert np.array_equal(codes.cpu().numpy(), want_c)
    assert np.array_equal(wd.cpu().numpy().view(np.uint32), want_w.view(np.uint32))


def slots_for(num_pages, T, rng):
    slots = rng.choice(num_pages * 64, size=T, replace=False).astype(np.int64)
    slots[rng.choice(T, size=max(1, T // 50), replace=False)] = -1
    slots[-1] = num_pages * 64 + 3                  # past the cache: skipped
    return slots


@pytest.mark.parametrize("T,num_pages,k_stride,page_pad", [(1, 3, 128, 0), (61, 3, 128, 0),
                                                           (1000, 40, 136, 48), (4097, 70, 256, 0)])
def test_k_quant_and_cache_bit_exact(dsa, T, num_pages, k_stride, page_pad):
    rng = np.random.default_rng(T)
    stride = synth.IDX_PAGE_BYTES + page_pad
    cache0 = rng.integers(0, 256, (num_pages, stride), dtype=np.uint8)
    wide = tricky_groups(T, seed=T + 7)
    kbuf = torch.zeros(T, k_stride, dtype=torch.bfloat16)
    kbuf[:, :128] = wide
    kbuf[:, 128:] = float("nan")                    # never read
    slots = slots_for(num_pages, T, rng)
    cache = torch.from_numpy(cache0.copy()).to(DEV)
    dsa.indexer_k_quant_and_cache(kbuf.to(DEV)[:, :128], torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    want = oracle.indexer_k_quant_and_cache(bf16_bits(wide), slots, cache0)
    got = cache.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, f"{bad.shape[0]} cache bytes differ, first at page/byte {tuple(bad[0])}"


@pytest.mark.parametrize("T,num_pages,lat_stride,rope_stride,page_pad", [(1, 2, 512, 64, 0), (100, 3, 576, 64, 8),
                                                                         (3000, 60, 1024, 72, 0)])
def test_latent_cache_write_bit_exact(dsa, T, num_pages, lat_stride, rope_stride, page_pad):
    rng = np.random.default_rng(T + 1)
    stride = 64 * 576 + page_pad
    cache0 = rng.integers(0, 65536, (num_pages, stride), dtype=np.uint16)
    lat = rng.integers(0, 65536, (T, lat_stride), dtype=np.uint16)
    rope = rng.integers(0, 65536, (T, rope_stride), dtype=np.uint16)
    slots = slots_for(num_pages, T, rng)
    as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    cache = as_bf16(cache0.copy())
    dsa.latent_cache_write(as_bf16(lat)[:, :512], as_bf16(rope)[:, :64], torch.from_numpy(slots).to(DEV), cache)
    torch.cuda.synchronize()
    want = oracle.latent_cache_write(lat[:, :512], rope[:, :64], slots, cache0)
    got = cache.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_writers_accept_empty_calls(dsa):
    cache = torch.zeros(2, synth.IDX_PAGE_BYTES, dtype=torch.uint8, device=DEV)
    dsa.indexer_k_quant_and_cache(torch.empty(0, 128, dtype=torch.bfloat16, device=DEV),
                                  torch.empty(0, dtype=torch.int64, device=DEV), cache)
    kv = torch.zeros(2, 64 * 576, dtype=torch.bfloat16, device=DEV)
    dsa.latent_cache_write(torch.empty(0, 512, dtype=torch.bfloat16, device=DEV),
                           torch.empty(0, 64, dtype=torch.bfloat16, device=DEV),
                           torch.empty(0, dtype=torch.int64, device=DEV), kv)
    c, w = dsa.indexer_q_quant_fp8(torch.empty(0, 64, 128, dtype=torch.bfloat16, device=DEV),
                                   torch.empty(0, 64, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert not cache.any() and not kv.view(torch.int16).any() and c.numel() == 0


def test_closed_loop_from_bf16_to_logits(dsa):
    """bf16 q and bf16 K tokens -> quantiser and K writer on the GPU -> paged
    indexer; the written cache must equal the oracle's byte for byte and the
    logits must match the oracle's logits over the oracle's own quantised
    inputs."""
    wl = synth.make_workload([700, 64, 1500], [1, 2, 1], 16, seed=21, spare_pages=3)
    g = torch.Generator().manual_seed(5)
    R, L = wl.num_rows, wl.seq_lens.numpy()
    q = torch.randn(R, 64, 128, generator=g).to(torch.bfloat16)
    w = torch.randn(R, 64, generator=g) / 8
    toks = [torch.randn(int(n), 128, generator=g).to(torch.bfloat16) for n in L]
    bt = wl.block_table.numpy()
    slots = np.concatenate([bt[b, np.arange(n) // 64].astype(np.int64) * 64 + np.arange(n) % 64
                            for b, n in enumerate(L)])
    kall = torch.cat(toks)
    cache0 = np.zeros((wl.num_pages, synth.IDX_PAGE_BYTES), np.uint8)
    cache = torch.from_numpy(cache0).to(DEV)
    dsa.indexer_k_quant_and_cache(kall.to(DEV), torch.from_numpy(slots).to(DEV), cache)
    q8, w2 = dsa.indexer_q_quant_fp8(q.to(DEV), w.to(DEV))
    batch, _ = to_dev(wl)
    stride = (wl.max_seq_len + 3) // 4 * 4
    logits = torch.empty(R, stride, dtype=torch.float32, device=DEV)
    dsa.indexer_logits_paged(batch, q8, w2, cache, logits, clean_logits=True)
    torch.cuda.synchronize()
    want_cache = oracle.indexer_k_quant_and_cache(bf16_bits(kall), slots, cache0)
    assert np.array_equal(cache.cpu().numpy(), want_cache)
    oq, ow = oracle.indexer_q_quant(bf16_bits(q), w.numpy())
    ref, mag, _ = oracle.indexer_logits(oq, ow, want_cache, bt, wl.seq_lens.numpy(), wl.query_start.numpy(),
                                        stride, clean=True)
    check_logits(logits.cpu().numpy(), ref, mag, "closed loop")
