"""Reference oracle for the DeepSeek-Sparse-Attention decode step (TEST INFRASTRUCTURE).

This is a plain, slow, CPU implementation in float64, used only by the test
suite, the package smoke check and the CPU-baseline leg of the benchmark to
decide whether the HIP library is right.  The library never imports it and
has no fallback to it.  It shares no code with the GPU path.

What it computes, and where each step comes from:

* FP8 decode.  The vLLM PR page "[Feature] TRITON_MLA_SPARSE backend for
  SM8x/11x/12x DSA Sparse MLA Support" (section Changes, item 2; section Tests)
  keeps the indexer K cache and q in FP8 and tests the decode of all 256 byte
  values.  The format is OCP E4M3 "fn" (bias 7, no infinities, one NaN pattern
  per sign): written out in ``e4m3fn_decode``.
* Indexer ("lightning indexer") logits.  Same page, Changes item 2: MQA logits
  from fp8 q and paged fp8 K, with the per-token K scale applied to the fp32
  dot output, 64 indexer heads of dim 128 reduced with per-head weights.  The
  pages name but do not print the head reduction; the reading taken is
  logit[r, s] = sum_h w[r, h] * relu(q[r, h] . k[s]) * kscale[s]
  (the DSA lightning-indexer form; without a per-head nonlinearity the 64 heads
  would collapse into one dot).  A token whose block maps to a page outside
  the cache is never read and its logit is -inf.  Row r of a sequence with L
  cached tokens and q_len queries sees keys [0, L - q_len + i + 1) ("per-row causal" bound).
  Keys come through the block table, 64 tokens per block (vllm-dsa-mtp-sm80
  README: pages addressed through their stride).
* Top-k.  The PR page review thread (chunked exact top-k discussion): the
  index_topk = 2048 largest logits of each row.  Order: larger value first,
  equal values to the lower index; the chosen indices are written in ascending
  index order, padded with -1 when a row has fewer than k keys.
* Sparse MLA.  Same page, Changes item 3: attention of each query row over only
  its selected latent rows, split-KV partials merged N-way by online softmax, a
  single-pass fast path, and -1e30 as the running-max sentinel of fully masked
  tiles.  Score z = scale * q[h, :576] . c[s, :576]; value = c[s, :512];
  out = softmax(z) @ V; lse = ln sum exp(z) (natural log).
* Quantisation and cache writes (the steps before the path).  The
  vllm-dsa-mtp-sm80 README (skew fixes 0 and 1) names the indexer-K cache
  writer and the per-token-group fp8 quantiser of the indexer q; the reading of
  their arithmetic (one amax / 448 scale per 128 values, round-to-nearest-even
  saturating e4m3fn codes, decided in fp32) is stated where they are written
  out, with the bf16 latent-cache writer beside them.
* FP8 latent cache.  The PR page (Limitations) names the bf16-only latent cache
  as a gap; the fp8 layout read here (4 scale groups of 128 latent values,
  bf16 rope) is defined where it is written out (``latent_cache_write_fp8``)
  and sparse MLA over it attends over the dequantised rows.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
IDX_HEADS = 64
IDX_DIM = 128
IDX_SCALE_OFFSET = PAGE * IDX_DIM
KV_DIM = 576
V_DIM = 512
MASK_SENTINEL = -1e30


# --------------------------------------------------------------------------
# element decoding

def e4m3fn_decode(codes) -> np.ndarray:
    """OCP E4M3 ("e4m3fn") byte -> float64.

    sign s = bit 7, exponent e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: subnormal (-1)^s * m * 2^-9.  e == 15 and m == 7: NaN (no
    infinities).  Otherwise (-1)^s * (8 + m) * 2^(e - 10), i.e. 1.m * 2^(e-7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_decode(u16) -> np.ndarray:
    """bfloat16 bit pattern -> float64 (the upper half of an IEEE binary32)."""
    u = np.asarray(u16).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# batch geometry

def row_extents(seq_lens, query_start):
    """(sequence of each row, e_r) with e_r = L_b - q_len_b + i + 1, floored at 0."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    qs = np.asarray(query_start, dtype=np.int64)
    R = int(qs[-1])
    seq = np.zeros(R, dtype=np.int64)
    ext = np.zeros(R, dtype=np.int64)
    for b in range(len(seq_lens)):
        q = int(qs[b + 1] - qs[b])
        for i in range(q):
            r = int(qs[b]) + i
            seq[r] = b
            ext[r] = max(0, int(seq_lens[b]) - q + i + 1)
    return seq, ext


def token_location(block_table_row, s):
    """Physical page and slot of logical token s: block s // 64, slot s % 64."""
    s = np.asarray(s, dtype=np.int64)
    return np.asarray(block_table_row, dtype=np.int64)[s // PAGE], s % PAGE


# --------------------------------------------------------------------------
# indexer logits

def indexer_keys(idx_cache, block_table_row, s):
    """Codes [n, 128] and fp32 scales [n] (as float64) of the logical tokens in s.

    An indexer page holds its 64 tokens' 128 e4m3 codes, then their 64 fp32
    scales starting at byte 8192 of the page.
    """
    cache = np.asarray(idx_cache, dtype=np.uint8)
    page, slot = token_location(block_table_row, s)
    codes = cache[page[:, None], slot[:, None] * IDX_DIM + np.arange(IDX_DIM)[None, :]]
    sc_cols = IDX_SCALE_OFFSET + 4 * slot[:, None] + np.arange(4)[None, :]
    scale_bytes = np.ascontiguousarray(cache[page[:, None], sc_cols])
    return codes, scale_bytes.view(np.float32).reshape(len(page)).astype(np.float64)


def indexer_logits(q_fp8, weights, idx_cache, block_table, seq_lens, query_start,
                   logits_stride, clean=True, rows=None):
    """Logits and magnitudes of the lightning indexer.

    Returns (logits, magnitude, e) where logits[r, s] for s < e_r is
    sum_h w[r,h] * max(q_h . k_s, 0) * kscale_s, magnitude[r, s] is the same sum
    with |w[r,h]| (the scale the comparison tolerance is relative to), and
    columns s >= e_r hold -inf when ``clean`` and NaN (meaning: not written)
    otherwise.  ``rows`` restricts the computation to the listed rows; the
    returned arrays then hold just those rows, in that order (e stays full).
    """
    q_fp8 = np.asarray(q_fp8, dtype=np.uint8)
    w = np.asarray(weights, dtype=np.float64)
    bt = np.asarray(block_table, dtype=np.int64)
    seq, ext = row_extents(seq_lens, query_start)
    row_list = list(range(len(ext))) if rows is None else [int(r) for r in rows]
    logits = np.full((len(row_list), logits_stride), np.nan)
    mag = np.full((len(row_list), logits_stride), np.nan)
    num_pages = np.asarray(idx_cache).shape[0]
    # The keys of a sequence are decoded once for all of its listed rows (a
    # row uses the prefix [0, e_r) of them); the arithmetic is per row.
    keys = {}
    for o, r in enumerate(row_list):
        e = int(ext[r])
        if clean:
            logits[o, e:] = -np.inf
        if e == 0:
            continue
        b = int(seq[r])
        if b not in keys:
            e_max = max(int(ext[x]) for x in row_list if seq[x] == b)
            page, _ = token_location(bt[b], np.arange(e_max))
            ok_b = (page >= 0) & (page < num_pages)
            s_b = np.nonzero(ok_b)[0]
            codes, scales_b = indexer_keys(idx_cache, bt[b], s_b)
            keys[b] = (s_b, e4m3fn_decode(codes), scales_b)
        s_b, K_b, scales_b = keys[b]
        n = int(np.searchsorted(s_b, e))       # the in-range tokens below e_r
        logits[o, :e] = -np.inf                # tokens on an out-of-range page stay masked
        mag[o, :e] = 0.0
        if n == 0:
            continue
        s, K, scales = s_b[:n], K_b[:n], scales_b[:n]
        Q = e4m3fn_decode(q_fp8[r])            # [64, 128]
        relu = np.maximum(Q @ K.T, 0.0)        # [64, n]
        logits[o, s] = (w[r] @ relu) * scales
        mag[o, s] = (np.abs(w[r]) @ relu) * scales
    return logits, mag, ext


# --------------------------------------------------------------------------
# top-k

def topk_row(values, e, k):
    """Indices of the k largest of values[0:e] (ties to the lower index), ascending, -1 padded."""
    v = np.asarray(values[:e], dtype=np.float64)
    n = min(int(k), int(e))
    out = np.full(int(k), -1, dtype=np.int64)
    if n == 0:
        return out
    order = np.lexsort((np.arange(e), -v))     # primary: -v ascending; secondary: index
    out[:n] = np.sort(order[:n])
    return out


def topk(logits, seq_lens, query_start, k, rows=None):
    """top-k of every row over its own causal extent.  With ``rows``, logits and
    the result hold just those rows, in that order."""
    _, ext = row_extents(seq_lens, query_start)
    row_list = list(range(len(ext))) if rows is None else [int(r) for r in rows]
    out = np.full((len(row_list), int(k)), -1, dtype=np.int64)
    for o, r in enumerate(row_list):
        out[o] = topk_row(logits[o], int(ext[r]), k)
    return out


# --------------------------------------------------------------------------
# sparse MLA

def _selected_rows(kv_cache, bt_row, idx_list, e, num_pages, kv_format="bf16"):
    """Latent rows [n, 576] (float64) of the valid entries of an index list.

    Valid entries are 0 <= s < e whose block maps to a page in [0, num_pages);
    everything else (the -1 padding included) is masked and never read.
    Duplicates are kept, in list order.  ``kv_format`` "fp8" reads the fp8
    latent cache (dequantised rows, see ``kv8_rows``).
    """
    kv = np.asarray(kv_cache)
    s = np.asarray(idx_list, dtype=np.int64)
    s = s[(s >= 0) & (s < e)]
    if s.size == 0:
        return np.zeros((0, KV_DIM))
    page, slot = token_location(bt_row, s)
    ok = (page >= 0) & (page < num_pages)
    page, slot = page[ok], slot[ok]
    if kv_format == "fp8":
        return kv8_rows(kv, page, slot) if page.size else np.zeros((0, KV_DIM))
    cols = slot[:, None] * KV_DIM + np.arange(KV_DIM)[None, :]
    return bf16_decode(kv[page[:, None], cols])


def sparse_mla(q_mla, kv_cache, block_table, seq_lens, query_start, indices,
               softmax_scale, num_pages=None, rows=None, kv_format="bf16"):
    """Single-pass sparse MLA: (out [R, H, 512] float64, lse [R, H] float64).

    For each row and head over the row's valid selected latent rows c_j:
    z_j = scale * q . c_j (576 dims); out = sum softmax(z)_j c_j[:512];
    lse = ln sum_j exp(z_j).  A row with no valid entry gives out = 0 and
    lse = -inf.  With ``rows``, ``indices`` and the outputs hold just those
    rows, in that order.  ``kv_format`` "fp8": the cache is the fp8 latent
    cache and c_j its dequantised rows.
    """
    q_u16 = np.asarray(q_mla)
    R, H, _ = q_u16.shape
    bt = np.asarray(block_table, dtype=np.int64)
    if num_pages is None:
        num_pages = int(np.asarray(kv_cache).shape[0])
    seq, ext = row_extents(seq_lens, query_start)
    row_list = list(range(R)) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(row_list), H, V_DIM))
    lse = np.full((len(row_list), H), -np.inf)
    for o, r in enumerate(row_list):
        C = _selected_rows(kv_cache, bt[seq[r]], indices[o], int(ext[r]), num_pages, kv_format)
        if C.shape[0] == 0:
            continue
        Q = bf16_decode(q_u16[r])                       # [H, 576]
        z = softmax_scale * (Q @ C.T)                   # [H, n]
        M = z.max(axis=1, keepdims=True)
        p = np.exp(z - M)
        l = p.sum(axis=1, keepdims=True)
        out[o] = (p @ C[:, :V_DIM]) / l
        lse[o] = (M + np.log(l))[:, 0]
    return out, lse


def sparse_mla_split(q_mla, kv_cache, block_table, seq_lens, query_start, indices,
                     softmax_scale, num_splits, num_pages=None, rows=None, kv_format="bf16"):
    """Split-KV sparse MLA with the N-way online-softmax merge.

    The k slots of each row's index list are cut into ``num_splits`` contiguous
    ranges of ceil(k / num_splits) slots.  Each range yields a running max m_i
    (starting from the -1e30 sentinel, so an all-masked range never forms
    (-inf) - (-inf)), a sum l_i = sum exp(z - m_i) and an unnormalised
    accumulator acc_i = sum exp(z - m_i) c[:512].  The merge takes
    M = max m_i, L = sum l_i exp(m_i - M), out = sum acc_i exp(m_i - M) / L and
    lse = M + ln L; L == 0 (nothing valid anywhere) gives out = 0, lse = -inf.
    """
    q_u16 = np.asarray(q_mla)
    R, H, _ = q_u16.shape
    idx = np.asarray(indices, dtype=np.int64)
    k = idx.shape[1]
    bt = np.asarray(block_table, dtype=np.int64)
    if num_pages is None:
        num_pages = int(np.asarray(kv_cache).shape[0])
    seq, ext = row_extents(seq_lens, query_start)
    per = -(-k // num_splits)
    row_list = list(range(R)) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(row_list), H, V_DIM))
    lse = np.full((len(row_list), H), -np.inf)
    for o, r in enumerate(row_list):
        Q = bf16_decode(q_u16[r])
        ms, ls, accs = [], [], []
        for i in range(num_splits):
            C = _selected_rows(kv_cache, bt[seq[r]], idx[o, i * per:(i + 1) * per],
                               int(ext[r]), num_pages, kv_format)
            m = np.full(H, MASK_SENTINEL)
            l = np.zeros(H)
            acc = np.zeros((H, V_DIM))
            if C.shape[0]:
                z = softmax_scale * (Q @ C.T)
                m = np.maximum(m, z.max(axis=1))
                p = np.exp(z - m[:, None])
                l = p.sum(axis=1)
                acc = p @ C[:, :V_DIM]
            ms.append(m)
            ls.append(l)
            accs.append(acc)
        M = np.max(ms, axis=0)
        wts = [np.exp(m - M) for m in ms]
        L = sum(l * wt for l, wt in zip(ls, wts))
        A = sum(a * wt[:, None] for a, wt in zip(accs, wts))
        ok = L > 0
        out[o][ok] = A[ok] / L[ok][:, None]
        lse[o][ok] = M[ok] + np.log(L[ok])
    return out, lse


# --------------------------------------------------------------------------
# quantisation and cache writes: the steps just before the path
#
# The vllm-dsa-mtp-sm80 README names them (skew fix 0: indexer_k_quant_and_cache
# writes the paged indexer K through the page stride; skew fix 1: the unfused
# per_token_group_quant_fp8 quantises the indexer q).  The pages print neither
# body.  The reading taken: one fp32 scale per 128-value group (a K token, or
# one (row, head) of q), scale = amax / 448 so the largest element lands on
# the largest finite e4m3fn value, codes = e4m3fn(x / scale) rounded to nearest
# with ties to the even code and saturated at +-448; an all-zero group takes
# scale 1.  Every fp32 step (amax, the scale division, x / scale) is taken in
# IEEE fp32, the precision the codes are decided in.  The q scale is folded
# into the indexer head weight: w'[r, h] = fp32(w[r, h] * scale[r, h]).

E4M3_MAX = 448.0
_E4M3_GRID = e4m3fn_decode(np.arange(127, dtype=np.uint8))   # codes 0x00..0x7E, ascending


def e4m3fn_encode(y) -> np.ndarray:
    """float -> OCP E4M3 code: nearest representable value, ties to the even
    code (even mantissa), |y| > 448 saturating to +-448, sign kept (so -0 and
    negative values that round to zero give 0x80).  NaN gives 0x7F / 0xFF."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    lo = np.clip(np.searchsorted(_E4M3_GRID, a, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    d_lo = a - _E4M3_GRID[lo]
    d_hi = _E4M3_GRID[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.int64)
    code = np.where(np.isnan(y), 0x7F, code)
    return (code | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def quantize_groups_fp8(x_bf16):
    """bf16 bit patterns [..., 128] -> (e4m3fn codes [..., 128], fp32 scales [...])."""
    x = bf16_decode(x_bf16).astype(np.float32)          # exact
    amax = np.max(np.abs(x), axis=-1)                    # exact
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)        # IEEE fp32 division
    return e4m3fn_encode(y), scale


def indexer_q_quant(q_bf16, weights):
    """Indexer q quantisation: q [R, 64, 128] bf16 bits and w [R, 64] fp32 ->
    (codes [R, 64, 128] uint8, w' [R, 64] fp32 with the q scale folded in)."""
    codes, scale = quantize_groups_fp8(np.asarray(q_bf16))
    w = np.asarray(weights, dtype=np.float32)
    return codes, (w * scale).astype(np.float32)


def _slot_targets(slot_mapping, num_pages):
    """(token, page, slot-in-page) of every token whose slot lands in the cache.

    slot = page * 64 + slot-in-page; a negative slot (a padding token) or one on
    a page outside [0, num_pages) writes nothing."""
    sm = np.asarray(slot_mapping, dtype=np.int64)
    ok = (sm >= 0) & (sm < np.int64(num_pages) * PAGE)
    t = np.nonzero(ok)[0]
    return t, sm[t] // PAGE, sm[t] % PAGE


def indexer_k_quant_and_cache(k_bf16, slot_mapping, idx_cache):
    """Quantise K [T, 128] bf16 bits per token and write it into a copy of the
    paged indexer cache [num_pages, page_stride] uint8: codes at
    page * stride + slot * 128, the fp32 scale at page * stride + 8192 + slot * 4.
    Bytes of other slots, and the page padding, keep their value."""
    cache = np.array(idx_cache, dtype=np.uint8, copy=True)
    codes, scale = quantize_groups_fp8(np.asarray(k_bf16))
    t, page, slot = _slot_targets(slot_mapping, cache.shape[0])
    for i, p, s in zip(t, page, slot):
        cache[p, s * IDX_DIM:(s + 1) * IDX_DIM] = codes[i]
        cache[p, IDX_SCALE_OFFSET + 4 * s:IDX_SCALE_OFFSET + 4 * s + 4] = \
            np.frombuffer(np.float32(scale[i]).tobytes(), dtype=np.uint8)
    return cache


def latent_cache_write(latent_bf16, rope_bf16, slot_mapping, kv_cache):
    """Write each token's latent row [512] followed by its rope part [64] (bf16
    bits, unchanged) into a copy of the paged latent cache [num_pages, stride]
    at page * stride + slot * 576."""
    cache = np.array(kv_cache, copy=True)
    lat = np.asarray(latent_bf16)
    rope = np.asarray(rope_bf16)
    t, page, slot = _slot_targets(slot_mapping, cache.shape[0])
    for i, p, s in zip(t, page, slot):
        cache[p, s * KV_DIM:s * KV_DIM + V_DIM] = lat[i]
        cache[p, s * KV_DIM + V_DIM:(s + 1) * KV_DIM] = rope[i]
    return cache


# --------------------------------------------------------------------------
# fp8 latent cache (the pages list the bf16-only latent cache as a limitation
# of their backend, PR page "Limitations"; they define no fp8 layout)
#
# Reading taken: the 512 latent values of a token are quantised in 4 groups of
# 128 with the same quantiser as the indexer (amax / 448 fp32 scale, RNE
# saturating e4m3fn); the 64 rope values stay bf16.  Page of 64 tokens: row
# t at byte 640 t holds the 512 codes then the 64 bf16 rope values (640 B);
# the 4 fp32 scales of token t sit at byte 40960 + 16 t.  A token's latent
# value d is scale[d // 128] * e4m3(code[d]).

KV8_ROW_BYTES = 640
KV8_SCALE_OFFSET = PAGE * KV8_ROW_BYTES           # 40960
KV8_PAGE_BYTES = KV8_SCALE_OFFSET + PAGE * 16     # 41984


def latent_cache_write_fp8(latent_bf16, rope_bf16, slot_mapping, kv8_cache):
    """Quantise each token's latent [512] (4 groups of 128) and write codes,
    rope bits and scales into a copy of the fp8 latent cache
    [num_pages, page_stride] uint8."""
    cache = np.array(kv8_cache, dtype=np.uint8, copy=True)
    lat = np.asarray(latent_bf16).reshape(-1, 4, 128)
    codes, scale = quantize_groups_fp8(lat)                 # [T, 4, 128], [T, 4]
    rope = np.ascontiguousarray(np.asarray(rope_bf16, dtype=np.uint16))
    t, page, slot = _slot_targets(slot_mapping, cache.shape[0])
    for i, p, s in zip(t, page, slot):
        row = s * KV8_ROW_BYTES
        cache[p, row:row + V_DIM] = codes[i].reshape(-1)
        cache[p, row + V_DIM:row + KV8_ROW_BYTES] = rope[i].view(np.uint8)
        cache[p, KV8_SCALE_OFFSET + 16 * s:KV8_SCALE_OFFSET + 16 * s + 16] = \
            np.ascontiguousarray(scale[i].astype(np.float32)).view(np.uint8)
    return cache


def kv8_rows(kv8_cache, page, slot):
    """Dequantised latent rows [n, 576] (float64) of (page, slot) pairs."""
    cache = np.asarray(kv8_cache, dtype=np.uint8)
    page = np.asarray(page, dtype=np.int64)
    slot = np.asarray(slot, dtype=np.int64)
    cols = slot[:, None] * KV8_ROW_BYTES + np.arange(KV8_ROW_BYTES)[None, :]
    raw = cache[page[:, None], cols]                                  # [n, 640]
    sc_cols = KV8_SCALE_OFFSET + 16 * slot[:, None] + np.arange(16)[None, :]
    scale = np.ascontiguousarray(cache[page[:, None], sc_cols]).view(np.float32).astype(np.float64)  # [n, 4]
    lat = e4m3fn_decode(raw[:, :V_DIM]).reshape(-1, 4, 128) * scale[:, :, None]
    rope = bf16_decode(np.ascontiguousarray(raw[:, V_DIM:]).view(np.uint16))
    return np.concatenate([lat.reshape(-1, V_DIM), rope], axis=1)
