"""fp64 CPU oracle for single-token decode attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP path and imports neither torch nor the kernel library.

What it computes, and where the pages say so:

* "KV cache" guide (this.guide/ai/kv-cache.html), section "A cache you keep
  because attention looks backwards": at generation step t the current
  token's query attends, through a causal mask, to the keys and values of
  every position up to t; the key and value of position i depend only on
  the hidden state at i, so caching them gives the same result as
  recomputing them.  The attention equation itself was lost when the page
  was extracted; this oracle uses the standard softmax(q.K^T * scale).V with
  scale = 1/sqrt(d_h) (1/sqrt(576) for the latent cache).
* Same guide, "Two tensors per layer": the cache of one layer and one
  sequence is a key tensor and a value tensor, each [n_kv, L, d_h].
* Same guide, "Fewer KV heads": grouped-query attention partitions the n_h
  query heads into n_kv groups that share one KV head.  Reading: the groups
  are contiguous, so query head i uses KV head i // (n_h / n_kv).
* Same guide, "Caching a compressed latent": with the key up-projection
  folded into the query, scores are taken directly against the cached
  latent; the value side folds into the output projection, so the weighted
  sum is taken over the latent itself.  The memory footnote fixes the row as
  a 512-wide latent plus a 64-wide shared rotary key.
* Podcast transcript (my-weird-prompts 640482), DeepSeek Sparse Attention
  passage: a top-k subset of stored positions is read; attention runs over
  those positions only.
* "KV cache" guide, "Fewer bits per number", and the podcast's KV
  quantization passage: the cache may be stored at lower precision, FP8
  being the common choice, one byte per number.  Reading (the pages name no
  layout): OCP FP8 E4M3 in its finite variant (the format whose largest
  value, 448, the DeepSeek FP4 section multiplies by 6), one float scale
  per tensor (keys, values); a stored number is code value x scale, and a
  new row is quantised as x * (1 / scale) in float32, rounded to nearest
  even and saturated to +-448.
* Podcast transcript, the 890-byte passage, and the DeepSeek article's FP4
  section: the main key/value cache may be FP4, E2M1 numbers with one E4M3
  scale per 16 channels and no second-level global scale (the pages call
  it MXFP4 but give these NVFP4-style parameters; the largest stored
  magnitude, 448 x 6 = 2688, is the article's bound), dequantised before
  attention.  Reading (no rounding rule is given): a block's scale is the
  E4M3 value nearest float32(amax / 6), each number the E2M1 value nearest
  float32(x / scale) with ties to the even code and saturation at 6, an
  all-zero scale stores zero codes; two codes per byte, even channel in the
  low nibble.
* Podcast transcript, DeepSeek Sparse Attention passage, and the "A
  Hundred Messages" blog's hierarchical-indexer passage: an indexer scores
  the visible prefix and a top-k subset of positions is kept (k = 2048); a
  deeper indexer picks its own top-k only among the positions of a candidate
  pool of 8-position blocks.  Reading (the pages give no tie rule): the k
  highest scores, equal scores ordered by lower position first; the kept
  positions are returned in ascending order (the order the sparse decode
  reads them), padded with -1 when fewer than k positions exist.
* "KV cache" guide, "The allocator, not the algorithm": instead of one
  contiguous reservation per sequence at its maximum length, the cache is
  cut into fixed-size blocks of beta positions held in a shared pool, and a
  per-sequence block table maps logical block k (positions [k*beta,
  (k+1)*beta)) to a physical block; each sequence then wastes at most
  beta - 1 slots.  Reading (the pages give no layout): a pool is
  [num_blocks, n_kv, beta, d]; a block-table entry outside [0, num_blocks)
  is invalid.
* "890 bytes a token" (bemiagent), SWA bounded replay passage: with a
  window W and a replayed segment starting at position s, a query at
  position i attends to keys [max(s, i - W + 1), i].  For decode the query
  is the newest position i = n - 1, so the keys are [max(s, n - W), n);
  s = 0 when every position is present.  (The guide's "Keeping fewer
  tokens" section describes the same bounded, most-recent window.)
* Podcast transcript, decode walk-through: each new token attends to the
  cache plus its own new pair, and its key and value are appended.  The
  oracle appends first and then attends over [0, seq_len), which is the
  same set of positions.

Storage convention: caches and inputs are held in their storage form,
float32 arrays or bf16 bit patterns in uint16 arrays.  Appends copy those
bits.  Arithmetic is float64 throughout.

Device-side conditions (defined here, mirrored by the library contract):
* append when seq_len is not in [0, L_max): no write, no increment,
  flag bit 0 (value 1) set;
* a top-k index outside [0, seq_len): skipped, flag bit 1 (value 2) set;
* a sequence with no positions to attend: output row 0, lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

FLAG_CACHE_FULL = 1
FLAG_BAD_INDEX = 2


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------
def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of fp32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def to_f64(raw: np.ndarray) -> np.ndarray:
    """Storage form -> float64.  uint16 is read as bf16, float32 as is."""
    raw = np.asarray(raw)
    if raw.dtype == np.uint16:
        return bf16_to_f64(raw)
    if raw.dtype in (np.float32, np.float64):
        return raw.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {raw.dtype}")


# --------------------------------------------------------------------------
# cache size ("KV cache" guide, "The size formula")
# --------------------------------------------------------------------------
def cache_bytes(n_l: int, n_kv: int, d_h: int, b: int, L: int, B: int) -> int:
    """Two tensors x layers x KV heads x head dim x bytes x length x batch.

    The guide's equation was lost in extraction; its prose lists exactly
    these factors, and notes that n_h does not appear.
    """
    return 2 * n_l * n_kv * d_h * b * L * B


def mla_cache_bytes(n_l: int, d_c: int, d_r: int, b: int, L: int, B: int) -> int:
    """One latent (d_c) plus one shared rotary key (d_r) per layer and token."""
    return n_l * (d_c + d_r) * b * L * B


# --------------------------------------------------------------------------
# append (podcast decode walk-through; guide "Two tensors per layer")
# --------------------------------------------------------------------------
def append(k_cache, v_cache, seq_lens, k_new, v_new) -> int:
    """Write the new token's key/value at slot seq_lens[b], then increment.

    k_cache, v_cache: [B, n_kv, L_max, d] storage arrays, modified in place.
    v_cache may be None for a single-tensor (latent) cache.
    seq_lens: int32 [B], modified in place.
    k_new, v_new: [B, n_kv, d].
    Returns the flag word (bit 0: a sequence had no free slot).
    """
    B, n_kv, L_max, d = k_cache.shape
    flag = 0
    for b in range(B):
        n = int(seq_lens[b])
        if n < 0 or n >= L_max:
            flag |= FLAG_CACHE_FULL
            continue
        k_cache[b, :, n, :] = k_new[b]
        if v_cache is not None:
            v_cache[b, :, n, :] = v_new[b]
        seq_lens[b] = n + 1
    return flag


# --------------------------------------------------------------------------
# attention of one query over a set of rows
# --------------------------------------------------------------------------
def _attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale * K q) . V for one query vector, plus its log-sum-exp.

    q: [d_qk], K: [n, d_qk], V: [n, d_v], all float64.  The max is
    subtracted before exponentiating (no change to the value, only to
    overflow).  n == 0 gives a zero row and lse = -inf.
    """
    n = K.shape[0]
    if n == 0:
        return np.zeros(V.shape[1]), -math.inf
    s = scale * (K @ q)
    m = s.max()
    w = np.exp(s - m)
    z = w.sum()
    return (w @ V) / z, m + math.log(z)


# --------------------------------------------------------------------------
# dense decode: MHA (G = 1), GQA (1 < G < n_h), MQA (n_kv = 1)
# --------------------------------------------------------------------------
def decode(q, k_cache, v_cache, seq_lens, scale: float):
    """Each query head attends over positions [0, seq_lens[b]) of its KV head.

    q: [B, n_h, d]; k_cache, v_cache: [B, n_kv, L_max, d] (storage form).
    Returns (o [B, n_h, d] float64, lse [B, n_h] float64, natural log).
    """
    B, n_h, d = q.shape
    n_kv = k_cache.shape[1]
    assert n_h % n_kv == 0
    G = n_h // n_kv
    o = np.zeros((B, n_h, v_cache.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    for b in range(B):
        n = int(seq_lens[b])
        for j in range(n_kv):
            K = to_f64(k_cache[b, j, :n])
            V = to_f64(v_cache[b, j, :n])
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse


# --------------------------------------------------------------------------
# top-k selection from indexer scores (DSA; hierarchical indexer pool)
# --------------------------------------------------------------------------
def topk_select(scores, seq_lens, K: int, pool=None, pool_block: int = 8):
    """Indices of the K highest scores among positions [0, seq_lens[b]) of
    each row scores[b, j, :], equal scores by lower position, returned in
    ascending position order and padded with -1.

    scores: [B, n_idx, L_max] float32.  pool (optional): [B, n_idx, P] int32
    block ids (-1 = unused); then only positions t < seq_lens[b] with
    t // pool_block in the row's pool are candidates.
    Returns int32 [B, n_idx, K]."""
    B, R, L = scores.shape
    out = np.full((B, R, K), -1, dtype=np.int32)
    for b in range(B):
        n = min(max(int(seq_lens[b]), 0), L)
        for j in range(R):
            if pool is None:
                cand = range(n)
            else:
                blocks = {int(x) for x in pool[b, j] if x >= 0}
                cand = [t for t in range(n) if t // pool_block in blocks]
            ranked = sorted(cand, key=lambda t: (-float(scores[b, j, t]), t))[:K]
            ranked.sort()
            out[b, j, :len(ranked)] = ranked
    return out


# --------------------------------------------------------------------------
# paged cache (guide "The allocator, not the algorithm")
# --------------------------------------------------------------------------
def paged_waste_fraction(lengths, beta: int) -> float:
    """Slots held but unused over slots used, when each sequence holds
    ceil(n / beta) blocks of beta slots."""
    held = sum(-(-int(n) // beta) * beta for n in lengths)
    used = sum(int(n) for n in lengths)
    return (held - used) / used


def paged_rows(pool, block_table, b: int, j: int, n: int, beta: int):
    """Rows [0, n) of (sequence b, KV head j) gathered through the block
    table, plus the list of positions whose block is invalid (skipped)."""
    rows, bad = [], []
    num_blocks = pool.shape[0]
    for t in range(n):
        blk = int(block_table[b, t // beta])
        if 0 <= blk < num_blocks:
            rows.append(pool[blk, j, t % beta])
        else:
            bad.append(t)
    shape = (len(rows),) + pool.shape[3:]
    return (np.stack(rows) if rows else np.zeros(shape, dtype=pool.dtype)), bad


def append_paged(k_pool, v_pool, block_table, seq_lens, k_new, v_new) -> int:
    """append() into a paged cache: slot n = seq_lens[b] lives in block
    block_table[b, n // beta] at offset n % beta.  A full table (n at or past
    max_blocks * beta) sets flag bit 0; an invalid block at the slot sets
    flag bit 1; either way nothing is written and the length stays."""
    beta = k_pool.shape[2]
    max_blocks = block_table.shape[1]
    flag = 0
    for b in range(seq_lens.shape[0]):
        n = int(seq_lens[b])
        if n < 0 or n >= max_blocks * beta:
            flag |= FLAG_CACHE_FULL
            continue
        blk = int(block_table[b, n // beta])
        if not 0 <= blk < k_pool.shape[0]:
            flag |= FLAG_BAD_INDEX
            continue
        k_pool[blk, :, n % beta] = k_new[b]
        v_pool[blk, :, n % beta] = v_new[b]
        seq_lens[b] = n + 1
    return flag


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float):
    """decode() over a paged cache: head i of sequence b attends over the
    positions [0, seq_lens[b]) gathered through the block table; positions
    in an invalid block are skipped and set flag bit 1.
    Returns (o, lse, flag)."""
    B, n_h, d = q.shape
    n_kv = k_pool.shape[1]
    beta = k_pool.shape[2]
    G = n_h // n_kv
    o = np.zeros((B, n_h, v_pool.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    flag = 0
    for b in range(B):
        n = min(max(int(seq_lens[b]), 0), block_table.shape[1] * beta)
        for j in range(n_kv):
            Kr, bad = paged_rows(k_pool, block_table, b, j, n, beta)
            Vr, _ = paged_rows(v_pool, block_table, b, j, n, beta)
            if bad:
                flag |= FLAG_BAD_INDEX
            K = to_f64(Kr)
            V = to_f64(Vr)
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse, flag


# --------------------------------------------------------------------------
# sliding-window decode (bounded replay's window rule)
# --------------------------------------------------------------------------
def window_range(n: int, window: int, start: int = 0):
    """Positions the newest query (position n - 1) attends: [lo, n) with
    lo = max(start, n - window), clamped to [0, n]."""
    lo = min(max(start, n - window, 0), n)
    return lo, n


def decode_window(q, k_cache, v_cache, seq_lens, scale: float, window: int,
                  win_start=None):
    """decode() restricted to the window: head i of sequence b attends over
    window_range(seq_lens[b], window, win_start[b]) (win_start None: 0)."""
    assert window >= 1
    B, n_h, d = q.shape
    n_kv = k_cache.shape[1]
    G = n_h // n_kv
    o = np.zeros((B, n_h, v_cache.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    for b in range(B):
        st = 0 if win_start is None else int(win_start[b])
        lo, n = window_range(int(seq_lens[b]), window, st)
        for j in range(n_kv):
            K = to_f64(k_cache[b, j, lo:n])
            V = to_f64(v_cache[b, j, lo:n])
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse


# --------------------------------------------------------------------------
# MLA latent decode (guide "Caching a compressed latent")
# --------------------------------------------------------------------------
def decode_mla(q, ckv, seq_lens, d_c: int, d_r: int, scale: float):
    """Attention over a latent cache with absorbed queries.

    q: [B, n_h, d_c + d_r]: the absorbed latent query, then the rotary query.
    ckv: [B, L_max, d_c + d_r]: per position the latent c, then the shared
    rotary key.  Score = scale * (q_lat . c + q_rope . k_rope); output is the
    softmax-weighted sum of the latents c (d_c wide).
    Returns (o [B, n_h, d_c], lse [B, n_h]).
    """
    B, n_h, D = q.shape
    assert D == d_c + d_r
    if ckv.ndim == 4:
        assert ckv.shape[1] == 1
        ckv = ckv[:, 0]
    o = np.zeros((B, n_h, d_c))
    lse = np.full((B, n_h), -math.inf)
    for b in range(B):
        n = int(seq_lens[b])
        rows = to_f64(ckv[b, :n])
        c, k_rope = rows[:, :d_c], rows[:, d_c:]
        for i in range(n_h):
            qi = to_f64(q[b, i])
            q_lat, q_rope = qi[:d_c], qi[d_c:]
            if n == 0:
                continue
            s = scale * (c @ q_lat + k_rope @ q_rope)
            m = s.max()
            w = np.exp(s - m)
            z = w.sum()
            o[b, i] = (w @ c) / z
            lse[b, i] = m + math.log(z)
    return o, lse


# --------------------------------------------------------------------------
# top-k sparse decode (podcast, DeepSeek Sparse Attention passage)
# --------------------------------------------------------------------------
def decode_topk(q, k_cache, v_cache, seq_lens, idx, scale: float):
    """Attend only over the listed positions: gather, then attend.

    idx: [B, n_kv, K] int.  An index outside [0, seq_lens[b]) is skipped and
    sets flag bit 1.  A position listed twice counts twice.
    Returns (o [B, n_h, d], lse [B, n_h], flag).
    """
    B, n_h, d = q.shape
    n_kv = k_cache.shape[1]
    G = n_h // n_kv
    o = np.zeros((B, n_h, v_cache.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    flag = 0
    for b in range(B):
        n = int(seq_lens[b])
        for j in range(n_kv):
            listed = [int(t) for t in idx[b, j]]
            kept = [t for t in listed if 0 <= t < n]
            if len(kept) != len(listed):
                flag |= FLAG_BAD_INDEX
            K = to_f64(k_cache[b, j][kept]) if kept else np.zeros((0, d))
            V = to_f64(v_cache[b, j][kept]) if kept else np.zeros((0, v_cache.shape[3]))
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse, flag


# --------------------------------------------------------------------------
# full recomputation with a causal mask (guide, first section)
# --------------------------------------------------------------------------
def full_causal(Q, K, V, scale: float):
    """Attention for every position of one sequence, recomputed from scratch.

    Q: [n, n_h, d]; K, V: [n, n_kv, d] (float64 or storage form).  Builds the
    n x n score matrix per head, adds the causal mask (-inf above the
    diagonal), takes a row softmax and multiplies by V.
    Returns O [n, n_h, d_v].
    """
    Q, K, V = to_f64(Q), to_f64(K), to_f64(V)
    n, n_h, _ = Q.shape
    n_kv = K.shape[1]
    G = n_h // n_kv
    mask = np.triu(np.full((n, n), -np.inf), k=1)
    O = np.zeros((n, n_h, V.shape[2]))
    for i in range(n_h):
        j = i // G
        S = scale * (Q[:, i, :] @ K[:, j, :].T) + mask
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P = P / P.sum(axis=1, keepdims=True)
        O[:, i, :] = P @ V[:, j, :]
    return O


# --------------------------------------------------------------------------
# log-sum-exp merge of partial results over a partition of the positions
# --------------------------------------------------------------------------
def merge_partials(os_, lses):
    """Combine per-part (o_p, lse_p) into the result over the union.

    o = sum_p exp(lse_p - LSE) o_p with LSE = log sum_p exp(lse_p).  Parts
    with lse_p = -inf contribute nothing.
    """
    lses = np.asarray(lses, dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(np.asarray(os_[0], dtype=np.float64)), -math.inf
    M = lses[~np.isneginf(lses)].max()
    w = np.exp(lses - M)
    Z = w.sum()
    o = sum(wi * np.asarray(oi, dtype=np.float64) for wi, oi in zip(w, os_)) / Z
    return o, M + math.log(Z)


# --------------------------------------------------------------------------
# FP8 E4M3 storage (guide "Fewer bits per number"; podcast KV quantization)
# --------------------------------------------------------------------------
FP8_E4M3_MAX = 448.0


def fp8_e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """E4M3 bit patterns (uint8) -> float64, exactly.

    Bit fields s eeee mmm, exponent bias 7.  e = 0: subnormal m * 2^-9;
    e = 15 with m = 7: NaN (the finite variant has no infinities); otherwise
    (1 + m/8) * 2^(e-7).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, val)


_FP8_POS = None


def _fp8_positive_values():
    """Values of the finite non-negative codes 0x00..0x7E (increasing)."""
    global _FP8_POS
    if _FP8_POS is None:
        _FP8_POS = fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    return _FP8_POS


def f64_to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code, saturating
    to +-448; NaN -> 0x7F.  Sign is kept for zero."""
    x = np.asarray(x, dtype=np.float64)
    vals = _fp8_positive_values()
    a = np.minimum(np.abs(x), FP8_E4M3_MAX)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == vals[hi], hi, code)
    out = code.astype(np.uint8) | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out).astype(np.uint8)


def quantize_fp8(x_raw, scale: float) -> np.ndarray:
    """Storage-form values -> E4M3 codes: float32(x) * float32(1/scale),
    then f64_to_fp8_e4m3 (the product is exact in float64)."""
    inv = np.float32(1.0) / np.float32(scale)
    y = to_f64(x_raw).astype(np.float32) * inv
    return f64_to_fp8_e4m3(y.astype(np.float64))


def append_fp8(k_cache8, v_cache8, seq_lens, k_new, v_new, k_scale, v_scale) -> int:
    """append() for an E4M3 cache: the new rows are quantised first."""
    return append(k_cache8, v_cache8, seq_lens, quantize_fp8(k_new, k_scale),
                  quantize_fp8(v_new, v_scale))


def decode_fp8(q, k_cache8, v_cache8, seq_lens, scale: float, k_scale: float,
               v_scale: float):
    """decode() over an E4M3 cache: stored keys are code value * k_scale,
    stored values code value * v_scale."""
    B, n_h, d = q.shape
    n_kv = k_cache8.shape[1]
    G = n_h // n_kv
    o = np.zeros((B, n_h, v_cache8.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    for b in range(B):
        n = int(seq_lens[b])
        for j in range(n_kv):
            K = fp8_e4m3_to_f64(k_cache8[b, j, :n]) * float(k_scale)
            V = fp8_e4m3_to_f64(v_cache8[b, j, :n]) * float(v_scale)
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse


# --------------------------------------------------------------------------
# FP4 block-scaled cache (DeepSeek article, FP4 section; podcast, the
# 890-byte passage): E2M1 numbers, one E4M3 scale per 16 channels, no
# second-level scale, dequantised before attention.  Reading of how a block
# is encoded (the pages give the format, not the rounding): scale = E4M3 of
# float32(amax / 6), every number float32(x / scale) rounded to the nearest
# E2M1 value, ties to the even code, magnitudes past 6 saturating.
# --------------------------------------------------------------------------
FP4_E2M1_MAX = 6.0
FP4_BLOCK = 16
# E2M1 magnitudes of codes 0..7 (sign in bit 3): exponent bias 1, one
# mantissa bit, code 1 subnormal.
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64, from the field definition:
    sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return np.where(c & 8, -mag, mag)


def f64_to_fp4_e2m1(q: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code, ties to the even code, |q| > 6 -> 6; the sign bit
    copies the sign of q (also for zero).  Written as a search over the
    eight magnitudes, like the E4M3 encoder."""
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    vals = np.asarray(_E2M1_MAG)
    best = np.zeros(a.shape, dtype=np.int64)
    for code in range(1, 8):
        d_new = np.abs(a - vals[code])
        d_best = np.abs(a - vals[best])
        take = (d_new < d_best) | ((d_new == d_best) & (code % 2 == 0))
        best = np.where(take, code, best)
    best = np.where(a > FP4_E2M1_MAX, 7, best)
    return (best | np.where(np.signbit(q), 8, 0)).astype(np.uint8)


def quantize_fp4(x_raw) -> tuple:
    """Storage-form rows [..., d] (d a multiple of 16) -> (codes [..., d/2]
    uint8, two per byte with the even channel in the low nibble; scales
    [..., d/16] uint8 E4M3 codes)."""
    x = to_f64(x_raw).astype(np.float32)
    shp = x.shape
    d = shp[-1]
    blk = x.reshape(shp[:-1] + (d // FP4_BLOCK, FP4_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    s_raw = amax / np.float32(FP4_E2M1_MAX)                       # float32 quotient
    sc = f64_to_fp8_e4m3(s_raw.astype(np.float64))
    s = fp8_e4m3_to_f64(sc).astype(np.float32)                    # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        q = blk / s[..., None]                                    # float32 quotient
    codes = f64_to_fp4_e2m1(q.astype(np.float64))
    codes = np.where((s == 0)[..., None], np.uint8(0), codes).astype(np.uint8)
    codes = codes.reshape(shp)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, sc.astype(np.uint8)


def dequantize_fp4(packed, scales) -> np.ndarray:
    """(codes, scales) as written by quantize_fp4 -> float64 rows."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = fp4_e2m1_to_f64(packed & 0xF)
    hi = fp4_e2m1_to_f64(packed >> 4)
    vals = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
    s = fp8_e4m3_to_f64(np.asarray(scales, dtype=np.uint8))
    return vals * np.repeat(s, FP4_BLOCK, axis=-1)


def append_fp4(k_codes, k_scales, v_codes, v_scales, seq_lens, k_new, v_new) -> int:
    """append() for an FP4 cache: the new rows are quantised, then codes and
    scales go to slot seq_lens[b] of their arrays (one length bump)."""
    kc, ks = quantize_fp4(k_new)
    vc, vs = quantize_fp4(v_new)
    lens2 = np.array(seq_lens, copy=True)
    flag = append(k_codes, v_codes, seq_lens, kc, vc)
    append(k_scales, v_scales, lens2, ks, vs)
    return flag


def decode_fp4(q, k_codes, k_scales, v_codes, v_scales, seq_lens, scale: float):
    """decode() over an FP4 cache: every stored number is its E2M1 value
    times the E4M3 scale of its 16-channel block (dequantise, then attend)."""
    B, n_h, d = q.shape
    n_kv = k_codes.shape[1]
    G = n_h // n_kv
    o = np.zeros((B, n_h, 2 * v_codes.shape[3]))
    lse = np.full((B, n_h), -math.inf)
    for b in range(B):
        n = int(seq_lens[b])
        for j in range(n_kv):
            K = dequantize_fp4(k_codes[b, j, :n], k_scales[b, j, :n])
            V = dequantize_fp4(v_codes[b, j, :n], v_scales[b, j, :n])
            for i in range(j * G, (j + 1) * G):
                o[b, i], lse[b, i] = _attend(to_f64(q[b, i]), K, V, scale)
    return o, lse
