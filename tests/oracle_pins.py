"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` takes an oracle object (the real module, or a copy with a
planted mistake) and raises AssertionError when the oracle disagrees with
the fact.  None of them re-types the oracle's formula: they use closed
forms, invariants, page figures, or an independent scalar brute force.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import kvc_synth as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _f64_case(rng, B, n_h, n_kv, d, lens, L_max=None, dv=None):
    """float64 storage-free case (float32 storage, so to_f64 is exact)."""
    L_max = L_max or max(int(max(lens)), 1)
    dv = dv or d
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    kc = rng.standard_normal((B, n_kv, L_max, d)).astype(np.float32)
    vc = rng.standard_normal((B, n_kv, L_max, dv)).astype(np.float32)
    return q, kc, vc, np.asarray(lens, dtype=np.int32)


# ---------------------------------------------------------------- brute force
def brute_attend(q, K, V, scale):
    """Scalar Python attention: math.exp and math.fsum, no numpy arithmetic."""
    q = [float(x) for x in q]
    s = [scale * math.fsum(qa * float(ka) for qa, ka in zip(q, row)) for row in K]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = math.fsum(w)
    dv = len(V[0])
    o = [math.fsum(w[t] * float(V[t][c]) for t in range(len(w))) / z for c in range(dv)]
    return o, m + math.log(z)


# ------------------------------------------------------------------- size
def pin_size_llama2(orc):
    """Podcast: Llama-2-7B at fp16, B = 1, 4096 tokens -> about two gigabytes."""
    g = golden()["llama2_7b_cache"]
    got = orc.cache_bytes(g["n_l"], g["n_kv"], g["d_h"], g["bytes_per_elem"], g["L"], g["B"])
    assert abs(got - g["approx_bytes"]) <= g["relative_tolerance"] * g["approx_bytes"], got
    # Doubling any one factor doubles the size; n_h does not enter.
    base = got
    assert orc.cache_bytes(g["n_l"] * 2, g["n_kv"], g["d_h"], 2, g["L"], 1) == 2 * base
    assert orc.cache_bytes(g["n_l"], g["n_kv"], g["d_h"], 1, g["L"], 1) * 2 == base


def pin_size_matches_storage(orc):
    """The size formula equals the bytes of the cache tensors actually built."""
    n_l, B, n_kv, d, L = 3, 2, 4, 64, 37
    total = 0
    for layer in range(n_l):
        c = syn.dense_case(B, 8, n_kv, d, L, [L] * B, syn.BF16, layer=layer, poison=False)
        total += c["k_cache"].nbytes + c["v_cache"].nbytes
    assert total == orc.cache_bytes(n_l, n_kv, d, 2, L, B), total
    m = syn.mla_case(B, 4, 512, 64, L, [L] * B, syn.BF16, poison=False)
    assert m["ckv"].nbytes == orc.mla_cache_bytes(1, 512, 64, 2, L, B)


# ---------------------------------------------------------------- causal
def pin_causal_equals_recompute(orc):
    """Guide, first section: cached decode step t equals row t of full causal
    attention recomputed from scratch."""
    rng = np.random.default_rng(7)
    n, n_h, n_kv, d = 9, 6, 3, 5
    Q = rng.standard_normal((n, n_h, d)).astype(np.float32)
    K = rng.standard_normal((n, n_kv, d)).astype(np.float32)
    V = rng.standard_normal((n, n_kv, d)).astype(np.float32)
    scale = 1 / math.sqrt(d)
    full = orc.full_causal(Q, K, V, scale)
    kc = np.full((1, n_kv, n, d), np.nan, dtype=np.float32)
    vc = np.full((1, n_kv, n, d), np.nan, dtype=np.float32)
    lens = np.zeros(1, dtype=np.int32)
    for t in range(n):
        flag = orc.append(kc, vc, lens, K[t][None], V[t][None])
        assert flag == 0 and lens[0] == t + 1
        o, _ = orc.decode(Q[t][None], kc, vc, lens, scale)
        np.testing.assert_allclose(o[0], full[t], rtol=0, atol=1e-12)


def pin_full_causal_bruteforce(orc):
    """full_causal row t equals a scalar brute force over positions 0..t."""
    rng = np.random.default_rng(11)
    n, n_h, n_kv, d = 5, 4, 2, 3
    Q = rng.standard_normal((n, n_h, d))
    K = rng.standard_normal((n, n_kv, d))
    V = rng.standard_normal((n, n_kv, d))
    full = orc.full_causal(Q, K, V, 0.7)
    G = n_h // n_kv
    for t in range(n):
        for i in range(n_h):
            j = i // G
            ref, _ = brute_attend(Q[t, i], K[:t + 1, j], V[:t + 1, j], 0.7)
            np.testing.assert_allclose(full[t, i], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------- brute force
def pin_decode_bruteforce(orc):
    """Dense GQA decode equals a scalar brute force (independent arithmetic),
    for ragged lengths including 0 and 1."""
    rng = np.random.default_rng(3)
    B, n_h, n_kv, d = 4, 6, 2, 4
    lens = [5, 1, 0, 7]
    q, kc, vc, sl = _f64_case(rng, B, n_h, n_kv, d, lens, L_max=8)
    kc[:, :, 7:] = np.nan  # never read: lens <= 7
    vc[:, :, 7:] = np.nan
    o, lse = orc.decode(q, kc, vc, sl, 0.5)
    G = n_h // n_kv
    for b in range(B):
        for i in range(n_h):
            n = lens[b]
            if n == 0:
                assert np.all(o[b, i] == 0) and lse[b, i] == -math.inf
                continue
            ref, rl = brute_attend(q[b, i], kc[b, i // G, :n], vc[b, i // G, :n], 0.5)
            np.testing.assert_allclose(o[b, i], ref, rtol=0, atol=1e-12)
            assert abs(lse[b, i] - rl) < 1e-12


# --------------------------------------------------------- closed forms
def pin_single_position(orc):
    """One position: weight 1, so o = v_0 exactly; lse = scale * q.k_0."""
    rng = np.random.default_rng(5)
    q, kc, vc, sl = _f64_case(rng, 2, 4, 2, 8, [1, 1], L_max=3)
    kc[:, :, 1:] = np.nan
    vc[:, :, 1:] = np.nan
    o, lse = orc.decode(q, kc, vc, sl, 0.25)
    for b in range(2):
        for i in range(4):
            assert np.array_equal(o[b, i], vc[b, i // 2, 0].astype(np.float64))
            s = 0.25 * math.fsum(float(a) * float(c) for a, c in zip(q[b, i], kc[b, i // 2, 0]))
            assert abs(lse[b, i] - s) < 1e-12


def pin_weights_sum_to_one(orc):
    """V = 1 everywhere gives o = 1 (the weights sum to one)."""
    rng = np.random.default_rng(6)
    q, kc, vc, sl = _f64_case(rng, 2, 8, 2, 16, [33, 70], L_max=70)
    vc[:] = 1.0
    o, _ = orc.decode(q * 3, kc, vc, sl, 1.0)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


def pin_two_positions(orc):
    """n = 2: o = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1, with hand scores.

    q = (1, 2), k0 = (1, 0), k1 = (0, 1), scale 1.5 -> s0 = 1.5, s1 = 3.
    """
    q = np.array([[[1.0, 2.0]]], dtype=np.float32)
    kc = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], dtype=np.float32)
    vc = np.array([[[[10.0, -1.0], [2.0, 4.0]]]], dtype=np.float32)
    o, lse = orc.decode(q, kc, vc, np.array([2], dtype=np.int32), 1.5)
    w0 = 1.0 / (1.0 + math.exp(3.0 - 1.5))
    w1 = 1.0 / (1.0 + math.exp(1.5 - 3.0))
    np.testing.assert_allclose(o[0, 0], [10 * w0 + 2 * w1, -1 * w0 + 4 * w1], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - (3.0 + math.log(1 + math.exp(-1.5)))) < 1e-14


def pin_uniform_query(orc):
    """q = 0 (or scale = 0): equal weights, o = mean of V rows; V[t] = t gives (n-1)/2."""
    for n in (1, 2, 17, 64):
        q = np.zeros((1, 2, 4), dtype=np.float32)
        kc = np.random.default_rng(n).standard_normal((1, 1, n, 4)).astype(np.float32)
        vc = np.repeat(np.arange(n, dtype=np.float32)[None, None, :, None], 4, axis=3)
        o, lse = orc.decode(q, kc, vc, np.array([n], dtype=np.int32), 0.125)
        np.testing.assert_allclose(o, (n - 1) / 2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, math.log(n), rtol=0, atol=1e-12)
        q1 = np.random.default_rng(1).standard_normal((1, 2, 4)).astype(np.float32)
        o0, _ = orc.decode(q1, kc, vc, np.array([n], dtype=np.int32), 0.0)
        np.testing.assert_allclose(o0, (n - 1) / 2, rtol=0, atol=1e-12)


def pin_saturation(orc):
    """Scores far apart: the softmax is one-hot on the max, with no overflow."""
    q = np.array([[[1.0]]], dtype=np.float32)
    kc = np.array([[[[1000.0], [-50.0], [999.0 - 40.0]]]], dtype=np.float32)
    vc = np.array([[[[3.0], [7.0], [11.0]]]], dtype=np.float32)
    o, lse = orc.decode(q, kc, vc, np.array([3], dtype=np.int32), 1.0)
    assert np.isfinite(o).all() and abs(o[0, 0, 0] - 3.0) < 1e-15
    assert abs(lse[0, 0] - 1000.0) < 1e-12


def pin_scale_is_multiplicative(orc):
    """Scaling q by a and scale by 1/a leaves the result unchanged; and the
    scale enters the scores (scale 0 vs 1 differ for random data)."""
    rng = np.random.default_rng(8)
    q, kc, vc, sl = _f64_case(rng, 1, 2, 1, 8, [20])
    o1, _ = orc.decode(q, kc, vc, sl, 0.5)
    o2, _ = orc.decode(q * 4, kc, vc, sl, 0.125)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    o3, _ = orc.decode(q, kc, vc, sl, 0.0)
    assert np.abs(o1 - o3).max() > 1e-3


# ------------------------------------------------------------- invariants
def pin_permutation(orc):
    """Permuting cached positions (K and V together) leaves o unchanged."""
    rng = np.random.default_rng(9)
    q, kc, vc, sl = _f64_case(rng, 1, 4, 2, 8, [31])
    o, lse = orc.decode(q, kc, vc, sl, 0.3)
    perm = rng.permutation(31)
    o2, lse2 = orc.decode(q, kc[:, :, perm], vc[:, :, perm], sl, 0.3)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def pin_split_merge(orc):
    """Decoding disjoint parts and merging by log-sum-exp equals one pass;
    lse equals log(sum(exp(s))) from a scalar brute force."""
    rng = np.random.default_rng(10)
    d, n = 8, 50
    q, kc, vc, sl = _f64_case(rng, 1, 1, 1, d, [n])
    o, lse = orc.decode(q, kc, vc, sl, 0.4)
    s = [0.4 * math.fsum(float(a) * float(b) for a, b in zip(q[0, 0], kc[0, 0, t])) for t in range(n)]
    m = max(s)
    assert abs(lse[0, 0] - (m + math.log(math.fsum(math.exp(x - m) for x in s)))) < 1e-12
    for cuts in ([25], [1, 2, 49], [10, 20, 30, 40], [0, 50]):
        bounds = [0] + cuts + [n]
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            po, pl = orc.decode(q, kc[:, :, a:b], vc[:, :, a:b], np.array([b - a], dtype=np.int32), 0.4)
            parts_o.append(po[0, 0])
            parts_l.append(pl[0, 0])
        mo, ml = orc.merge_partials(parts_o, parts_l)
        np.testing.assert_allclose(mo, o[0, 0], rtol=0, atol=1e-12)
        assert abs(ml - lse[0, 0]) < 1e-12


def pin_gqa_head_mapping(orc):
    """Guide, 'Fewer KV heads': groups of G query heads share one KV head.
    With V_j = j + 1 everywhere, head i returns i // G + 1; GQA equals MHA
    with each KV head repeated G times; MQA is the n_kv = 1 case."""
    rng = np.random.default_rng(12)
    B, n_h, n_kv, d = 2, 12, 3, 8
    G = n_h // n_kv
    q, kc, vc, sl = _f64_case(rng, B, n_h, n_kv, d, [13, 40], L_max=40)
    vconst = vc.copy()
    for j in range(n_kv):
        vconst[:, j] = j + 1
    o, _ = orc.decode(q, kc, vconst, sl, 0.35)
    for i in range(n_h):
        np.testing.assert_allclose(o[:, i], i // G + 1, rtol=0, atol=1e-13)
    og, lg = orc.decode(q, kc, vc, sl, 0.35)
    om, lm = orc.decode(q, np.repeat(kc, G, axis=1), np.repeat(vc, G, axis=1), sl, 0.35)
    np.testing.assert_allclose(og, om, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lg, lm, rtol=0, atol=1e-13)
    oq, _ = orc.decode(q, kc[:, :1], vc[:, :1], sl, 0.35)
    om1, _ = orc.decode(q, np.repeat(kc[:, :1], n_h, axis=1), np.repeat(vc[:, :1], n_h, axis=1), sl, 0.35)
    np.testing.assert_allclose(oq, om1, rtol=0, atol=1e-13)


# -------------------------------------------------------------------- MLA
def pin_mla_dims_and_scale():
    """Guide footnote: 512 + 64 per row, so the score scale 1/sqrt(576) = 1/24."""
    g = golden()["mla_row"]
    assert math.sqrt(g["d_c"] + g["d_r"]) == 24.0
    assert syn.C4.d_c == g["d_c"] and syn.C4.d_r == g["d_r"] and syn.C4.scale == 1 / 24


def pin_mla_reduces_to_dense(orc):
    """MLA equals dense MQA decode with K = the whole row (latent and rotary
    key) and V = the latent part only; checked also against brute force with
    the two score terms written separately."""
    rng = np.random.default_rng(13)
    B, n_h, d_c, d_r = 2, 5, 12, 4
    L_max = 20
    lens = np.array([20, 3], dtype=np.int32)
    q = rng.standard_normal((B, n_h, d_c + d_r)).astype(np.float32)
    ckv = rng.standard_normal((B, L_max, d_c + d_r)).astype(np.float32)
    o, lse = orc.decode_mla(q, ckv, lens, d_c, d_r, 0.2)
    od, ld = orc.decode(q, ckv[:, None], np.ascontiguousarray(ckv[:, None, :, :d_c]), lens, 0.2)
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-13)
    for b in range(B):
        n = int(lens[b])
        for i in range(n_h):
            s = [0.2 * (math.fsum(float(a) * float(c) for a, c in zip(q[b, i, :d_c], ckv[b, t, :d_c]))
                        + math.fsum(float(a) * float(c) for a, c in zip(q[b, i, d_c:], ckv[b, t, d_c:])))
                 for t in range(n)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            ref = [math.fsum(w[t] * float(ckv[b, t, c]) for t in range(n)) / z for c in range(d_c)]
            np.testing.assert_allclose(o[b, i], ref, rtol=0, atol=1e-12)


def pin_mla_rope_matters(orc):
    """The rotary part enters the score: zeroing q_rope changes the result,
    and a latent-orthogonal rotary key alone can decide the weights."""
    q = np.zeros((1, 1, 3), dtype=np.float32)
    q[0, 0, 2] = 1.0  # rotary query only
    ckv = np.array([[[5.0, 0.0, 100.0], [7.0, 1.0, 0.0]]], dtype=np.float32)
    o, _ = orc.decode_mla(q, ckv, np.array([2], dtype=np.int32), 2, 1, 1.0)
    np.testing.assert_allclose(o[0, 0], [5.0, 0.0], rtol=0, atol=1e-12)


# ------------------------------------------------------------------ top-k
def pin_topk(orc):
    """Podcast, DSA passage: attend over the listed positions only.

    * all positions listed -> dense decode;
    * a subset -> dense decode of the gathered sub-cache;
    * q = 0 and V[t, 0] = t -> o[0] = mean of the listed indices;
    * out-of-range indices are skipped and raise flag bit 1.
    """
    rng = np.random.default_rng(14)
    B, n_h, n_kv, d, L = 2, 4, 2, 8, 64
    lens = np.array([64, 40], dtype=np.int32)
    q, kc, vc, _ = _f64_case(rng, B, n_h, n_kv, d, [L, L], L_max=L)
    allidx = np.broadcast_to(np.arange(40, dtype=np.int32), (B, n_kv, 40)).copy()
    o, lse, flag = orc.decode_topk(q, kc, vc, np.array([40, 40], dtype=np.int32), allidx, 0.3)
    od, ld = orc.decode(q, kc, vc, np.array([40, 40], dtype=np.int32), 0.3)
    assert flag == 0
    np.testing.assert_allclose(o, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-13)

    idx = np.stack([np.stack([np.sort(rng.choice(int(lens[b]), 11, replace=False))
                              for _ in range(n_kv)]) for b in range(B)]).astype(np.int32)
    o, lse, flag = orc.decode_topk(q, kc, vc, lens, idx, 0.3)
    assert flag == 0
    G = n_h // n_kv
    for b in range(B):
        for i in range(n_h):
            I = idx[b, i // G]
            ref, rl = brute_attend(q[b, i], kc[b, i // G, I], vc[b, i // G, I], 0.3)
            np.testing.assert_allclose(o[b, i], ref, rtol=0, atol=1e-12)
            assert abs(lse[b, i] - rl) < 1e-12

    vt = np.zeros_like(vc)
    vt[..., 0] = np.arange(L, dtype=np.float32)[None, None, :]
    o, _, _ = orc.decode_topk(np.zeros_like(q), kc, vt, lens, idx, 0.3)
    for b in range(B):
        for i in range(n_h):
            assert abs(o[b, i, 0] - idx[b, i // G].mean()) < 1e-12

    bad = idx.copy()
    bad[1, 0, 0] = 45      # >= lens[1] = 40
    bad[0, 1, 3] = -1
    o, _, flag = orc.decode_topk(np.zeros_like(q), kc, vt, lens, bad, 0.3)
    assert flag == orc.FLAG_BAD_INDEX
    assert abs(o[1, 0, 0] - idx[1, 0, 1:].mean()) < 1e-12


# ----------------------------------------------------------------- append
def pin_append(orc):
    """Append copies bits (NaN payloads, -0.0, bf16 patterns), increments the
    length, touches nothing else; a full cache sets flag bit 0 and is left
    untouched."""
    B, n_kv, L_max, d = 3, 2, 4, 5
    kc = np.full((B, n_kv, L_max, d), 0xABCD, dtype=np.uint16)
    vc = np.full((B, n_kv, L_max, d), 0x1234, dtype=np.uint16)
    lens = np.array([0, 2, 4], dtype=np.int32)
    kn = np.arange(B * n_kv * d, dtype=np.uint16).reshape(B, n_kv, d) | 0x7F80
    vn = np.array([0x8000, 0x7FC1, 0xFFFF, 0x0001, 0x3F80] * (B * n_kv), dtype=np.uint16).reshape(B, n_kv, d)
    k0, v0 = kc.copy(), vc.copy()
    flag = orc.append(kc, vc, lens, kn, vn)
    assert flag == orc.FLAG_CACHE_FULL
    assert lens.tolist() == [1, 3, 4]
    for b, slot in ((0, 0), (1, 2)):
        assert np.array_equal(kc[b, :, slot], kn[b]) and np.array_equal(vc[b, :, slot], vn[b])
        keep = [t for t in range(L_max) if t != slot]
        assert np.array_equal(kc[b, :, keep], k0[b, :, keep])
        assert np.array_equal(vc[b, :, keep], v0[b, :, keep])
    assert np.array_equal(kc[2], k0[2]) and np.array_equal(vc[2], v0[2])
    # float32 storage: -0.0 and a NaN payload survive bit for bit
    kf = np.zeros((1, 1, 2, 2), dtype=np.float32)
    vf = np.zeros((1, 1, 2, 2), dtype=np.float32)
    nan_payload = np.array([0x7FC00123], dtype=np.uint32).view(np.float32)[0]
    new = np.array([[[-0.0, nan_payload]]], dtype=np.float32)
    lf = np.array([1], dtype=np.int32)
    orc.append(kf, vf, lf, new, new)
    assert kf[0, 0, 1].view(np.uint32).tolist() == [0x80000000, 0x7FC00123]
    assert lf[0] == 2


def pin_bf16_decoding(orc):
    """bf16 is the top half of an IEEE float32."""
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], dtype=np.uint16)
    got = orc.bf16_to_f64(bits)
    want = [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, -0.0, 3.140625]
    assert got.tolist() == want
    assert math.copysign(1.0, got[5]) == -1.0


# ---------------------------------------------------------------- FP8 E4M3
# Code values from the format's bit fields (sign, 4-bit exponent with bias 7,
# 3-bit mantissa; exponent 0 subnormal; 0x7F/0xFF NaN), and the page's
# figure for its largest value.
_FP8_KNOWN = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3A: 1.25, 0x3C: 1.5, 0x3F: 1.875,
              0x40: 2.0, 0x44: 3.0, 0x4C: 6.0, 0x7D: 416.0, 0x7E: 448.0,
              0x80: -0.0, 0xB8: -1.0, 0xC0: -2.0, 0xFE: -448.0}


def pin_fp8_page_max(orc):
    """The DeepSeek article's headroom bound: the block format tops out at
    448 x 6 = 2688, 448 being the largest E4M3 value."""
    g = golden()["fp8_e4m3_max"]
    assert g["e4m3_max"] * g["e2m1_max"] == g["product"]
    assert orc.FP8_E4M3_MAX == g["e4m3_max"]
    assert float(orc.fp8_e4m3_to_f64(np.array([0x7E], np.uint8))[0]) == g["e4m3_max"]
    # nothing finite above it
    allv = orc.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.nanmax(np.abs(allv)) == g["e4m3_max"]


def pin_fp8_codes(orc):
    """Known code values; NaN codes; 127 finite non-negative values,
    strictly increasing with the code."""
    codes = np.array(sorted(_FP8_KNOWN), dtype=np.uint8)
    got = orc.fp8_e4m3_to_f64(codes)
    for c, v in zip(codes.tolist(), got.tolist()):
        assert v == _FP8_KNOWN[c], (hex(c), v)
    assert math.copysign(1.0, float(orc.fp8_e4m3_to_f64(np.array([0x80], np.uint8))[0])) == -1.0
    assert np.isnan(orc.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()
    pos = orc.fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    # negative codes mirror positive ones
    neg = orc.fp8_e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(-pos[1:], neg[1:])


def pin_fp8_roundtrip(orc):
    """Every finite code encodes back to itself."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = orc.f64_to_fp8_e4m3(orc.fp8_e4m3_to_f64(codes))
    assert np.array_equal(back, codes)


def _nearest_even_code(x, table):
    """Scalar brute force over (code, value) pairs: nearest value, ties to
    the even code, saturating at the largest magnitude."""
    a = min(abs(x), 448.0)
    best = None
    for c, v in table:
        dist = abs(a - v)
        key = (dist, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    return c | (0x80 if math.copysign(1.0, x) < 0 else 0)


def pin_fp8_rounding(orc):
    """Round to nearest, ties to even, saturate: worked ties, the clamp,
    and a scalar brute force over random float32 values."""
    cases = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02,
             1e6: 0x7E, -1e6: 0xFE, 464.0: 0x7E, 447.0: 0x7E, 432.0: 0x7E,
             431.0: 0x7D, 0.0: 0x00}
    xs = np.array(list(cases), dtype=np.float64)
    got = orc.f64_to_fp8_e4m3(xs)
    for x, c in zip(xs.tolist(), got.tolist()):
        assert c == cases[x], (x, hex(c))
    assert orc.f64_to_fp8_e4m3(np.array([-0.0])).tolist() == [0x80]
    rng = np.random.default_rng(7)
    ys = (rng.standard_normal(400) * np.exp2(rng.integers(-12, 10, 400))).astype(np.float32).astype(np.float64)
    got = orc.f64_to_fp8_e4m3(ys)
    full = [(c, float(2.0 ** -9 * (c & 7)) if (c >> 3) == 0 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7))
            for c in range(0x7F)]
    for y, c in zip(ys.tolist(), got.tolist()):
        assert c == _nearest_even_code(y, full), (y, hex(c))


def pin_fp8_quantize_scale(orc):
    """A stored code times the scale gives the number back: 3.0 stored with
    scale 2 is code 1.5 (0x3C), with scale 0.5 it is code 6.0 (0x4C)."""
    x = syn.bf16_bits(np.array([3.0, -3.0], np.float32))
    assert orc.quantize_fp8(x, 2.0).tolist() == [0x3C, 0xBC]
    assert orc.quantize_fp8(x, 0.5).tolist() == [0x4C, 0xCC]
    # float32 inputs too
    assert orc.quantize_fp8(np.array([448.0 * 4], np.float32), 4.0).tolist() == [0x7E]


def pin_fp8_decode(orc):
    """decode_fp8 equals scalar brute-force attention over values taken
    from known codes (times the scales); append_fp8 stores quantised rows
    at the length slot."""
    rng = np.random.default_rng(11)
    known = np.array([c for c in _FP8_KNOWN if c not in (0x80,)], dtype=np.uint8)
    B, n_h, n_kv, d, L = 1, 4, 2, 8, 6
    kc = rng.choice(known, size=(B, n_kv, L, d)).astype(np.uint8)
    vc = rng.choice(known, size=(B, n_kv, L, d)).astype(np.uint8)
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    lens = np.array([5], np.int32)
    ks, vs = 0.25, 1.5
    o, l = orc.decode_fp8(q, kc, vc, lens, 0.3, ks, vs)
    for i in range(n_h):
        j = i // (n_h // n_kv)
        Kf = [[_FP8_KNOWN[int(c)] * ks for c in row] for row in kc[0, j, :5]]
        Vf = [[_FP8_KNOWN[int(c)] * vs for c in row] for row in vc[0, j, :5]]
        bo, bl = brute_attend(q[0, i], Kf, Vf, 0.3)
        assert np.allclose(o[0, i], bo, rtol=1e-12, atol=1e-12)
        assert abs(l[0, i] - bl) < 1e-12
    k8 = np.zeros((1, 1, 4, 2), np.uint8)
    v8 = np.zeros((1, 1, 4, 2), np.uint8)
    sl = np.array([2], np.int32)
    kn = syn.bf16_bits(np.array([[[1.0, -2.0]]], np.float32))
    vn = syn.bf16_bits(np.array([[[3.0, 0.5]]], np.float32))
    f = orc.append_fp8(k8, v8, sl, kn, vn, 1.0, 0.5)
    assert f == 0 and int(sl[0]) == 3
    assert k8[0, 0, 2].tolist() == [0x38, 0xC0] and v8[0, 0, 2].tolist() == [0x4C, 0x38]
    assert not k8[0, 0, [0, 1, 3]].any()


# ------------------------------------------------------------ FP4 (E2M1)
# E2M1 magnitudes from the OCP element definition (1 sign, 2 exponent bits
# with bias 1, 1 mantissa bit; exponent field 0 is subnormal: 0 and 0.5).
_E2M1_TABLE = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def _e4m3_positive():
    """All finite positive E4M3 values, from the field definition."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return sorted(set(vals))


def pin_fp4_format(orc):
    """The 890-byte passage: E2M1 with one E4M3 scale per 16 channels, no
    global scale; the article's bound 448 x 6 = 2688 is the largest stored
    magnitude.  Codes decode to the OCP E2M1 table and every code survives
    decode then encode."""
    g = golden()
    f = g["fp4_block_format"]
    assert f["block_channels"] == orc.FP4_BLOCK and not f["global_scale"]
    assert orc.FP4_E2M1_MAX == g["fp8_e4m3_max"]["e2m1_max"]
    for c, v in _E2M1_TABLE.items():
        assert float(orc.fp4_e2m1_to_f64(np.array([c]))[0]) == v
        assert float(orc.fp4_e2m1_to_f64(np.array([c | 8]))[0]) == -v
    codes = np.arange(16)
    assert (orc.f64_to_fp4_e2m1(orc.fp4_e2m1_to_f64(codes)) == codes).all()
    # a block whose largest magnitude is the format's maximum
    x = np.zeros((1, 16), np.float32)
    x[0, 3] = g["fp8_e4m3_max"]["product"]
    x[0, 5] = -g["fp8_e4m3_max"]["product"]
    pk, sc = orc.quantize_fp4(syn.bf16_bits(x))
    assert int(sc[0, 0]) == 0x7E                      # scale 448
    deq = orc.dequantize_fp4(pk, sc)
    assert deq[0, 3] == 2688.0 and deq[0, 5] == -2688.0 and not deq[0, [0, 1, 2, 4]].any()


def pin_fp4_rounding(orc):
    """Nearest E2M1 value, ties to the even code, saturation past 6, sign
    kept for zero; checked at every midpoint and against a brute-force
    nearest search over the eight magnitudes."""
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in mids.items():
        assert int(orc.f64_to_fp4_e2m1(np.array([x]))[0]) == c
        assert int(orc.f64_to_fp4_e2m1(np.array([-x]))[0]) == c | 8
    assert int(orc.f64_to_fp4_e2m1(np.array([100.0]))[0]) == 7
    assert int(orc.f64_to_fp4_e2m1(np.array([-0.0]))[0]) == 8
    rng = np.random.default_rng(12)
    xs = rng.uniform(-7, 7, 500)
    mags = sorted(_E2M1_TABLE.items(), key=lambda t: t[1])
    for x in xs:
        a = min(abs(x), 6.0)
        best = min(mags, key=lambda t: (abs(a - t[1]), t[0] % 2))
        got = int(orc.f64_to_fp4_e2m1(np.array([x]))[0])
        assert got == (best[0] | (8 if x < 0 else 0)), (x, got, best)


def pin_fp4_blocks(orc):
    """Block encoding: scale = the E4M3 value nearest float32(amax / 6)
    (found by brute force over all E4M3 values), each number the E2M1 code
    nearest float32(x / scale); even channel in the low nibble; an all-zero
    block stores zeros.  decode_fp4 is plain attention over the dequantised
    rows."""
    e4 = np.array(_e4m3_positive())
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((3, 48)) * np.array([[1.0], [0.01], [40.0]])).astype(np.float32)
    x[1, 16:32] = 0.0
    raw = syn.bf16_bits(x)
    xf = (raw.astype(np.uint32) << 16).view(np.float32)        # bf16 bits -> float32
    pk, sc = orc.quantize_fp4(raw)
    assert pk.shape == (3, 24) and sc.shape == (3, 3)
    deq = orc.dequantize_fp4(pk, sc)
    mags = np.array(sorted(_E2M1_TABLE.values()))
    for r in range(3):
        for blk in range(3):
            v = xf[r, 16 * blk:16 * blk + 16]
            amax = np.float32(np.max(np.abs(v)))
            s_raw = float(amax / np.float32(6.0))
            cand = np.concatenate([[0.0], e4])
            dist = np.abs(cand - s_raw)
            s = cand[np.argmin(dist)]
            if np.count_nonzero(dist == dist.min()) > 1:
                s = None        # a tie between two scales: checked by the code's parity below
            if s is not None:
                assert orc.fp8_e4m3_to_f64(sc[r, blk:blk + 1])[0] == s
            s = orc.fp8_e4m3_to_f64(sc[r, blk:blk + 1])[0]
            for c in range(16):
                want = 0.0
                if s > 0:
                    qv = float(np.float32(v[c]) / np.float32(s))
                    a = min(abs(qv), 6.0)
                    m = min(mags, key=lambda t: (abs(a - t), list(mags).index(t) % 2))
                    want = math.copysign(m, qv) * s
                assert deq[r, 16 * blk + c] == want, (r, blk, c)
    assert not pk[1, 8:16].any() and int(sc[1, 1]) == 0
    # nibble order
    y = np.zeros((1, 16), np.float32)
    y[0, 0], y[0, 1] = 6.0, -1.0
    p2, s2 = orc.quantize_fp4(syn.bf16_bits(y))
    assert int(s2[0, 0]) == 0x38 and int(p2[0, 0]) == (0x7 | (0xA << 4))
    # decode over dequantised rows
    B, n_h, n_kv, d, L = 1, 2, 1, 16, 5
    kx = rng.standard_normal((B, n_kv, L, d)).astype(np.float32)
    vx = rng.standard_normal((B, n_kv, L, d)).astype(np.float32)
    kc, ks = orc.quantize_fp4(syn.bf16_bits(kx))
    vc, vs = orc.quantize_fp4(syn.bf16_bits(vx))
    q = rng.standard_normal((B, n_h, d)).astype(np.float32)
    lens = np.array([4], np.int32)
    o, l = orc.decode_fp4(q, kc, ks, vc, vs, lens, 0.25)
    Kf = orc.dequantize_fp4(kc[0, 0, :4], ks[0, 0, :4])
    Vf = orc.dequantize_fp4(vc[0, 0, :4], vs[0, 0, :4])
    for i in range(n_h):
        bo, bl = brute_attend(q[0, i], Kf.tolist(), Vf.tolist(), 0.25)
        assert np.allclose(o[0, i], bo, rtol=1e-12, atol=1e-12) and abs(l[0, i] - bl) < 1e-12
    # append: codes and scales at slot n, one length bump
    kcache = np.zeros((1, 1, 3, 8), np.uint8)
    kscal = np.zeros((1, 1, 3, 1), np.uint8)
    vcache = np.zeros((1, 1, 3, 8), np.uint8)
    vscal = np.zeros((1, 1, 3, 1), np.uint8)
    sl = np.array([1], np.int32)
    f = orc.append_fp4(kcache, kscal, vcache, vscal, sl, syn.bf16_bits(kx[:, :, 0]),
                       syn.bf16_bits(vx[:, :, 0]))
    assert f == 0 and int(sl[0]) == 2
    assert (kcache[0, 0, 1] == kc[0, 0, 0]).all() and (kscal[0, 0, 1] == ks[0, 0, 0]).all()
    assert (vcache[0, 0, 1] == vc[0, 0, 0]).all() and (vscal[0, 0, 1] == vs[0, 0, 0]).all()
    assert not kcache[0, 0, [0, 2]].any() and not vscal[0, 0, [0, 2]].any()


# ---------------------------------------------------------- sliding window
def _window_lo_from_page_rule(n, W, s):
    """The page's rule for the query at position i = n - 1: keys from
    max(s, i - W + 1) through i.  Written with i, as the page states it."""
    i = n - 1
    return min(max(s, i - W + 1, 0), n)


def pin_window(orc):
    """Bounded-replay window rule (DeepSeek article): brute force over the
    page's [max(s, i - W + 1), i]; W >= n reduces to plain decode; W = 1
    returns the newest value row; the window and the positions before it
    merge (log-sum-exp) into the full decode; n_win = 128 attends exactly 128
    positions (closed-form mean); an empty window gives zeros and -inf."""
    g = golden()["swa_bounded_replay"]
    assert g["layers"] * g["n_win"] == g["replay_tokens"]
    rng = np.random.default_rng(21)
    B, n_h, n_kv, d = 3, 4, 2, 8
    lens = [1, 37, 90]
    q, kc, vc, sl = _f64_case(rng, B, n_h, n_kv, d, lens, L_max=90)
    for W, starts in ((1, None), (5, None), (33, [0, 10, 80]), (64, [0, 36, 0]), (200, None)):
        o, lse = orc.decode_window(q, kc, vc, sl, 0.3, W, starts)
        for b in range(B):
            st = 0 if starts is None else starts[b]
            lo = _window_lo_from_page_rule(lens[b], W, st)
            for i in range(n_h):
                j = i // (n_h // n_kv)
                if lo == lens[b]:
                    assert (o[b, i] == 0).all() and lse[b, i] == -math.inf
                    continue
                bo, bl = brute_attend(q[b, i], kc[b, j, lo:lens[b]], vc[b, j, lo:lens[b]], 0.3)
                assert np.allclose(o[b, i], bo, rtol=1e-12, atol=1e-12), (W, b, i)
                assert abs(lse[b, i] - bl) < 1e-12
    ofull, lfull = orc.decode(q, kc, vc, sl, 0.3)
    ow, lw = orc.decode_window(q, kc, vc, sl, 0.3, 10 ** 6)
    np.testing.assert_allclose(ow, ofull, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lw, lfull, rtol=0, atol=1e-13)
    o1, l1 = orc.decode_window(q, kc, vc, sl, 0.3, 1)
    for b in range(B):
        for i in range(n_h):
            j = i // (n_h // n_kv)
            np.testing.assert_allclose(o1[b, i], vc[b, j, lens[b] - 1], rtol=0, atol=1e-14)
            s_last = 0.3 * math.fsum(float(x) * float(y) for x, y in zip(q[b, i], kc[b, j, lens[b] - 1]))
            assert abs(l1[b, i] - s_last) < 1e-12
    # window W plus the positions before it = everything (merge by lse)
    W = 20
    ow, lw = orc.decode_window(q, kc, vc, sl, 0.3, W)
    n = lens[2]
    oh, lh = orc.decode(q[2:3], kc[2:3], vc[2:3], np.array([n - W], np.int32), 0.3)
    for i in range(n_h):
        mo, ml = orc.merge_partials([oh[0, i], ow[2, i]], [lh[0, i], lw[2, i]])
        np.testing.assert_allclose(mo, ofull[2, i], rtol=0, atol=1e-12)
        assert abs(ml - lfull[2, i]) < 1e-12
    # the page's window of 128: q = 0 weighs every attended position equally,
    # and V[t] = t averages to the middle of [n - 128, n)
    n = 300
    qz = np.zeros((1, 2, 4), np.float32)
    kz = rng.standard_normal((1, 1, n, 4)).astype(np.float32)
    vt = np.repeat(np.arange(n, dtype=np.float32)[None, None, :, None], 4, axis=3)
    o, lse = orc.decode_window(qz, kz, vt, np.array([n], np.int32), 0.5, g["n_win"])
    np.testing.assert_allclose(o, (2 * n - g["n_win"] - 1) / 2, rtol=0, atol=1e-9)
    np.testing.assert_allclose(lse, math.log(g["n_win"]), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ paging
def _to_pool(cache, beta, perm_rng=None, extra_blocks=0):
    """Lay a contiguous [B, n_kv, L, d] cache out as a pool [num_blocks,
    n_kv, beta, d] plus a block table, with explicit loops (physical block
    order shuffled when perm_rng is given)."""
    B, n_kv, L, d = cache.shape
    mb = L // beta
    nblk = B * mb + extra_blocks
    order = list(range(nblk))
    if perm_rng is not None:
        perm_rng.shuffle(order)
    pool = np.zeros((nblk, n_kv, beta, d), dtype=cache.dtype)
    table = np.full((B, mb), -1, dtype=np.int32)
    for b in range(B):
        for k in range(mb):
            phys = order[b * mb + k]
            table[b, k] = phys
            for j in range(n_kv):
                for o in range(beta):
                    pool[phys, j, o] = cache[b, j, k * beta + o]
    return pool, table


def pin_paged(orc):
    """Guide, 'The allocator, not the algorithm': a sequence wastes at most
    beta - 1 slots, under 3% at beta = 16 and mean length 512; decoding
    through a block table (any physical order, shared prefix blocks) equals
    decoding the contiguous cache; append writes exactly slot n of the
    mapped block; invalid blocks are skipped and flagged."""
    g = golden()["paged_waste_bound"]
    beta, mean = g["beta"], g["mean_len"]
    worst = [mean - beta + 1 + beta * k for k in (-2, -1, 0, 1, 2)]      # each wastes beta - 1
    assert sum(worst) / len(worst) == mean - beta + 1
    assert orc.paged_waste_fraction(worst, beta) == (beta - 1) / (mean - beta + 1)
    assert orc.paged_waste_fraction([mean + 1] * 7, beta) < g["bound_below"]
    assert orc.paged_waste_fraction([beta * 3] * 4, beta) == 0.0

    rng = np.random.default_rng(31)
    B, n_h, n_kv, d, beta, L = 3, 8, 2, 8, 4, 32
    lens = [0, 13, 32]
    q, kc, vc, sl = _f64_case(rng, B, n_h, n_kv, d, lens, L_max=L)
    o_ref, l_ref = orc.decode(q, kc, vc, sl, 0.45)
    for prng in (None, np.random.default_rng(5)):
        kp, table = _to_pool(kc, beta, prng, extra_blocks=3)
        vp, table2 = _to_pool(vc, beta, None if prng is None else np.random.default_rng(5), 3)
        assert np.array_equal(table, table2)
        o, lse, flag = orc.decode_paged(q, kp, vp, table, sl, 0.45)
        assert flag == 0
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-13)
    # shared prefix: sequence 1 points its first two blocks at sequence 2's
    kp, table = _to_pool(kc, beta)
    vp, _ = _to_pool(vc, beta)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[1, :, :2 * beta] = kc[2, :, :2 * beta]
    vc2[1, :, :2 * beta] = vc[2, :, :2 * beta]
    t2 = table.copy()
    t2[1, :2] = table[2, :2]
    o_sh, l_sh, _ = orc.decode_paged(q, kp, vp, t2, sl, 0.45)
    o_cp, l_cp = orc.decode(q, kc2, vc2, sl, 0.45)
    np.testing.assert_allclose(o_sh, o_cp, rtol=0, atol=1e-13)
    # an invalid block: its positions are skipped (brute force) and flagged
    t3 = table.copy()
    t3[2, 1] = kp.shape[0] + 7
    o3, l3, f3 = orc.decode_paged(q, kp, vp, t3, sl, 0.45)
    assert f3 == orc.FLAG_BAD_INDEX
    keep = [t for t in range(lens[2]) if t // beta != 1]
    for i in range(n_h):
        j = i // (n_h // n_kv)
        bo, bl = brute_attend(q[2, i], kc[2, j, keep], vc[2, j, keep], 0.45)
        assert np.allclose(o3[2, i], bo, rtol=1e-12, atol=1e-12)
        assert abs(l3[2, i] - bl) < 1e-12
    np.testing.assert_allclose(o3[:2], o_ref[:2], rtol=0, atol=1e-13)
    # append: exactly slot n of its block; full table and invalid block flagged
    kp = np.zeros((6, 2, 4, 3), np.float32)
    vp = np.zeros((6, 2, 4, 3), np.float32)
    table = np.array([[4, 1], [0, 5], [2, 77]], np.int32)
    sl = np.array([5, 8, 4], np.int32)          # b0: block 1 slot 1; b1: full; b2: block 77
    kn = np.arange(18, dtype=np.float32).reshape(3, 2, 3) + 1
    vn = -kn
    f = orc.append_paged(kp, vp, table, sl, kn, vn)
    assert f == orc.FLAG_CACHE_FULL | orc.FLAG_BAD_INDEX
    assert sl.tolist() == [6, 8, 4]
    assert np.array_equal(kp[1, :, 1], kn[0]) and np.array_equal(vp[1, :, 1], vn[0])
    kp[1, :, 1] = 0
    vp[1, :, 1] = 0
    assert not kp.any() and not vp.any()


# ------------------------------------------------------------ top-k select
def _heap_topk(scores_row, cand, K):
    """Independent selection: heapq.nlargest on (score, -position), then
    ascending positions."""
    import heapq
    best = heapq.nlargest(K, ((float(scores_row[t]), -t) for t in cand))
    return sorted(-t for _, t in best)


def pin_topk_select(orc):
    """DSA keeps the k = 2048 highest-scoring positions; the hierarchical
    indexer's pool is 2048 blocks of 8 positions (16,384 candidates) and its
    top-512 comes only from the pool.  Checked against an independent heap
    selection, ties (lower position first), a known permutation, short
    sequences (-1 padding) and the pool restriction."""
    g = golden()
    assert g["dsa_topk"]["k"] == 2048
    hp = g["hierarchical_indexer_pool"]
    assert hp["pool_blocks"] * hp["block_positions"] == hp["candidates"]
    rng = np.random.default_rng(41)
    B, R, L = 2, 3, 700
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    sc[0, 1, 100:400] = 0.5                      # a run of ties
    sl = np.array([700, 333], np.int32)
    K = 64
    got = orc.topk_select(sc, sl, K)
    for b in range(B):
        for j in range(R):
            want = _heap_topk(sc[b, j], range(int(sl[b])), K)
            assert got[b, j].tolist() == want, (b, j)
    # all equal: the first K positions
    eq = np.zeros((1, 1, 50), np.float32)
    assert orc.topk_select(eq, np.array([50]), 7)[0, 0].tolist() == list(range(7))
    # a permutation of 0..n-1 as scores: the top K are where n-K..n-1 sit
    perm = rng.permutation(300)
    ps = perm.astype(np.float32)[None, None]
    want = sorted(np.nonzero(perm >= 300 - 20)[0].tolist())
    assert orc.topk_select(ps, np.array([300]), 20)[0, 0].tolist() == want
    # fewer positions than K: all of them, then -1
    short = orc.topk_select(sc[:1, :1], np.array([5], np.int32), 8)[0, 0].tolist()
    assert short == [0, 1, 2, 3, 4, -1, -1, -1]
    # pool of 8-position blocks: candidates only from the listed blocks
    pool = np.full((B, R, 16), -1, np.int32)
    for b in range(B):
        for j in range(R):
            pool[b, j, :10] = rng.choice(L // 8, 10, replace=False)
    gp = orc.topk_select(sc, sl, 32, pool=pool, pool_block=hp["block_positions"])
    for b in range(B):
        for j in range(R):
            blocks = set(pool[b, j, :10].tolist())
            cand = [t for t in range(int(sl[b])) if t // 8 in blocks]
            want = _heap_topk(sc[b, j], cand, 32)
            assert gp[b, j, :len(want)].tolist() == want and (gp[b, j, len(want):] == -1).all()


ALL_PINS = [
    pin_size_llama2, pin_size_matches_storage, pin_causal_equals_recompute,
    pin_full_causal_bruteforce, pin_decode_bruteforce, pin_single_position,
    pin_weights_sum_to_one, pin_two_positions, pin_uniform_query,
    pin_saturation, pin_scale_is_multiplicative, pin_permutation,
    pin_split_merge, pin_gqa_head_mapping, pin_mla_reduces_to_dense,
    pin_mla_rope_matters, pin_topk, pin_append, pin_bf16_decoding,
    pin_fp8_page_max, pin_fp8_codes, pin_fp8_roundtrip, pin_fp8_rounding,
    pin_fp8_quantize_scale, pin_fp8_decode, pin_window, pin_paged, pin_topk_select,
    pin_fp4_format, pin_fp4_rounding, pin_fp4_blocks,
]
