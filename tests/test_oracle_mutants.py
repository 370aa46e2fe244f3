"""Planted mistakes in copies of the oracle must each trip at least one pin.

Each mutant is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one).  The mistakes live only in this file and
only run on the CPU.
"""
import math
import types

import numpy as np
import pytest

import oracle
import oracle_pins as P
from oracle import kvc_oracle as K


def _copy():
    return types.SimpleNamespace(**{k: getattr(K, k) for k in dir(K) if not k.startswith("__")})


def _decode_with(attend=None, head_of=None, length_of=None):
    attend = attend or K._attend

    def decode(q, k_cache, v_cache, seq_lens, scale):
        B, n_h, d = q.shape
        n_kv = k_cache.shape[1]
        G = n_h // n_kv
        o = np.zeros((B, n_h, v_cache.shape[3]))
        lse = np.full((B, n_h), -math.inf)
        for b in range(B):
            n = int(seq_lens[b]) if length_of is None else length_of(int(seq_lens[b]))
            for i in range(n_h):
                j = i // G if head_of is None else head_of(i, G, n_kv)
                Kb = K.to_f64(k_cache[b, j, :n])
                Vb = K.to_f64(v_cache[b, j, :n])
                o[b, i], lse[b, i] = attend(K.to_f64(q[b, i]), Kb, Vb, scale)
        return o, lse
    return decode


def _attend_variant(kind):
    def attend(q, Kr, Vr, scale):
        n = Kr.shape[0]
        if n == 0:
            return np.zeros(Vr.shape[1]), -math.inf
        if kind == "no_scale":
            s = Kr @ q
        elif kind == "neg":
            s = -scale * (Kr @ q)
        elif kind == "swap_kv":
            s = scale * (Vr @ q[:Vr.shape[1]]) if Vr.shape[1] == q.shape[0] else scale * (Kr @ q)
            Vr = Kr[:, :Vr.shape[1]]
        else:
            s = scale * (Kr @ q)
        if kind == "no_max":
            w = np.exp(s)
            z = w.sum()
            return (w @ Vr) / z, math.log(z)
        m = s.max()
        w = np.exp(s - m)
        z = w.sum()
        if kind == "log2_lse":
            return (w @ Vr) / z, m + math.log2(z)
        if kind == "no_norm":
            return (w @ Vr), m + math.log(z)
        return (w @ Vr) / z, m + math.log(z)
    return attend


def mutants():
    out = {}
    for kind in ("no_scale", "neg", "swap_kv", "no_max", "log2_lse", "no_norm"):
        m = _copy()
        m.decode = _decode_with(attend=_attend_variant(kind))
        m._attend = _attend_variant(kind)
        out["attend_" + kind] = m
    m = _copy()
    m.decode = _decode_with(head_of=lambda i, G, n_kv: i % n_kv)
    out["gqa_interleaved_heads"] = m
    m = _copy()
    m.decode = _decode_with(length_of=lambda n: max(n - 1, 0))
    out["drop_newest_position"] = m

    m = _copy()

    def append_no_inc(kc, vc, sl, kn, vn):
        sl0 = sl.copy()
        f = K.append(kc, vc, sl, kn, vn)
        sl[:] = sl0
        return f
    m.append = append_no_inc
    out["append_no_increment"] = m

    m = _copy()

    def append_next_slot(kc, vc, sl, kn, vn):
        B, n_kv, L_max, d = kc.shape
        f = 0
        for b in range(B):
            n = int(sl[b])
            if n >= L_max:
                f |= 1
                continue
            t = min(n + 1, L_max - 1)
            kc[b, :, t] = kn[b]
            if vc is not None:
                vc[b, :, t] = vn[b]
            sl[b] = n + 1
        return f
    m.append = append_next_slot
    out["append_wrong_slot"] = m

    m = _copy()

    def mla_no_rope(q, ckv, seq_lens, d_c, d_r, scale):
        q2 = q.copy()
        q2[..., d_c:] = 0
        return K.decode_mla(q2, ckv, seq_lens, d_c, d_r, scale)
    m.decode_mla = mla_no_rope
    out["mla_drops_rope_term"] = m

    m = _copy()

    def mla_rope_in_value(q, ckv, seq_lens, d_c, d_r, scale):
        o, l = K.decode(q, ckv[:, None] if ckv.ndim == 3 else ckv,
                        ckv[:, None] if ckv.ndim == 3 else ckv, seq_lens, scale)
        return o[..., :d_c] * 0 + o[..., d_r:d_r + d_c], l
    m.decode_mla = mla_rope_in_value
    out["mla_value_misaligned"] = m

    m = _copy()

    def topk_dense(q, kc, vc, sl, idx, scale):
        o, l = K.decode(q, kc, vc, sl, scale)
        return o, l, 0
    m.decode_topk = topk_dense
    out["topk_ignores_indices"] = m

    m = _copy()

    def topk_no_skip(q, kc, vc, sl, idx, scale):
        idx2 = np.clip(idx, 0, None)
        return K.decode_topk(q, kc, vc, np.full_like(sl, kc.shape[2]), idx2, scale)
    m.decode_topk = topk_no_skip
    out["topk_no_range_check"] = m

    m = _copy()
    m.bf16_to_f64 = lambda u: (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    out["bf16_wrong_shift"] = m

    m = _copy()
    m.cache_bytes = lambda n_l, n_kv, d_h, b, L, B: n_l * n_kv * d_h * b * L * B
    out["size_missing_factor_two"] = m

    m = _copy()

    def full_causal_leaky(Q, Kk, V, scale):
        Q, Kk, V = K.to_f64(Q), K.to_f64(Kk), K.to_f64(V)
        n, n_h, _ = Q.shape
        G = n_h // Kk.shape[1]
        mask = np.triu(np.full((n, n), -np.inf), k=2)
        O = np.zeros((n, n_h, V.shape[2]))
        for i in range(n_h):
            S = scale * (Q[:, i] @ Kk[:, i // G].T) + mask
            P_ = np.exp(S - S.max(axis=1, keepdims=True))
            O[:, i] = (P_ / P_.sum(axis=1, keepdims=True)) @ V[:, i // G]
        return O
    m.full_causal = full_causal_leaky
    out["causal_mask_off_by_one"] = m

    m = _copy()

    def merge_unweighted(os_, lses):
        return sum(np.asarray(o) for o in os_) / len(os_), max(lses)
    m.merge_partials = merge_unweighted
    out["merge_ignores_lse"] = m

    # FP8 E4M3 slips
    def fp8_decode_variant(bias=7, sub=2.0 ** -9):
        def dec(codes):
            c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
            sign = np.where((c >> 7) & 1, -1.0, 1.0)
            e, mm = (c >> 3) & 15, c & 7
            mag = np.where(e == 0, mm * sub, (1.0 + mm / 8.0) * np.exp2(e - float(bias)))
            return np.where((e == 15) & (mm == 7), np.nan, sign * mag)
        return dec
    m = _copy()
    m.fp8_e4m3_to_f64 = fp8_decode_variant(bias=8)
    out["fp8_exponent_bias_8"] = m
    m = _copy()
    m.fp8_e4m3_to_f64 = fp8_decode_variant(sub=2.0 ** -10)
    out["fp8_subnormal_scale"] = m

    def fp8_encode_variant(ties_up=False, saturate=True):
        def enc(x):
            x = np.asarray(x, dtype=np.float64)
            vals = K.fp8_e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
            a = np.abs(x)
            over = a > 448.0
            a = np.minimum(a, 448.0)
            hi = np.clip(np.searchsorted(vals, a), 0, 0x7E)
            lo = np.maximum(hi - 1, 0)
            d_lo, d_hi = a - vals[lo], vals[hi] - a
            pick = (d_hi < d_lo) | ((d_hi == d_lo) & (True if ties_up else (hi % 2 == 0)))
            code = np.where(a == vals[hi], hi, np.where(pick, hi, lo)).astype(np.uint8)
            code = code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
            if not saturate:
                code = np.where(over, np.uint8(0x7F), code)
            return code.astype(np.uint8)
        return enc
    m = _copy()
    m.f64_to_fp8_e4m3 = fp8_encode_variant(ties_up=True)
    out["fp8_ties_away_from_zero"] = m
    m = _copy()
    m.f64_to_fp8_e4m3 = fp8_encode_variant(saturate=False)
    out["fp8_overflow_to_nan"] = m

    m = _copy()

    def quantize_multiplies(x, scale):
        y = K.to_f64(x).astype(np.float32) * np.float32(scale)
        return K.f64_to_fp8_e4m3(y.astype(np.float64))
    m.quantize_fp8 = quantize_multiplies
    out["fp8_quantize_multiplies_scale"] = m

    m = _copy()

    def decode_fp8_no_vscale(q, kc, vc, sl, scale, ks, vs):
        return K.decode_fp8(q, kc, vc, sl, scale, ks, 1.0)
    m.decode_fp8 = decode_fp8_no_vscale
    out["fp8_decode_ignores_value_scale"] = m

    # sliding window
    def window_variant(lo_of):
        def decode_window(q, kc, vc, sl, scale, window, win_start=None):
            B, n_h, d = q.shape
            n_kv = kc.shape[1]
            G = n_h // n_kv
            o = np.zeros((B, n_h, vc.shape[3]))
            lse = np.full((B, n_h), -math.inf)
            for b in range(B):
                n = int(sl[b])
                st = 0 if win_start is None else int(win_start[b])
                lo = min(max(lo_of(n, window, st), 0), n)
                hi = n if lo_of is not _front else min(window, n)
                for i in range(n_h):
                    j = i // G
                    o[b, i], lse[b, i] = K._attend(K.to_f64(q[b, i]), K.to_f64(kc[b, j, lo:hi]),
                                                   K.to_f64(vc[b, j, lo:hi]), scale)
            return o, lse
        return decode_window

    def _front(n, W, st):
        return 0
    for name, lo_of in (("window_one_short", lambda n, W, st: max(st, n - W + 1)),
                        ("window_one_long", lambda n, W, st: max(st, n - W - 1)),
                        ("window_ignores_start", lambda n, W, st: n - W),
                        ("window_from_front", _front)):
        m = _copy()
        m.decode_window = window_variant(lo_of)
        out[name] = m

    # paging
    def rows_variant(kind):
        def paged_rows(pool, table, b, j, n, beta):
            rows, bad = [], []
            for t in range(n):
                k = t // beta if kind != "next_block" else (t + 1) // beta
                k = min(k, table.shape[1] - 1)
                blk = int(table[b, k]) if kind != "no_table" else b * table.shape[1] + t // beta
                if not 0 <= blk < pool.shape[0]:
                    bad.append(t)
                    continue
                off = t % beta if kind != "offset_swapped" else (t // beta) % beta
                rows.append(pool[blk, j, off])
            shape = (len(rows),) + pool.shape[3:]
            return (np.stack(rows) if rows else np.zeros(shape, dtype=pool.dtype)), bad
        return paged_rows
    for kind in ("next_block", "no_table", "offset_swapped"):
        m = _copy()
        m.paged_rows = rows_variant(kind)

        def decode_paged(q, kp, vp, table, sl, scale, _m=m):
            B, n_h, d = q.shape
            n_kv, beta = kp.shape[1], kp.shape[2]
            G = n_h // n_kv
            o = np.zeros((B, n_h, vp.shape[3]))
            lse = np.full((B, n_h), -math.inf)
            flag = 0
            for b in range(B):
                n = min(max(int(sl[b]), 0), table.shape[1] * beta)
                for j in range(n_kv):
                    Kr, bad = _m.paged_rows(kp, table, b, j, n, beta)
                    Vr, _ = _m.paged_rows(vp, table, b, j, n, beta)
                    flag |= K.FLAG_BAD_INDEX if bad else 0
                    for i in range(j * G, (j + 1) * G):
                        o[b, i], lse[b, i] = K._attend(K.to_f64(q[b, i]), K.to_f64(Kr), K.to_f64(Vr), scale)
            return o, lse, flag
        m.decode_paged = decode_paged
        out["paged_" + kind] = m

    def append_paged_slot_plus_one(kp, vp, table, sl, kn, vn):
        beta = kp.shape[2]
        flag = 0
        for b in range(sl.shape[0]):
            n = int(sl[b])
            if n >= table.shape[1] * beta:
                flag |= K.FLAG_CACHE_FULL
                continue
            blk = int(table[b, n // beta])
            if not 0 <= blk < kp.shape[0]:
                flag |= K.FLAG_BAD_INDEX
                continue
            kp[blk, :, (n + 1) % beta] = kn[b]
            vp[blk, :, (n + 1) % beta] = vn[b]
            sl[b] = n + 1
        return flag
    m = _copy()
    m.append_paged = append_paged_slot_plus_one
    out["append_paged_wrong_slot"] = m

    # top-k selection
    def select_variant(kind):
        def topk_select(scores, seq_lens, K, pool=None, pool_block=8):
            B, R, L = scores.shape
            out = np.full((B, R, K), -1, dtype=np.int32)
            for b in range(B):
                n = min(max(int(seq_lens[b]), 0), L)
                for j in range(R):
                    if pool is None or kind == "ignores_pool":
                        cand = range(n)
                    else:
                        blocks = {int(x) for x in pool[b, j] if x >= 0}
                        shift = 1 if kind == "pool_block_off_by_one" else 0
                        cand = [t for t in range(n) if t // pool_block + shift in blocks]
                    tie = (lambda t: -t) if kind == "ties_high" else (lambda t: t)
                    ranked = sorted(cand, key=lambda t: (-float(scores[b, j, t]), tie(t)))
                    ranked = ranked[:K - 1] if kind == "one_short" else ranked[:K]
                    if kind != "score_order":
                        ranked.sort()
                    out[b, j, :len(ranked)] = ranked
            return out
        return topk_select
    for kind in ("ties_high", "one_short", "score_order", "ignores_pool", "pool_block_off_by_one"):
        m = _copy()
        m.topk_select = select_variant(kind)
        out["topk_select_" + kind] = m

    # FP4 block format: each variant rebuilds the encoder / decoder chain
    def e2m1_encode(ties_away=False):
        def enc(q):
            q = np.asarray(q, dtype=np.float64)
            a = np.abs(q)
            vals = np.asarray(K._E2M1_MAG)
            best = np.zeros(a.shape, dtype=np.int64)
            for code in range(1, 8):
                d_new = np.abs(a - vals[code])
                d_best = np.abs(a - vals[best])
                tie = (code > best) if ties_away else (code % 2 == 0)
                best = np.where((d_new < d_best) | ((d_new == d_best) & tie), code, best)
            best = np.where(a > 6.0, 7, best)
            return (best | np.where(np.signbit(q), 8, 0)).astype(np.uint8)
        return enc

    def fp4_variant(kind):
        enc = e2m1_encode(ties_away=(kind == "ties_away"))
        block = 32 if kind == "block_32" else 16

        def decode_e2m1(codes):
            v = K.fp4_e2m1_to_f64(codes)
            return v * 2.0 if kind == "exponent_bias_0" else v

        def quantize(x_raw):
            x = K.to_f64(x_raw).astype(np.float32)
            shp = x.shape
            blk = x.reshape(shp[:-1] + (shp[-1] // block, block))
            amax = np.max(np.abs(blk), axis=-1)
            s_raw = amax if kind == "scale_amax" else amax / np.float32(6.0)
            sc = K.f64_to_fp8_e4m3(s_raw.astype(np.float64))
            s = K.fp8_e4m3_to_f64(sc).astype(np.float32)
            if kind == "scale_unrounded":
                s = s_raw.astype(np.float32)
            with np.errstate(divide="ignore", invalid="ignore"):
                q = blk / s[..., None]
            codes = np.where((s == 0)[..., None], np.uint8(0), enc(q.astype(np.float64)))
            codes = codes.astype(np.uint8).reshape(shp)
            lo, hi = (codes[..., 1::2], codes[..., 0::2]) if kind == "nibbles_swapped" else \
                     (codes[..., 0::2], codes[..., 1::2])
            packed = (lo | (hi << 4)).astype(np.uint8)
            if block == 32:
                sc = np.repeat(sc, 2, axis=-1)
            return packed, sc.astype(np.uint8)

        def dequantize(packed, scales):
            packed = np.asarray(packed, dtype=np.uint8)
            lo = decode_e2m1(packed & 0xF)
            hi = decode_e2m1(packed >> 4)
            vals = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
            s = K.fp8_e4m3_to_f64(np.asarray(scales, dtype=np.uint8))
            return vals * np.repeat(s, 16, axis=-1)

        m = _copy()
        m.f64_to_fp4_e2m1 = enc
        m.fp4_e2m1_to_f64 = decode_e2m1
        m.quantize_fp4 = quantize
        m.dequantize_fp4 = dequantize
        return m
    for kind in ("scale_amax", "ties_away", "nibbles_swapped", "block_32", "exponent_bias_0",
                 "scale_unrounded"):
        out["fp4_" + kind] = fp4_variant(kind)
    return out


MUTANTS = mutants()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    m = MUTANTS[name]
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


def test_real_oracle_passes_all():
    for pin in P.ALL_PINS:
        pin(oracle)
