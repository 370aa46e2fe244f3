"""FP8 E4M3 cache: HIP path vs the fp64 oracle through the C ABI (MI355X).

Codes written by kvc_append_fp8 must equal the oracle's bit for bit
(rounding ties, saturation, signed zero, subnormals, NaN included).  Decode
over E4M3 caches takes its cache codes from the oracle's quantiser on the
host and must match the oracle's decode within the bf16 tolerance (2e-2
max-abs on the output, 4e-3 on lse).  Every one of the 254 finite codes is
also checked exactly through the decode kernel's widening of keys and of
values.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import kvc_synth as syn
import oracle
from gpu_helpers import compare, compare_lse, dev, host, host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import kv_cache_decode_kvc_amd as kvc  # noqa: E402

NAN_CODE = 0x7F


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' elsewhere)")
    kvc.kvc_set_split_override(0)
    yield
    kvc.kvc_set_split_override(0)
    torch.cuda.synchronize()


def fp8_case(B, n_h, n_kv, d, L_max, pre, cfg_id, k_scale, v_scale):
    """bf16 inputs from the seeded generator; the cached rows are the oracle's
    E4M3 codes of the generated rows, the unused slots the NaN code."""
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, "bf16", cfg_id=cfg_id, poison=False)
    k8 = np.full((B, n_kv, L_max, d), NAN_CODE, np.uint8)
    v8 = np.full((B, n_kv, L_max, d), NAN_CODE, np.uint8)
    for b in range(B):
        n = int(pre[b])
        k8[b, :, :n] = oracle.quantize_fp8(case["k_cache"][b, :, :n], k_scale)
        v8[b, :, :n] = oracle.quantize_fp8(case["v_cache"][b, :, :n], v_scale)
    case["k8"], case["v8"] = k8, v8
    return case


def run_fp8_step(case, scale, k_scale, v_scale, split=0):
    k8, v8, sl = dev(case["k8"]), dev(case["v8"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_fp8(k8, v8, sl, kn, vn, k_scale, v_scale, flag=flag)
    B, n_h, d = q.shape
    n_kv, L_max = k8.shape[1], k8.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(B, n_h, n_kv, L_max, d))
    kvc.kvc_decode_attn_fp8(q, k8, v8, sl, out, k_scale, v_scale, lse, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert int(ws[:4 * B * n_kv].view(torch.int32).abs().sum()) == 0, "tickets not reset"
    return out, lse, sl, k8, v8, flag


def oracle_fp8_step(case, scale, k_scale, v_scale):
    k8, v8, sl = case["k8"].copy(), case["v8"].copy(), case["seq_lens"].copy()
    flag = oracle.append_fp8(k8, v8, sl, case["k_new"], case["v_new"], k_scale, v_scale)
    o, lse = oracle.decode_fp8(case["q"], k8, v8, sl, scale, k_scale, v_scale)
    return o, lse, sl, k8, v8, flag


# ------------------------------------------------------------------ append
def _special_row(d, k_scale):
    """bf16 values whose quotient by the (power-of-two) scale lands on the
    E4M3 grid's hard cases: ties between codes, the subnormal boundary, the
    saturation edge, signed zero, infinities and NaN."""
    q = [1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, -2.0 ** -10, 0.0, -0.0,
         448.0, 464.0, 447.0, 432.0, 431.0, 480.0, 1e6, -1e6,
         np.inf, -np.inf, np.nan, 2.0 ** -6, 2.0 ** -7 * 1.5, 0.5 + 2.0 ** -5, 240.0, 248.0]
    vals = np.zeros(d, np.float32)
    vals[:len(q)] = np.array(q, np.float64) * k_scale
    rest = np.random.default_rng(7).standard_normal(d - len(q)).astype(np.float32)
    vals[len(q):] = rest * np.float32(k_scale) * np.exp2(np.linspace(-12, 10, d - len(q))).astype(np.float32)
    return syn.bf16_bits(vals)


@pytest.mark.parametrize("k_scale,v_scale", [(0.25, 1.0), (1.0 / 64, 0.0625), (0.037, 3.3)])
def test_fp8_append_bit_exact(k_scale, v_scale):
    B, n_kv, d, L_max = 5, 3, 128, 9
    pre = [0, 4, 8, 9, 7]          # 9 == L_max: full, must flag and not write
    case = fp8_case(B, n_kv, n_kv, d, L_max, pre, 110, k_scale, v_scale)
    case["k_new"][1, 2] = _special_row(d, k_scale)
    case["v_new"][2, 0] = _special_row(d, v_scale)
    k8, v8, sl = dev(case["k8"]), dev(case["v8"]), dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_fp8(k8, v8, sl, dev(case["k_new"]), dev(case["v_new"]), k_scale, v_scale,
                       flag=flag)
    torch.cuda.synchronize()
    k_o, v_o, sl_o = case["k8"].copy(), case["v8"].copy(), case["seq_lens"].copy()
    f_o = oracle.append_fp8(k_o, v_o, sl_o, case["k_new"], case["v_new"], k_scale, v_scale)
    assert host(sl).tolist() == sl_o.tolist()
    assert int(host(flag)[0]) == f_o == 1
    gk, gv = host(k8), host(v8)
    bad = np.argwhere(gk != k_o)
    assert bad.size == 0, f"key codes differ at {bad[:5].tolist()}: {gk[tuple(bad[0])]:#x} vs {k_o[tuple(bad[0])]:#x}"
    assert np.array_equal(gv, v_o)


# ------------------------------------------------------------------ decode
FP8_CASES = [
    # (n_h, n_kv, pre-append lengths, L_max, split)
    (64, 8, [0, 30, 31, 32, 127, 128, 1000, 2047], 2048, 0),     # GQA G=8, ragged
    (32, 32, [4096], 4097, 0),                                    # MHA
    (16, 1, [5, 300], 512, 0),                                    # MQA G=16
    (8, 4, [100, 0, 255], 256, 0),                                # G=2
    (64, 8, [2999, 1000, 129], 3000, 128),                        # split sweep
    (64, 8, [2999, 1000, 129], 3000, 384),
    (64, 8, [2999, 1000, 129], 3000, 8192),
]


@pytest.mark.parametrize("n_h,n_kv,pre,L_max,split", FP8_CASES)
def test_fp8_decode_parity(n_h, n_kv, pre, L_max, split):
    k_scale, v_scale = 1.0 / 64, 0.02
    case = fp8_case(len(pre), n_h, n_kv, 128, L_max, pre, 111, k_scale, v_scale)
    scale = 1 / math.sqrt(128)
    out, lse, sl, k8, v8, flag = run_fp8_step(case, scale, k_scale, v_scale, split=split)
    o_ref, l_ref, sl_ref, k_ref, v_ref, f_ref = oracle_fp8_step(case, scale, k_scale, v_scale)
    assert host(sl).tolist() == sl_ref.tolist()
    assert np.array_equal(host(k8), k_ref) and np.array_equal(host(v8), v_ref)
    assert int(host(flag)[0]) == f_ref
    compare(host_f64(out), o_ref, 2e-2, f"fp8 {n_h}/{n_kv} split {split}")
    compare_lse(host(lse), l_ref, 4e-3)


def test_fp8_every_code_exact():
    """One cached position per sequence: the output is that position's value
    row times v_scale, and with a one-hot query at column c the lse is
    scale * k_scale * key[c].  All 256 codes are laid out over two sequences
    (the two NaN codes replaced by zero), so every finite code is widened
    through both operands; the one-hot columns also pin the key column
    order against the query's."""
    B, n_h, n_kv, d, L_max = 2, 128, 8, 128, 4
    G = n_h // n_kv
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    k8 = np.zeros((B, n_kv, L_max, d), np.uint8)
    v8 = np.zeros((B, n_kv, L_max, d), np.uint8)
    q = np.zeros((B, n_h, d), np.float32)
    for b in range(B):
        for j in range(n_kv):
            v8[b, j, 0] = codes[b * 128:(b + 1) * 128]
            k8[b, j, 0] = np.random.default_rng(b * 8 + j).integers(0, 0x7F, d)
            for h in range(G):
                c = j * G + h
                k8[b, j, 0, c] = codes[b * 128 + c]
                q[b, j * G + h, c] = 1.0
    k_scale, v_scale, scale = 0.125, 0.5, 0.25
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    qd = dev(syn.bf16_bits(q))
    out = torch.empty(B, n_h, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(B, n_h, n_kv, L_max, d))
    kvc.kvc_decode_attn_fp8(qd, dev(k8), dev(v8), sl, out, k_scale, v_scale, lse, scale=scale,
                            workspace=ws)
    torch.cuda.synchronize()
    o = host_f64(out)
    want_v = oracle.fp8_e4m3_to_f64(v8[:, :, 0]) * v_scale            # [B, n_kv, d]
    for b in range(B):
        for j in range(n_kv):
            assert np.array_equal(o[b, j * G:(j + 1) * G], np.broadcast_to(want_v[b, j], (G, d)))
    want_l = np.array([[scale * k_scale * oracle.fp8_e4m3_to_f64(k8[b, i // G, 0, i])
                        for i in range(n_h)] for b in range(B)])
    got_l = host(lse).astype(np.float64)
    assert np.abs(got_l - want_l).max() <= 1e-6 * np.abs(want_l).max() + 1e-7


def test_fp8_graph_replay_matches_oracle_loop():
    """Append + decode captured once and replayed: each replay appends one
    more token and matches the oracle's append/decode loop."""
    n_h, n_kv, d, L_max = 64, 8, 128, 1200
    pre = [1000, 3, 600]
    k_scale, v_scale = 1.0 / 32, 1.0 / 64
    case = fp8_case(len(pre), n_h, n_kv, d, L_max, pre, 112, k_scale, v_scale)
    B = len(pre)
    k8, v8, sl = dev(case["k8"]), dev(case["v8"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    out = torch.empty_like(q)
    ws = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(B, n_h, n_kv, L_max, d))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        kvc.kvc_append_fp8(k8, v8, sl, kn, vn, k_scale, v_scale)
        kvc.kvc_decode_attn_fp8(q, k8, v8, sl, out, k_scale, v_scale,
                                    scale=1 / math.sqrt(d), workspace=ws)
    k_o, v_o, sl_o = case["k8"].copy(), case["v8"].copy(), case["seq_lens"].copy()
    for step in range(3):
        g.replay()
        torch.cuda.synchronize()
        oracle.append_fp8(k_o, v_o, sl_o, case["k_new"], case["v_new"], k_scale, v_scale)
        o_ref, _ = oracle.decode_fp8(case["q"], k_o, v_o, sl_o, 1 / math.sqrt(d), k_scale, v_scale)
        assert host(sl).tolist() == sl_o.tolist()
        compare(host_f64(out), o_ref, 2e-2, f"fp8 replay {step}")
    assert np.array_equal(host(k8), k_o) and np.array_equal(host(v8), v_o)
