"""FP4 block-scaled cache (E2M1 codes, one E4M3 scale per 16 channels): HIP
path vs the fp64 oracle through the C ABI (MI355X).

Codes and scales written by kvc_append_fp4 must equal the oracle's bit for
bit (E2M1 ties at every midpoint, saturation, signed zero, zero blocks,
scale rounding and saturation at 448).  Decode over FP4 caches takes its
codes from the oracle's quantiser on the host and must match the oracle's
decode within the bf16 tolerance (2e-2 max-abs on the output, 4e-3 on lse).
Every one of the 16 codes under a range of scales is also checked exactly
through the decode kernel's dequantisation of keys and of values.
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


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' elsewhere)")
    kvc.kvc_set_split_override(0)
    yield
    kvc.kvc_set_split_override(0)
    torch.cuda.synchronize()


def fp4_case(B, n_h, n_kv, d, L_max, pre, cfg_id):
    """bf16 inputs from the seeded generator; the cached rows are the oracle's
    FP4 codes and scales of the generated rows, unused slots filled with
    0xFF codes and the 0x7F (NaN) scale so that any read of them shows."""
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, "bf16", cfg_id=cfg_id, poison=False)
    kc = np.full((B, n_kv, L_max, d // 2), 0xFF, np.uint8)
    vc = np.full((B, n_kv, L_max, d // 2), 0xFF, np.uint8)
    ks = np.full((B, n_kv, L_max, d // 16), 0x7F, np.uint8)
    vs = np.full((B, n_kv, L_max, d // 16), 0x7F, np.uint8)
    for b in range(B):
        n = int(pre[b])
        kc[b, :, :n], ks[b, :, :n] = oracle.quantize_fp4(case["k_cache"][b, :, :n])
        vc[b, :, :n], vs[b, :, :n] = oracle.quantize_fp4(case["v_cache"][b, :, :n])
    case.update(kc=kc, ks=ks, vc=vc, vs=vs)
    return case


def run_fp4_step(case, scale, split=0):
    kc, ks, vc, vs = dev(case["kc"]), dev(case["ks"]), dev(case["vc"]), dev(case["vs"])
    sl = dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_fp4(kc, ks, vc, vs, sl, kn, vn, flag=flag)
    B, n_h, d = q.shape
    n_kv, L_max = kc.shape[1], kc.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_fp4_workspace_size(B, n_h, n_kv, L_max, d))
    kvc.kvc_decode_attn_fp4(q, kc, ks, vc, vs, sl, out, lse, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert int(ws[:4 * B * n_kv].view(torch.int32).abs().sum()) == 0, "tickets not reset"
    return out, lse, sl, kc, ks, vc, vs, flag


def oracle_fp4_step(case, scale):
    kc, ks, vc, vs = (case[k].copy() for k in ("kc", "ks", "vc", "vs"))
    sl = case["seq_lens"].copy()
    flag = oracle.append_fp4(kc, ks, vc, vs, sl, case["k_new"], case["v_new"])
    o, lse = oracle.decode_fp4(case["q"], kc, ks, vc, vs, sl, scale)
    return o, lse, sl, kc, ks, vc, vs, flag


# ------------------------------------------------------------------ append
def _special_rows(d):
    """Blocks that hit the hard cases: quotients on every E2M1 midpoint (a
    block whose amax is 6 has scale exactly 1), saturation, signed zero, an
    all-zero block, tiny blocks (scale subnormal or rounding to zero),
    scales at and past 448, and a block whose scale rounds down so that its
    largest quotient exceeds 6."""
    blocks = []
    b = np.zeros(16, np.float32)
    b[:8] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    b[8:16] = [-0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -0.0]
    blocks.append(b)
    blocks.append(np.zeros(16, np.float32))
    blocks.append(np.full(16, -0.0, np.float32))
    blocks.append(np.linspace(-3e-3, 3e-3, 16).astype(np.float32))      # tiny: subnormal scale
    blocks.append(np.full(16, 1e-6, np.float32))                        # scale rounds to zero
    blocks.append(np.linspace(-2688.0, 2688.0, 16).astype(np.float32))  # scale 448
    blocks.append(np.array([1e5] + [1.0] * 15, np.float32))             # scale saturates
    blocks.append(np.array([6.6] + [-3.3, 1.1] * 7 + [0.1], np.float32))  # amax/6 rounds down
    x = np.concatenate(blocks)
    rest = np.random.default_rng(9).standard_normal(d * 2 - x.size).astype(np.float32)
    x = np.concatenate([x, rest * np.exp2(np.linspace(-8, 8, rest.size)).astype(np.float32)])
    return syn.bf16_bits(x[:d]), syn.bf16_bits(x[d:2 * d])


def test_fp4_append_bit_exact():
    B, n_kv, d, L_max = 5, 3, 128, 9
    pre = [0, 4, 8, 9, 7]          # 9 == L_max: full, must flag and not write
    case = fp4_case(B, n_kv, n_kv, d, L_max, pre, 120)
    r0, r1 = _special_rows(d)
    case["k_new"][1, 2], case["v_new"][2, 0] = r0, r1
    case["k_new"][4, 1], case["v_new"][0, 2] = r1, r0
    kc, ks, vc, vs = dev(case["kc"]), dev(case["ks"]), dev(case["vc"]), dev(case["vs"])
    sl = dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_fp4(kc, ks, vc, vs, sl, dev(case["k_new"]), dev(case["v_new"]), flag=flag)
    torch.cuda.synchronize()
    ref = {k: case[k].copy() for k in ("kc", "ks", "vc", "vs")}
    sl_o = case["seq_lens"].copy()
    f_o = oracle.append_fp4(ref["kc"], ref["ks"], ref["vc"], ref["vs"], sl_o, case["k_new"],
                            case["v_new"])
    assert host(sl).tolist() == sl_o.tolist()
    assert int(host(flag)[0]) == f_o == 1
    for name, got in (("kc", kc), ("ks", ks), ("vc", vc), ("vs", vs)):
        g = host(got)
        bad = np.argwhere(g != ref[name])
        assert bad.size == 0, f"{name} differs at {bad[:5].tolist()}: " \
                              f"{g[tuple(bad[0])]:#x} vs {ref[name][tuple(bad[0])]:#x}"


# ------------------------------------------------------------------ decode
FP4_CASES = [
    # (n_h, n_kv, pre-append lengths, L_max, split)
    (64, 8, [0, 30, 31, 32, 127, 128, 1000, 2047], 2048, 0),     # GQA G=8, ragged
    (32, 32, [4096], 4097, 0),                                    # MHA
    (16, 1, [5, 300], 512, 0),                                    # MQA G=16
    (8, 4, [100, 0, 255], 256, 0),                                # G=2
    (64, 8, [2999, 1000, 129], 3000, 128),                        # split sweep
    (64, 8, [2999, 1000, 129], 3000, 384),
    (64, 8, [2999, 1000, 129], 3000, 8192),
]


@pytest.mark.parametrize("n_h,n_kv,pre,L_max,split", FP4_CASES)
def test_fp4_decode_parity(n_h, n_kv, pre, L_max, split):
    case = fp4_case(len(pre), n_h, n_kv, 128, L_max, pre, 121)
    scale = 1 / math.sqrt(128)
    out, lse, sl, kc, ks, vc, vs, flag = run_fp4_step(case, scale, split=split)
    o_ref, l_ref, sl_ref, kc_r, ks_r, vc_r, vs_r, f_ref = oracle_fp4_step(case, scale)
    assert host(sl).tolist() == sl_ref.tolist()
    for got, want in ((kc, kc_r), (ks, ks_r), (vc, vc_r), (vs, vs_r)):
        assert np.array_equal(host(got), want)
    assert int(host(flag)[0]) == f_ref
    compare(host_f64(out), o_ref, 2e-2, f"fp4 {n_h}/{n_kv} split {split}")
    compare_lse(host(lse), l_ref, 4e-3)


@pytest.mark.parametrize("n_h", [128, 64])
def test_fp4_every_code_exact(n_h):
    """One cached position per sequence: the output is that position's value
    row dequantised, and with a one-hot query at column c the lse is
    scale * key[c].  The 2 x 8 x 8 blocks of each operand pattern take every
    finite non-negative E4M3 scale code 0x00 .. 0x7E (zero, the subnormals
    up to 448) in a different order for keys and values, and each block
    holds all 16 E2M1 codes in a rotated order, so every code meets every
    scale through both operands; the one-hot columns pin the key column
    order against the query's.  16 heads per KV head (every score column
    used) and 8 (half of them padding); sequence b holds pattern b % 2 and
    its heads read columns h + G * (b // 2), so each pattern's 128 columns
    are all read."""
    n_kv, d, L_max = 8, 128, 4
    G = n_h // n_kv
    B = 2 * (128 // G)
    all_scales = np.concatenate([np.arange(0x7F), [0x38]]).astype(np.uint8)   # 128 blocks
    v_scales = all_scales.reshape(2, n_kv, 8)
    k_scales = np.roll(all_scales, 37).reshape(2, n_kv, 8)
    kc = np.zeros((B, n_kv, L_max, d // 2), np.uint8)
    vc = np.zeros((B, n_kv, L_max, d // 2), np.uint8)
    ks = np.zeros((B, n_kv, L_max, d // 16), np.uint8)
    vs = np.zeros((B, n_kv, L_max, d // 16), np.uint8)
    q = np.zeros((B, n_h, d), np.float32)
    col = np.zeros((B, n_h), np.int64)
    for b in range(B):
        pb = b % 2
        for j in range(n_kv):
            codes = np.concatenate([np.roll(np.arange(16), j + blk + 3 * pb) for blk in range(8)])
            kcodes = np.roll(codes, 5 * j + pb)
            vc[b, j, 0] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
            kc[b, j, 0] = (kcodes[0::2] | (kcodes[1::2] << 4)).astype(np.uint8)
            ks[b, j, 0] = k_scales[pb, j]
            vs[b, j, 0] = v_scales[pb, j]
            for h in range(G):
                col[b, j * G + h] = h + G * (b // 2)
                q[b, j * G + h, col[b, j * G + h]] = 1.0
    scale = 0.25
    sl = torch.ones(B, dtype=torch.int32, device="cuda")
    qd = dev(syn.bf16_bits(q))
    out = torch.empty(B, n_h, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_fp4_workspace_size(B, n_h, n_kv, L_max, d))
    kvc.kvc_decode_attn_fp4(qd, dev(kc), dev(ks), dev(vc), dev(vs), sl, out, lse, scale=scale,
                            workspace=ws)
    torch.cuda.synchronize()
    o = host_f64(out)
    want_v = oracle.dequantize_fp4(vc[:, :, 0], vs[:, :, 0])          # [B, n_kv, d]
    want_k = oracle.dequantize_fp4(kc[:, :, 0], ks[:, :, 0])
    for b in range(B):
        for j in range(n_kv):
            assert np.array_equal(o[b, j * G:(j + 1) * G], np.broadcast_to(want_v[b, j], (G, d)))
    got_l = host(lse).astype(np.float64)
    want_l = np.array([[scale * want_k[b, i // G, col[b, i]] for i in range(n_h)] for b in range(B)])
    # a zero key gives lse = 0 (one position, weight 1)
    assert np.abs(got_l - want_l).max() <= 1e-6 * np.abs(want_l).max() + 1e-7
