"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Inputs are seeded (kvc_synth), in storage form (bf16 bits or float32), with
NaN poison at every position a kernel must not read.  Append and index
handling must match bit for bit; outputs within 1e-5 (float32 inputs) or
2e-2 (bf16 inputs) max-abs.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import kvc_synth as syn
import oracle
from gpu_helpers import compare, compare_lse, dev, host, host_f64, tol_for

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


def lse_tol(dtype):
    return 4e-3 if dtype == "bf16" else 1e-5


# ----------------------------------------------------------------- helpers
def run_dense_step(case, scale, split=0, lse=True):
    """Append the new token, then decode; returns (out, lse, seq_lens, caches, flag)."""
    kc, vc = dev(case["k_cache"]), dev(case["v_cache"])
    sl = dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append(kc, vc, sl, kn, vn, flag=flag)
    B, n_h, d = q.shape
    n_kv, L_max = kc.shape[1], kc.shape[2]
    out = torch.empty_like(q)
    lse_t = torch.empty(B, n_h, dtype=torch.float32, device="cuda") if lse else None
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, kvc._dtype_code(q)))
    kvc.kvc_decode_attn(q, kc, vc, sl, out, lse_t, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert int(ws[:4 * B * n_kv].view(torch.int32).abs().sum()) == 0, "tickets not reset"
    return out, lse_t, sl, kc, vc, flag


def oracle_dense_step(case, scale):
    kc, vc = case["k_cache"].copy(), case["v_cache"].copy()
    sl = case["seq_lens"].copy()
    flag = oracle.append(kc, vc, sl, case["k_new"], case["v_new"])
    o, lse = oracle.decode(case["q"], kc, vc, sl, scale)
    return o, lse, sl, kc, vc, flag


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 576), ("bf16", 3)])
def test_append_bit_exact(dtype, d):
    B, n_kv, L_max = 5, 3, 9
    pre = [0, 4, 8, 9, 7]     # 9 == L_max: full, must flag and not write
    case = syn.dense_case(B, n_kv, n_kv, d, L_max, pre, dtype, cfg_id=90)
    kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append(kc, vc, sl, dev(case["k_new"]), dev(case["v_new"]), flag=flag)
    torch.cuda.synchronize()
    _, _, sl_o, kc_o, vc_o, flag_o = oracle_dense_step(case, 1.0)
    assert host(sl).tolist() == sl_o.tolist()
    assert np.array_equal(host(kc).view(np.uint8), kc_o.view(np.uint8))
    assert np.array_equal(host(vc).view(np.uint8), vc_o.view(np.uint8))
    assert int(host(flag)[0]) == flag_o == oracle.FLAG_CACHE_FULL


def test_append_latent_single_tensor():
    B, L_max, D = 3, 6, 576
    case = syn.mla_case(B, 64, 512, 64, L_max, [0, 5, 6], "bf16", cfg_id=91)
    ckv, sl = dev(case["ckv"]), dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append(ckv, None, sl, dev(case["ckv_new"]), None, flag=flag)
    torch.cuda.synchronize()
    c4 = case["ckv"][:, None].copy()
    sl_o = case["seq_lens"].copy()
    f = oracle.append(c4, None, sl_o, case["ckv_new"][:, None], None)
    assert host(sl).tolist() == sl_o.tolist() and int(host(flag)[0]) == f
    assert np.array_equal(host(ckv), c4[:, 0])


# ------------------------------------------------------------- dense decode
def test_c1_tiny_gqa_fp32():
    """C1: B=1, 8 query heads over 2 KV heads, d=64, 256 cached + 1 appended."""
    c = syn.C1
    case = syn.dense_case(c.B, c.n_h, c.n_kv, c.d, c.L_max, syn.pre_append_lens(c), c.dtype, cfg_id=c.cfg_id)
    out, lse, sl, kc, vc, flag = run_dense_step(case, c.scale)
    o_ref, l_ref, sl_ref, kc_ref, vc_ref, f_ref = oracle_dense_step(case, c.scale)
    assert host(sl).tolist() == sl_ref.tolist() == [257]
    assert np.array_equal(host(kc), kc_ref) or np.array_equal(host(kc).view(np.uint32), kc_ref.view(np.uint32))
    compare(host_f64(out), o_ref, 1e-5, "C1 out")
    compare_lse(host(lse), l_ref, lse_tol("f32"))


DENSE_CASES = [
    # (n_h, n_kv, d, dtype, pre-append lengths, L_max)
    (32, 32, 128, "bf16", [4096], 4097),                 # MHA, C2 layer shape
    (64, 8, 128, "bf16", [0, 30, 31, 32, 127, 128, 1000, 2047], 2048),   # GQA G=8, ragged
    (16, 1, 128, "bf16", [5, 300], 512),                 # MQA G=16
    (8, 4, 128, "bf16", [100, 0, 255], 256),             # G=2
    (12, 3, 128, "bf16", [77, 600], 700),                # G=4
    (15, 5, 128, "bf16", [700, 33], 800),                # G=3 (does not divide 16)
    (12, 1, 128, "bf16", [1999, 40], 2000),              # G=12, 16 splits: two merge batches
    (8, 2, 64, "bf16", [0, 1, 129, 500], 600),           # generic kernel, bf16 d=64
    (16, 4, 128, "f32", [0, 64, 65, 999], 1000),         # generic kernel, f32 d=128
    (6, 6, 64, "f32", [1, 2, 3], 8),                     # tiny, many empty chunk slots
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,pre,L_max", DENSE_CASES)
def test_dense_parity(n_h, n_kv, d, dtype, pre, L_max):
    B = len(pre)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, dtype, cfg_id=92)
    scale = 1 / math.sqrt(d)
    out, lse, sl, kc, vc, flag = run_dense_step(case, scale)
    o_ref, l_ref, sl_ref, _, _, f_ref = oracle_dense_step(case, scale)
    assert host(sl).tolist() == sl_ref.tolist()
    assert int(host(flag)[0]) == f_ref
    compare(host_f64(out), o_ref, tol_for(dtype), f"dense {n_h}/{n_kv} d{d} {dtype}")
    compare_lse(host(lse), l_ref, lse_tol(dtype))


@pytest.mark.parametrize("split", [128, 256, 384, 1024, 8192])
def test_dense_split_sweep(split):
    """Any split size merges to the same result (log-sum-exp combine)."""
    case = syn.dense_case(3, 64, 8, 128, 3000, [2999, 1000, 129], "bf16", cfg_id=93)
    out, lse, *_ = run_dense_step(case, 1 / math.sqrt(128), split=split)
    o_ref, l_ref, *_ = oracle_dense_step(case, 1 / math.sqrt(128))
    compare(host_f64(out), o_ref, 2e-2, f"split {split}")
    compare_lse(host(lse), l_ref, lse_tol("bf16"))


@pytest.mark.parametrize("n_h,n_kv", [(32, 32), (16, 1), (15, 5)])
def test_dense_many_splits_merge(n_h, n_kv):
    """Up to 250 splits of 32 positions: the merge takes several batches of
    partial rows per thread, with 1, 16 and 3 heads per KV head."""
    case = syn.dense_case(2, n_h, n_kv, 128, 8000, [7999, 300], "bf16", cfg_id=94)
    out, lse, *_ = run_dense_step(case, 1 / math.sqrt(128), split=32)
    o_ref, l_ref, *_ = oracle_dense_step(case, 1 / math.sqrt(128))
    compare(host_f64(out), o_ref, 2e-2, f"many splits {n_h}/{n_kv}")
    compare_lse(host(lse), l_ref, lse_tol("bf16"))


def test_dense_uniform_and_sum_to_one():
    """q = 0: every weight is exactly 1/n, so o is the mean of V.  Position t
    is stored as two bf16-exact columns (t // 64, t % 64), so both means are
    known in closed form.  V = 1 everywhere gives o = 1."""
    B, n_h, n_kv, d, L_max = 2, 16, 2, 128, 1000
    pre = [999, 300]
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, "bf16", cfg_id=94)
    case["q"][:] = 0
    t = np.arange(L_max)
    for b in range(B):
        case["v_cache"][b, :, :pre[b], 0] = syn.bf16_bits((t[:pre[b]] // 64).astype(np.float32))
        case["v_cache"][b, :, :pre[b], 1] = syn.bf16_bits((t[:pre[b]] % 64).astype(np.float32))
        case["v_new"][b, :, 0] = syn.bf16_bits(np.array([pre[b] // 64], np.float32))[0]
        case["v_new"][b, :, 1] = syn.bf16_bits(np.array([pre[b] % 64], np.float32))[0]
    out, *_ = run_dense_step(case, 0.1)
    o = host_f64(out)
    for b in range(B):
        used = np.arange(pre[b] + 1)
        for col, want in ((0, (used // 64).mean()), (1, (used % 64).mean())):
            assert np.abs(o[b, :, col] - want).max() <= want * 2 ** -8 + 1e-4, (b, col)
    case2 = syn.dense_case(B, n_h, n_kv, d, L_max, pre, "bf16", cfg_id=95)
    for b in range(B):
        case2["v_cache"][b, :, :pre[b]] = 0x3F80
    case2["v_new"][:] = 0x3F80
    out2, *_ = run_dense_step(case2, 1 / math.sqrt(d))
    assert np.abs(host_f64(out2) - 1.0).max() <= 2 ** -8


def test_dense_saturated_scores():
    """Huge scores: no overflow, the max position wins."""
    B, n_h, n_kv, d, L_max = 1, 8, 1, 128, 256
    case = syn.dense_case(B, n_h, n_kv, d, L_max, [255], "bf16", cfg_id=96)
    case["k_cache"][0, 0, :255] = syn.bf16_bits(np.zeros((255, d), np.float32))
    case["k_cache"][0, 0, 17] = syn.bf16_bits(np.full(d, 8.0, np.float32))
    case["q"][:] = syn.bf16_bits(np.full((B, n_h, d), 8.0, np.float32))
    case["k_new"][:] = 0
    out, lse, *_ = run_dense_step(case, 1.0)
    o_ref, l_ref, *_ = oracle_dense_step(case, 1.0)
    compare(host_f64(out), o_ref, 2e-2, "saturated")


# ------------------------------------------------------------------- top-k
TOPK_CASES = [
    # (n_h, n_kv, d, dtype, K, lens, L_max)
    (64, 8, 128, "bf16", 2048, [20000, 4000], 20001),    # C5 head shape, ragged lengths
    (64, 8, 128, "bf16", 100, [500, 101], 600),           # K not a multiple of 32
    (16, 16, 128, "bf16", 33, [64], 64),
    (8, 2, 64, "bf16", 70, [90, 300], 300),               # generic kernel
    (8, 4, 128, "f32", 129, [200], 256),                  # generic kernel f32
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,K,lens,L_max", TOPK_CASES)
def test_topk_parity(n_h, n_kv, d, dtype, K, lens, L_max):
    B = len(lens)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, lens, dtype, cfg_id=97)
    idx = np.empty((B, n_kv, K), dtype=np.int32)
    for b in range(B):
        idx[b] = syn.topk_indices(97, 0, 1, n_kv, K, lens[b], index_set=b)[0]
    scale = 1 / math.sqrt(d)
    q, kc, vc, sl = dev(case["q"]), dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, K, d, kvc._dtype_code(q)))
    kvc.kvc_decode_attn_topk(q, kc, vc, sl, dev(idx), out, lse, scale=scale, flag=flag, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref, f_ref = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"],
                                             case["seq_lens"], idx, scale)
    assert int(host(flag)[0]) == f_ref == 0
    compare(host_f64(out), o_ref, tol_for(dtype), f"topk K={K} {dtype}")
    compare_lse(host(lse), l_ref, lse_tol(dtype))


def test_topk_bad_indices_and_exact_selection():
    """q = 0 and V[t, 0] = t: column 0 is the mean of the used indices, so the
    used set is checked exactly; out-of-range indices are skipped and flagged."""
    B, n_h, n_kv, d, L_max, K = 2, 16, 2, 128, 4096, 256
    lens = [4096, 1000]
    case = syn.dense_case(B, n_h, n_kv, d, L_max, lens, "bf16", cfg_id=98)
    case["q"][:] = 0
    # position t stored in two bf16-exact halves: t = 64*hi + lo
    t = np.arange(L_max)
    case["v_cache"][..., 0] = syn.bf16_bits((t // 64).astype(np.float32))[None, None, :]
    case["v_cache"][..., 1] = syn.bf16_bits((t % 64).astype(np.float32))[None, None, :]
    idx = np.stack([syn.topk_indices(98, 0, 1, n_kv, K, lens[b], index_set=b)[0] for b in range(B)])
    idx[0, 1, 5] = -3
    idx[1, 0, 200] = 1000          # == seq_len: out of range
    idx[1, 1, 7] = 2 ** 30
    q, kc, vc, sl = dev(case["q"]), dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    out = torch.empty_like(q)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, K, d, 1))
    kvc.kvc_decode_attn_topk(q, kc, vc, sl, dev(idx), out, None, scale=0.1, flag=flag,
                             workspace=ws)
    torch.cuda.synchronize()
    o_ref, _, f_ref = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"], case["seq_lens"], idx, 0.1)
    assert f_ref == oracle.FLAG_BAD_INDEX and int(host(flag)[0]) == f_ref
    o = host_f64(out)
    G = n_h // n_kv
    for b in range(B):
        for i in range(n_h):
            used = [x for x in idx[b, i // G] if 0 <= x < lens[b]]
            hi = np.mean([x // 64 for x in used])
            lo = np.mean([x % 64 for x in used])
            assert abs(o[b, i, 0] - hi) <= 2e-2 * max(1, hi) / 2 + 0.07
            assert abs(o[b, i, 1] - lo) <= 0.3
    compare(o, o_ref, 0.5, "topk mean-index")   # values up to 64: bf16 output spacing 0.25


# --------------------------------------------------------------------- MLA
MLA_CASES = [
    # (B, n_h, pre-append lens, L_max)
    (3, 128, [0, 100, 700], 800),
    (2, 64, [8192, 31], 8193),
    (1, 256, [1000], 1001),
]


@pytest.mark.parametrize("B,n_h,pre,L_max", MLA_CASES)
@pytest.mark.parametrize("split", [0, 256, 96])
def test_mla_parity(B, n_h, pre, L_max, split):
    case = syn.mla_case(B, n_h, 512, 64, L_max, pre, "bf16", cfg_id=99)
    ckv, sl = dev(case["ckv"]), dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append(ckv, None, sl, dev(case["ckv_new"]), None, flag=flag)
    q = dev(case["q"])
    out = torch.empty(B, n_h, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_mla_workspace_size(B, n_h, L_max, 512, 64))
    kvc.kvc_decode_attn_mla(q, ckv, sl, out, lse, scale=1 / 24, workspace=ws)
    torch.cuda.synchronize()
    c4 = case["ckv"][:, None].copy()
    sl_o = case["seq_lens"].copy()
    oracle.append(c4, None, sl_o, case["ckv_new"][:, None], None)
    assert host(sl).tolist() == sl_o.tolist()
    o_ref, l_ref = oracle.decode_mla(case["q"], c4[:, 0], sl_o, 512, 64, 1 / 24)
    compare(host_f64(out), o_ref, 2e-2, f"mla B{B} h{n_h} split{split}")
    compare_lse(host(lse), l_ref, lse_tol("bf16"))
    if ws is not None:
        groups = n_h // (128 if n_h % 128 == 0 else 64)
        assert int(ws[:4 * B * groups].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("n_h", [128, 64])
@pytest.mark.parametrize("split", [0, 96])
def test_mla_score_jump(n_h, split):
    """Rows whose score lies far above every earlier score of the split (by
    about 90 and about 1200 in log2 units): the weights must not overflow
    and the result is the exact softmax, dominated by those rows."""
    B, L_max, pre = 2, 400, [300, 390]
    case = syn.mla_case(B, n_h, 512, 64, L_max, pre, "bf16", cfg_id=98)
    ckv, qb = case["ckv"], case["q"]
    qf = oracle.bf16_to_f64(qb).astype(np.float32)
    ckv[0, 200:204, :512] = syn.bf16_bits(3.0 * qf[0, 5, :512])
    ckv[0, 200:204, 512:] = syn.bf16_bits(np.zeros(64, np.float32))
    ckv[1, 350:352, :512] = syn.bf16_bits(40.0 * qf[1, 7, :512])
    ckv[1, 350:352, 512:] = syn.bf16_bits(np.zeros(64, np.float32))
    ckv_d, sl = dev(ckv), dev(case["seq_lens"])
    q = dev(qb)
    out = torch.empty(B, n_h, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_mla_workspace_size(B, n_h, L_max, 512, 64))
    kvc.kvc_decode_attn_mla(q, ckv_d, sl, out, lse, scale=1 / 24, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_mla(qb, ckv, case["seq_lens"], 512, 64, 1 / 24)
    assert l_ref[0, 5] > 50 and l_ref[1, 7] > 500   # the jumps are real (natural log units)
    got = host_f64(out)
    assert np.isfinite(got).all()
    # the dominated heads' outputs are 3x and 40x a query row: bf16 rounding
    # of the output is relative, so scale the 2e-2 contract by max(1, |o|)
    mag = np.maximum(1.0, np.abs(o_ref))
    compare(got / mag, o_ref / mag, 2e-2, f"mla jump h{n_h} split{split}")
    compare_lse(host(lse), l_ref, 4e-3 * max(1.0, float(np.abs(l_ref).max()) / 100))


# ------------------------------------------------------------------ causal
def test_causal_loop_on_gpu():
    """Guide, first section: appending one token at a time and decoding gives
    every row of full causal attention recomputed from scratch."""
    n, n_h, n_kv, d = 40, 16, 2, 128
    rng = np.random.default_rng(1234)
    Q = syn.bf16_bits(rng.standard_normal((n, n_h, d)).astype(np.float32))
    K = syn.bf16_bits(rng.standard_normal((n, n_kv, d)).astype(np.float32))
    V = syn.bf16_bits(rng.standard_normal((n, n_kv, d)).astype(np.float32))
    full = oracle.full_causal(Q, K, V, 1 / math.sqrt(d))
    kc = dev(np.full((1, n_kv, n, d), syn.BF16_QNAN, np.uint16))
    vc = dev(np.full((1, n_kv, n, d), syn.BF16_QNAN, np.uint16))
    sl = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_workspace_size(1, n_h, n_kv, n, d, 1))
    outs = []
    for t in range(n):
        kvc.kvc_append(kc, vc, sl, dev(K[t][None]), dev(V[t][None]))
        q = dev(Q[t][None])
        out = torch.empty_like(q)
        kvc.kvc_decode_attn(q, kc, vc, sl, out, None, scale=1 / math.sqrt(d), workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    got = np.stack([host_f64(o)[0] for o in outs])
    compare(got, full, 2e-2, "causal loop")


# ------------------------------------------------------------ graph replay
def test_graph_replay_matches_eager():
    """Append + decode captured in a HIP graph: every replay (with eager work
    and syncs in between) equals the eager result from the same state."""
    case = syn.dense_case(4, 64, 8, 128, 1024, [1000, 10, 500, 0], "bf16", cfg_id=100)
    kc0, vc0, sl0 = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    kc, vc, sl = kc0.clone(), vc0.clone(), sl0.clone()
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    out = torch.empty_like(q)
    ws = kvc.workspace(kvc.kvc_decode_attn_workspace_size(4, 64, 8, 1024, 128, 1))
    kvc.kvc_append(kc, vc, sl, kn, vn)
    kvc.kvc_decode_attn(q, kc, vc, sl, out, None, scale=1 / math.sqrt(128), workspace=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    kc.copy_(kc0); vc.copy_(vc0); sl.copy_(sl0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        kvc.kvc_append(kc, vc, sl, kn, vn)
        kvc.kvc_decode_attn(q, kc, vc, sl, out, None, scale=1 / math.sqrt(128), workspace=ws)
    for rep in range(4):
        kc.copy_(kc0); vc.copy_(vc0); sl.copy_(sl0); out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert host(sl).tolist() == [1001, 11, 501, 1]


# -------------------------------------------------------------- diagnostics
def test_copy_and_stream_read():
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    kvc.kvc_copy(dst, src)
    sink = torch.empty(kvc.kvc_stream_read_sink_floats(src.numel() * 4), dtype=torch.float32, device="cuda")
    kvc.kvc_stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


# ------------------------------------------------- fused append + attend
FUSED_CASES = [
    # (n_h, n_kv, d, dtype, pre-append lengths, L_max, split)
    (32, 32, 128, "bf16", [4096], 4097, 0),                      # MHA layer, C2 shape
    (64, 8, 128, "bf16", [0, 31, 255, 256, 1000, 2047, 2048], 2048, 0),   # incl. full cache
    (64, 8, 128, "bf16", [0, 31, 255, 256, 1000, 2047], 2048, 256),
    (16, 1, 128, "bf16", [511, 3], 512, 0),
    # last splits of 0..4 chunks: every choice of the wave that attends the
    # new row from registers
    (16, 2, 128, "bf16", [0, 1, 95, 96, 97, 200, 319, 320], 400, 96),
    (16, 2, 128, "bf16", [0, 31, 32, 63, 64, 159, 160, 161], 400, 160),
    (8, 2, 64, "bf16", [0, 129, 599, 600], 600, 0),              # generic kernel
    (16, 4, 128, "f32", [0, 999, 64], 1000, 0),                  # generic kernel f32
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,pre,L_max,split", FUSED_CASES)
def test_fused_append_decode(n_h, n_kv, d, dtype, pre, L_max, split):
    """One launch = kvc_append then kvc_decode_attn: cache bytes and lengths
    bit-exact, outputs within tolerance, full cache flagged and untouched."""
    B = len(pre)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, dtype, cfg_id=101)
    scale = 1 / math.sqrt(d)
    kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_set_split_override(split)
    code = kvc._dtype_code(q)
    ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, code))
    kvc.kvc_append_decode_attn(q, kc, vc, sl, kn, vn, out, lse, scale=scale, flag=flag, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref, sl_ref, kc_ref, vc_ref, f_ref = oracle_dense_step(case, scale)
    assert host(sl).tolist() == sl_ref.tolist()
    assert int(host(flag)[0]) == f_ref
    assert np.array_equal(host(kc).view(np.uint8), kc_ref.view(np.uint8))
    assert np.array_equal(host(vc).view(np.uint8), vc_ref.view(np.uint8))
    compare(host_f64(out), o_ref, tol_for(dtype), f"fused {n_h}/{n_kv} d{d} {dtype}")
    compare_lse(host(lse), l_ref, lse_tol(dtype))
    # counters: per-unit tickets at the front (when splits exist), one
    # arrival counter per sequence in the last 256-byte-rounded block
    tail = -(-4 * (B + B * n_kv) // 256) * 256
    w32 = ws.view(torch.int32)
    assert int(w32[-tail // 4:].abs().sum()) == 0, "arrival counters not reset"
    if ws.numel() > tail:
        assert int(w32[:B * n_kv].abs().sum()) == 0, "tickets not reset"


def test_fused_graph_replay_and_repeat():
    """Repeated fused steps (one appended token each) match the oracle's
    append/decode loop, also when replayed from a captured graph."""
    n_h, n_kv, d, L_max = 64, 8, 128, 1200
    pre = [1000, 3, 600]
    B = len(pre)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, "bf16", cfg_id=102)
    kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    out = torch.empty_like(q)
    ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, 1))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        kvc.kvc_append_decode_attn(q, kc, vc, sl, kn, vn, out, scale=1 / math.sqrt(d),
                                   workspace=ws)
    kc_o, vc_o, sl_o = case["k_cache"].copy(), case["v_cache"].copy(), case["seq_lens"].copy()
    for step in range(3):
        g.replay()
        torch.cuda.synchronize()
        oracle.append(kc_o, vc_o, sl_o, case["k_new"], case["v_new"])
        o_ref, _ = oracle.decode(case["q"], kc_o, vc_o, sl_o, 1 / math.sqrt(d))
        assert host(sl).tolist() == sl_o.tolist()
        compare(host_f64(out), o_ref, 2e-2, f"fused replay {step}")
    assert np.array_equal(host(kc), kc_o)
