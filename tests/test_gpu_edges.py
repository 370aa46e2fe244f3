"""Edge cases of the method on the GPU, every output and workspace inside
guard bands (MI355X).

Sources: podcast transcript, DeepSeek Sparse Attention passage (the sparse
decode attends only over the listed positions: one position, all of them,
or none that exist); "KV cache" guide, first section (a sequence with
nothing cached yet has nothing to attend) and "Caching a compressed latent"
(the latent decode over sequences of every length, any number of heads).

Each call writes into buffers with 0xA5 guard bands before and after
(`Guarded`): a store outside a buffer fails the test, and a row left
unwritten fails the finite check (outputs start as NaN).  Outputs are
compared with the fp64 oracle within the contract (2e-2 bf16, 1e-5 f32);
empty rows must be exactly zero with lse = -inf; flags exactly.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import kvc_synth as syn
import oracle
from gpu_helpers import Guarded, compare, compare_lse, dev, guarded_workspace, host, host_f64, tol_for

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


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def check_counters_zero(ws, nwords, what):
    """The counters at the front of a workspace are back at zero."""
    if ws is not None and nwords:
        assert int(ws.t[:4 * nwords].view(torch.int32).abs().sum()) == 0, f"{what}: counters not reset"


# ------------------------------------------------------------------- top-k
def run_topk_guarded(case, idx, K, scale, split=0):
    B, n_h, d = case["q"].shape
    n_kv = case["k_cache"].shape[1]
    dt = torch_dtype(case["dtype"])
    q, kc, vc, sl = dev(case["q"]), dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    out = Guarded((B, n_h, d), dt)
    lse = Guarded((B, n_h), torch.float32)
    flag = Guarded((1,), torch.int32, zero=True)
    kvc.kvc_set_split_override(split)
    ws = guarded_workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, K, d,
                                                                   kvc._dtype_code(q)))
    kvc.kvc_decode_attn_topk(q, kc, vc, sl, dev(idx), out.t, lse.t, scale=scale, flag=flag.t,
                             workspace=None if ws is None else ws.t)
    torch.cuda.synchronize()
    for g, nm in ((out, "out"), (lse, "lse"), (flag, "flag")):
        g.check(f"top-k {nm}")
    if ws is not None:
        ws.check("top-k workspace")
        check_counters_zero(ws, B * n_kv, "top-k")
    return out.t, lse.t, int(host(flag.t)[0])


TOPK_EDGE = [
    # (n_h, n_kv, d, dtype, K, lens, L_max, split)
    (64, 8, 128, "bf16", 1, [1, 500, 3000], 3000, 0),        # K = 1 (MFMA kernel)
    (64, 8, 128, "bf16", 1, [7, 2], 64, 0),
    (8, 2, 64, "bf16", 1, [1, 40], 40, 0),                   # K = 1, generic kernel
    (16, 4, 128, "f32", 1, [3, 90], 96, 0),                  # K = 1, generic kernel f32
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,K,lens,L_max,split", TOPK_EDGE)
def test_topk_k_equals_one(n_h, n_kv, d, dtype, K, lens, L_max, split):
    """One listed position: every head returns that position's value row
    (its only weight is exactly 1)."""
    B = len(lens)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, lens, dtype, cfg_id=150)
    idx = np.stack([syn.topk_indices(150, 0, 1, n_kv, K, lens[b], index_set=b)[0]
                    for b in range(B)])
    scale = 1 / math.sqrt(d)
    out, lse, flag = run_topk_guarded(case, idx, K, scale, split)
    o_ref, l_ref, f_ref = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"],
                                             case["seq_lens"], idx, scale)
    assert flag == f_ref == 0
    G = n_h // n_kv
    got = host_f64(out)
    for b in range(B):
        for i in range(n_h):
            want = oracle.to_f64(case["v_cache"][b, i // G, idx[b, i // G, 0]])
            # bf16 output of an exact copy: the stored row itself
            assert np.abs(got[b, i] - want).max() <= (0 if dtype == "bf16" else 1e-6), (b, i)
    compare(got, o_ref, tol_for(dtype), f"top-k K=1 {dtype} d{d}")
    compare_lse(host(lse), l_ref, lse_tol(dtype))


@pytest.mark.parametrize("split", [0, 128])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_topk_k_equals_length(dtype, d, split):
    """K = n_b: listing every position of a sequence equals the dense decode
    of that sequence (the same positions); the other sequence's subset is
    checked against the oracle's gather."""
    n_h, n_kv = 32, 4
    lens = [700, 1500]
    K = lens[0]
    B = len(lens)
    case = syn.dense_case(B, n_h, n_kv, d, 1500, lens, dtype, cfg_id=151)
    idx = np.empty((B, n_kv, K), np.int32)
    idx[0] = np.arange(K, dtype=np.int32)[None]
    idx[1] = syn.topk_indices(151, 0, 1, n_kv, K, lens[1])[0]
    scale = 1 / math.sqrt(d)
    out, lse, flag = run_topk_guarded(case, idx, K, scale, split)
    assert flag == 0
    o_dense, l_dense = oracle.decode(case["q"], case["k_cache"], case["v_cache"],
                                     case["seq_lens"], scale)
    o_ref, l_ref, _ = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"],
                                         case["seq_lens"], idx, scale)
    got = host_f64(out)
    compare(got[0], o_dense[0], tol_for(dtype), f"top-k K=n vs dense {dtype} d{d}")
    compare_lse(host(lse)[0], l_dense[0], lse_tol(dtype))
    compare(got, o_ref, tol_for(dtype), f"top-k K=n {dtype} d{d}")
    compare_lse(host(lse), l_ref, lse_tol(dtype))


@pytest.mark.parametrize("split", [0, 128])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_topk_all_indices_invalid(dtype, d, split):
    """A (sequence, KV head) whose every listed index is out of range has
    nothing to attend: zero row, lse = -inf, bad-index flag; the other
    units of the batch are unaffected."""
    n_h, n_kv, K = 16, 4, 300
    lens = [1000, 400]
    B = len(lens)
    case = syn.dense_case(B, n_h, n_kv, d, 1000, lens, dtype, cfg_id=152)
    idx = np.stack([syn.topk_indices(152, 0, 1, n_kv, K, lens[b], index_set=b)[0]
                    for b in range(B)])
    idx[0, 1] = np.arange(K, dtype=np.int32) + lens[0]      # all >= n_b
    idx[1, 3, :150] = -1 - np.arange(150, dtype=np.int32)    # negative ...
    idx[1, 3, 150:] = lens[1] + 7                            # ... and past the end
    scale = 1 / math.sqrt(d)
    out, lse, flag = run_topk_guarded(case, idx, K, scale, split)
    o_ref, l_ref, f_ref = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"],
                                             case["seq_lens"], idx, scale)
    assert f_ref == oracle.FLAG_BAD_INDEX == flag
    G = n_h // n_kv
    got, got_l = host_f64(out), host(lse)
    for b, j in ((0, 1), (1, 3)):
        rows = slice(j * G, (j + 1) * G)
        assert np.all(got[b, rows] == 0.0) and not np.signbit(got[b, rows]).any(), (b, j)
        assert np.all(np.isneginf(got_l[b, rows])), (b, j)
    compare(got, o_ref, tol_for(dtype), f"top-k all-invalid {dtype}")
    compare_lse(got_l, l_ref, lse_tol(dtype))


# --------------------------------------------------------------------- MLA
MLA_EDGE = [
    # (B, n_h, lengths (no append), L_max): B % 8 == 0 takes the XCD-local
    # block numbering, other B the plain one; n_h = 192 is three 64-head
    # groups, 256 two 128-head groups
    (8, 64, [0, 300, 17, 0, 1, 640, 33, 128], 640),
    (8, 192, [512, 0, 96, 97, 1, 0, 250, 31], 512),
    (16, 256, [0, 1, 2, 30, 31, 32, 33, 95, 96, 97, 300, 0, 401, 64, 65, 450], 450),
    (9, 128, [0, 0, 200, 1, 0, 333, 96, 0, 400], 400),
    (3, 128, [0, 0, 0], 64),                                # nothing to attend anywhere
]


@pytest.mark.parametrize("B,n_h,lens,L_max", MLA_EDGE)
@pytest.mark.parametrize("split", [0, 96])
def test_mla_empty_rows_and_head_groups(B, n_h, lens, L_max, split):
    """Latent decode with no append first: sequences of length 0 (zero row,
    lse = -inf, skipped by the split merge) next to sequences cut at chunk
    and split boundaries, with one to three head groups per sequence."""
    case = syn.mla_case(B, n_h, 512, 64, L_max, lens, "bf16", cfg_id=153)
    q, ckv, sl = dev(case["q"]), dev(case["ckv"]), dev(case["seq_lens"])
    out = Guarded((B, n_h, 512), torch.bfloat16)
    lse = Guarded((B, n_h), torch.float32)
    kvc.kvc_set_split_override(split)
    ws = guarded_workspace(kvc.kvc_decode_attn_mla_workspace_size(B, n_h, L_max, 512, 64))
    kvc.kvc_decode_attn_mla(q, ckv, sl, out.t, lse.t, scale=1 / 24,
                            workspace=None if ws is None else ws.t)
    torch.cuda.synchronize()
    out.check("mla out")
    lse.check("mla lse")
    if ws is not None:
        ws.check("mla workspace")
    assert host(sl).tolist() == list(lens)
    o_ref, l_ref = oracle.decode_mla(case["q"], case["ckv"], case["seq_lens"], 512, 64, 1 / 24)
    got, got_l = host_f64(out.t), host(lse.t)
    for b in range(B):
        if lens[b] == 0:
            assert np.all(got[b] == 0.0) and not np.signbit(got[b]).any(), b
            assert np.all(np.isneginf(got_l[b])), b
    compare(got, o_ref, 2e-2, f"mla edges B{B} h{n_h} split{split}")
    compare_lse(got_l, l_ref, lse_tol("bf16"))


# ------------------------------------------------------------ dense, fused
GUARDED_DENSE = [
    # (n_h, n_kv, d, dtype, pre-append lengths, L_max, split)
    (32, 32, 128, "bf16", [4096], 4097, 0),
    (64, 8, 128, "bf16", [0, 31, 32, 1000, 2047], 2048, 0),
    (64, 8, 128, "bf16", [0, 31, 32, 1000, 2047], 2048, 32),
    (15, 5, 128, "bf16", [700, 0], 800, 128),
    (8, 2, 64, "bf16", [0, 129, 599], 600, 128),
    (16, 4, 128, "f32", [0, 64, 999], 1000, 0),
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,pre,L_max,split", GUARDED_DENSE)
def test_dense_and_fused_guarded(n_h, n_kv, d, dtype, pre, L_max, split):
    """Append then decode, and the fused append-and-attend, with guard
    bands round every output and workspace; both against the oracle."""
    B = len(pre)
    scale = 1 / math.sqrt(d)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, dtype, cfg_id=154)
    kc_o, vc_o, sl_o = case["k_cache"].copy(), case["v_cache"].copy(), case["seq_lens"].copy()
    f_o = oracle.append(kc_o, vc_o, sl_o, case["k_new"], case["v_new"])
    o_ref, l_ref = oracle.decode(case["q"], kc_o, vc_o, sl_o, scale)
    dt = torch_dtype(dtype)
    code = kvc.KVC_BF16 if dtype == "bf16" else kvc.KVC_F32
    kvc.kvc_set_split_override(split)
    for fused in (False, True):
        kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
        q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
        out = Guarded((B, n_h, d), dt)
        lse = Guarded((B, n_h), torch.float32)
        flag = Guarded((1,), torch.int32, zero=True)
        if fused:
            ws = guarded_workspace(kvc.kvc_append_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, code))
            kvc.kvc_append_decode_attn(q, kc, vc, sl, kn, vn, out.t, lse.t, scale=scale, flag=flag.t,
                                       workspace=ws.t)
        else:
            kvc.kvc_append(kc, vc, sl, kn, vn, flag=flag.t)
            ws = guarded_workspace(kvc.kvc_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, code))
            kvc.kvc_decode_attn(q, kc, vc, sl, out.t, lse.t, scale=scale,
                                workspace=None if ws is None else ws.t)
        torch.cuda.synchronize()
        what = f"{'fused' if fused else 'dense'} {n_h}/{n_kv} d{d} {dtype} split {split}"
        for g, nm in ((out, "out"), (lse, "lse"), (flag, "flag")):
            g.check(f"{what} {nm}")
        if ws is not None:
            ws.check(f"{what} workspace")
            if fused:
                tail = -(-4 * (B + B * n_kv) // 256) * 256
                assert int(ws.t[-tail:].view(torch.int32).abs().sum()) == 0, "arrival counters"
            if kvc.kvc_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, code):
                check_counters_zero(ws, B * n_kv, what)     # split tickets
        assert host(sl).tolist() == sl_o.tolist()
        assert int(host(flag.t)[0]) == f_o
        assert np.array_equal(host(kc).view(np.uint8), kc_o.view(np.uint8))
        assert np.array_equal(host(vc).view(np.uint8), vc_o.view(np.uint8))
        compare(host_f64(out.t), o_ref, tol_for(dtype), what)
        compare_lse(host(lse.t), l_ref, lse_tol(dtype))
