"""kvc_append_decode_attn_noalloc against kvc_append_decode_attn (MI355X).

The no-allocation variant runs the same kernels on the library's own
scratch instead of a caller's workspace, so for the same inputs it must give
the same cache bytes, lengths and flag, and the same output and lse bits;
both are also checked against the fp64 oracle within the contract.  The
calls come in a row on one GPU, each later one smaller than the first (a
different split plan and counter layout over the same scratch, which keeps
the previous call's contents).
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

# (n_h, n_kv, d, dtype, pre-append lengths, L_max), called in this order
CALLS = [
    (64, 8, 128, "bf16", [3071, 17, 2000, 0, 1024, 2999, 512, 1] * 4, 3072),   # 12 splits per unit
    (16, 2, 128, "bf16", [100, 0, 700], 800),                                 # 7 splits, fewer units
    (32, 32, 128, "bf16", [1000], 1001),                                      # one sequence, MHA
    (8, 2, 64, "f32", [0, 63, 64, 257], 257),                                 # generic kernel; a full cache
]


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' elsewhere)")
    kvc.kvc_set_split_override(0)
    yield
    torch.cuda.synchronize()


def run(case, noalloc):
    B, n_h, d = case["q"].shape
    n_kv, L_max = case["k_cache"].shape[1], case["k_cache"].shape[2]
    kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, n_h), float("nan"), dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(d)
    if noalloc:
        kvc.kvc_append_decode_attn_noalloc(q, kc, vc, sl, kn, vn, out, lse, scale=scale, flag=flag)
    else:
        ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(B, n_h, n_kv, L_max, d,
                                                                     kvc._dtype_code(q)))
        kvc.kvc_append_decode_attn(q, kc, vc, sl, kn, vn, out, lse, scale=scale, flag=flag,
                                   workspace=ws)
    torch.cuda.synchronize()
    return dict(out=host(out), lse=host(lse), sl=host(sl), flag=int(host(flag)[0]),
                kc=host(kc), vc=host(vc))


def test_noalloc_matches_workspace_call_in_a_row():
    for k, (n_h, n_kv, d, dtype, pre, L_max) in enumerate(CALLS):
        B = len(pre)
        print(f"call {k}: B={B} n_h={n_h} n_kv={n_kv} d={d} {dtype} L_max={L_max}", flush=True)
        case = syn.dense_case(B, n_h, n_kv, d, L_max, pre, dtype, cfg_id=160 + k)
        want = run(case, noalloc=False)
        got = run(case, noalloc=True)
        assert got["sl"].tolist() == want["sl"].tolist()
        assert got["flag"] == want["flag"]
        assert np.array_equal(got["kc"].view(np.uint8), want["kc"].view(np.uint8))
        assert np.array_equal(got["vc"].view(np.uint8), want["vc"].view(np.uint8))
        assert np.array_equal(got["out"].view(np.uint8), want["out"].view(np.uint8)), f"call {k}: out"
        assert np.array_equal(got["lse"].view(np.uint8), want["lse"].view(np.uint8)), f"call {k}: lse"

        kc, vc, sl = case["k_cache"].copy(), case["v_cache"].copy(), case["seq_lens"].copy()
        f_ref = oracle.append(kc, vc, sl, case["k_new"], case["v_new"])
        o_ref, l_ref = oracle.decode(case["q"], kc, vc, sl, 1 / math.sqrt(d))
        assert got["sl"].tolist() == sl.tolist() and got["flag"] == f_ref
        assert np.array_equal(got["kc"].view(np.uint8), kc.view(np.uint8))
        compare(oracle.to_f64(got["out"]), o_ref, tol_for(dtype), f"noalloc call {k}")
        compare_lse(got["lse"], l_ref, 4e-3 if dtype == "bf16" else 1e-5)
