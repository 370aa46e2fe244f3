"""Sliding-window decode: HIP path vs the fp64 oracle through the C ABI (MI355X).

Every head attends over [max(s, n - W), n) (the bounded-replay window rule
for the newest query).  Rows below that range are NaN-poisoned in the inputs,
as are rows at or past the sequence length, so any read of them shows up in
the output.  Outputs within 2e-2 (bf16) / 1e-5 (fp32) max-abs.
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


WINDOW_CASES = [
    # (n_h, n_kv, d, dtype, lengths, L_max, window, starts, split)
    (64, 8, 128, "bf16", [0, 1, 31, 32, 127, 128, 1000, 2047], 2048, 128, None, 0),
    (64, 8, 128, "bf16", [0, 1, 31, 32, 127, 128, 1000, 2047], 2048, 1, None, 0),
    (64, 8, 128, "bf16", [0, 1, 31, 32, 127, 128, 1000, 2047], 2048, 300,
     [0, 0, 5, 40, 100, 200, 999, 1500], 0),
    (32, 32, 128, "bf16", [4096], 4097, 5000, None, 0),          # window covers everything
    (16, 1, 128, "bf16", [5, 300], 512, 33, [0, 290], 0),       # MQA, window not a chunk multiple
    (64, 8, 128, "bf16", [2999, 1000, 129], 3000, 1500, None, 128),
    (64, 8, 128, "bf16", [2999, 1000, 129], 3000, 1500, [0, 600, 0], 384),
    (8, 2, 64, "bf16", [0, 1, 129, 500], 600, 77, [0, 0, 100, 490], 0),   # generic kernel
    (16, 4, 128, "f32", [0, 64, 65, 999], 1000, 200, None, 0),            # generic kernel, fp32
]


@pytest.mark.parametrize("n_h,n_kv,d,dtype,lens,L_max,window,starts,split", WINDOW_CASES)
def test_window_parity(n_h, n_kv, d, dtype, lens, L_max, window, starts, split):
    B = len(lens)
    case = syn.dense_case(B, n_h, n_kv, d, L_max, lens, dtype, cfg_id=120)
    kc, vc = case["k_cache"], case["v_cache"]
    poison = syn.poison_value(dtype)
    for b in range(B):
        lo, _ = oracle.window_range(lens[b], window, 0 if starts is None else starts[b])
        kc[b, :, :lo] = poison
        vc[b, :, :lo] = poison
    sl = np.asarray(lens, np.int32)
    st = None if starts is None else np.asarray(starts, np.int32)
    scale = 1 / math.sqrt(d)
    o_ref, l_ref = oracle.decode_window(case["q"], kc, vc, sl, scale, window, st)

    q = dev(case["q"])
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_window_workspace_size(B, n_h, n_kv, L_max, d,
                                                                 kvc._dtype_code(q), window))
    kvc.kvc_decode_attn_window(q, dev(kc), dev(vc), dev(sl), out, window,
                               win_start=None if st is None else dev(st), lse=lse,
                               scale=scale, workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert int(ws[:4 * B * n_kv].view(torch.int32).abs().sum()) == 0, "tickets not reset"
    compare(host_f64(out), o_ref, tol_for(dtype), f"window {window} {n_h}/{n_kv} d{d} {dtype}")
    compare_lse(host(lse), l_ref, 4e-3 if dtype == "bf16" else 1e-5)


def test_window_one_is_newest_value_row():
    """W = 1: every head returns the value row at position n - 1 exactly."""
    B, n_h, n_kv, d, L_max = 3, 16, 2, 128, 700
    lens = [1, 333, 700]
    case = syn.dense_case(B, n_h, n_kv, d, L_max, lens, "bf16", cfg_id=121)
    q = dev(case["q"])
    out = torch.empty_like(q)
    ws = kvc.workspace(kvc.kvc_decode_attn_window_workspace_size(B, n_h, n_kv, L_max, d, 1, 1))
    kvc.kvc_decode_attn_window(q, dev(case["k_cache"]), dev(case["v_cache"]),
                               dev(np.asarray(lens, np.int32)), out, 1,
                               scale=1 / math.sqrt(d), workspace=ws)
    torch.cuda.synchronize()
    got = host(out)
    G = n_h // n_kv
    for b in range(B):
        for i in range(n_h):
            assert np.array_equal(got[b, i], case["v_cache"][b, i // G, lens[b] - 1])
