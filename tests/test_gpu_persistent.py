"""Parity of the persistent dense form at the lengths its item list treats
differently.

A GQA layer of 16 sequences x 8 KV heads at L_max = 8192 (bf16, d = 128)
is decoded in the persistent form: 512 workgroups take (sequence, KV head,
split) items from a device counter, whole splits of S = 1024 positions
first, then every unit's last, shorter split in four classes by length
(longest first), or the empty item of a unit with nothing to attend.  The
lengths below put units in every class, on both sides of every split edge,
at zero and at the full cache, and compare with the oracle (the pages'
definition of decode attention: "KV cache" guide, "A cache you keep because
attention looks backwards"; the podcast's decode walk-through for the
append).  Rows past each length hold NaN, so a read past a split or a
sequence shows up as a non-finite output."""
from __future__ import annotations

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import kv_cache_decode_kvc_amd as kvc  # noqa: E402
import kvc_synth as syn  # noqa: E402
import oracle  # noqa: E402
from gpu_helpers import compare, compare_lse, dev, host, host_f64  # noqa: E402

B, N_H, N_KV, D, L_MAX = 16, 64, 8, 128, 8192
S = 1024          # the split size the library picks for this shape (checked below)
# attended lengths: every class of last item (remainder >= 3S/4 down to
# < S/4), exact multiples of S (no last item), split edges +- 1, one
# position, the full cache
LENS = [1, 2, 32, 33, 1023, 1024, 1025, 2048, 2049, 3000, 4096, 5000, 6144, 7000, 7900, 8192]


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' elsewhere)")
    kvc.kvc_set_split_override(0)
    yield
    torch.cuda.synchronize()


def _check_counters(ws):
    """Tickets (front) and the two scheduling words (last 256-byte block)
    are back to zero."""
    w32 = ws.view(torch.int32)
    assert int(w32[:B * N_KV].abs().sum()) == 0, "tickets not reset"
    assert int(w32[-64:-62].abs().sum()) == 0, "scheduling counters not reset"


def test_plan_is_persistent_with_1024_splits():
    # 128 units x 32 pieces of 256 positions is a large problem (fixed
    # splits); the persistent plan aims at about 1792 items: 8192 / 14
    # rounded up to a whole 1024
    assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, B, B * N_KV, L_MAX) == 256
    plain = kvc.kvc_decode_attn_workspace_size(B, N_H, N_KV, L_MAX, D, kvc.KVC_BF16)
    # partials for 8 splits (+ tickets, lengths and the scheduling block)
    P = L_MAX // S
    assert plain >= B * N_H * P * D * 4
    assert plain < B * N_H * (P + 1) * D * 4 + (1 << 16)


@pytest.mark.parametrize("with_empty", [False, True])
def test_persistent_decode_lengths(with_empty):
    """Plain decode at the listed lengths (and, with_empty, two sequences of
    length 0: the empty item, a zero row and lse = -inf)."""
    lens = list(LENS)
    if with_empty:
        lens[1] = 0
        lens[7] = 0
    case = syn.dense_case(B, N_H, N_KV, D, L_MAX, lens, "bf16", cfg_id=120)
    scale = 1 / math.sqrt(D)
    kc, vc, sl, q = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"]), dev(case["q"])
    out = torch.full((B, N_H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, N_H), float("nan"), dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_workspace_size(B, N_H, N_KV, L_MAX, D, kvc.KVC_BF16))
    kvc.kvc_decode_attn(q, kc, vc, sl, out, lse, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(case["q"], case["k_cache"], case["v_cache"], case["seq_lens"], scale)
    compare(host_f64(out), o_ref, 2e-2, f"persistent decode (empty={with_empty})")
    compare_lse(host(lse), l_ref, 4e-3)
    if with_empty:
        assert np.all(host_f64(out)[[1, 7]] == 0.0)
    _check_counters(ws)


def test_persistent_fused_lengths():
    """Append-and-attend in the persistent form: cached lengths n = LENS - 1
    (so 0 cached rows: the empty item plus the new row; 8191: the cache ends
    full), cache bytes and lengths bit-exact, outputs within tolerance; then
    a second call on the grown cache (every length moved by one across the
    split edges)."""
    pre = [n - 1 for n in LENS]
    case = syn.dense_case(B, N_H, N_KV, D, L_MAX, pre, "bf16", cfg_id=121)
    scale = 1 / math.sqrt(D)
    kc, vc, sl = dev(case["k_cache"]), dev(case["v_cache"]), dev(case["seq_lens"])
    q, kn, vn = dev(case["q"]), dev(case["k_new"]), dev(case["v_new"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(B, N_H, N_KV, L_MAX, D,
                                                                 kvc.KVC_BF16))
    kc_ref, vc_ref, sl_ref = case["k_cache"].copy(), case["v_cache"].copy(), case["seq_lens"].copy()
    for step in range(2):
        out = torch.full((B, N_H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, N_H), float("nan"), dtype=torch.float32, device="cuda")
        kvc.kvc_append_decode_attn(q, kc, vc, sl, kn, vn, out, lse, scale=scale, flag=flag,
                                   workspace=ws)
        torch.cuda.synchronize()
        f_ref = oracle.append(kc_ref, vc_ref, sl_ref, case["k_new"], case["v_new"])
        o_ref, l_ref = oracle.decode(case["q"], kc_ref, vc_ref, sl_ref, scale)
        assert host(sl).tolist() == sl_ref.tolist()
        assert np.array_equal(host(kc).view(np.uint8), kc_ref.view(np.uint8))
        assert np.array_equal(host(vc).view(np.uint8), vc_ref.view(np.uint8))
        compare(host_f64(out), o_ref, 2e-2, f"persistent fused step {step}")
        compare_lse(host(lse), l_ref, 4e-3)
        w32 = ws.view(torch.int32)
        assert int(w32[-64:-62].abs().sum()) == 0, "scheduling counters not reset"
        if step == 1:
            # the second step found the last sequence's cache full
            assert int(host(flag)[0]) == f_ref == oracle.FLAG_CACHE_FULL
