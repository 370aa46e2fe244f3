"""Paged KV cache: HIP path vs the fp64 oracle through the C ABI (MI355X).

Pools [num_blocks, n_kv, beta, d] with blocks in shuffled physical order;
blocks no sequence maps, and table entries past a sequence's blocks, hold
NaN poison / out-of-range ids, so any stray read shows.  Appends and lengths
must match bit for bit; outputs within 2e-2 (bf16).
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


def paged_case(B, n_h, n_kv, d, lens, beta, max_blocks, dtype, cfg_id, spare=5, seed=0):
    """A contiguous seeded case laid out in a shuffled pool.  Each sequence
    maps ceil((len + 1) / beta) blocks (room for the append); the rest of its
    table row holds out-of-range ids; spare blocks are poisoned."""
    L = max_blocks * beta
    case = syn.dense_case(B, n_h, n_kv, d, L, lens, dtype, cfg_id=cfg_id)
    need = [min(-(-(n + 1) // beta), max_blocks) for n in lens]
    nblk = sum(need) + spare
    order = np.random.default_rng(seed).permutation(nblk)
    sd = syn.storage_dtype(dtype)
    kp = np.full((nblk, n_kv, beta, d), syn.poison_value(dtype), dtype=sd)
    vp = kp.copy()
    table = np.full((B, max_blocks), 1 << 30, dtype=np.int32)
    at = 0
    for b in range(B):
        for k in range(need[b]):
            phys = int(order[at])
            at += 1
            table[b, k] = phys
            kp[phys] = case["k_cache"][b, :, k * beta:(k + 1) * beta]
            vp[phys] = case["v_cache"][b, :, k * beta:(k + 1) * beta]
    case.update(k_pool=kp, v_pool=vp, table=table)
    return case


PAGED_CASES = [
    # (n_h, n_kv, lens, beta, max_blocks, split)
    (64, 8, [0, 1, 15, 16, 17, 127, 1000, 2046], 16, 128, 0),
    (64, 8, [0, 31, 32, 33, 500, 2047], 32, 64, 0),
    (32, 32, [4095], 64, 64, 0),
    (16, 1, [5, 300], 8, 64, 0),
    (64, 8, [2990, 1000, 129], 16, 188, 128),
    (64, 8, [2990, 1000, 129], 16, 188, 384),
]


@pytest.mark.parametrize("n_h,n_kv,lens,beta,max_blocks,split", PAGED_CASES)
def test_paged_append_then_decode(n_h, n_kv, lens, beta, max_blocks, split):
    B, d = len(lens), 128
    case = paged_case(B, n_h, n_kv, d, lens, beta, max_blocks, "bf16", 130)
    kp, vp, tab, sl = dev(case["k_pool"]), dev(case["v_pool"]), dev(case["table"]), dev(case["seq_lens"])
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_paged(kp, vp, tab, sl, dev(case["k_new"]), dev(case["v_new"]), flag=flag)
    q = dev(case["q"])
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    kvc.kvc_set_split_override(split)
    ws = kvc.workspace(kvc.kvc_decode_attn_paged_workspace_size(B, n_h, n_kv, max_blocks, beta, d, 1))
    kvc.kvc_decode_attn_paged(q, kp, vp, tab, sl, out, lse, scale=1 / math.sqrt(d), flag=flag,
                              workspace=ws)
    torch.cuda.synchronize()
    if ws is not None:
        assert int(ws[:4 * B * n_kv].view(torch.int32).abs().sum()) == 0, "tickets not reset"

    k_o, v_o, sl_o = case["k_pool"].copy(), case["v_pool"].copy(), case["seq_lens"].copy()
    f_o = oracle.append_paged(k_o, v_o, case["table"], sl_o, case["k_new"], case["v_new"])
    o_ref, l_ref, f2 = oracle.decode_paged(case["q"], k_o, v_o, case["table"], sl_o, 1 / math.sqrt(d))
    assert host(sl).tolist() == sl_o.tolist()
    assert np.array_equal(host(kp), k_o) and np.array_equal(host(vp), v_o)
    assert int(host(flag)[0]) == (f_o | f2) == 0
    compare(host_f64(out), o_ref, 2e-2, f"paged beta {beta} split {split}")
    compare_lse(host(lse), l_ref, 4e-3)


def test_paged_shared_prefix_and_bad_blocks():
    """Two sequences share their first blocks (the same physical blocks);
    one table entry inside a sequence is invalid: its positions are skipped
    and the bad-index flag is set.  A full table and an invalid slot block
    on append set flags and write nothing."""
    B, n_h, n_kv, d, beta, mb = 3, 32, 4, 128, 16, 40
    lens = [300, 300, 200]
    case = paged_case(B, n_h, n_kv, d, lens, beta, mb, "bf16", 131, seed=3)
    tab = case["table"].copy()
    tab[1, :6] = tab[0, :6]                   # shared prefix (96 positions)
    tab[2, 4] = case["k_pool"].shape[0] + 9   # invalid block inside sequence 2
    sl = np.asarray(lens, np.int32)
    q = dev(case["q"])
    out = torch.empty_like(q)
    lse = torch.empty(B, n_h, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_paged_workspace_size(B, n_h, n_kv, mb, beta, d, 1))
    kvc.kvc_decode_attn_paged(q, dev(case["k_pool"]), dev(case["v_pool"]), dev(tab), dev(sl), out,
                              lse, scale=1 / math.sqrt(d), flag=flag, workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref, f_ref = oracle.decode_paged(case["q"], case["k_pool"], case["v_pool"], tab, sl,
                                              1 / math.sqrt(d))
    assert f_ref == oracle.FLAG_BAD_INDEX == int(host(flag)[0])
    compare(host_f64(out), o_ref, 2e-2, "paged shared/bad")
    compare_lse(host(lse), l_ref, 4e-3)

    kp, vp = dev(case["k_pool"]), dev(case["v_pool"])
    tab2 = case["table"].copy()
    sl2 = np.array([mb * beta, 32, 200], np.int32)      # full; slot 32 -> entry 2; ok
    tab2[1, 2] = -5
    fl = torch.zeros(1, dtype=torch.int32, device="cuda")
    sl2_d = dev(sl2)
    kvc.kvc_append_paged(kp, vp, dev(tab2), sl2_d, dev(case["k_new"]), dev(case["v_new"]), flag=fl)
    torch.cuda.synchronize()
    k_o, v_o, s_o = case["k_pool"].copy(), case["v_pool"].copy(), sl2.copy()
    f_o = oracle.append_paged(k_o, v_o, tab2, s_o, case["k_new"], case["v_new"])
    assert f_o == oracle.FLAG_CACHE_FULL | oracle.FLAG_BAD_INDEX == int(host(fl)[0])
    assert host(sl2_d).tolist() == s_o.tolist() == [mb * beta, 32, 201]
    assert np.array_equal(host(kp), k_o) and np.array_equal(host(vp), v_o)


def test_paged_append_f32():
    """The paged append is a bit copy for float32 rows too (d = 64)."""
    B, n_kv, d, beta, mb = 4, 2, 64, 8, 6
    lens = [0, 7, 8, 30]
    case = paged_case(B, n_kv, n_kv, d, lens, beta, mb, "f32", 132)
    kp, vp, sl = dev(case["k_pool"]), dev(case["v_pool"]), dev(case["seq_lens"])
    kvc.kvc_append_paged(kp, vp, dev(case["table"]), sl, dev(case["k_new"]), dev(case["v_new"]))
    torch.cuda.synchronize()
    k_o, v_o, s_o = case["k_pool"].copy(), case["v_pool"].copy(), case["seq_lens"].copy()
    oracle.append_paged(k_o, v_o, case["table"], s_o, case["k_new"], case["v_new"])
    assert host(sl).tolist() == s_o.tolist()
    assert np.array_equal(host(kp).view(np.uint32), k_o.view(np.uint32))
    assert np.array_equal(host(vp).view(np.uint32), v_o.view(np.uint32))
