"""Top-k selection from indexer scores: HIP path vs the oracle, bit for bit.

The selected positions (ascending, -1 padded) must equal the oracle's for
random scores, heavy ties (lower position first), signed zeros, short rows,
the pool-restricted variant, and at the sparse workload's full size on
sampled rows.  Selection followed by the sparse decode matches the oracle's
decode over the same positions.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import kvc_synth as syn
import oracle
from gpu_helpers import compare, dev, host, host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import kv_cache_decode_kvc_amd as kvc  # noqa: E402


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' elsewhere)")
    yield
    torch.cuda.synchronize()


def run_select(scores, lens, K, pool=None, pool_block=8, ws=False):
    """ws: pass a workspace (the segmented form where the shape has one)."""
    B, R, L = scores.shape
    out = torch.full((B, R, K), 12345, dtype=torch.int32, device="cuda")
    w = kvc.workspace(kvc.kvc_topk_select_workspace_size(B, R, L, K)) if ws else None
    kvc.kvc_topk_select(dev(scores), dev(np.asarray(lens, np.int32)), out,
                        pool=None if pool is None else dev(pool), pool_block=pool_block,
                        workspace=w)
    torch.cuda.synchronize()
    return host(out)


# Rows of several 16384-position steps take the segmented form when a
# workspace is given: both forms against the oracle.
SEG_CASES = [
    # (kind, R, L, lens, K)
    ("normal", 4, 70000, [70000, 33000], 2048),
    ("normal", 2, 40000, [16384, 16385, 0, 32769], 700),   # segment edges, an empty row
    ("coarse", 4, 50000, [50000, 49999], 2048),            # many equal keys at the threshold
    ("ties", 4, 50000, [50000, 20000], 2048),              # lists overflow: whole-row fallback
    ("zeros", 4, 40000, [40000], 500),                     # -0 and +0 equal
    ("few", 2, 50000, [1500, 2048, 2049], 2048),           # fewer than, exactly, one more than K
    ("normal", 1, 262144, [262144], 4096),                 # the longest row of the form
    ("lastmax", 2, 40000, [32769, 32770, 32771, 39999], 300),   # top scores in the row's last 3
    # the K largest far above the rest, at positions the row's sample skips
    # (offsets 64..2047 of each 2048-position block): the bound comes from
    # the rest, and the K-th lies more than 2^22 key steps above it
    ("hidden", 4, 70000, [70000, 65536], 512),
]


@pytest.mark.parametrize("kind,R,L,lens,K", SEG_CASES)
@pytest.mark.parametrize("ws", [False, True])
def test_select_segmented_matches_oracle(kind, R, L, lens, K, ws):
    rng = np.random.default_rng(sum(map(ord, kind)) * 7919 + R * 131 + L + K)
    B = len(lens)
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    if kind == "coarse":
        sc = (np.round(sc * 64) / 64).astype(np.float32)
    elif kind == "ties":
        sc = rng.integers(0, 4, size=(B, R, L)).astype(np.float32)
    elif kind == "zeros":
        sc = np.where(rng.random((B, R, L)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        sc[:, :, ::9] = 1.0
    elif kind == "hidden":
        for b, n in enumerate(lens):
            unsampled = np.arange(n)[np.arange(n) % 2048 >= 64]
            for r in range(R):
                pos = rng.choice(unsampled, size=K + 64, replace=False)
                sc[b, r, pos] = np.float32(1000.0) + rng.random(K + 64).astype(np.float32)
    elif kind == "lastmax":
        # the highest scores sit in the last positions of each row (lengths
        # not multiples of 4: a 16-byte load straddles the end)
        for b, n in enumerate(lens):
            sc[b, :, n - 3:n] = np.float32(50.0) + np.arange(3, dtype=np.float32)
    if ws:
        assert kvc.kvc_topk_select_workspace_size(B, R, L, K) > 0
    got = run_select(sc, lens, K, ws=ws)
    want = oracle.topk_select(sc, np.asarray(lens), K)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "short"])
def test_select_matches_oracle(kind):
    rng = np.random.default_rng({"normal": 1, "ties": 2, "zeros": 3, "short": 4}[kind])
    B, R, L, K = 3, 4, 5000, 256
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    lens = [5000, 4097, 1]
    if kind == "ties":
        sc = rng.integers(0, 4, size=(B, R, L)).astype(np.float32)
    elif kind == "zeros":
        sc = np.where(rng.random((B, R, L)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        sc[:, :, ::7] = 1.0
    elif kind == "short":
        lens = [0, 100, 255]
    got = run_select(sc, lens, K)
    want = oracle.topk_select(sc, np.asarray(lens), K)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("kind", ["overflow", "long"])
def test_select_multipass_paths(kind):
    """Rows the one-extra-pass route cannot take: a threshold bin of more
    than 8192 equal keys (20000 ones among zeros), and rows longer than 2^18
    positions; both go through the further histogram passes and the ordered
    row walk."""
    rng = np.random.default_rng(7 if kind == "overflow" else 8)
    if kind == "overflow":
        B, R, L, K = 2, 2, 40000, 1000
        sc = (rng.random((B, R, L)) < 0.5).astype(np.float32)
        lens = [40000, 33333]
    else:
        B, R, L, K = 1, 2, 300000, 2048
        sc = rng.standard_normal((B, R, L)).astype(np.float32)
        lens = [299999]
    got = run_select(sc, lens, K)
    want = oracle.topk_select(sc, np.asarray(lens), K)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("kind", ["equal", "ties", "short", "pool"])
def test_select_long_rows(kind):
    """Rows of 140000 positions: every score equal (the lowest K positions;
    the threshold bin overflows the lists), coarse ties, rows ending early,
    and a pool."""
    rng = np.random.default_rng({"equal": 21, "ties": 22, "short": 23, "pool": 25}[kind])
    B, R, L, K = 2, 3, 140000, 2048
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    lens = [L, 100000]
    pool = None
    if kind == "equal":
        sc[:] = 0.5
    elif kind == "ties":
        sc = np.round(sc * 4).astype(np.float32) / 4
    elif kind == "short":
        lens = [33000, 70000]
    elif kind == "pool":
        nblk = -(-L // 8)
        pool = np.stack([np.stack([rng.choice(nblk, 2000, replace=False) for _ in range(R)])
                         for _ in range(B)]).astype(np.int32)
    got = run_select(sc, lens, K, pool=pool, pool_block=8)
    want = oracle.topk_select(sc, np.asarray(lens), K, pool=pool, pool_block=8)
    assert np.array_equal(got, want), (kind, np.argwhere(got != want)[:5])


@pytest.mark.parametrize("seed", range(12))
def test_select_random_sweep(seed):
    """Seeded shapes across both passes' short and general steps: K from 1
    to past the row, lengths off the 16384-position step, coarse ties,
    negative-only and infinite scores, with and without a pool."""
    rng = np.random.default_rng(1000 + seed)
    B, R = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    L = int(rng.choice([700, 16384, 20000, 50001, 70000]))
    K = int(rng.choice([1, 17, 256, 2048, L, L + 5]))
    K = max(1, min(K, L))
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    kind = seed % 4
    if kind == 1:
        sc = np.round(sc * 8).astype(np.float32) / 8          # coarse ties
    elif kind == 2:
        sc = -np.abs(sc) - 1.0                                # every score negative
    elif kind == 3:
        sc.reshape(-1)[rng.integers(0, sc.size, 40)] = np.inf
        sc.reshape(-1)[rng.integers(0, sc.size, 40)] = -np.inf
    lens = [int(x) for x in rng.integers(0, L + 1, B)]
    lens[0] = L
    pool = None
    if seed % 3 == 2:
        nblk = -(-L // 8)
        P = int(min(nblk, 600))
        pool = np.stack([np.stack([rng.choice(nblk, P, replace=False) for _ in range(R)])
                         for _ in range(B)]).astype(np.int32)
    got = run_select(sc, lens, K, pool=pool, pool_block=8)
    want = oracle.topk_select(sc, np.asarray(lens), K, pool=pool, pool_block=8)
    assert np.array_equal(got, want), (seed, np.argwhere(got != want)[:5])


def test_select_pool_variant():
    rng = np.random.default_rng(5)
    B, R, L, K, blk = 2, 3, 20000, 512, 8
    sc = rng.standard_normal((B, R, L)).astype(np.float32)
    pool = np.full((B, R, 300), -1, np.int32)
    for b in range(B):
        for j in range(R):
            pool[b, j, :250] = rng.choice(L // blk, 250, replace=False)
    pool[0, 0, 250:260] = [10 ** 7, -3, 5, 5, 5, 7, 99999, 0, 0, 1]   # out of range and repeats
    lens = [20000, 15000]
    got = run_select(sc, lens, K, pool=pool, pool_block=blk)
    want = oracle.topk_select(sc, np.asarray(lens), K, pool=pool, pool_block=blk)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ws", [False, True])
def test_select_fullsize_sampled_rows(ws):
    """The sparse workload's shape: 8 sequences x 8 KV heads, 2048 of 131072
    (with a workspace: the segmented form, as timed)."""
    c = syn.C5
    B, R, L, K = c.B, c.n_kv, c.pre_len, c.K
    g = torch.Generator(device="cuda")
    g.manual_seed(syn.device_seed(c.cfg_id, 0, "idx"))
    scores = torch.randn(B, R, L, generator=g, device="cuda", dtype=torch.float32)
    out = torch.empty(B, R, K, dtype=torch.int32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    units = [(0, 0), (3, 5), (7, 7)]
    rows = {u: host(scores[u[0]:u[0] + 1, u[1]:u[1] + 1]) for u in units}   # before the call
    w = kvc.workspace(kvc.kvc_topk_select_workspace_size(B, R, L, K)) if ws else None
    if ws:
        assert w is not None
    kvc.kvc_topk_select(scores, lens, out, workspace=w)
    torch.cuda.synchronize()
    got = host(out)
    for b, j in units:
        want = oracle.topk_select(rows[(b, j)], np.array([L]), K)
        assert np.array_equal(got[b, j], want[0, 0]), (b, j)


def test_select_then_sparse_decode():
    """Selection feeding the sparse decode equals the oracle's decode over
    the oracle's selection."""
    rng = np.random.default_rng(6)
    B, n_h, n_kv, d, L, K = 2, 32, 4, 128, 3000, 300
    lens = [3000, 1200]
    case = syn.dense_case(B, n_h, n_kv, d, L, lens, "bf16", cfg_id=140)
    sc = rng.standard_normal((B, n_kv, L)).astype(np.float32)
    idx = torch.empty(B, n_kv, K, dtype=torch.int32, device="cuda")
    sl = dev(np.asarray(lens, np.int32))
    kvc.kvc_topk_select(dev(sc), sl, idx)
    q = dev(case["q"])
    out = torch.empty_like(q)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, K, d, 1))
    kvc.kvc_decode_attn_topk(q, dev(case["k_cache"]), dev(case["v_cache"]), sl, idx, out,
                             scale=1 / math.sqrt(d), flag=flag, workspace=ws)
    torch.cuda.synchronize()
    sel = oracle.topk_select(sc, np.asarray(lens), K)
    assert np.array_equal(host(idx), sel)
    o_ref, _, f_ref = oracle.decode_topk(case["q"], case["k_cache"], case["v_cache"],
                                        np.asarray(lens, np.int32), sel, 1 / math.sqrt(d))
    assert f_ref == 0 == int(host(flag)[0])
    compare(host_f64(out), o_ref, 2e-2, "select + sparse decode")
