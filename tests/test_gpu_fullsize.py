"""Parity at the benchmark's full sizes (MI355X).

Each test builds one layer of a benchmark workload at its real shape on the
device (seeded N(0,1), the same generators and split policy the benchmark
uses), runs the calls the benchmark times, and checks a sample of the
outputs against the fp64 oracle on host copies of just the rows those
outputs depend on.  Those host copies are taken before any library call (so
no oracle input passes through the HIP path); the appended row is the
generated new row itself, or the oracle's own quantisation of it, and the
row the library wrote is checked against it bit for bit, as are the lengths.
"""
from __future__ import annotations

import numpy as np
import pytest

import kvc_synth as syn
import oracle
from gpu_helpers import compare, compare_lse, host

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
    torch.cuda.empty_cache()


def normal(shape, cfg_id, layer, tensor):
    t = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
    return syn.device_normal_(t, syn.device_seed(cfg_id, layer, tensor))


def bits(t):
    """bf16 (or uint8) device tensor -> host copy of its storage."""
    return host(t.contiguous())


def sample_units(pre, n_kv, count, seed):
    """(b, j) pairs: the longest and shortest sequences plus a seeded draw."""
    rng = np.random.default_rng(seed)
    bs = {int(np.argmax(pre)), int(np.argmin(pre))}
    bs |= set(int(x) for x in rng.choice(len(pre), size=min(count, len(pre)), replace=False))
    return [(b, int(rng.integers(n_kv))) for b in sorted(bs)]


def snapshot(units, pre, **tensors):
    """Host copies, taken before the library runs, of what the sampled
    units' outputs depend on: cached rows [0, pre[b]) of each [B, n_kv, L, .]
    tensor given, and the unit's slice of each [B, n_kv, .] new-row tensor."""
    snap = {}
    for b, j in units:
        for name, t in tensors.items():
            snap[(name, b, j)] = bits(t[b, j, :int(pre[b])] if t.dim() == 4 else t[b, j])
    return snap


def check_dense_units(cfg, pre, q_h, snap, out, lse, units, what):
    """Oracle decode over the snapshot rows plus the generated new row."""
    G = cfg.n_h // cfg.n_kv
    for b, j in units:
        n = int(pre[b]) + 1
        kb = np.concatenate([snap[("K", b, j)], snap[("kn", b, j)][None]])[None, None]
        vb = np.concatenate([snap[("V", b, j)], snap[("vn", b, j)][None]])[None, None]
        qb = q_h[b, j * G:(j + 1) * G][None]
        o_ref, l_ref = oracle.decode(qb, kb, vb, np.array([n], np.int32), cfg.scale)
        got = oracle.to_f64(bits(out[b, j * G:(j + 1) * G]))
        compare(got, o_ref[0], 2e-2, f"{what} b={b} j={j} n={n}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)


def test_fullsize_mha_layer():
    """32-head MHA layer, 4096 cached + 1 appended, fused append + attend."""
    c = syn.C2
    _fused_dense(c, units=[(0, j) for j in range(c.n_kv)])


def test_fullsize_gqa_layer():
    """GQA layer, B = 32, lengths U[1024, 32768], fused append + attend."""
    c = syn.C3
    pre = syn.pre_append_lens(c)
    _fused_dense(c, units=sample_units(pre, c.n_kv, 4, 31))


@pytest.mark.parametrize("grown", [1, 17, 34])
def test_fullsize_mha_layer_grown(grown):
    """The MHA layer as the benchmark times it after `grown` steps: the
    cache reserves the benchmark's slack (4097 + slack positions) and holds
    4096 + grown rows, so the fused call attends 4097 + grown positions over
    the plan those lengths take (15 splits of 288 cached rows, the new row
    from registers), not the 16 x 256 of exactly 4096."""
    import bench
    c = syn.C2
    pre = syn.pre_append_lens(c) + grown
    _fused_dense(c, units=[(0, j) for j in range(c.n_kv)], pre=pre,
                 L_max=int(c.L_max + bench.reservation_slack()))


def _fused_dense(c, units, pre=None, L_max=None):
    if pre is None:
        pre = syn.pre_append_lens(c)
    if L_max is None:
        L_max = int(max(c.L_max, pre.max() + 1))
    K = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "k")
    V = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "v")
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    snap = snapshot(units, pre, K=K, V=V, kn=kn, vn=vn)
    q_h = bits(q)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(c.B, c.n_h, c.n_kv, L_max, c.d,
                                                                 kvc.KVC_BF16))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_append_decode_attn(q, K, V, sl, kn, vn, out, lse, scale=c.scale, flag=flag,
                               workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    assert int(host(flag)[0]) == 0
    for b, j in units:
        assert np.array_equal(bits(K[b, j, pre[b]]), snap[("kn", b, j)])
        assert np.array_equal(bits(V[b, j, pre[b]]), snap[("vn", b, j)])
    check_dense_units(c, pre, q_h, snap, out, lse, units, c.name)


def _random_codes(shape, tensor, c, lo=0, hi=256):
    """Seeded uniform bytes on the device (the benchmark's cache fill)."""
    t = torch.empty(*shape, dtype=torch.uint8, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(syn.device_seed(c.cfg_id, 0, tensor))
    t.copy_(torch.randint(lo, hi, t.shape, generator=g, device="cuda",
                          dtype=torch.int32).to(torch.uint8))
    return t


def test_fullsize_gqa_layer_fp8():
    """The GQA layer over E4M3 caches: append_fp8 then decode_fp8."""
    c = syn.C3
    pre = syn.pre_append_lens(c)
    L_max = int(max(c.L_max, pre.max() + 1))
    ks, vs = 1.0 / 64, 1.0 / 64
    G = c.n_h // c.n_kv

    def codes(tensor, scale):
        t = torch.empty(c.B, c.n_kv, L_max, c.d, dtype=torch.uint8, device="cuda")
        flat = t.view(-1)
        g = torch.Generator(device="cuda")
        g.manual_seed(syn.device_seed(c.cfg_id, 0, tensor))
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            e = min(flat.numel(), s + step)
            x = torch.randn(e - s, generator=g, device="cuda", dtype=torch.float32) / scale
            flat[s:e].copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
        return t

    K8, V8 = codes("k", ks), codes("v", vs)
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    units = sample_units(pre, c.n_kv, 4, 33)
    snap = snapshot(units, pre, K=K8, V=V8, kn=kn, vn=vn)
    q_h = bits(q)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(c.B, c.n_h, c.n_kv, L_max, c.d))
    kvc.kvc_append_fp8(K8, V8, sl, kn, vn, ks, vs)
    kvc.kvc_decode_attn_fp8(q, K8, V8, sl, out, ks, vs, lse, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    for b, j in units:
        n = int(pre[b]) + 1
        k_new = oracle.quantize_fp8(snap[("kn", b, j)], ks)
        v_new = oracle.quantize_fp8(snap[("vn", b, j)], vs)
        assert np.array_equal(host(K8[b, j, pre[b]]), k_new)
        assert np.array_equal(host(V8[b, j, pre[b]]), v_new)
        kb = np.concatenate([snap[("K", b, j)], k_new[None]])[None, None]
        vb = np.concatenate([snap[("V", b, j)], v_new[None]])[None, None]
        o_ref, l_ref = oracle.decode_fp8(q_h[b, j * G:(j + 1) * G][None], kb, vb,
                                         np.array([n], np.int32), c.scale, ks, vs)
        got = oracle.to_f64(bits(out[b, j * G:(j + 1) * G]))
        compare(got, o_ref[0], 2e-2, f"fp8 b={b} j={j} n={n}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)


def test_fullsize_gqa_layer_fp4():
    """The GQA layer over FP4 caches (E2M1 codes, E4M3 scales per 16
    channels): append_fp4 then decode_fp4, as the benchmark's FP4 workload."""
    c = syn.C3
    pre = syn.pre_append_lens(c)
    L_max = int(max(c.L_max, pre.max() + 1))
    G = c.n_h // c.n_kv
    cshape, sshape = (c.B, c.n_kv, L_max, c.d // 2), (c.B, c.n_kv, L_max, c.d // 16)
    KC, VC = _random_codes(cshape, "k", c), _random_codes(cshape, "v", c)
    KS = _random_codes(sshape, "k_scales", c, 0x20, 0x30)
    VS = _random_codes(sshape, "v_scales", c, 0x20, 0x30)
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    units = sample_units(pre, c.n_kv, 4, 34)
    snap = snapshot(units, pre, KC=KC, VC=VC, KS=KS, VS=VS, kn=kn, vn=vn)
    q_h = bits(q)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_fp4_workspace_size(c.B, c.n_h, c.n_kv, L_max, c.d))
    kvc.kvc_append_fp4(KC, KS, VC, VS, sl, kn, vn)
    kvc.kvc_decode_attn_fp4(q, KC, KS, VC, VS, sl, out, lse, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    for b, j in units:
        n = int(pre[b]) + 1
        kc_new, ks_new = oracle.quantize_fp4(snap[("kn", b, j)])
        vc_new, vs_new = oracle.quantize_fp4(snap[("vn", b, j)])
        assert np.array_equal(host(KC[b, j, pre[b]]), kc_new)
        assert np.array_equal(host(KS[b, j, pre[b]]), ks_new)
        assert np.array_equal(host(VC[b, j, pre[b]]), vc_new)
        assert np.array_equal(host(VS[b, j, pre[b]]), vs_new)
        cat = lambda old, new: np.concatenate([snap[(old, b, j)], new[None]])[None, None]
        o_ref, l_ref = oracle.decode_fp4(q_h[b, j * G:(j + 1) * G][None], cat("KC", kc_new),
                                         cat("KS", ks_new), cat("VC", vc_new), cat("VS", vs_new),
                                         np.array([n], np.int32), c.scale)
        got = oracle.to_f64(bits(out[b, j * G:(j + 1) * G]))
        compare(got, o_ref[0], 2e-2, f"fp4 b={b} j={j} n={n}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)


def test_fullsize_mla_layer():
    """Latent-cache layer: B = 64, 128 heads, 8192 cached + 1 appended."""
    c = syn.C4
    D = c.d_c + c.d_r
    L_max = c.L_max
    C = normal((c.B, L_max, D), c.cfg_id, 0, "ckv")
    q = normal((c.B, c.n_h, D), c.cfg_id, 0, "q")
    cn = normal((c.B, D), c.cfg_id, 0, "ckv_new")
    check = (0, 37, 63)
    snap = {b: (bits(C[b, :c.pre_len]), bits(cn[b]), bits(q[b])) for b in check}
    pre = np.full(c.B, c.pre_len, dtype=np.int32)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty(c.B, c.n_h, c.d_c, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_mla_workspace_size(c.B, c.n_h, L_max, c.d_c, c.d_r))
    kvc.kvc_append(C, None, sl, cn, None)
    kvc.kvc_decode_attn_mla(q, C, sl, out, lse, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    refs = {}
    for b in check:
        rows, new, qb = snap[b]
        assert np.array_equal(bits(C[b, c.pre_len]), new)
        o_ref, l_ref = oracle.decode_mla(qb[None], np.concatenate([rows, new[None]])[None],
                                         np.array([c.pre_len + 1], np.int32), c.d_c, c.d_r, c.scale)
        refs[b] = o_ref[0]
        compare(oracle.to_f64(bits(out[b])), o_ref[0], 2e-2, f"mla b={b}")
        compare_lse(host(lse[b]), l_ref[0], 4e-3)

    # What the split exchange adds: the same decode as one split per
    # sequence (no partials) against the benchmark's plan (partials stored in
    # bf16, merged in float32).  Both are printed against the oracle, and
    # their difference over the whole batch relative to its rms.
    kvc.kvc_set_split_override(L_max + 31)
    out1 = torch.empty_like(out)
    kvc.kvc_decode_attn_mla(q, C, sl, out1, None, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    for b in check:
        compare(oracle.to_f64(bits(out1[b])), refs[b], 2e-2, f"mla one split b={b}")
    a, a1 = out.float(), out1.float()
    rms = float(a1.pow(2).mean().sqrt())
    dd = (a - a1).abs()
    print(f"[mla split partials vs one split, whole batch] max|d|/rms={float(dd.max()) / rms:.3e} "
          f"rms|d|/rms={float(dd.pow(2).mean().sqrt()) / rms:.3e} rms={rms:.3e}")
    assert float(dd.max()) <= 2e-2


def test_fullsize_topk_layer():
    """Top-k layer: B = 8, 2048 listed positions of 131072 per KV head."""
    c = syn.C5
    L_max = c.L_max
    K = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "k")
    V = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "v")
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    idx_h = syn.topk_indices(c.cfg_id, 0, c.B, c.n_kv, c.K, c.pre_len, index_set=0)
    idx = torch.from_numpy(idx_h).cuda()
    pre = np.full(c.B, c.pre_len, dtype=np.int32)
    units = [(0, 0), (3, 5), (7, 7)]
    snap = snapshot(units, pre, K=K, V=V, kn=kn, vn=vn)
    q_h = bits(q)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(c.B, c.n_h, c.n_kv, c.K, c.d,
                                                               kvc.KVC_BF16))
    kvc.kvc_append(K, V, sl, kn, vn)
    kvc.kvc_decode_attn_topk(q, K, V, sl, idx, out, lse, scale=c.scale, flag=flag, workspace=ws)
    torch.cuda.synchronize()
    assert int(host(flag)[0]) == 0
    G = c.n_h // c.n_kv
    for b, j in units:
        n = c.pre_len + 1
        kb = np.concatenate([snap[("K", b, j)], snap[("kn", b, j)][None]])[None, None]
        vb = np.concatenate([snap[("V", b, j)], snap[("vn", b, j)][None]])[None, None]
        qb = q_h[b, j * G:(j + 1) * G][None]
        o_ref, l_ref, f_ref = oracle.decode_topk(qb, kb, vb, np.array([n], np.int32),
                                                 idx_h[b:b + 1, j:j + 1], c.scale)
        assert f_ref == 0
        compare(oracle.to_f64(bits(out[b, j * G:(j + 1) * G])), o_ref[0], 2e-2, f"topk b={b} j={j}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)


def test_fullsize_gqa_layer_window():
    """The GQA layer attending its newest 128 positions (append, then the
    window decode), as the benchmark's window workload runs it."""
    c = syn.C3
    W = 128
    pre = syn.pre_append_lens(c)
    L_max = int(max(c.L_max, pre.max() + 1))
    K = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "k")
    V = normal((c.B, c.n_kv, L_max, c.d), c.cfg_id, 0, "v")
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    units = sample_units(pre, c.n_kv, 4, 35)
    snap = snapshot(units, pre, K=K, V=V, kn=kn, vn=vn)
    q_h = bits(q)
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_window_workspace_size(c.B, c.n_h, c.n_kv, L_max, c.d,
                                                                 kvc.KVC_BF16, W))
    kvc.kvc_append(K, V, sl, kn, vn)
    kvc.kvc_decode_attn_window(q, K, V, sl, out, W, lse=lse, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    G = c.n_h // c.n_kv
    for b, j in units:
        n = int(pre[b]) + 1
        lo = n - W
        kb = np.concatenate([snap[("K", b, j)], snap[("kn", b, j)][None]])[lo:n]
        vb = np.concatenate([snap[("V", b, j)], snap[("vn", b, j)][None]])[lo:n]
        o_ref, l_ref = oracle.decode_window(q_h[b, j * G:(j + 1) * G][None], kb[None, None],
                                            vb[None, None], np.array([W], np.int32), c.scale, W)
        compare(oracle.to_f64(bits(out[b, j * G:(j + 1) * G])), o_ref[0], 2e-2, f"window b={b} j={j}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)


def test_fullsize_gqa_layer_paged():
    """The GQA layer over a paged cache of 16-position blocks in shuffled
    order (pools sized to the lengths), as the benchmark's paged workload."""
    c = syn.C3
    beta = 16
    pre = syn.pre_append_lens(c)
    need = [-(-int(n + 1) // beta) for n in pre]
    nblk = int(sum(need))
    mb = -(-int(pre.max() + 1) // beta)
    order = np.random.default_rng(7).permutation(nblk)
    table = np.full((c.B, mb), 1 << 30, dtype=np.int32)
    at = 0
    for b in range(c.B):
        table[b, :need[b]] = order[at:at + need[b]]
        at += need[b]
    K = normal((nblk, c.n_kv, beta, c.d), c.cfg_id, 0, "k")
    V = normal((nblk, c.n_kv, beta, c.d), c.cfg_id, 0, "v")
    q = normal((c.B, c.n_h, c.d), c.cfg_id, 0, "q")
    kn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "k_new")
    vn = normal((c.B, c.n_kv, c.d), c.cfg_id, 0, "v_new")
    units = sample_units(pre, c.n_kv, 3, 37)
    # rows [0, pre) of each sampled unit, gathered through its block table
    # before the library runs
    snap = {}
    for b, j in units:
        blocks = torch.from_numpy(table[b, :need[b]].astype(np.int64)).cuda()
        snap[("K", b, j)] = bits(K.index_select(0, blocks)[:, j].reshape(-1, c.d)[:int(pre[b])])
        snap[("V", b, j)] = bits(V.index_select(0, blocks)[:, j].reshape(-1, c.d)[:int(pre[b])])
        snap[("kn", b, j)], snap[("vn", b, j)] = bits(kn[b, j]), bits(vn[b, j])
    q_h = bits(q)
    tab = torch.from_numpy(table).cuda()
    sl = torch.tensor(pre, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(c.B, c.n_h, dtype=torch.float32, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_decode_attn_paged_workspace_size(c.B, c.n_h, c.n_kv, mb, beta, c.d,
                                                                kvc.KVC_BF16))
    kvc.kvc_append_paged(K, V, tab, sl, kn, vn, flag=flag)
    kvc.kvc_decode_attn_paged(q, K, V, tab, sl, out, lse, scale=c.scale, flag=flag, workspace=ws)
    torch.cuda.synchronize()
    assert host(sl).tolist() == (pre + 1).tolist()
    assert int(host(flag)[0]) == 0
    G = c.n_h // c.n_kv
    for b, j in units:
        n = int(pre[b]) + 1
        slot_blk, slot_off = int(table[b, pre[b] // beta]), int(pre[b]) % beta
        assert np.array_equal(bits(K[slot_blk, j, slot_off]), snap[("kn", b, j)])
        assert np.array_equal(bits(V[slot_blk, j, slot_off]), snap[("vn", b, j)])
        kb = np.concatenate([snap[("K", b, j)], snap[("kn", b, j)][None]])
        vb = np.concatenate([snap[("V", b, j)], snap[("vn", b, j)][None]])
        o_ref, l_ref = oracle.decode(q_h[b, j * G:(j + 1) * G][None], kb[None, None],
                                     vb[None, None], np.array([n], np.int32), c.scale)
        compare(oracle.to_f64(bits(out[b, j * G:(j + 1) * G])), o_ref[0], 2e-2, f"paged b={b} j={j}")
        compare_lse(host(lse[b, j * G:(j + 1) * G]), l_ref[0], 4e-3)
