"""Run-to-run repeatability of every decode path at sizes that use their
split merges, the persistent schedule and every tile-copy stage.

The same call on the same inputs must give the same bits: each kernel's
arithmetic order is fixed by the lengths alone (the split merges combine
partials in split order, whatever order the workgroups finish in).  A
difference between two runs means a race: a read of a tile stage before its
copy landed, a stage overwritten while still read, a partial read before it
was written.  Outputs start as NaN each time, so a row left unwritten also
shows.  Inputs are generated on the device (no oracle is involved: the
parity tests compare against the oracle at smaller sizes)."""
from __future__ import annotations

import math

import numpy as np
import pytest

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


def _gen(seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _bf16(shape, g):
    return torch.randn(*shape, device="cuda", generator=g).to(torch.bfloat16)


def _lens(B, lo, hi, seed):
    rng = np.random.default_rng(seed)
    return torch.tensor(rng.integers(lo, hi + 1, size=B), dtype=torch.int32, device="cuda")


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _repeat(run, n=3):
    """run() -> list of output tensors; every repetition must match the first
    bit for bit."""
    first = None
    for rep in range(n):
        outs = run()
        torch.cuda.synchronize()
        outs = [_bits(o).clone() for o in outs]
        if first is None:
            first = outs
            continue
        for i, (a, b) in enumerate(zip(first, outs)):
            nd = int((a != b).sum())
            assert nd == 0, f"repetition {rep}: output {i} differs in {nd} elements"


def _nan(shape, dtype=torch.bfloat16):
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def test_fused_persistent_repeatable():
    """Append-and-attend on a GQA layer large enough for the persistent
    schedule (128 units, ragged lengths up to 16k, several splits each)."""
    B, n_h, n_kv, d, L_max = 16, 64, 8, 128, 16384
    g = _gen(11)
    K0, V0 = _bf16((B, n_kv, L_max, d), g), _bf16((B, n_kv, L_max, d), g)
    q, kn, vn = _bf16((B, n_h, d), g), _bf16((B, n_kv, d), g), _bf16((B, n_kv, d), g)
    sl0 = _lens(B, 1, L_max - 1, 11)
    ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, 1))
    K, V = torch.empty_like(K0), torch.empty_like(V0)

    def run():
        K.copy_(K0)
        V.copy_(V0)
        sl = sl0.clone()
        out, lse = _nan((B, n_h, d)), _nan((B, n_h), torch.float32)
        kvc.kvc_append_decode_attn(q, K, V, sl, kn, vn, out, lse, scale=1 / math.sqrt(d),
                                   workspace=ws)
        return [out, lse, sl]

    _repeat(run)


def test_decode_small_and_large_repeatable():
    """Plain decode in the small-problem mode (splits cut from the actual
    lengths) and in the large-problem mode."""
    for B, L_max, lo in ((2, 4096, 1000), (32, 8192, 1)):
        n_h, n_kv, d = 64, 8, 128
        g = _gen(12 + B)
        K, V = _bf16((B, n_kv, L_max, d), g), _bf16((B, n_kv, L_max, d), g)
        q = _bf16((B, n_h, d), g)
        sl = _lens(B, lo, L_max, 12 + B)
        ws = kvc.workspace(kvc.kvc_decode_attn_workspace_size(B, n_h, n_kv, L_max, d, 1))

        def run():
            out, lse = _nan((B, n_h, d)), _nan((B, n_h), torch.float32)
            kvc.kvc_decode_attn(q, K, V, sl, out, lse, scale=1 / math.sqrt(d), workspace=ws)
            return [out, lse]

        _repeat(run)


def test_latent_repeatable():
    """The latent path at the 128-head width with several splits per
    sequence (four-stage tile copies, the split merge), lengths that end
    mid-chunk."""
    B, n_h, L_max = 64, 128, 8200
    g = _gen(13)
    ckv = _bf16((B, L_max, 576), g)
    q = _bf16((B, n_h, 576), g)
    sl = _lens(B, 5000, L_max, 13)
    ws = kvc.workspace(kvc.kvc_decode_attn_mla_workspace_size(B, n_h, L_max, 512, 64))

    def run():
        out, lse = _nan((B, n_h, 512)), _nan((B, n_h), torch.float32)
        kvc.kvc_decode_attn_mla(q, ckv, sl, out, lse, scale=1 / 24, workspace=ws)
        return [out, lse]

    _repeat(run)


def test_topk_and_paged_repeatable():
    B, n_h, n_kv, d, L_max, K = 8, 64, 8, 128, 16384, 2048
    g = _gen(14)
    Kc, Vc = _bf16((B, n_kv, L_max, d), g), _bf16((B, n_kv, L_max, d), g)
    q = _bf16((B, n_h, d), g)
    sl = torch.full((B,), L_max, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(14)
    idx = np.stack([np.stack([np.sort(rng.choice(L_max, K, replace=False)) for _ in range(n_kv)])
                    for _ in range(B)]).astype(np.int32)
    idx_d = torch.from_numpy(idx).cuda()
    ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, K, d, 1))

    def run_topk():
        out, lse = _nan((B, n_h, d)), _nan((B, n_h), torch.float32)
        kvc.kvc_decode_attn_topk(q, Kc, Vc, sl, idx_d, out, lse, scale=1 / math.sqrt(d),
                                 workspace=ws)
        return [out, lse]

    _repeat(run_topk)

    beta, max_blocks = 16, L_max // 16
    Bp = 4
    nblk = Bp * max_blocks
    kp, vp = _bf16((nblk, n_kv, beta, d), g), _bf16((nblk, n_kv, beta, d), g)
    table = torch.from_numpy(rng.permutation(nblk).astype(np.int32).reshape(Bp, max_blocks)).cuda()
    slp = _lens(Bp, 1, L_max, 15)
    qp = _bf16((Bp, n_h, d), g)
    wsp = kvc.workspace(kvc.kvc_decode_attn_paged_workspace_size(Bp, n_h, n_kv, max_blocks, beta,
                                                                 d, 1))

    def run_paged():
        out, lse = _nan((Bp, n_h, d)), _nan((Bp, n_h), torch.float32)
        kvc.kvc_decode_attn_paged(qp, kp, vp, table, slp, out, lse, scale=1 / math.sqrt(d),
                                  workspace=wsp)
        return [out, lse]

    _repeat(run_paged)


def test_quantised_repeatable():
    """E4M3 and E2M1 caches (codes drawn over their finite values)."""
    B, n_h, n_kv, d, L_max = 16, 64, 8, 128, 16384
    g = _gen(16)
    q = _bf16((B, n_h, d), g)
    sl = _lens(B, 1, L_max, 16)

    def codes8(shape):
        c = torch.randint(0, 0x7F, shape, device="cuda", dtype=torch.int32, generator=g)
        s = torch.randint(0, 2, shape, device="cuda", dtype=torch.int32, generator=g) << 7
        return (c | s).to(torch.uint8)     # 0x7F and 0xFF (NaN) never drawn

    k8, v8 = codes8((B, n_kv, L_max, d)), codes8((B, n_kv, L_max, d))
    ws8 = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(B, n_h, n_kv, L_max, d))

    def run8():
        out, lse = _nan((B, n_h, d)), _nan((B, n_h), torch.float32)
        kvc.kvc_decode_attn_fp8(q, k8, v8, sl, out, 0.05, 0.05, lse, scale=1 / math.sqrt(d),
                                workspace=ws8)
        return [out, lse]

    _repeat(run8)

    def u8(shape, lo, hi):
        return torch.randint(lo, hi, shape, device="cuda", dtype=torch.int32,
                             generator=g).to(torch.uint8)

    kc, vc = u8((B, n_kv, L_max, d // 2), 0, 256), u8((B, n_kv, L_max, d // 2), 0, 256)
    # scale bytes: positive E4M3 values between 2^-4 and 2^1
    ks, vs = u8((B, n_kv, L_max, d // 16), 0x18, 0x40), u8((B, n_kv, L_max, d // 16), 0x18, 0x40)
    ws4 = kvc.workspace(kvc.kvc_decode_attn_fp4_workspace_size(B, n_h, n_kv, L_max, d))

    def run4():
        out, lse = _nan((B, n_h, d)), _nan((B, n_h), torch.float32)
        kvc.kvc_decode_attn_fp4(q, kc, ks, vc, vs, sl, out, lse, scale=1 / math.sqrt(d),
                                workspace=ws4)
        return [out, lse]

    _repeat(run4)
