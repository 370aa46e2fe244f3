"""C-ABI checks that need no GPU: the library loads, exports every function
include/kvc.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import kv_cache_decode_kvc_amd as kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

# fake, never-dereferenced device addresses with chosen alignment
A16 = ctypes.c_void_p(0x10000)
A4 = ctypes.c_void_p(0x10004)
A8 = ctypes.c_void_p(0x10008)
NULL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return kvc.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in range(-9, 1):
        assert kvc.kvc_status_string(code)
    assert kvc.kvc_status_string(-99) == "unknown status"


def dense(L, **kw):
    a = dict(q=A16, k=A16, v=A16, sl=A4, out=A16, lse=NULL, B=2, n_h=8, n_kv=2,
             L_max=64, d=128, scale=0.1, dt=kvc.KVC_BF16, ws=A16, wsb=1 << 30,
             stream=NULL)
    a.update(kw)
    return L.kvc_decode_attn(a["q"], a["k"], a["v"], a["sl"], a["out"], a["lse"],
                             a["B"], a["n_h"], a["n_kv"], a["L_max"], a["d"],
                             a["scale"], a["dt"], a["ws"], a["wsb"], a["stream"])


def test_dense_validation(L):
    assert dense(L, q=NULL) == -1
    assert dense(L, sl=NULL) == -1
    assert dense(L, n_h=7) == -2                  # n_h % n_kv
    assert dense(L, L_max=0) == -2
    assert dense(L, B=-1) == -2
    assert dense(L, dt=5) == -3
    assert dense(L, d=96) == -4
    assert dense(L, n_h=34, n_kv=2) == -4         # group of 17 > 16
    assert dense(L, L_max=1 << 23) == -2          # 2^23 * 256 B >= 2^31
    assert dense(L, q=A8) == -6
    assert dense(L, out=A4) == -6
    assert dense(L, scale=float("nan")) == -8
    assert dense(L, scale=float("inf")) == -8
    assert dense(L, B=0) == 0                     # empty batch: nothing to do


def test_dense_workspace_rules(L):
    need = L.kvc_decode_attn_workspace_size(4, 64, 8, 32768, 128, kvc.KVC_BF16)
    assert need > 0
    assert dense(L, B=4, n_h=64, n_kv=8, L_max=32768, ws=NULL, wsb=need) == -1
    assert dense(L, B=4, n_h=64, n_kv=8, L_max=32768, wsb=need - 1) == -5
    assert dense(L, B=4, n_h=64, n_kv=8, L_max=32768, ws=ctypes.c_void_p(0x10010), wsb=need) == -6
    # a single split needs no workspace
    assert L.kvc_decode_attn_workspace_size(1, 8, 2, 64, 64, kvc.KVC_F32) == 0
    assert L.kvc_decode_attn_workspace_size(1, 8, 2, 64, 96, kvc.KVC_F32) == 0  # unsupported -> 0


def test_split_policy_and_override(L):
    S = kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 32, 256, 32768)
    assert S % 128 == 0 and 256 * -(-32768 // S) <= 4608
    # small problem: one round of 512 workgroups -> at most 16 splits of 4097,
    # whole chunks: 288 (15 splits)
    assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 1, 32, 4097) == 288
    assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 1, 32, 4096) == 256
    # top-k 2048 of 64 units: 8 splits of 256
    assert kvc.kvc_split_positions(kvc.KVC_KIND_TOPK, 8, 64, 2048) == 512
    # tiny problem: at least 128 positions per split
    assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 1, 4, 300) == 128
    # at most 256 splits per sequence
    assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 1, 1, 1 << 20) >= (1 << 20) // 256
    Sm = kvc.kvc_split_positions(kvc.KVC_KIND_MLA, 64, 128, 8193)
    assert Sm % 32 == 0 and Sm >= 256
    try:
        kvc.kvc_set_split_override(300)
        assert kvc.kvc_split_positions(kvc.KVC_KIND_DENSE, 1, 1, 1000) == 320
        assert kvc.kvc_split_positions(kvc.KVC_KIND_MLA, 1, 1, 1000) == 320
    finally:
        kvc.kvc_set_split_override(0)
    assert L.kvc_set_split_override(-1) == -8
    assert L.kvc_split_positions(7, 1, 1, 1) == -8


def test_append_validation(L):
    def ap(**kw):
        a = dict(k=A16, v=A16, sl=A4, kn=A16, vn=A16, B=2, n_kv=2, L_max=8, d=64,
                 dt=kvc.KVC_BF16, flag=NULL, stream=NULL)
        a.update(kw)
        return L.kvc_append(a["k"], a["v"], a["sl"], a["kn"], a["vn"], a["B"],
                            a["n_kv"], a["L_max"], a["d"], a["dt"], a["flag"], a["stream"])
    assert ap(k=NULL) == -1
    assert ap(v=NULL) == -1          # v_cache NULL needs v_new NULL
    assert ap(vn=NULL) == -1
    assert ap(dt=2) == -3
    assert ap(d=0) == -2
    assert ap(k=A8) == -6
    assert ap(sl=ctypes.c_void_p(0x10002)) == -6
    assert ap(B=0) == 0


def test_mla_validation(L):
    def ml(**kw):
        a = dict(q=A16, c=A16, sl=A4, out=A16, lse=NULL, B=2, n_h=128, L_max=100,
                 d_c=512, d_r=64, scale=1 / 24, dt=kvc.KVC_BF16, ws=A16, wsb=1 << 30,
                 stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_mla(a["q"], a["c"], a["sl"], a["out"], a["lse"], a["B"],
                                     a["n_h"], a["L_max"], a["d_c"], a["d_r"], a["scale"],
                                     a["dt"], a["ws"], a["wsb"], a["stream"])
    assert ml(c=NULL) == -1
    assert ml(dt=kvc.KVC_F32) == -4
    assert ml(d_c=256) == -4
    assert ml(n_h=96) == -4
    assert ml(n_h=0) == -2
    assert ml(out=A8) == -6
    assert ml(scale=float("nan")) == -8
    assert ml(B=0) == 0
    assert L.kvc_decode_attn_mla_workspace_size(64, 128, 8193, 512, 64) > 0


def test_topk_validation(L):
    def tk(**kw):
        a = dict(q=A16, k=A16, v=A16, sl=A4, idx=A16, K=16, out=A16, lse=NULL, B=2,
                 n_h=8, n_kv=2, L_max=64, d=128, scale=0.1, dt=kvc.KVC_BF16,
                 flag=NULL, ws=A16, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_topk(a["q"], a["k"], a["v"], a["sl"], a["idx"], a["K"],
                                      a["out"], a["lse"], a["B"], a["n_h"], a["n_kv"],
                                      a["L_max"], a["d"], a["scale"], a["dt"], a["flag"],
                                      a["ws"], a["wsb"], a["stream"])
    assert tk(idx=NULL) == -1
    assert tk(K=0) == -2
    assert tk(K=65) == -2
    assert tk(idx=A8) == -6
    assert tk(B=0) == 0


def test_diag_validation(L):
    assert L.kvc_stream_read(NULL, 16, A16, NULL) == -1
    assert L.kvc_stream_read(A16, 8, A16, NULL) == -6
    assert L.kvc_copy(A16, A8, 16, NULL) == -6
    assert L.kvc_copy(A16, A16, 0, NULL) == 0


def test_fused_validation(L):
    def fz(**kw):
        a = dict(q=A16, k=A16, v=A16, sl=A4, kn=A16, vn=A16, out=A16, lse=NULL, B=2, n_h=8,
                 n_kv=2, L_max=64, d=128, scale=0.1, dt=kvc.KVC_BF16, flag=NULL, ws=A16,
                 wsb=1 << 30, stream=NULL)
        a.update(kw)
        return L.kvc_append_decode_attn(a["q"], a["k"], a["v"], a["sl"], a["kn"], a["vn"],
                                        a["out"], a["lse"], a["B"], a["n_h"], a["n_kv"],
                                        a["L_max"], a["d"], a["scale"], a["dt"], a["flag"],
                                        a["ws"], a["wsb"], a["stream"])
    assert fz(kn=NULL) == -1
    assert fz(vn=A8) == -6
    assert fz(ws=NULL) == -1              # always needs its arrival counters
    assert fz(wsb=16) == -5
    assert fz(n_h=6, n_kv=4) == -2
    assert fz(B=0) == 0
    assert L.kvc_append_decode_attn_workspace_size(1, 8, 2, 64, 128, kvc.KVC_BF16) > 0


def test_fp8_validation(L):
    def ap(**kw):
        a = dict(k=A16, v=A16, sl=A4, kn=A16, vn=A16, B=2, n_kv=2, L_max=8, d=128,
                 ks=0.1, vs=0.1, flag=NULL, stream=NULL)
        a.update(kw)
        return L.kvc_append_fp8(a["k"], a["v"], a["sl"], a["kn"], a["vn"], a["B"], a["n_kv"],
                                a["L_max"], a["d"], a["ks"], a["vs"], a["flag"], a["stream"])
    assert ap(v=NULL) == -1           # both caches are required
    assert ap(vn=NULL) == -1
    assert ap(d=120) == -2            # rows are whole 16-byte pieces
    assert ap(ks=0.0) == -8
    assert ap(vs=float("inf")) == -8
    assert ap(ks=-1.0) == -8
    assert ap(k=A8) == -6
    assert ap(B=0) == 0

    def dc(**kw):
        a = dict(q=A16, k=A16, v=A16, sl=A4, out=A16, lse=NULL, B=2, n_h=8, n_kv=2,
                 L_max=64, d=128, scale=0.1, ks=0.1, vs=0.1, ws=A16, wsb=1 << 30,
                 stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_fp8(a["q"], a["k"], a["v"], a["sl"], a["out"], a["lse"],
                                     a["B"], a["n_h"], a["n_kv"], a["L_max"], a["d"],
                                     a["scale"], a["ks"], a["vs"], a["ws"], a["wsb"],
                                     a["stream"])
    assert dc(k=NULL) == -1
    assert dc(d=64) == -4
    assert dc(n_h=7) == -2
    assert dc(n_h=64, n_kv=2) == -4   # group of 32 heads
    assert dc(scale=float("nan")) == -8
    assert dc(ks=0.0) == -8
    assert dc(vs=float("nan")) == -8
    assert dc(out=A8) == -6
    assert dc(B=0) == 0
    # (E4M3 caches have their own split plan in the persistent form: the
    # workspace is the one their size query returns, and a byte less is
    # refused before anything is enqueued)
    w8 = L.kvc_decode_attn_fp8_workspace_size(32, 64, 8, 32768, 128)
    assert w8 > 0
    assert dc(B=32, n_h=64, n_kv=8, L_max=32768, wsb=w8 - 1) == -5
    assert L.kvc_decode_attn_fp8_workspace_size(32, 64, 8, 32768, 64) == 0


def test_fp4_validation(L):
    def ap(**kw):
        a = dict(kc=A16, ks=A16, vc=A16, vs=A16, sl=A4, kn=A16, vn=A16, B=2, n_kv=2, L_max=8,
                 d=128, flag=NULL, stream=NULL)
        a.update(kw)
        return L.kvc_append_fp4(a["kc"], a["ks"], a["vc"], a["vs"], a["sl"], a["kn"], a["vn"],
                                a["B"], a["n_kv"], a["L_max"], a["d"], a["flag"], a["stream"])
    assert ap(ks=NULL) == -1          # scales are required
    assert ap(vc=NULL) == -1
    assert ap(vn=NULL) == -1
    assert ap(d=120) == -2            # whole 16-channel blocks
    assert ap(kc=A4) == -6            # codes: 8-byte stores
    assert ap(kn=A8) == -6
    assert ap(B=0) == 0

    def dc(**kw):
        a = dict(q=A16, kc=A16, ks=A16, vc=A16, vs=A16, sl=A4, out=A16, lse=NULL, B=2, n_h=8,
                 n_kv=2, L_max=64, d=128, scale=0.1, ws=A16, wsb=1 << 30, stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_fp4(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["sl"],
                                     a["out"], a["lse"], a["B"], a["n_h"], a["n_kv"],
                                     a["L_max"], a["d"], a["scale"], a["ws"], a["wsb"],
                                     a["stream"])
    assert dc(kc=NULL) == -1
    assert dc(vs=NULL) == -1
    assert dc(d=64) == -4
    assert dc(n_h=7) == -2
    assert dc(n_h=64, n_kv=2) == -4   # group of 32 heads
    assert dc(scale=float("nan")) == -8
    assert dc(ks=A4) == -6            # scale arrays 8-byte aligned (the header's contract)
    assert dc(out=A8) == -6
    assert dc(B=0) == 0
    # FP4 caches take their own persistent split size (8192 positions for
    # 256 units at L_max 32768: 4 splits where bf16 caches take 7), so the
    # partials are fewer; the size query is still what the call checks
    w4 = L.kvc_decode_attn_fp4_workspace_size(32, 64, 8, 32768, 128)
    assert 0 < w4 < L.kvc_decode_attn_workspace_size(32, 64, 8, 32768, 128, kvc.KVC_BF16)
    assert w4 >= 32 * 64 * 4 * 128 * 4
    big = dict(B=32, n_h=64, n_kv=8, L_max=32768)
    assert dc(wsb=w4 - 1, **big) == -5
    assert L.kvc_decode_attn_fp4_workspace_size(32, 64, 8, 32768, 64) == 0


def test_window_validation(L):
    def wd(**kw):
        a = dict(q=A16, k=A16, v=A16, sl=A4, st=NULL, W=128, out=A16, lse=NULL, B=2, n_h=8,
                 n_kv=2, L_max=4096, d=128, scale=0.1, dt=kvc.KVC_BF16, ws=A16,
                 wsb=1 << 30, stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_window(a["q"], a["k"], a["v"], a["sl"], a["st"], a["W"],
                                        a["out"], a["lse"], a["B"], a["n_h"], a["n_kv"],
                                        a["L_max"], a["d"], a["scale"], a["dt"], a["ws"],
                                        a["wsb"], a["stream"])
    assert wd(W=0) == -8
    assert wd(W=-3) == -8
    assert wd(st=ctypes.c_void_p(0x10002)) == -6
    assert wd(k=NULL) == -1
    assert wd(n_h=7) == -2
    assert wd(B=0) == 0
    full = L.kvc_decode_attn_workspace_size(32, 64, 8, 32768, 128, kvc.KVC_BF16)
    win = L.kvc_decode_attn_window_workspace_size(32, 64, 8, 32768, 128, kvc.KVC_BF16, 128)
    assert 0 <= win <= full
    assert L.kvc_decode_attn_window_workspace_size(32, 64, 8, 32768, 128, kvc.KVC_BF16, 0) == 0
    assert L.kvc_decode_attn_window_workspace_size(1, 8, 2, 64, 128, kvc.KVC_BF16, 10 ** 6) == \
        L.kvc_decode_attn_workspace_size(1, 8, 2, 64, 128, kvc.KVC_BF16)


def test_paged_validation(L):
    def dp(**kw):
        a = dict(q=A16, k=A16, v=A16, t=A4, mb=64, sl=A4, out=A16, lse=NULL, B=2, n_h=8, n_kv=2,
                 nb=100, bs=16, d=128, scale=0.1, dt=kvc.KVC_BF16, flag=NULL, ws=A16,
                 wsb=1 << 30, stream=NULL)
        a.update(kw)
        return L.kvc_decode_attn_paged(a["q"], a["k"], a["v"], a["t"], a["mb"], a["sl"], a["out"],
                                       a["lse"], a["B"], a["n_h"], a["n_kv"], a["nb"], a["bs"],
                                       a["d"], a["scale"], a["dt"], a["flag"], a["ws"], a["wsb"],
                                       a["stream"])
    assert dp(t=NULL) == -1
    assert dp(bs=12) == -2          # not a power of two
    assert dp(bs=4) == -2           # below 8
    assert dp(nb=0) == -2
    assert dp(nb=1 << 20, bs=64) == -2      # pool beyond 2^31 bytes
    assert dp(d=64) == -4
    assert dp(dt=kvc.KVC_F32) == -4
    assert dp(t=ctypes.c_void_p(0x10002)) == -6
    assert dp(B=0) == 0

    def ap(**kw):
        a = dict(k=A16, v=A16, t=A4, mb=64, sl=A4, kn=A16, vn=A16, B=2, n_kv=2, nb=100, bs=16,
                 d=128, dt=kvc.KVC_BF16, flag=NULL, stream=NULL)
        a.update(kw)
        return L.kvc_append_paged(a["k"], a["v"], a["t"], a["mb"], a["sl"], a["kn"], a["vn"],
                                  a["B"], a["n_kv"], a["nb"], a["bs"], a["d"], a["dt"], a["flag"],
                                  a["stream"])
    assert ap(v=NULL) == -1
    assert ap(d=4) == -2            # 8 bytes per row: not whole 16-byte pieces
    assert ap(bs=24) == -2
    assert ap(dt=3) == -3
    assert ap(k=A8) == -6
    assert ap(B=0) == 0
    assert L.kvc_decode_attn_paged_workspace_size(32, 64, 8, 2048, 16, 128, kvc.KVC_BF16) == \
        L.kvc_decode_attn_workspace_size(32, 64, 8, 32768, 128, kvc.KVC_BF16)
    assert L.kvc_decode_attn_paged_workspace_size(32, 64, 8, 2048, 12, 128, kvc.KVC_BF16) == 0


def test_select_validation(L):
    def sel(**kw):
        a = dict(s=A4, sl=A4, pool=NULL, P=0, pb=8, out=A4, B=2, R=8, L=131072, K=2048,
                 ws=NULL, wn=0, stream=NULL)
        a.update(kw)
        return L.kvc_topk_select(a["s"], a["sl"], a["pool"], a["P"], a["pb"], a["out"], a["B"],
                                 a["R"], a["L"], a["K"], a["ws"], a["wn"], a["stream"])
    need = L.kvc_topk_select_workspace_size(2, 8, 131072, 2048)
    assert need > 0
    assert sel(ws=A16, wn=need - 1) == -5                  # workspace too small
    assert sel(ws=ctypes.c_void_p(0x10010), wn=need) == -6  # workspace not 256-byte aligned
    # the one-workgroup form needs none: long rows, a device-filling row count
    assert L.kvc_topk_select_workspace_size(2, 8, (1 << 18) + 1, 2048) == 0
    assert L.kvc_topk_select_workspace_size(64, 8, 131072, 2048) == 0
    assert L.kvc_topk_select_workspace_size(4, 4, 16384, 100) == 0    # one step per row
    assert L.kvc_topk_select_workspace_size(0, 8, 131072, 2048) == 0
    assert sel(s=NULL) == -1
    assert sel(out=NULL) == -1
    assert sel(K=0) == -2
    assert sel(R=0) == -2
    assert sel(pool=A4, P=0) == -2
    assert sel(pool=A4, P=16, pb=0) == -2
    assert sel(pool=A4, P=16, pb=1, L=1 << 20) == -4     # pool bitmap beyond LDS
    assert sel(L=1 << 29) == -4                          # rows beyond 32-bit byte offsets
    assert sel(L=(1 << 29) - 1, B=0) == 0
    assert sel(s=ctypes.c_void_p(0x10002)) == -6
    assert sel(B=0) == 0


def test_header_enum_and_signatures():
    """The element-type enum's values are the binding's codes, and the
    latent workspace query takes the five shape arguments only."""
    text = open(HEADER).read()
    assert re.search(r"typedef enum kvc_dtype\s*(:\s*int\s*)?\{\s*KVC_F32 = 0, KVC_BF16 = 1\s*\}", text)
    assert (kvc.KVC_F32, kvc.KVC_BF16) == (0, 1)
    decl = re.search(r"size_t kvc_decode_attn_mla_workspace_size\(([^)]*)\)", text).group(1)
    assert [a.split()[-1] for a in decl.split(",")] == ["B", "n_h", "L_max", "d_c", "d_r"]
    # every call that takes an element type declares it as kvc_dtype
    flat = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    assert "int dtype" not in flat


def test_binding_requires_scale():
    """The score scale is always the caller's: the binding computes no
    default (it fails before touching any device pointer)."""
    import torch
    q = torch.zeros(1, 8, 128)
    kc = torch.zeros(1, 2, 16, 128)
    sl = torch.zeros(1, dtype=torch.int32)
    for call in (lambda: kvc.kvc_decode_attn(q, kc, kc, sl, q),
                 lambda: kvc.kvc_append_decode_attn(q, kc, kc, sl, q, q, q),
                 lambda: kvc.kvc_decode_attn_window(q, kc, kc, sl, q, 4),
                 lambda: kvc.kvc_decode_attn_topk(q, kc, kc, sl, sl.view(1, 1, 1), q)):
        with pytest.raises(TypeError, match="scale is required"):
            call()


def test_noalloc_limits_and_validation(L):
    """The no-allocation fused call checks arguments like the workspace
    variant and rejects calls that do not fit the library's scratch
    (KVC_ERR_SCRATCH), all before any HIP call."""
    def na(**kw):
        a = dict(q=A16, k=A16, v=A16, sl=A4, kn=A16, vn=A16, out=A16, lse=NULL, B=2, n_h=8,
                 n_kv=2, L_max=64, d=128, scale=0.1, dt=kvc.KVC_BF16, flag=NULL, stream=NULL)
        a.update(kw)
        return L.kvc_append_decode_attn_noalloc(a["q"], a["k"], a["v"], a["sl"], a["kn"], a["vn"],
                                                a["out"], a["lse"], a["B"], a["n_h"], a["n_kv"],
                                                a["L_max"], a["d"], a["scale"], a["dt"], a["flag"],
                                                a["stream"])
    assert na(kn=NULL) == -1
    assert na(n_h=7) == -2
    assert na(dt=7) == -3
    assert na(d=96) == -4
    assert na(q=A8) == -6
    assert na(scale=float("nan")) == -8
    assert na(B=0) == 0
    # more (sequence, KV head) units than counter slots
    assert na(B=2049, n_h=64, n_kv=8, L_max=4096) == -9
    # split partials beyond the scratch: 64 sequences x 128 fp32 heads at
    # 32768 (eight splits of float32 partials: 33.5 MB)
    assert na(B=64, n_h=128, n_kv=8, L_max=32768, dt=kvc.KVC_F32) == -9
    # the benchmark's GQA layer shape fits (its own workspace is below 32 MiB)
    need = L.kvc_append_decode_attn_workspace_size(32, 64, 8, 32807, 128, kvc.KVC_BF16)
    assert 0 < need < 32 << 20
