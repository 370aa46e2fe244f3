#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C2] [--others C3,C4,C5]

A step is one decode step of every layer of the workload: per layer, the new
token's key/value are appended (kvc_append) and the token attends over the
cache (kvc_decode_attn / _mla / _topk).  The step is captured once in a HIP
graph and replayed; W untimed replays, then K replays between HIP events.
Each replay appends one more token, so the attended length grows by one per
step (as in real decoding).

The headline (`value`) is the Llama-2-7B-like MHA workload (32 layers,
B = 1, 32 heads, d = 128, 4096 cached + 1 appended, bf16): achieved HBM
GB/s over the algorithmic bytes of a step (cache read + q read + out write +
new k/v read and written + lengths).  `roofline` is the dense decode kernel
alone, timed with HIP events over back-to-back launches of one step's
layers.  `also` carries the same figures for the GQA, MLA and top-k
workloads, for the GQA workload over FP8 E4M3 caches (C3F8) and over FP4
caches (C3F4: E2M1 codes, one E4M3 scale per 16 channels), for the GQA
workload attending a sliding window of its newest 128 positions (C3W128) and
over a paged cache of 16-position blocks (C3P16), and for the top-k
selection that feeds the sparse workload (C5S).  `cpu_baseline` is the fp64 oracle on the same inputs (copied to
the host), on a time-bounded sample of layer-steps.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import kvc_synth as syn  # noqa: E402

PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
CPU_BUDGET_S = 12.0        # oracle sample budget


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C2", choices=["C2", "C3", "C4", "C5", "C3F8", "C3F4", "C3W128", "C3P16", "C5S"])
    ap.add_argument("--others", default="C3,C4,C5,C3F8,C3F4,C3W128,C3P16,C5S",
                    help="also-measured workloads (comma list; 'none' for none)")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


# ---------------------------------------------------------------- workloads
class DenseWorkload:
    """MHA/GQA layers over [B, n_kv, L_max, d] caches (C2, C3).  Each layer
    runs the fused append-and-attend call (one kernel per layer-step)."""

    kernel = "dense_mfma_kernel<false, true, false, false, false> (append + attend)"
    kernel_appends = True

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(max(cfg.L_max, self.pre.max() + 1) + slack)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        dt = torch.bfloat16
        self.K, self.V = [], []
        for i in range(self.nbuf):
            self.K.append(syn.device_normal_(torch.empty(B, n_kv, self.L_max, d, dtype=dt, device="cuda"),
                                             syn.device_seed(cfg.cfg_id, i, "k")))
            self.V.append(syn.device_normal_(torch.empty(B, n_kv, self.L_max, d, dtype=dt, device="cuda"),
                                             syn.device_seed(cfg.cfg_id, i, "v")))
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.q = [mk((B, n_h, d), l, "q") for l in range(self.layers)]
        self.kn = [mk((B, n_kv, d), l, "k_new") for l in range(self.layers)]
        self.vn = [mk((B, n_kv, d), l, "v_new") for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, d, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(
            B, n_h, n_kv, self.L_max, d, kvc.KVC_BF16))
        self.ws_plain = kvc.workspace(kvc.kvc_decode_attn_workspace_size(
            B, n_h, n_kv, self.L_max, d, kvc.KVC_BF16))

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append_decode_attn(self.q[l], self.K[b], self.V[b], self.sl[l],
                                            self.kn[l], self.vn[l], self.out[l], None,
                                            scale=self.cfg.scale, workspace=self.ws)

    kernel_only = step

    def decode_only(self):
        """Attention without the append (no state change)."""
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn(self.q[l], self.K[b], self.V[b], self.sl[l], self.out[l],
                                     None, scale=self.cfg.scale, workspace=self.ws_plain)

    def lens_after(self, steps_done):
        """Attended lengths during the step that follows `steps_done` steps."""
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * c.d * 2 * n.sum() + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def step_bytes(self, steps_done):
        c = self.cfg
        n = self.lens_after(steps_done)
        per_layer = self.kernel_bytes(n) + 4 * c.B * c.n_kv * c.d * 2 + 4 * c.B
        return per_layer * self.layers

    def launch_bytes(self, steps_done):
        """Algorithmic bytes of one fused launch (append included)."""
        return self.step_bytes(steps_done) // self.layers

    def describe(self):
        c = self.cfg
        lens = ("%d cached + 1 appended" % c.pre_len) if c.pre_len is not None else \
            "seq_lens ~ U[%d, %d] (post-append)" % c.len_range
        return (f"{c.name}: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} bf16, {lens}, "
                f"{self.layers} layers ({self.nbuf} distinct cache buffers)")

    # oracle on the host, one layer-step at a time
    def cpu_sample(self, budget_s, oracle):
        torch, c = self.torch, self.cfg
        done_bytes, secs, layers = 0, 0.0, 0
        for l in range(self.layers):
            b = l % self.nbuf
            h = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
            kc, vc = h(self.K[b]), h(self.V[b])
            q, kn, vn = h(self.q[l]), h(self.kn[l]), h(self.vn[l])
            sl = self.pre.astype(np.int32).copy()
            t0 = time.perf_counter()
            oracle.append(kc, vc, sl, kn, vn)
            oracle.decode(q, kc, vc, sl, c.scale)
            secs += time.perf_counter() - t0
            layers += 1
            done_bytes += self.step_bytes(0) // self.layers
            del kc, vc
            if secs >= budget_s:
                break
        return done_bytes, secs, f"{layers} of {self.layers} layer-steps of the same workload"


class MlaWorkload:
    """Latent-cache layers, [B, L_max, 576] per layer buffer (C4)."""

    kernel = "mla_kernel + mla_merge_kernel"
    kernel_appends = False

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, D = cfg.B, cfg.n_h, cfg.d_c + cfg.d_r
        self.pre = np.full(B, cfg.pre_len, dtype=np.int64)
        self.L_max = int(cfg.L_max + slack)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        dt = torch.bfloat16
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.C = [mk((B, self.L_max, D), i, "ckv") for i in range(self.nbuf)]
        self.q = [mk((B, n_h, D), l, "q") for l in range(self.layers)]
        self.cn = [mk((B, D), l, "ckv_new") for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, cfg.d_c, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_decode_attn_mla_workspace_size(
            B, n_h, self.L_max, cfg.d_c, cfg.d_r))

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append(self.C[b], None, self.sl[l], self.cn[l], None)
            self.kvc.kvc_decode_attn_mla(self.q[l], self.C[b], self.sl[l], self.out[l], None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_mla(self.q[l], self.C[b], self.sl[l], self.out[l], None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def kernel_only(self):
        self.decode_only()

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def kernel_bytes(self, n):
        c = self.cfg
        D = c.d_c + c.d_r
        return int(D * 2 * n.sum() + c.B * c.n_h * (D * 2 + c.d_c * 2) + 4 * c.B)

    def step_bytes(self, steps_done):
        c = self.cfg
        per_layer = self.kernel_bytes(self.lens_after(steps_done)) + 2 * c.B * (c.d_c + c.d_r) * 2 + 4 * c.B
        return per_layer * self.layers

    def describe(self):
        c = self.cfg
        return (f"{c.name}: B={c.B} n_h={c.n_h} latent {c.d_c} + rope {c.d_r} bf16, "
                f"{c.pre_len} cached + 1 appended, scale 1/24, {self.layers} layers")


class TopKWorkload:
    """Top-k sparse GQA over [B, n_kv, L_max, d] caches (C5)."""

    kernel = "dense_mfma_kernel<true, false, false, false, false> (top-k)"
    kernel_appends = False

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.pre = np.full(B, cfg.pre_len, dtype=np.int64)
        self.L_max = int(cfg.L_max + slack)
        self.layers = cfg.index_sets
        self.nbuf = cfg.distinct_buffers
        dt = torch.bfloat16
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.K = [mk((B, n_kv, self.L_max, d), i, "k") for i in range(self.nbuf)]
        self.V = [mk((B, n_kv, self.L_max, d), i, "v") for i in range(self.nbuf)]
        self.q = [mk((B, n_h, d), l, "q") for l in range(self.layers)]
        self.kn = [mk((B, n_kv, d), l, "k_new") for l in range(self.layers)]
        self.vn = [mk((B, n_kv, d), l, "v_new") for l in range(self.layers)]
        self.idx = [torch.from_numpy(syn.topk_indices(cfg.cfg_id, 0, B, n_kv, cfg.K, cfg.pre_len,
                                                      index_set=l)).cuda()
                    for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, d, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_decode_attn_topk_workspace_size(B, n_h, n_kv, cfg.K, d, kvc.KVC_BF16))

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append(self.K[b], self.V[b], self.sl[l], self.kn[l], self.vn[l])
            self.kvc.kvc_decode_attn_topk(self.q[l], self.K[b], self.V[b], self.sl[l], self.idx[l],
                                          self.out[l], None, scale=self.cfg.scale, workspace=self.ws)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_topk(self.q[l], self.K[b], self.V[b], self.sl[l], self.idx[l],
                                          self.out[l], None, scale=self.cfg.scale, workspace=self.ws)

    def kernel_bytes(self, n=None):
        c = self.cfg
        return int(c.B * c.n_kv * c.K * (2 * c.d * 2 + 4) + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def kernel_only(self):
        self.decode_only()

    def launch_bytes(self, steps_done):
        return self.kernel_bytes()

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def step_bytes(self, steps_done):
        c = self.cfg
        return (self.kernel_bytes() + 4 * c.B * c.n_kv * c.d * 2 + 4 * c.B) * self.layers

    def describe(self):
        c = self.cfg
        return (f"{c.name}: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} bf16, K={c.K} sorted distinct "
                f"indices of L={c.pre_len}, {self.layers} index sets over {self.nbuf} cache buffers")


class Fp8DenseWorkload:
    """The GQA layers of C3 over FP8 E4M3 caches (uint8 [B, n_kv, L_max, d],
    one float32 scale per tensor).  A layer-step is kvc_append_fp8 then
    kvc_decode_attn_fp8."""

    kernel = "dense_mfma_kernel<false, false, true, false, false> (fp8 E4M3 cache)"
    kernel_appends = False
    K_SCALE = 1.0 / 64      # N(0,1) / (1/64) stays within +-448
    V_SCALE = 1.0 / 64

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(max(cfg.L_max, self.pre.max() + 1) + slack)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        dt = torch.bfloat16
        codes = lambda i, t, sc: self._fp8_fill(
            torch.empty(B, n_kv, self.L_max, d, dtype=torch.uint8, device="cuda"),
            syn.device_seed(cfg.cfg_id, i, t), sc)
        self.K = [codes(i, "k", self.K_SCALE) for i in range(self.nbuf)]
        self.V = [codes(i, "v", self.V_SCALE) for i in range(self.nbuf)]
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.q = [mk((B, n_h, d), l, "q") for l in range(self.layers)]
        self.kn = [mk((B, n_kv, d), l, "k_new") for l in range(self.layers)]
        self.vn = [mk((B, n_kv, d), l, "v_new") for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, d, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_decode_attn_fp8_workspace_size(B, n_h, n_kv, self.L_max, d))

    def _fp8_fill(self, t, seed, scale, chunk=1 << 26):
        """Synthetic cache contents: seeded N(0,1) / scale as E4M3 codes
        (torch's float8_e4m3fn cast lays the data out; input set-up only)."""
        torch = self.torch
        flat = t.view(-1)
        g = torch.Generator(device=t.device)
        g.manual_seed(seed)
        for s in range(0, flat.numel(), chunk):
            e = min(flat.numel(), s + chunk)
            x = torch.randn(e - s, generator=g, device=t.device, dtype=torch.float32) / scale
            flat[s:e].copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
            del x
        return t

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append_fp8(self.K[b], self.V[b], self.sl[l], self.kn[l], self.vn[l],
                                    self.K_SCALE, self.V_SCALE)
            self.kvc.kvc_decode_attn_fp8(self.q[l], self.K[b], self.V[b], self.sl[l], self.out[l],
                                         self.K_SCALE, self.V_SCALE, None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_fp8(self.q[l], self.K[b], self.V[b], self.sl[l], self.out[l],
                                         self.K_SCALE, self.V_SCALE, None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def kernel_only(self):
        self.decode_only()

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * c.d * 1 * n.sum() + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def step_bytes(self, steps_done):
        c = self.cfg
        append = 2 * c.B * c.n_kv * c.d * (2 + 1) + 8 * c.B
        return (self.kernel_bytes(self.lens_after(steps_done)) + append) * self.layers

    def describe(self):
        c = self.cfg
        return (f"{c.name} over FP8 E4M3 caches: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d}, "
                f"seq_lens ~ U[{c.len_range[0]}, {c.len_range[1]}] (post-append), "
                f"{self.layers} layers ({self.nbuf} distinct cache buffers), bf16 q/out")


class Fp4DenseWorkload:
    """The GQA layers of C3 over FP4 block-scaled caches: E2M1 codes
    (uint8 [B, n_kv, L_max, d/2]) and one E4M3 scale per 16 channels (uint8
    [B, n_kv, L_max, d/16]).  A layer-step is kvc_append_fp4 then
    kvc_decode_attn_fp4."""

    kernel = "dense_mfma_kernel<false, false, false, false, true> (fp4 E2M1 cache)"
    kernel_appends = False

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(max(cfg.L_max, self.pre.max() + 1) + slack)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        dt = torch.bfloat16
        fill = lambda shape, i, t, lo, hi: self._bytes(
            torch.empty(*shape, dtype=torch.uint8, device="cuda"), syn.device_seed(cfg.cfg_id, i, t),
            lo, hi)
        cshape, sshape = (B, n_kv, self.L_max, d // 2), (B, n_kv, self.L_max, d // 16)
        # any byte is a pair of E2M1 codes; scale codes 0x20..0x2F are E4M3
        # 0.125 .. 0.47, so stored values have about unit rms, like N(0,1) data
        self.KC = [fill(cshape, i, "k", 0, 256) for i in range(self.nbuf)]
        self.VC = [fill(cshape, i, "v", 0, 256) for i in range(self.nbuf)]
        self.KS = [fill(sshape, i, "k_scales", 0x20, 0x30) for i in range(self.nbuf)]
        self.VS = [fill(sshape, i, "v_scales", 0x20, 0x30) for i in range(self.nbuf)]
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.q = [mk((B, n_h, d), l, "q") for l in range(self.layers)]
        self.kn = [mk((B, n_kv, d), l, "k_new") for l in range(self.layers)]
        self.vn = [mk((B, n_kv, d), l, "v_new") for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, d, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_decode_attn_fp4_workspace_size(B, n_h, n_kv, self.L_max, d))

    def _bytes(self, t, seed, lo, hi):
        """Seeded uniform bytes in [lo, hi) (input set-up only)."""
        g = self.torch.Generator(device=t.device)
        g.manual_seed(seed)
        t.copy_(self.torch.randint(lo, hi, t.shape, generator=g, device=t.device,
                                   dtype=self.torch.int32).to(self.torch.uint8))
        return t

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append_fp4(self.KC[b], self.KS[b], self.VC[b], self.VS[b], self.sl[l],
                                    self.kn[l], self.vn[l])
            self.kvc.kvc_decode_attn_fp4(self.q[l], self.KC[b], self.KS[b], self.VC[b],
                                         self.VS[b], self.sl[l], self.out[l], None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_fp4(self.q[l], self.KC[b], self.KS[b], self.VC[b],
                                         self.VS[b], self.sl[l], self.out[l], None,
                                         scale=self.cfg.scale, workspace=self.ws)

    def kernel_only(self):
        self.decode_only()

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def row_bytes(self):
        return self.cfg.d // 2 + self.cfg.d // 16          # codes + scales per position

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * self.row_bytes() * n.sum() + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def step_bytes(self, steps_done):
        c = self.cfg
        append = 2 * c.B * c.n_kv * (c.d * 2 + self.row_bytes()) + 8 * c.B
        return (self.kernel_bytes(self.lens_after(steps_done)) + append) * self.layers

    def describe(self):
        c = self.cfg
        return (f"{c.name} over FP4 caches (E2M1 + E4M3 scale per 16 channels): B={c.B} "
                f"n_h={c.n_h} n_kv={c.n_kv} d={c.d}, seq_lens ~ U[{c.len_range[0]}, "
                f"{c.len_range[1]}] (post-append), {self.layers} layers ({self.nbuf} distinct "
                f"cache buffers), bf16 q/out")


class WindowWorkload(DenseWorkload):
    """The GQA layers of C3 attending only the newest WINDOW positions (the
    DeepSeek article's n_win = 128).  A layer-step is kvc_append then
    kvc_decode_attn_window."""

    kernel = "dense_mfma_kernel<false, false, false, false, false> (window 128)"
    kernel_appends = False
    WINDOW = 128

    def __init__(self, cfg, slack, torch, kvc):
        super().__init__(cfg, slack, torch, kvc)
        self.ws_win = kvc.workspace(kvc.kvc_decode_attn_window_workspace_size(
            cfg.B, cfg.n_h, cfg.n_kv, self.L_max, cfg.d, kvc.KVC_BF16, self.WINDOW))

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append(self.K[b], self.V[b], self.sl[l], self.kn[l], self.vn[l])
            self.kvc.kvc_decode_attn_window(self.q[l], self.K[b], self.V[b], self.sl[l],
                                            self.out[l], self.WINDOW, scale=self.cfg.scale,
                                            workspace=self.ws_win)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_window(self.q[l], self.K[b], self.V[b], self.sl[l],
                                            self.out[l], self.WINDOW, scale=self.cfg.scale,
                                            workspace=self.ws_win)

    def kernel_only(self):
        self.decode_only()

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * c.d * 2 * np.minimum(n, self.WINDOW).sum()
                   + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def step_bytes(self, steps_done):
        c = self.cfg
        per_layer = self.kernel_bytes(self.lens_after(steps_done)) + 4 * c.B * c.n_kv * c.d * 2 + 8 * c.B
        return per_layer * self.layers

    def describe(self):
        return super().describe().replace(", seq_lens", f", window {self.WINDOW} of seq_lens")


class PagedWorkload:
    """The GQA layers of C3 over a paged cache: pools of 16-position blocks
    sized to the sequences' lengths, blocks in shuffled physical order, one
    block table per layer buffer.  A layer-step is kvc_append_paged then
    kvc_decode_attn_paged."""

    kernel = "dense_mfma_kernel<false, false, false, true, false> (paged, 16-position blocks)"
    kernel_appends = False
    BETA = 16

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(self.pre.max() + 1 + slack)
        self.max_blocks = -(-self.L_max // self.BETA)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        need = [-(-int(n + 1 + slack) // self.BETA) for n in self.pre]
        self.num_blocks = int(sum(need))
        order = np.random.default_rng(1000 + cfg.cfg_id).permutation(self.num_blocks)
        table = np.full((B, self.max_blocks), 1 << 30, dtype=np.int32)
        at = 0
        for b in range(B):
            table[b, :need[b]] = order[at:at + need[b]]
            at += need[b]
        self.table = torch.from_numpy(table).cuda()
        dt = torch.bfloat16
        pool = lambda i, t: syn.device_normal_(
            torch.empty(self.num_blocks, n_kv, self.BETA, d, dtype=dt, device="cuda"),
            syn.device_seed(cfg.cfg_id, i, t))
        self.K = [pool(i, "k") for i in range(self.nbuf)]
        self.V = [pool(i, "v") for i in range(self.nbuf)]
        mk = lambda shape, l, t: syn.device_normal_(torch.empty(*shape, dtype=dt, device="cuda"),
                                                    syn.device_seed(cfg.cfg_id, l, t))
        self.q = [mk((B, n_h, d), l, "q") for l in range(self.layers)]
        self.kn = [mk((B, n_kv, d), l, "k_new") for l in range(self.layers)]
        self.vn = [mk((B, n_kv, d), l, "v_new") for l in range(self.layers)]
        self.out = [torch.empty(B, n_h, d, dtype=dt, device="cuda") for _ in range(self.layers)]
        pre_t = torch.tensor(self.pre, dtype=torch.int32)
        self.sl = [pre_t.clone().cuda() for _ in range(self.layers)]
        self.ws = kvc.workspace(kvc.kvc_decode_attn_paged_workspace_size(
            B, n_h, n_kv, self.max_blocks, self.BETA, d, kvc.KVC_BF16))

    def step(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_append_paged(self.K[b], self.V[b], self.table, self.sl[l], self.kn[l],
                                      self.vn[l])
            self.kvc.kvc_decode_attn_paged(self.q[l], self.K[b], self.V[b], self.table, self.sl[l],
                                           self.out[l], scale=self.cfg.scale, workspace=self.ws)

    def decode_only(self):
        for l in range(self.layers):
            b = l % self.nbuf
            self.kvc.kvc_decode_attn_paged(self.q[l], self.K[b], self.V[b], self.table, self.sl[l],
                                           self.out[l], scale=self.cfg.scale, workspace=self.ws)

    def kernel_only(self):
        self.decode_only()

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * c.d * 2 * n.sum() + 4 * (-(-n // self.BETA)).sum()
                   + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def step_bytes(self, steps_done):
        c = self.cfg
        per_layer = self.kernel_bytes(self.lens_after(steps_done)) + 4 * c.B * c.n_kv * c.d * 2 + 12 * c.B
        return per_layer * self.layers

    def describe(self):
        c = self.cfg
        return (f"{c.name} over a paged cache: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} bf16, "
                f"{self.BETA}-position blocks ({self.num_blocks} in shuffled order), seq_lens ~ "
                f"U[{c.len_range[0]}, {c.len_range[1]}] (post-append), {self.layers} layers "
                f"({self.nbuf} distinct pools)")


class SelectWorkload:
    """Top-k selection for the sparse workload's shape: per sequence and KV
    head, the 2048 highest of 131072 indexer scores (float32, seeded N(0,1)),
    32 index sets over 16 distinct score buffers (512 MB)."""

    kernel = "topk_select_kernel"
    kernel_appends = False
    NBUF = 16

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, R, L = cfg.B, cfg.n_kv, cfg.pre_len
        self.layers = cfg.index_sets
        self.S = []
        for i in range(self.NBUF):
            g = torch.Generator(device="cuda")
            g.manual_seed(syn.device_seed(cfg.cfg_id, 100 + i, "idx"))
            self.S.append(torch.randn(B, R, L, generator=g, device="cuda", dtype=torch.float32))
        self.lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        self.out = [torch.empty(B, R, cfg.K, dtype=torch.int32, device="cuda")
                    for _ in range(self.layers)]

    def step(self):
        for l in range(self.layers):
            self.kvc.kvc_topk_select(self.S[l % self.NBUF], self.lens, self.out[l])

    decode_only = step
    kernel_only = step

    def lens_after(self, steps_done):
        return np.full(self.cfg.B, self.cfg.pre_len)

    def kernel_bytes(self, n=None):
        c = self.cfg
        return int(c.B * c.n_kv * (c.pre_len * 4 + c.K * 4) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes()

    def step_bytes(self, steps_done):
        return self.kernel_bytes() * self.layers

    def describe(self):
        c = self.cfg
        return (f"top-k selection: B={c.B} x {c.n_kv} rows, K={c.K} of {c.pre_len} float32 scores, "
                f"{self.layers} index sets over {self.NBUF} score buffers")


WORKLOADS = {"C2": (syn.C2, DenseWorkload), "C3": (syn.C3, DenseWorkload),
             "C4": (syn.C4, MlaWorkload), "C5": (syn.C5, TopKWorkload),
             "C3F8": (syn.C3, Fp8DenseWorkload), "C3W128": (syn.C3, WindowWorkload),
             "C3P16": (syn.C3, PagedWorkload), "C3F4": (syn.C3, Fp4DenseWorkload), "C5S": (syn.C5, SelectWorkload)}


# ---------------------------------------------------------------- timing
def time_graph(torch, fn, reps):
    """Capture fn once, replay `reps` times between HIP events on the
    replay stream; returns (ms total, graph)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def measure(name, args, torch, kvc):
    cfg, cls = WORKLOADS[name]
    slack = args.warmup + args.steps + args.kernel_reps + 4
    wl = cls(cfg, slack, torch, kvc)
    wl.decode_only()            # first launches outside capture (no state change)
    torch.cuda.synchronize()

    g = time_graph(torch, wl.step, 1)
    done = 0
    for _ in range(args.warmup):
        g.replay()
        done += 1
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    bytes_total = sum(wl.step_bytes(done + i) for i in range(args.steps))
    done += args.steps
    ms_step = ms / args.steps
    gbs = bytes_total / (ms * 1e-3) / 1e9

    # the dominant kernel alone: one launch per layer, back to back
    gk = time_graph(torch, wl.kernel_only, 1)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for _ in range(args.kernel_reps):
        gk.replay()
    k1.record()
    torch.cuda.synchronize()
    k_us = k0.elapsed_time(k1) * 1e3 / (args.kernel_reps * wl.layers)
    if wl.kernel_appends:
        k_bytes = sum(wl.launch_bytes(done + r) for r in range(args.kernel_reps)) // args.kernel_reps
        done += args.kernel_reps
    else:
        k_bytes = wl.launch_bytes(done)
    res = dict(
        workload=wl.describe(), layers=wl.layers, ms_per_step=ms_step,
        us_per_layer_step=ms_step * 1e3 / wl.layers, gbs=gbs, pct_of_peak=100 * gbs / PEAK_GBS,
        kernel=wl.kernel, kernel_us=k_us, kernel_bytes=k_bytes,
        kernel_gbs=k_bytes / (k_us * 1e-6) / 1e9,
        bytes_per_step=bytes_total / args.steps)
    return wl, res


def calibrate_copy(torch, kvc, nbytes=1 << 30):
    """One plain copy of known size: hardware byte counters (FETCH_SIZE,
    WRITE_SIZE) read for this dispatch scale the attention kernels' counts."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    kvc.kvc_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def read_ceiling(torch, kvc, nbytes=4 << 30, reps=10):
    buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    buf.fill_(1.0)
    sink = torch.empty(kvc.kvc_stream_read_sink_floats(nbytes), dtype=torch.float32, device="cuda")
    kvc.kvc_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kvc.kvc_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return gbs


def measured_traffic(name):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter runs (profiles/traffic.json), or None if that kernel's
    sources changed since those counters were taken."""
    try:
        from kv_cache_decode_kvc_amd.profile_summary import source_hash
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f).get(name)
        if not rec or rec["source_sha256"] != source_hash(name):
            return None
        return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)
    import torch

    import kv_cache_decode_kvc_amd as kvc
    kvc.lib()
    torch.cuda.set_device(0)

    wl, head = measure(args.config, args, torch, kvc)
    line = {
        "metric": "decode-attention achieved HBM GB/s (% of peak) and us/layer-step",
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16 round-to-nearest-even)",
        "config": {"workload": head["workload"], "layers_per_step": head["layers"],
                   "pct_of_peak": round(head["pct_of_peak"], 2),
                   "us_per_layer_step": round(head["us_per_layer_step"], 3)},
        "roofline": {"bound": "hbm", "achieved": round(head["kernel_gbs"], 2),
                     "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["kernel_gbs"] / PEAK_GBS, 4),
                     "traffic": measured_traffic(args.config),
                     "kernel": head["kernel"], "kernel_us": round(head["kernel_us"], 3),
                     "algorithmic_bytes_per_launch": head["kernel_bytes"]},
    }

    if not args.no_cpu:
        import oracle
        nbytes, secs, sample = wl.cpu_sample(CPU_BUDGET_S, oracle)
        line["cpu_baseline"] = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s",
                                "cores": blas_threads(), "kind": "oracle",
                                "sample": f"{sample}, {secs:.1f} s"}
    del wl
    torch.cuda.empty_cache()

    calibrate_copy(torch, kvc)
    line["read_ceiling_gbs"] = round(read_ceiling(torch, kvc), 1)
    also = {}
    for name in [x for x in args.others.split(",") if x in WORKLOADS and x != args.config]:
        w, r = measure(name, args, torch, kvc)
        also[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
        also[name]["traffic"] = measured_traffic(name)
        del w
        torch.cuda.empty_cache()
    if also:
        line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
