#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config C3] [--others C4,C5,...]

A step is one decode step of every layer of the workload: per layer, the new
token's key/value are appended and the token attends over the cache.  The
step is captured once in a HIP graph and replayed; W untimed replays, then K
replays between HIP events.  Each replay appends one more token, so the
attended lengths grow by one per step (as in real decoding).

The headline (`value`) is the Llama-3.1-70B-like GQA workload (80 layers,
B = 32, 64 query heads over 8 KV heads, d = 128, bf16, lengths drawn from
[1024, 32768]): achieved HBM GB/s over the algorithmic bytes of a step
(cache read + q read + out write + new k/v read and written + lengths).
Every workload line carries:

  roofline      the dominant kernel alone (one launch per layer, back to
                back in a graph, HIP events on the replay stream): algorithmic
                bytes per launch / average launch time against the 8 TB/s
                HBM peak, plus the counter-measured HBM bytes per launch
                (`traffic`, from the committed rocprofv3 runs in profiles/,
                null once the kernel's sources have changed);
  cpu_baseline  the fp64 oracle on a bounded sample of (sequence, KV head)
                units of the same layer-step, on host copies of their inputs.

`also` holds the other workloads: the latent cache (C4), top-k (C5), the
tiny float32 case (C1, reported in us per layer-step: launch-bound), the
Llama-2-7B-like MHA layer (C2), the GQA layers over FP8 and FP4 caches
(C3F8, C3F4), over a paged cache of 16-position blocks (C3P16), attending a
sliding window of the newest 128 positions (C3W128), and the top-k selection
feeding the sparse decode (C5S).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import kvc_synth as syn  # noqa: E402

PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
HEAD_CPU_BUDGET_S = 12.0   # oracle sample budget, headline workload
CPU_BUDGET_S = 3.0         # oracle sample budget, every other workload
DEFAULT_STEPS, DEFAULT_WARMUP, DEFAULT_KERNEL_REPS = 20, 5, 10
ALL = ["C3", "C4", "C5", "C1", "C2", "C3F8", "C3F4", "C3P16", "C3W128", "C5S"]


def reservation_slack(warmup=DEFAULT_WARMUP, steps=DEFAULT_STEPS, kernel_reps=DEFAULT_KERNEL_REPS):
    """Positions each cache reserves beyond its starting lengths: every
    replay (untimed and timed steps, untimed and timed kernel-only) appends
    one token."""
    return 2 * warmup + steps + kernel_reps + 4


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=DEFAULT_STEPS)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP)
    ap.add_argument("--config", default="C3", choices=ALL)
    ap.add_argument("--others", default=",".join(c for c in ALL if c != "C3"),
                    help="also-measured workloads (comma list; 'none' for none)")
    ap.add_argument("--kernel-reps", type=int, default=DEFAULT_KERNEL_REPS)
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


def to_host(t):
    """Device tensor -> numpy storage array (bf16 as uint16 bits)."""
    import torch
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# ---------------------------------------------------------------- workloads
class Workload:
    """Shared parts: the oracle sample over (sequence, KV head) units."""

    kernel_appends = False
    unit_name = "(sequence, KV head) units"

    def units(self):
        return [(b, j) for b in range(self.cfg.B) for j in range(self.cfg.n_kv)]

    def cpu_sample(self, budget_s, oracle):
        """Run the oracle on units of the first layer-step (seeded order)
        until `budget_s` seconds of oracle time; host copies are made
        outside the timed region.  Returns (bytes, seconds, description)."""
        units = self.units()
        order = np.random.default_rng(7).permutation(len(units))
        done, secs, n = 0, 0.0, 0
        for k in order:
            b, j = units[k]
            nbytes, dt = self.cpu_unit(b, j, oracle)
            done += nbytes
            secs += dt
            n += 1
            if secs >= budget_s:
                break
        return done, secs, f"{n} of {len(units)} {self.unit_name} of one layer-step"


class DenseWorkload(Workload):
    """MHA/GQA layers over [B, n_kv, L_max, d] caches (C1, C2, C3).  Each
    layer runs the fused append-and-attend call (one kernel per layer-step)."""

    kernel_appends = True

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.be = 2 if cfg.dtype == syn.BF16 else 4
        dt = torch.bfloat16 if cfg.dtype == syn.BF16 else torch.float32
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(max(cfg.L_max, self.pre.max() + 1) + slack)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
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
        self.pre_l = [self.pre.copy() for _ in range(self.layers)]
        self.sl = [torch.tensor(p, dtype=torch.int32).cuda() for p in self.pre_l]
        code = kvc.KVC_BF16 if cfg.dtype == syn.BF16 else kvc.KVC_F32
        self.ws = kvc.workspace(kvc.kvc_append_decode_attn_workspace_size(
            B, n_h, n_kv, self.L_max, d, code))
        self.ws_plain = kvc.workspace(kvc.kvc_decode_attn_workspace_size(
            B, n_h, n_kv, self.L_max, d, code))

    @property
    def kernel(self):
        c = self.cfg
        if c.dtype == syn.BF16 and c.d == 128:
            if c.B * c.n_kv >= 64:   # the long GQA layer: the persistent form
                return "dense_persist_kernel<true, false, false, false> (append + attend)"
            return "dense_mfma_kernel<false, true, false, false, false> (append + attend)"
        return "dense_generic_kernel<float, %d, false, true> (append + attend)" % c.d

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
        return int(2 * c.n_kv * c.d * self.be * n.sum() + c.B * c.n_h * c.d * 2 * self.be + 4 * c.B)

    def step_bytes(self, steps_done):
        c = self.cfg
        n = self.lens_after(steps_done)
        per_layer = self.kernel_bytes(n) + 4 * c.B * c.n_kv * c.d * self.be + 4 * c.B
        return per_layer * self.layers

    def launch_bytes(self, steps_done):
        """Algorithmic bytes of one fused launch (append included)."""
        return self.step_bytes(steps_done) // self.layers

    def unit_bytes(self, n, G):
        """One unit's share of a layer-step: n rows of K and V read, G query
        and output rows, the new K/V row read and written."""
        d = self.cfg.d
        return 2 * n * d * self.be + 2 * G * d * self.be + 4 * d * self.be

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        G = c.n_h // c.n_kv
        n = int(self.pre[b])
        kr, vr = to_host(self.K[0][b, j, :n]), to_host(self.V[0][b, j, :n])
        kc = np.zeros((1, 1, n + 1, c.d), kr.dtype)
        vc = np.zeros((1, 1, n + 1, c.d), vr.dtype)
        kc[0, 0, :n], vc[0, 0, :n] = kr, vr
        q = to_host(self.q[0][b, j * G:(j + 1) * G])[None]
        kn, vn = to_host(self.kn[0][b, j])[None, None], to_host(self.vn[0][b, j])[None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append(kc, vc, sl, kn, vn)
        oracle.decode(q, kc, vc, sl, c.scale)
        return self.unit_bytes(n + 1, G), time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        lens = ("%d cached + 1 appended" % c.pre_len) if c.pre_len is not None else \
            "seq_lens ~ U[%d, %d] (post-append)" % c.len_range
        dt = "bf16" if c.dtype == syn.BF16 else "fp32"
        return (f"{c.name}: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} {dt}, {lens}, "
                f"{self.layers} layers ({self.nbuf} distinct cache buffers)")


class MlaWorkload(Workload):
    """Latent-cache layers, [B, L_max, 576] per layer buffer (C4)."""

    kernel = "mla_kernel + mla_merge_kernel"
    unit_name = "sequences (all 128 heads)"

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

    def units(self):
        return [(b, 0) for b in range(self.cfg.B)]

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

    kernel_only = decode_only

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

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

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        D = c.d_c + c.d_r
        n = int(self.pre[b])
        rows = to_host(self.C[0][b, :n])
        c4 = np.zeros((1, 1, n + 1, D), rows.dtype)
        c4[0, 0, :n] = rows
        q, cn = to_host(self.q[0][b])[None], to_host(self.cn[0][b])[None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append(c4, None, sl, cn, None)
        oracle.decode_mla(q, c4[:, 0], sl, c.d_c, c.d_r, c.scale)
        nbytes = (n + 1) * D * 2 + c.n_h * (D + c.d_c) * 2 + 2 * D * 2
        return nbytes, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"{c.name}: B={c.B} n_h={c.n_h} latent {c.d_c} + rope {c.d_r} bf16, "
                f"{c.pre_len} cached + 1 appended, scale 1/24, {self.layers} layers "
                f"({self.nbuf} distinct cache buffers)")


class TopKWorkload(Workload):
    """Top-k sparse GQA over [B, n_kv, L_max, d] caches (C5)."""

    kernel = "dense_mfma_kernel<true, false, false, false, false> (top-k)"

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
        self.idx_h = [syn.topk_indices(cfg.cfg_id, 0, B, n_kv, cfg.K, cfg.pre_len, index_set=l)
                      for l in range(self.layers)]
        self.idx = [torch.from_numpy(x).cuda() for x in self.idx_h]
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

    kernel_only = decode_only

    def kernel_bytes(self, n=None):
        c = self.cfg
        return int(c.B * c.n_kv * c.K * (2 * c.d * 2 + 4) + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes()

    def lens_after(self, steps_done):
        return np.minimum(self.pre + 1 + steps_done, self.L_max)

    def step_bytes(self, steps_done):
        c = self.cfg
        return (self.kernel_bytes() + 4 * c.B * c.n_kv * c.d * 2 + 4 * c.B) * self.layers

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        G = c.n_h // c.n_kv
        n = int(self.pre[b])
        kc = np.zeros((1, 1, n + 1, c.d), np.uint16)
        vc = np.zeros((1, 1, n + 1, c.d), np.uint16)
        kc[0, 0, :n], vc[0, 0, :n] = to_host(self.K[0][b, j, :n]), to_host(self.V[0][b, j, :n])
        q = to_host(self.q[0][b, j * G:(j + 1) * G])[None]
        kn, vn = to_host(self.kn[0][b, j])[None, None], to_host(self.vn[0][b, j])[None, None]
        idx = self.idx_h[0][b, j][None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append(kc, vc, sl, kn, vn)
        oracle.decode_topk(q, kc, vc, sl, idx, c.scale)
        nbytes = c.K * (2 * c.d * 2 + 4) + 2 * G * c.d * 2 + 4 * c.d * 2
        return nbytes, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"{c.name}: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} bf16, K={c.K} sorted distinct "
                f"indices of L={c.pre_len}, {self.layers} index sets over {self.nbuf} cache buffers")


class Fp8DenseWorkload(DenseWorkload):
    """The GQA layers of C3 over FP8 E4M3 caches (uint8 [B, n_kv, L_max, d],
    one float32 scale per tensor).  A layer-step is kvc_append_fp8 then
    kvc_decode_attn_fp8."""

    kernel = "dense_persist_kernel<false, true, false, false> (fp8 E4M3 cache)"
    kernel_appends = False
    K_SCALE = 1.0 / 64      # N(0,1) / (1/64) stays within +-448
    V_SCALE = 1.0 / 64

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.be = 2
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

    kernel_only = decode_only

    def kernel_bytes(self, n):
        c = self.cfg
        return int(2 * c.n_kv * c.d * 1 * n.sum() + c.B * c.n_h * c.d * (2 + 2) + 4 * c.B)

    def launch_bytes(self, steps_done):
        return self.kernel_bytes(self.lens_after(steps_done - 1))

    def step_bytes(self, steps_done):
        c = self.cfg
        append = 2 * c.B * c.n_kv * c.d * (2 + 1) + 8 * c.B
        return (self.kernel_bytes(self.lens_after(steps_done)) + append) * self.layers

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        G = c.n_h // c.n_kv
        n = int(self.pre[b])
        kc = np.zeros((1, 1, n + 1, c.d), np.uint8)
        vc = np.zeros((1, 1, n + 1, c.d), np.uint8)
        kc[0, 0, :n], vc[0, 0, :n] = to_host(self.K[0][b, j, :n]), to_host(self.V[0][b, j, :n])
        q = to_host(self.q[0][b, j * G:(j + 1) * G])[None]
        kn, vn = to_host(self.kn[0][b, j])[None, None], to_host(self.vn[0][b, j])[None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append_fp8(kc, vc, sl, kn, vn, self.K_SCALE, self.V_SCALE)
        oracle.decode_fp8(q, kc, vc, sl, c.scale, self.K_SCALE, self.V_SCALE)
        nbytes = 2 * (n + 1) * c.d + 2 * G * c.d * 2 + 2 * c.d * (2 + 1)
        return nbytes, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"{c.name} over FP8 E4M3 caches: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d}, "
                f"seq_lens ~ U[{c.len_range[0]}, {c.len_range[1]}] (post-append), "
                f"{self.layers} layers ({self.nbuf} distinct cache buffers), bf16 q/out")


class Fp4DenseWorkload(DenseWorkload):
    """The GQA layers of C3 over FP4 block-scaled caches: E2M1 codes
    (uint8 [B, n_kv, L_max, d/2]) and one E4M3 scale per 16 channels (uint8
    [B, n_kv, L_max, d/16]).  A layer-step is kvc_append_fp4 then
    kvc_decode_attn_fp4."""

    kernel = "dense_persist_kernel<false, false, false, true> (fp4 E2M1 cache)"
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

    kernel_only = decode_only

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

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        G = c.n_h // c.n_kv
        n = int(self.pre[b])
        arrs = []
        for src, w in ((self.KC, c.d // 2), (self.KS, c.d // 16), (self.VC, c.d // 2), (self.VS, c.d // 16)):
            a = np.zeros((1, 1, n + 1, w), np.uint8)
            a[0, 0, :n] = to_host(src[0][b, j, :n])
            arrs.append(a)
        kc, ks, vc, vs = arrs
        q = to_host(self.q[0][b, j * G:(j + 1) * G])[None]
        kn, vn = to_host(self.kn[0][b, j])[None, None], to_host(self.vn[0][b, j])[None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append_fp4(kc, ks, vc, vs, sl, kn, vn)
        oracle.decode_fp4(q, kc, ks, vc, vs, sl, c.scale)
        nbytes = 2 * (n + 1) * self.row_bytes() + 2 * G * c.d * 2 + 2 * (c.d * 2 + self.row_bytes())
        return nbytes, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"{c.name} over FP4 caches (E2M1 + E4M3 scale per 16 channels): B={c.B} "
                f"n_h={c.n_h} n_kv={c.n_kv} d={c.d}, seq_lens ~ U[{c.len_range[0]}, "
                f"{c.len_range[1]}] (post-append), {self.layers} layers ({self.nbuf} distinct "
                f"cache buffers), bf16 q/out")


class WindowWorkload(DenseWorkload):
    """The GQA layers of C3 attending only the newest WINDOW positions (the
    DeepSeek article's n_win = 128).  A layer-step is kvc_append then
    kvc_decode_attn_window.

    In a real model every layer has its own cache, so the 80 layers' windows
    are 80 distinct regions of memory.  Two buffers stand in for the 80
    here, so the layers sharing a buffer get lengths offset by 128 positions
    from one another (wrapping inside the drawn range [1023, 32767]): each
    layer reads its own 17 MB of window rows, 1.3 GB per step, well beyond
    the 256 MB last-level cache.  Every length stays above the window, so
    the attended positions and bytes per layer are those of C3 at W = 128."""

    kernel = "dense_mfma_kernel<false, false, false, false, false> (window 128)"
    kernel_appends = False
    WINDOW = 128

    def __init__(self, cfg, slack, torch, kvc):
        super().__init__(cfg, slack, torch, kvc)
        lo, hi = cfg.len_range[0] - 1, cfg.len_range[1] - 1
        self.pre_l = [lo + (self.pre - lo - self.WINDOW * (l // self.nbuf)) % (hi - lo + 1)
                      for l in range(self.layers)]
        self.sl = [torch.tensor(p, dtype=torch.int32).cuda() for p in self.pre_l]
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

    kernel_only = decode_only

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

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        G = c.n_h // c.n_kv
        n = int(self.pre[b])
        lo = max(0, n + 1 - self.WINDOW)
        kc = np.zeros((1, 1, n + 1, c.d), np.uint16)    # rows below the window are never read
        vc = np.zeros((1, 1, n + 1, c.d), np.uint16)
        kc[0, 0, lo:n], vc[0, 0, lo:n] = to_host(self.K[0][b, j, lo:n]), to_host(self.V[0][b, j, lo:n])
        q = to_host(self.q[0][b, j * G:(j + 1) * G])[None]
        kn, vn = to_host(self.kn[0][b, j])[None, None], to_host(self.vn[0][b, j])[None, None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append(kc, vc, sl, kn, vn)
        oracle.decode_window(q, kc, vc, sl, c.scale, self.WINDOW)
        nbytes = 2 * min(n + 1, self.WINDOW) * c.d * 2 + 2 * G * c.d * 2 + 4 * c.d * 2
        return nbytes, time.perf_counter() - t0

    def describe(self):
        return (super().describe().replace(", seq_lens", f", window {self.WINDOW} of seq_lens")
                + ", per-layer lengths offset by the window so each layer reads its own rows")


class PagedWorkload(DenseWorkload):
    """The GQA layers of C3 over a paged cache: pools of 16-position blocks
    sized to the sequences' lengths, blocks in shuffled physical order, one
    block table per layer buffer.  A layer-step is kvc_append_paged then
    kvc_decode_attn_paged."""

    kernel = "dense_persist_kernel<false, false, true, false> (paged, 16-position blocks)"
    kernel_appends = False
    unit_name = "sequences (all KV heads)"
    BETA = 16

    def __init__(self, cfg, slack, torch, kvc):
        self.cfg, self.torch, self.kvc = cfg, torch, kvc
        B, n_h, n_kv, d = cfg.B, cfg.n_h, cfg.n_kv, cfg.d
        self.be = 2
        self.pre = syn.pre_append_lens(cfg).astype(np.int64)
        self.L_max = int(self.pre.max() + 1 + slack)
        self.max_blocks = -(-self.L_max // self.BETA)
        self.layers = cfg.layers
        self.nbuf = cfg.distinct_buffers
        self.need = [-(-int(n + 1 + slack) // self.BETA) for n in self.pre]
        self.num_blocks = int(sum(self.need))
        order = np.random.default_rng(1000 + cfg.cfg_id).permutation(self.num_blocks)
        table = np.full((B, self.max_blocks), 1 << 30, dtype=np.int32)
        at = 0
        for b in range(B):
            table[b, :self.need[b]] = order[at:at + self.need[b]]
            at += self.need[b]
        self.table_h = table
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

    def units(self):
        return [(b, 0) for b in range(self.cfg.B)]

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

    kernel_only = decode_only

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

    def cpu_unit(self, b, j, oracle):
        """One sequence, all KV heads: its blocks copied out in table order
        (a pool of its own, table entries renumbered 0..)."""
        c = self.cfg
        n = int(self.pre[b])
        blocks = self.torch.from_numpy(self.table_h[b, :self.need[b]].astype(np.int64)).cuda()
        kp, vp = to_host(self.K[0][blocks]), to_host(self.V[0][blocks])
        tab = np.arange(self.need[b], dtype=np.int32)[None]
        q = to_host(self.q[0][b])[None]
        kn, vn = to_host(self.kn[0][b])[None], to_host(self.vn[0][b])[None]
        sl = np.array([n], np.int32)
        t0 = time.perf_counter()
        oracle.append_paged(kp, vp, tab, sl, kn, vn)
        oracle.decode_paged(q, kp, vp, tab, sl, c.scale)
        nbytes = (c.n_kv * (2 * (n + 1) * c.d * 2 + 4 * c.d * 2) + 2 * c.n_h * c.d * 2
                  + 4 * -(-(n + 1) // self.BETA))
        return nbytes, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"{c.name} over a paged cache: B={c.B} n_h={c.n_h} n_kv={c.n_kv} d={c.d} bf16, "
                f"{self.BETA}-position blocks ({self.num_blocks} in shuffled order), seq_lens ~ "
                f"U[{c.len_range[0]}, {c.len_range[1]}] (post-append), {self.layers} layers "
                f"({self.nbuf} distinct pools)")


class SelectWorkload(Workload):
    """Top-k selection for the sparse workload's shape: per sequence and KV
    head, the 2048 highest of 131072 indexer scores (float32, seeded N(0,1)),
    32 index sets over 16 distinct score buffers (512 MB)."""

    kernel = "seg_select_kernel"
    unit_name = "score rows"
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
        self.ws = kvc.workspace(kvc.kvc_topk_select_workspace_size(B, R, L, cfg.K))

    def step(self):
        for l in range(self.layers):
            self.kvc.kvc_topk_select(self.S[l % self.NBUF], self.lens, self.out[l],
                                     workspace=self.ws)

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

    def cpu_unit(self, b, j, oracle):
        c = self.cfg
        row = to_host(self.S[0][b, j])[None, None]
        t0 = time.perf_counter()
        oracle.topk_select(row, np.array([c.pre_len]), c.K)
        return c.pre_len * 4 + c.K * 4, time.perf_counter() - t0

    def describe(self):
        c = self.cfg
        return (f"top-k selection: B={c.B} x {c.n_kv} rows, K={c.K} of {c.pre_len} float32 scores, "
                f"{self.layers} index sets over {self.NBUF} score buffers")


# C1 is one tiny layer (256 cached + 1 appended): a graph of one kernel
# measures the graph launch, not the layer-step.  It is timed as 16
# independent layers of that shape launched back to back (each its own
# cache, lengths growing by one per step), like the C2 layer sweep.
C1_LAYERS = dataclasses.replace(syn.C1, layers=16, distinct_buffers=16)

WORKLOADS = {"C1": (C1_LAYERS, DenseWorkload), "C2": (syn.C2, DenseWorkload),
             "C3": (syn.C3, DenseWorkload), "C4": (syn.C4, MlaWorkload),
             "C5": (syn.C5, TopKWorkload), "C3F8": (syn.C3, Fp8DenseWorkload),
             "C3W128": (syn.C3, WindowWorkload), "C3P16": (syn.C3, PagedWorkload),
             "C3F4": (syn.C3, Fp4DenseWorkload), "C5S": (syn.C5, SelectWorkload)}


# ---------------------------------------------------------------- timing
def capture(torch, fn):
    """Capture fn once into a HIP graph (on a side stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def measure(name, args, torch, kvc):
    cfg, cls = WORKLOADS[name]
    slack = reservation_slack(args.warmup, args.steps, args.kernel_reps)
    wl = cls(cfg, slack, torch, kvc)
    wl.decode_only()            # first launches outside capture (no state change)
    torch.cuda.synchronize()

    g = capture(torch, wl.step)
    done = 0
    for _ in range(args.warmup):
        g.replay()
        done += 1
    torch.cuda.synchronize()
    # (graph replays run on the current stream, which the events record on)
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

    # the dominant kernel alone: one launch per layer, back to back, after
    # the same number of untimed replays as the step (a graph's first
    # replays run slower: 139.8 then 134 -> 129.5 us per launch over the
    # first eight replays of the FP4 layer graph)
    gk = capture(torch, wl.kernel_only)
    for _ in range(args.warmup):
        gk.replay()
    if wl.kernel_appends:
        done += args.warmup
    torch.cuda.synchronize()
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
    k_gbs = k_bytes / (k_us * 1e-6) / 1e9
    res = dict(
        workload=wl.describe(), layers=wl.layers, ms_per_step=ms_step,
        us_per_layer_step=ms_step * 1e3 / wl.layers, gbs=gbs, pct_of_peak=100 * gbs / PEAK_GBS,
        bytes_per_step=bytes_total / args.steps,
        roofline={"bound": "hbm", "achieved": round(k_gbs, 2), "peak": PEAK_GBS, "unit": "GB/s",
                  "frac": round(k_gbs / PEAK_GBS, 4), "traffic": measured_traffic(name),
                  "kernel": wl.kernel, "kernel_us": round(k_us, 3),
                  "algorithmic_bytes_per_launch": int(k_bytes)})
    return wl, res


def cpu_baseline(wl, budget_s):
    import oracle
    nbytes, secs, sample = wl.cpu_sample(budget_s, oracle)
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle", "sample": f"{sample}, {secs:.1f} s of oracle time"}


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
    """Streaming read of 4 GiB with the decode kernels' load pattern and
    cache policy: the achievable read rate of this part, in the same run."""
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
    print(f"[bench] {args.config}: {head['gbs']:.1f} GB/s, kernel {head['roofline']['kernel_us']} us",
          file=sys.stderr, flush=True)
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
        "dtype": "bf16" if WORKLOADS[args.config][0].dtype == syn.BF16 else "f32",
        "data": "synthetic (seeded N(0,1), bf16 round-to-nearest-even)",
        "config": {"workload": head["workload"], "layers_per_step": head["layers"],
                   "pct_of_peak": round(head["pct_of_peak"], 2),
                   "us_per_layer_step": round(head["us_per_layer_step"], 3)},
        "roofline": head["roofline"],
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, HEAD_CPU_BUDGET_S)
    del wl
    torch.cuda.empty_cache()

    calibrate_copy(torch, kvc)
    line["read_ceiling_gbs"] = round(read_ceiling(torch, kvc), 1)
    line["roofline"]["frac_of_read_ceiling"] = round(
        line["roofline"]["achieved"] / line["read_ceiling_gbs"], 4)
    also = {}
    for name in [x for x in args.others.split(",") if x in WORKLOADS and x != args.config]:
        w, r = measure(name, args, torch, kvc)
        print(f"[bench] {name}: {r['gbs']:.1f} GB/s, kernel {r['roofline']['kernel_us']} us",
              file=sys.stderr, flush=True)
        e = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items()}
        if not args.no_cpu:
            e["cpu_baseline"] = cpu_baseline(w, CPU_BUDGET_S)
        also[name] = e
        del w
        torch.cuda.empty_cache()
    if also:
        line["also"] = also
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
