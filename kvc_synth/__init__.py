"""Seeded synthetic inputs for single-token decode attention over a KV cache.

This module is shared by the fp64 CPU oracle's tests and by the HIP path's
tests and benchmark.  It draws random numbers, rounds them to the storage
dtype and lays them out; it holds none of the attention arithmetic.

Workloads follow the shapes the source pages discuss:

* "KV cache" guide (this.guide), section "Two tensors per layer": one cache
  pair per layer, each shaped [n_kv, L, d_h] per sequence.  Here a batch of
  sequences is stored as [B, n_kv, L_max, d_h] with a per-sequence length.
* Same guide, "Where the memory actually goes" footnote: an MLA row is a
  512-wide latent plus a 64-wide shared rotary key.
* Podcast transcript (my-weird-prompts 640482), DeepSeek Sparse Attention
  passage: a top-k of 2048 stored positions per query.

Every tensor chunk (one sequence b and one KV head j) is drawn from its own
``numpy.random.SeedSequence([1000 + cfg, layer, tensor_id, b, j])`` so any
chunk can be regenerated on its own.  Values are N(0, 1) in float32; bf16
storage uses round-to-nearest-even done with integer operations.  Positions
at or beyond a sequence's pre-append length are NaN-poisoned in parity
inputs so that a kernel reading past the valid range is caught.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "k_new": 3, "v_new": 4,
              "seq_lens": 5, "idx": 6, "ckv": 7, "ckv_new": 8,
              "k_scales": 9, "v_scales": 10}

F32 = "f32"
BF16 = "bf16"

BF16_QNAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# bf16 storage
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even.

    Integer-only: add 0x7FFF plus the lowest kept bit, then drop 16 bits.
    NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    rounded[np.isnan(x)] = BF16_QNAN
    return rounded


def storage_dtype(dtype: str):
    return np.uint16 if dtype == BF16 else np.float32


def poison_value(dtype: str):
    if dtype == BF16:
        return BF16_QNAN
    return np.float32(np.nan)


def _rng(cfg: int, layer: int, tensor: str, b: int, j: int):
    seq = np.random.SeedSequence([1000 + cfg, layer, TENSOR_IDS[tensor], b, j])
    return np.random.default_rng(seq)


def normal_chunk(cfg: int, layer: int, tensor: str, b: int, j: int,
                 shape, dtype: str) -> np.ndarray:
    """One seeded N(0,1) chunk in storage form (float32 or bf16 bits)."""
    x = _rng(cfg, layer, tensor, b, j).standard_normal(shape, dtype=np.float32)
    return bf16_bits(x) if dtype == BF16 else x


# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class DenseConfig:
    """Dense (MHA/GQA/MQA) decode workload.  Lengths are pre-append."""
    name: str
    cfg_id: int
    B: int
    n_h: int
    n_kv: int
    d: int
    dtype: str
    layers: int
    L_max: int
    pre_len: int | None          # fixed pre-append length, or None = drawn
    len_range: tuple | None      # post-append length range (inclusive)
    distinct_buffers: int        # layer buffers cycled in timing runs

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    name: str
    cfg_id: int
    B: int
    n_h: int
    d_c: int
    d_r: int
    dtype: str
    layers: int
    L_max: int
    pre_len: int
    distinct_buffers: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_c + self.d_r)


@dataclasses.dataclass(frozen=True)
class TopKConfig:
    name: str
    cfg_id: int
    B: int
    n_h: int
    n_kv: int
    d: int
    dtype: str
    L_max: int
    pre_len: int
    K: int
    distinct_buffers: int
    index_sets: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads.  Lengths: C1 holds 256 cached positions and attends 257
# after the append.  C2/C4 hold L and attend L+1.  C3 draws post-append
# lengths in [1024, 32768] (pre-append = draw - 1) so L_max = 32768 holds
# them.  C5 holds L = 131072 valid positions; the append writes slot 131072.
C1 = DenseConfig("tiny_gqa_fp32", 1, B=1, n_h=8, n_kv=2, d=64, dtype=F32,
                 layers=1, L_max=257, pre_len=256, len_range=None,
                 distinct_buffers=1)
C2 = DenseConfig("mha_llama2_7b_layer", 2, B=1, n_h=32, n_kv=32, d=128,
                 dtype=BF16, layers=32, L_max=4097, pre_len=4096,
                 len_range=None, distinct_buffers=32)
C3 = DenseConfig("gqa_llama3_70b_layer", 3, B=32, n_h=64, n_kv=8, d=128,
                 dtype=BF16, layers=80, L_max=32768, pre_len=None,
                 len_range=(1024, 32768), distinct_buffers=2)
C4 = MLAConfig("mla_latent_512_64", 4, B=64, n_h=128, d_c=512, d_r=64,
               dtype=BF16, layers=4, L_max=8193, pre_len=8192,
               distinct_buffers=4)
C5 = TopKConfig("topk_gqa_2048_of_131072", 5, B=8, n_h=64, n_kv=8, d=128,
                dtype=BF16, L_max=131073, pre_len=131072, K=2048,
                distinct_buffers=2, index_sets=32)

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}


def draw_post_append_lens(cfg_id: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence post-append lengths, uniform integers in [lo, hi]."""
    rng = _rng(cfg_id, 0, "seq_lens", 0, 0)
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def pre_append_lens(cfg: DenseConfig) -> np.ndarray:
    if cfg.pre_len is not None:
        return np.full(cfg.B, cfg.pre_len, dtype=np.int32)
    lo, hi = cfg.len_range
    return draw_post_append_lens(cfg.cfg_id, cfg.B, lo, hi) - 1


# --------------------------------------------------------------------------
# host-side (numpy) case builders
# --------------------------------------------------------------------------
def dense_case(B, n_h, n_kv, d, L_max, pre_lens, dtype, cfg_id=0, layer=0,
               poison=True) -> dict:
    """Dense decode inputs in storage form.

    Returns q [B,n_h,d], k_cache/v_cache [B,n_kv,L_max,d], seq_lens [B]
    (pre-append, int32), k_new/v_new [B,n_kv,d].  Query heads of KV head j
    are drawn in one chunk per (b, j).
    """
    assert n_h % n_kv == 0
    G = n_h // n_kv
    pre_lens = np.asarray(pre_lens, dtype=np.int32).reshape(B)
    sd = storage_dtype(dtype)
    fill = poison_value(dtype) if poison else sd(0)
    kc = np.full((B, n_kv, L_max, d), fill, dtype=sd)
    vc = np.full((B, n_kv, L_max, d), fill, dtype=sd)
    q = np.empty((B, n_h, d), dtype=sd)
    kn = np.empty((B, n_kv, d), dtype=sd)
    vn = np.empty((B, n_kv, d), dtype=sd)
    for b in range(B):
        n = int(pre_lens[b])
        assert 0 <= n <= L_max
        for j in range(n_kv):
            kc[b, j, :n] = normal_chunk(cfg_id, layer, "k", b, j, (n, d), dtype)
            vc[b, j, :n] = normal_chunk(cfg_id, layer, "v", b, j, (n, d), dtype)
            q[b, j * G:(j + 1) * G] = normal_chunk(cfg_id, layer, "q", b, j, (G, d), dtype)
            kn[b, j] = normal_chunk(cfg_id, layer, "k_new", b, j, (d,), dtype)
            vn[b, j] = normal_chunk(cfg_id, layer, "v_new", b, j, (d,), dtype)
    return dict(q=q, k_cache=kc, v_cache=vc, seq_lens=pre_lens.copy(),
                k_new=kn, v_new=vn, dtype=dtype)


def mla_case(B, n_h, d_c, d_r, L_max, pre_lens, dtype, cfg_id=0, layer=0,
             poison=True) -> dict:
    """MLA latent-cache inputs in storage form.

    ckv [B,L_max,d_c+d_r] holds the latent then the rotary key per position;
    q [B,n_h,d_c+d_r] holds the absorbed latent query then the rotary query;
    ckv_new [B,d_c+d_r] is the new token's row.
    """
    pre_lens = np.asarray(pre_lens, dtype=np.int32).reshape(B)
    D = d_c + d_r
    sd = storage_dtype(dtype)
    fill = poison_value(dtype) if poison else sd(0)
    ckv = np.full((B, L_max, D), fill, dtype=sd)
    q = np.empty((B, n_h, D), dtype=sd)
    cn = np.empty((B, D), dtype=sd)
    for b in range(B):
        n = int(pre_lens[b])
        assert 0 <= n <= L_max
        ckv[b, :n] = normal_chunk(cfg_id, layer, "ckv", b, 0, (n, D), dtype)
        q[b] = normal_chunk(cfg_id, layer, "q", b, 0, (n_h, D), dtype)
        cn[b] = normal_chunk(cfg_id, layer, "ckv_new", b, 0, (D,), dtype)
    return dict(q=q, ckv=ckv, seq_lens=pre_lens.copy(), ckv_new=cn,
                dtype=dtype)


def topk_indices(cfg_id, layer, B, n_kv, K, L, index_set=0) -> np.ndarray:
    """[B,n_kv,K] int32: per (b, j) a sorted draw of K distinct values in [0, L)."""
    idx = np.empty((B, n_kv, K), dtype=np.int32)
    for b in range(B):
        for j in range(n_kv):
            rng = _rng(cfg_id, layer * 1000 + index_set, "idx", b, j)
            idx[b, j] = np.sort(rng.choice(L, size=K, replace=False))
    return idx


# --------------------------------------------------------------------------
# device-side (torch) fills for full-size timing runs
# --------------------------------------------------------------------------
def device_normal_(t, seed: int, chunk_elems: int = 1 << 28):
    """Fill a CUDA tensor (float32 or bfloat16) with seeded N(0,1) in place.

    Uses torch's Philox generator on the device; bf16 is the round-to-
    nearest-even of the float32 draw.  Filling proceeds in slices so the
    float32 staging stays bounded.
    """
    import torch
    flat = t.view(-1)
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    for s in range(0, flat.numel(), chunk_elems):
        e = min(flat.numel(), s + chunk_elems)
        x = torch.randn(e - s, generator=g, device=t.device, dtype=torch.float32)
        flat[s:e].copy_(x.to(t.dtype))
        del x
    return t


def device_seed(cfg_id: int, layer: int, tensor: str) -> int:
    return (1000 + cfg_id) * 1_000_003 + layer * 101 + TENSOR_IDS[tensor]
