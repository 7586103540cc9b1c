"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only *draws* data: Gaussian Q/K/V rounded to bf16, per-head window
lengths, per-head sink logits, block-selection matrices and sampled query rows.
It holds none of the attention arithmetic, so the float64 oracle and the HIP
path can both be fed from it without sharing any part of the method.

Every random stream is a numpy ``default_rng`` seeded with a list
``[seed, cfg, tensor_id, h]`` so that a single head of a 128K-token problem can
be regenerated on its own.  Tensor ids: Q=0, K=1, V=2, sink=3, windows=4,
block scores=5, sampled rows=6, upstream gradient dO=7, decode sequence
lengths=8 (K/V cache rows and decode queries reuse the K, V and Q ids with
the sequence index in place of the head).

The workloads mirror the shapes on the pages: ViT token grids from 14-pixel
patches (448/896/1792 px give 1,024/4,096/16,384 tokens; "Semantic Head
Specialization Guides Hybrid ViT Attention", cost slide), 16 heads per layer
(same page, self-attention slide), a 4096-token LM whose heads pick causal
windows from {512, 1024, 2048, 4096} ("Asymmetric Attention Heads", Table 2),
and 128K-token block-sparse prefill that keeps about half of the causal blocks
("RRAttention", abstract and section 2.1).
"""

from __future__ import annotations

import math

import numpy as np

Q_ID, K_ID, V_ID, SINK_ID, WIN_ID, BLOCK_ID, ROWS_ID, DO_ID, LEN_ID = 0, 1, 2, 3, 4, 5, 6, 7, 8


def child_rng(seed: int, cfg: int, tensor_id: int, h: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, cfg, tensor_id, h])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # NaN stays NaN (quiet bit forced); finite values round to nearest even.
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(seed: int, cfg: int, tensor_id: int, h: int, shape) -> np.ndarray:
    """N(0,1) float32 draws for one head, rounded to bf16 bits."""
    x = child_rng(seed, cfg, tensor_id, h).standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x)


def qkv_bf16(seed: int, cfg: int, B: int, H: int, L: int, D: int, Hkv: int | None = None):
    """Q [B, H, L, D] and K, V [B, Hkv, L, D] (Hkv defaults to H) as uint16 bf16 bits, one stream per
    tensor and head."""
    out = []
    for tid in (Q_ID, K_ID, V_ID):
        nh = H if (tid == Q_ID or Hkv is None) else Hkv
        t = np.empty((B, nh, L, D), dtype=np.uint16)
        for h in range(nh):
            t[:, h] = gaussian_bf16(seed, cfg, tid, h, (B, L, D))
        out.append(t)
    return tuple(out)


def grad_out_bf16(seed: int, cfg: int, B: int, H: int, L: int, D: int) -> np.ndarray:
    """Upstream gradient dO ~ N(0,1) as uint16 bf16 bits in [B, H, L, D] order."""
    t = np.empty((B, H, L, D), dtype=np.uint16)
    for h in range(H):
        t[:, h] = gaussian_bf16(seed, cfg, DO_ID, h, (B, L, D))
    return t


def qkv_f32(seed: int, cfg: int, B: int, H: int, L: int, D: int):
    """The same draws as :func:`qkv_bf16` before rounding (float32, [B, H, L, D])."""
    out = []
    for tid in (Q_ID, K_ID, V_ID):
        t = np.empty((B, H, L, D), dtype=np.float32)
        for h in range(H):
            t[:, h] = child_rng(seed, cfg, tid, h).standard_normal((B, L, D), dtype=np.float32)
        out.append(t)
    return tuple(out)


def head_windows(seed: int, cfg: int, H: int = 16, sizes=(512, 1024, 2048, 4096)) -> np.ndarray:
    """Per-head causal window lengths: each size used H/len(sizes) times, seeded permutation."""
    reps = H // len(sizes)
    base = np.repeat(np.asarray(sizes, dtype=np.int64), reps)
    return child_rng(seed, cfg, WIN_ID).permutation(base)


def head_sinks(seed: int, cfg: int, H: int) -> np.ndarray:
    """Per-head sink logits ~ N(0,1), float32."""
    return child_rng(seed, cfg, SINK_ID).standard_normal(H, dtype=np.float32)


def block_matrix_top_half(seed: int, cfg: int, H: int, nb: int) -> np.ndarray:
    """Lower-triangular block-selection matrices, uint8 [H, nb, nb].

    Row m keeps block 0 and the diagonal block m.  Of the remaining causal
    blocks n in [1, m-1] it keeps the ceil(R/2) (R = m-1) with the highest
    seeded U[0,1) score; equal scores prefer the lower n.
    """
    out = np.zeros((H, nb, nb), dtype=np.uint8)
    for h in range(H):
        scores = child_rng(seed, cfg, BLOCK_ID, h).random((nb, nb))
        for m in range(nb):
            out[h, m, 0] = 1
            out[h, m, m] = 1
            r = m - 1
            if r <= 0:
                continue
            k = (r + 1) // 2
            cand = np.arange(1, m)
            order = np.argsort(-scores[m, 1:m], kind="stable")
            out[h, m, cand[order[:k]]] = 1
    return out


def sampled_rows(seed: int, cfg: int, H: int, L: int, n: int) -> np.ndarray:
    """n distinct query rows per head, uniform without replacement, sorted: int64 [H, n]."""
    rows = np.empty((H, n), dtype=np.int64)
    for h in range(H):
        rows[h] = np.sort(child_rng(seed, cfg, ROWS_ID, h).choice(L, size=n, replace=False))
    return rows


# ---------------------------------------------------------------------------
# Workload catalogue.  A mask is a plain dict understood by both the binding
# and the oracle:  kind in {"full", "chunk", "window", "block"}; "causal";
# "chunk" (C); "left"/"right" (window half-widths, inclusive); "head_left"
# (per-head left reach); "block" (token block size) and "block_mask"
# (uint8 [Hb, nb, nb]).
# ---------------------------------------------------------------------------

def workload(name: str, seed: int = 0) -> dict:
    """Return {"cfg", "B", "H", "Hkv", "L", "D", "masks": {label: mask}, "sink": array|None,
    "rows": int|None}; Hkv is the number of K/V heads (H unless the workload groups query heads)."""
    w = _workload(name, seed)
    w.setdefault("Hkv", w["H"])
    return w


def _workload(name: str, seed: int) -> dict:
    if name == "tiny_chunk":
        return dict(cfg=1, B=1, H=2, L=256, D=64, sink=None, rows=None,
                    masks={"chunk64": dict(kind="chunk", chunk=64)})
    if name == "vit896":
        return dict(cfg=2, B=1, H=16, L=4096, D=80, sink=None, rows=None,
                    masks={"full": dict(kind="full"),
                           "chunk256": dict(kind="chunk", chunk=256),
                           "swa128": dict(kind="window", left=128, right=128)})
    if name == "vit1792":
        return dict(cfg=3, B=1, H=16, L=16384, D=80, sink=None, rows=512,
                    masks={"full": dict(kind="full"),
                           "swa512": dict(kind="window", left=512, right=512)})
    if name == "lm_headwin":
        H = 16
        w = head_windows(seed, 4, H)
        return dict(cfg=4, B=1, H=H, L=4096, D=128, sink=head_sinks(seed, 4, H), rows=None,
                    windows=w,
                    masks={"headwin": dict(kind="window", causal=True, left=0, right=0,
                                           head_left=(w - 1).astype(np.int64))})
    if name == "blocksparse128k":
        H, L, bs = 32, 131072, 128
        nb = math.ceil(L / bs)
        return dict(cfg=5, B=1, H=H, L=L, D=128, sink=None, rows=512,
                    masks={"block50": dict(kind="block", block=bs,
                                           block_mask=block_matrix_top_half(seed, 5, H, nb))})
    if name == "swa576_d256":
        # prefill of the SWA-vs-linear-attention article's speed-test layer (16 query heads on 4 K/V
        # heads, head dim 256) over a 128K-token prompt: causal window of 576 keys, learned sink
        H = 16
        return dict(cfg=6, B=1, H=H, Hkv=4, L=131072, D=256, sink=head_sinks(seed, 6, H), rows=512,
                    masks={"swa576": dict(kind="window", left=575, right=0, causal=True)})
    raise KeyError(name)


WORKLOADS = ("tiny_chunk", "vit896", "vit1792", "lm_headwin", "blocksparse128k", "swa576_d256")


# ---------------------------------------------------------------------------
# Decode: one new query per sequence against a key/value cache.
# ---------------------------------------------------------------------------

def decode_lengths(seed: int, cfg: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Cached-token counts of B sequences, uniform integers in [lo, hi]: int32 [B]."""
    return child_rng(seed, cfg, LEN_ID).integers(lo, hi + 1, size=B).astype(np.int32)


def decode_queries(seed: int, cfg: int, B: int, H: int, D: int) -> np.ndarray:
    """The new query token of every sequence, N(0,1) rounded to bf16: uint16 [B, H, D]."""
    return np.stack([gaussian_bf16(seed, cfg, Q_ID, b, (H, D)) for b in range(B)])


def decode_cache_rows(seed: int, cfg: int, b: int, n: int, Hkv: int, D: int, head_rows: int, tail_rows: int):
    """The cache rows of sequence b (n cached tokens) that a run fills with data: the first
    head_rows and the last tail_rows positions (every position when they cover all n).
    Returns (positions int64 [m] ascending, K uint16 [Hkv, m, D], V uint16 [Hkv, m, D])."""
    pos = np.union1d(np.arange(min(head_rows, n)), np.arange(max(0, n - tail_rows), n)).astype(np.int64)
    k = gaussian_bf16(seed, cfg, K_ID, b, (Hkv, len(pos), D))
    v = gaussian_bf16(seed, cfg, V_ID, b, (Hkv, len(pos), D))
    return pos, k, v


def decode_workload(name: str, seed: int = 0) -> dict:
    """Decode shapes of the sliding-window vs linear-attention article: attention of a Qwen3-4B-like
    layer (32 query heads on 8 K/V heads, head dim 128) and the Qwen3.5-4B-like speed test
    (16 on 4, head dim 256); windows of 576 keys with a learned sink, 572 + 4 prefix tokens, and
    full attention at a 128K-token prompt.  Returns {"cfg", "B", "H", "Hkv", "D", "Lmax",
    "lens" int32 [B], "window", "prefix", "sink" float32 [H] or None}."""
    if name == "decode_swa576":
        B, H, Hkv, D, L = 64, 32, 8, 128, 131072
        return dict(cfg=10, B=B, H=H, Hkv=Hkv, D=D, Lmax=L, lens=decode_lengths(seed, 10, B, 1024, L),
                    window=576, prefix=0, sink=head_sinks(seed, 10, H))
    if name == "decode_swa572_prefix4":
        B, H, Hkv, D, L = 64, 32, 8, 128, 131072
        return dict(cfg=11, B=B, H=H, Hkv=Hkv, D=D, Lmax=L, lens=decode_lengths(seed, 11, B, 1024, L),
                    window=572, prefix=4, sink=None)
    if name == "decode_full128k":
        B, H, Hkv, D, L = 1, 32, 8, 128, 131072
        return dict(cfg=12, B=B, H=H, Hkv=Hkv, D=D, Lmax=L, lens=np.full(B, L, np.int32),
                    window=0, prefix=0, sink=None)
    if name == "decode_swa576_d256":
        B, H, Hkv, D, L = 64, 16, 4, 256, 131072
        return dict(cfg=13, B=B, H=H, Hkv=Hkv, D=D, Lmax=L, lens=decode_lengths(seed, 13, B, 1024, L),
                    window=576, prefix=0, sink=head_sinks(seed, 13, H))
    raise KeyError(name)


DECODE_WORKLOADS = ("decode_swa576", "decode_swa572_prefix4", "decode_full128k", "decode_swa576_d256")
