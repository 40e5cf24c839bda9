"""Seeded synthetic workloads for the token-sparse attention path.

This module only draws random numbers and shapes them into inputs: it holds
none of the method's arithmetic, and both the HIP path's tests/benchmark and
the CPU oracle consume what it returns.  Everything is numpy on the host; a
tensor is returned as bf16 bit patterns (``uint16``) so that the GPU and the
oracle see the very same values (``to_f64`` upcasts them exactly).

Workloads (shapes follow the video and 3D settings the pages measure on; the
pages' own models and prompts are not available, so these seeded generators
stand in for them):

  tiny     B=1 H=2  N=1024  D=64  C=64 : N(0,1) + 2*(rank-8 factor shared by
           Q, K, V of a head); keys also pulled toward one of 16 centroids by
           token id mod 16.
  small    B=1 H=12 N=32760 (21x30x52 grid) D=128 C=128
  large    B=1 H=40 N=75600 (21x45x80 grid) D=128 C=128
  long     B=1 H=24 N=118800 (33x45x80 grid) D=128 C=128
           video-like: Q and K share a smooth function of the (t, y, x)
           position (random Fourier features of length scales (1.5, 3, 3)
           cells, rotated by a per-head orthogonal matrix, amplitude a with
           a^2 = 8 sqrt(D) so the peak logit is about 8) plus 0.5*N(0,1)
           noise; V ~ N(0,1).
  asset3d  B=1 H=16 N=49152 D=64 C=64 : Q and K drawn around 256 per-head
           Gaussian centres (sigma 0.3), independently assigned; V ~ N(0,1).

Between steps every tensor drifts: X <- bf16(X + sigma * N(0,1)).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids used in seeds
_T_Q, _T_K, _T_V, _T_FACTOR, _T_CENTROID, _T_RFF, _T_ROT, _T_ASSIGN = 1, 2, 3, 4, 5, 6, 7, 8


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    H: int
    N: int
    D: int
    C: int
    densities: tuple
    kind: str
    drift: float
    reuse_steps: int
    grid: tuple = field(default=())


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 1024, 64, 64, (0.25,), "tiny", 0.05, 1),
    "small": Workload("small", 2, 1, 12, 32760, 128, 128, (0.20,), "video", 0.03, 4, (21, 30, 52)),
    "large": Workload("large", 3, 1, 40, 75600, 128, 128, (0.20,), "video", 0.03, 1, (21, 45, 80)),
    "long": Workload("long", 4, 1, 24, 118800, 128, 128, (0.25, 0.15), "video", 0.03, 9, (33, 45, 80)),
    "asset3d": Workload("asset3d", 5, 1, 16, 49152, 64, 64, (0.15,), "clusters", 0.02, 9),
}


# ---------------------------------------------------------------------------
# bf16 storage helpers (round-to-nearest-even, the rounding of a bf16 store)
# ---------------------------------------------------------------------------

def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    return to_f32(bits).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """Values rounded to the nearest bf16, returned as float64."""
    return to_f64(to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


# ---------------------------------------------------------------------------
# per-head generators (float32 values before bf16 rounding)
# ---------------------------------------------------------------------------

def _tiny_head(cfg: int, b: int, h: int, N: int, D: int):
    f = _rng(cfg, _T_FACTOR, b, h)
    low = f.standard_normal((N, 8), dtype=np.float32) @ (
        f.standard_normal((8, D), dtype=np.float32) / np.float32(math.sqrt(8.0)))
    cents = _rng(cfg, _T_CENTROID, b, h).standard_normal((16, D), dtype=np.float32)
    q = _rng(cfg, _T_Q, 0, b, h).standard_normal((N, D), dtype=np.float32) + 2.0 * low
    k = (_rng(cfg, _T_K, 0, b, h).standard_normal((N, D), dtype=np.float32) + 2.0 * low
         + 2.0 * cents[np.arange(N) % 16])
    v = _rng(cfg, _T_V, 0, b, h).standard_normal((N, D), dtype=np.float32) + 2.0 * low
    return q, k, v


def _grid_positions(grid) -> np.ndarray:
    T, Y, X = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Y), np.arange(X), indexing="ij")
    # token n = (t*Y + y)*X + x
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float32)


def _orthogonal(rng: np.random.Generator, D: int) -> np.ndarray:
    a = rng.standard_normal((D, D))
    qm, r = np.linalg.qr(a)
    return (qm * np.sign(np.diag(r))).astype(np.float32)


def _video_head(cfg: int, b: int, h: int, grid, D: int, pos: np.ndarray):
    rf = _rng(cfg, _T_RFF, b, h)
    lengths = np.array([1.5, 3.0, 3.0], dtype=np.float32)
    omega = rf.standard_normal((D, 3), dtype=np.float32) / lengths      # F = D features
    phase = rf.uniform(0.0, 2.0 * math.pi, size=D).astype(np.float32)
    feat = np.float32(math.sqrt(2.0 / D)) * np.cos(pos @ omega.T + phase)
    amp = np.float32(math.sqrt(8.0 * math.sqrt(D)))
    shared = amp * (feat @ _orthogonal(_rng(cfg, _T_ROT, b, h), D))
    n = pos.shape[0]
    q = shared + 0.5 * _rng(cfg, _T_Q, 0, b, h).standard_normal((n, D), dtype=np.float32)
    k = shared + 0.5 * _rng(cfg, _T_K, 0, b, h).standard_normal((n, D), dtype=np.float32)
    v = _rng(cfg, _T_V, 0, b, h).standard_normal((n, D), dtype=np.float32)
    return q, k, v


def _cluster_head(cfg: int, b: int, h: int, N: int, D: int):
    centres = _rng(cfg, _T_CENTROID, b, h).standard_normal((256, D), dtype=np.float32)
    assign = _rng(cfg, _T_ASSIGN, b, h)
    a_k = assign.integers(0, 256, size=N)
    a_q = assign.integers(0, 256, size=N)
    k = centres[a_k] + 0.3 * _rng(cfg, _T_K, 0, b, h).standard_normal((N, D), dtype=np.float32)
    q = centres[a_q] + 0.3 * _rng(cfg, _T_Q, 0, b, h).standard_normal((N, D), dtype=np.float32)
    v = _rng(cfg, _T_V, 0, b, h).standard_normal((N, D), dtype=np.float32)
    return q, k, v


def generate(name: str, heads=None):
    """Anchor-step inputs of a workload as bf16 bits: dict q, k, v of [B, H, N, D].

    ``heads`` optionally restricts generation to a list of (b, h) pairs (the
    result then has shape [1, len(heads), N, D]); every head is drawn from its
    own seed, so a head's values do not depend on which others are generated.
    """
    w = WORKLOADS[name]
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    shape = (1, len(pairs)) if heads is not None else (w.B, w.H)
    out = {t: np.empty(shape + (w.N, w.D), dtype=np.uint16) for t in ("q", "k", "v")}
    pos = _grid_positions(w.grid) if w.kind == "video" else None

    def one(i: int) -> None:
        b, h = pairs[i]
        if w.kind == "tiny":
            q, k, v = _tiny_head(w.cfg_id, b, h, w.N, w.D)
        elif w.kind == "video":
            q, k, v = _video_head(w.cfg_id, b, h, w.grid, w.D, pos)
        else:
            q, k, v = _cluster_head(w.cfg_id, b, h, w.N, w.D)
        bi, hi = divmod(i, shape[1])
        out["q"][bi, hi] = to_bf16_bits(q)
        out["k"][bi, hi] = to_bf16_bits(k)
        out["v"][bi, hi] = to_bf16_bits(v)

    _map_heads(one, len(pairs))
    return out


def _map_heads(fn, n: int) -> None:
    """Runs fn(i) for i < n; heads are independent, so a few threads share them."""
    workers = min(n, max(1, min(16, (os.cpu_count() or 1))))
    if workers == 1:
        for i in range(n):
            fn(i)
        return
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fn, range(n)))


def drift(name: str, tensors: dict, step: int, heads=None) -> dict:
    """Next step's inputs: X <- bf16(X + sigma * N(0,1)), fresh draws per step."""
    w = WORKLOADS[name]
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    out = {}
    for t, tid in (("q", _T_Q), ("k", _T_K), ("v", _T_V)):
        x = tensors[t]
        y = np.empty_like(x)
        nh = x.shape[1]

        def one(i: int, x=x, y=y, tid=tid, nh=nh) -> None:
            b, h = pairs[i]
            bi, hi = divmod(i, nh)
            noise = _rng(w.cfg_id, tid, step, b, h).standard_normal(x.shape[2:], dtype=np.float32)
            y[bi, hi] = to_bf16_bits(to_f32(x[bi, hi]) + np.float32(w.drift) * noise)

        _map_heads(one, len(pairs))
        out[t] = y
    return out


# ---------------------------------------------------------------------------
# generic inputs for parity and edge-case tests
# ---------------------------------------------------------------------------

def gaussian(shape, seed: int, scale: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """bf16 bits of mean + scale * N(0,1), drawn in independent chunks of 2^20 values."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 20

    def one(i: int) -> None:
        lo, hi = i * chunk, min(n, (i + 1) * chunk)
        x = _rng(9000, seed, i).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = to_bf16_bits(np.float32(mean) + np.float32(scale) * x)

    _map_heads(one, -(-n // chunk))
    return out.reshape(shape)


def random_perm(B: int, H: int, N: int, seed: int) -> np.ndarray:
    """Independent uniform permutations of 0..N-1 per (b, h): int32 [B, H, N]."""
    r = _rng(9100, seed)
    return np.stack([np.stack([r.permutation(N) for _ in range(H)]) for _ in range(B)]).astype(np.int32)


def random_index_sets(B: int, H: int, G: int, K: int, N: int, seed: int,
                      ascending: bool = True) -> np.ndarray:
    """Per (b, h, g) a uniform K-subset of 0..N-1: int32 [B, H, G, K]."""
    r = _rng(9200, seed)
    keys = r.random((B, H, G, N))
    sub = np.argpartition(keys, K - 1, axis=-1)[..., :K] if K < N else np.broadcast_to(
        np.arange(N), (B, H, G, N)).copy()
    if ascending:
        sub = np.sort(sub, axis=-1)
    return sub.astype(np.int32)


def stratified_index_sets(B: int, H: int, G: int, K: int, N: int, seed: int) -> np.ndarray:
    """Per (b, h, g) one uniform id in each of K equal strata of 0..N-1 (ascending,
    distinct): int32 [B, H, G, K]; cheap at full workload sizes."""
    lo = ((np.arange(K, dtype=np.int64) * N) // K).astype(np.int32)
    width = (((np.arange(1, K + 1, dtype=np.int64) * N) // K) - lo).astype(np.int32)
    widthf = width.astype(np.float32)
    out = np.empty((B * H, G, K), dtype=np.int32)

    def one(i: int) -> None:
        u = _rng(9400, seed, i).random((G, K), dtype=np.float32)
        off = (u * widthf).astype(np.int32)
        np.minimum(off, width - 1, out=off)
        out[i] = off + lo

    _map_heads(one, B * H)
    return out.reshape(B, H, G, K)


def growing_scores(N: int, D: int, seed: int, step: float, tile: int = 64):
    """bf16 bits of q, k, v [1, 1, N, D] whose scores q.k grow tile by tile.

    Every query is 3u + 0.3 N(0,1) and key j is (step * (j // tile)) u +
    0.3 N(0,1) for the unit vector u = (1, ..., 1)/sqrt(D), so with a unit
    scale the scores of key tile t sit near 3 * step * t: a later tile
    outranks all earlier ones by a wide margin.  v ~ N(0,1).
    """
    r = _rng(9400, seed)
    u = np.full(D, 1.0 / np.sqrt(D))
    q = 3.0 * u + 0.3 * r.standard_normal((1, 1, N, D))
    t = (np.arange(N) // tile).astype(np.float64)
    k = (step * t)[:, None] * u + 0.3 * r.standard_normal((1, 1, N, D))
    v = r.standard_normal((1, 1, N, D))
    return tuple(to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))


def mass_rows(rows: int, N: int, seed: int, ties: bool = True) -> np.ndarray:
    """Non-negative float32 score rows for top-K tests, optionally with many ties."""
    r = _rng(9300, seed)
    x = r.exponential(1e-3, size=(rows, N)).astype(np.float32)
    if ties:
        # quantise a third of the entries onto a coarse grid so equal values occur
        m = r.random((rows, N)) < 0.33
        x[m] = np.round(x[m] * 2e3).astype(np.float32) / np.float32(2e3)
        x[:, ::97] = 0.0
    return x
