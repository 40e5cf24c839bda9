"""Work and traffic accounting for the token-sparse attention path.

Conventions (they reproduce the per-layer cache sizes and FLOP counts printed
on the ai.info page, section "Main Findings", bullet on cache transfers):

  * K, the per-group KV budget at density s, is 128 * floor(s * N / 128);
  * G = ceil(N / C) query groups per head (the last one may be short);
  * KV ids are int32, the residual is bf16 with the layout of the output;
  * sparse attention costs 4 * N * K * D FLOPs per head (QK^T and PV, two
    FLOPs per multiply-add), dense attention 4 * N^2 * D;
  * the pages' kernel efficiency is speedup * s (speedup over the ideal 1/s).
"""
from __future__ import annotations


def k_from_density(s: float, N: int, multiple: int = 128) -> int:
    """Per-group KV budget K = multiple * floor(s * N / multiple), at least 1."""
    return max(1, multiple * int((s * N) // multiple))


def num_groups(N: int, C: int) -> int:
    return -(-N // C)


def sparse_flops(B: int, H: int, N: int, K: int, D: int) -> float:
    return 4.0 * B * H * N * K * D


def dense_flops(B: int, H: int, N: int, D: int) -> float:
    return 4.0 * B * H * N * N * D


def select_flops(B: int, H: int, N: int, D: int) -> float:
    """The probability-recovery pass: QK^T only, half a dense attention."""
    return 2.0 * B * H * N * N * D


def cache_bytes(N: int, H: int, D: int, K: int, C: int, B: int = 1) -> int:
    """Bytes of one layer's reusable metadata: KV ids (int32) and residual (bf16)."""
    return B * (num_groups(N, C) * K * H * 4 + N * H * D * 2)


def kernel_efficiency(speedup: float, density: float) -> float:
    """Fraction of the ideal 1/s speedup reached."""
    return speedup * density


def sparse_gather_bytes(B: int, H: int, N: int, K: int, D: int, C: int) -> float:
    """K and V rows pulled through the memory hierarchy by the sparse kernel."""
    return float(B * H * num_groups(N, C) * K * 2 * D * 2)


def sparse_compulsory_bytes(B: int, H: int, N: int, K: int, D: int, C: int,
                            residual: bool = True) -> float:
    """Bytes the sparse kernel must move at least once: Q, K, V, O (+R), ids, perm."""
    tensors = (5 if residual else 4) * B * H * N * D * 2
    return float(tensors + B * H * num_groups(N, C) * K * 4 + B * H * N * 4)
