"""Benchmark of the MSA forward path on one MI355X (filled in below)."""
from __future__ import annotations


def flops_gqa_eq12(N: int, H_q: int, d_h: int) -> int:
    """Dense causal GQA attention FLOPs as counted by Eq. 12 (MSA paper review, section 3)."""
    return 2 * H_q * d_h * N * N


def flops_msa_eq12(N: int, H_q: int, H_kv: int, d_h: int, d_idx: int, B_k: int, k: int) -> int:
    """MSA FLOPs as counted by Eq. 12: index branch H_kv d_idx N^2 + main branch 4 H_q d_h N k B_k."""
    return H_kv * d_idx * N * N + 4 * H_q * d_h * N * k * B_k
