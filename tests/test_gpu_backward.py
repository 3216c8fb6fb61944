"""GPU parity of the Main Branch backward (gradients of Eq. 8, selection fixed)
against the oracle, which recomputes the forward in fp64.

Tolerance: P and dS enter the MFMAs as bf16 (relative rounding 2^-9) and o, lse
come from the GPU forward, so each gradient element carries a relative error of a
few 1e-3 of the terms it sums; the tests allow max-abs 1e-2 and mean-abs 1e-3,
each relative to the largest reference magnitude of that gradient (at least 1:
the inputs are O(1), and a gradient that is exactly 0 in fp64 comes out at
rounding level).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def check_grads(got, ref, what, floor=1.0):
    """Max error <= 1e-2 and mean error <= 1e-3 of max(max |ref|, floor); None skips."""
    stats = {}
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        if a is None:
            continue
        a = a.cpu().double().numpy()
        scale = max(np.abs(b).max(), floor)
        err = np.abs(a - b)
        stats[name] = (float(err.max() / scale), float(err.mean() / scale))
        assert err.max() <= 1e-2 * scale, (what, name, stats[name])
        assert err.mean() <= 1e-3 * scale, (what, name, stats[name])
    return stats


def _run(msa, inp, bi_d, seed):
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi_d)
    g = torch.Generator(device=DEV).manual_seed(seed)
    dO = torch.randn(inp.q.shape, generator=g, device=DEV).to(torch.bfloat16)
    grads = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi_d)
    return dO, o, lse, grads


BWD_SHAPES = [  # N, H_q, H_kv, k
    (1000, 16, 2, 4),
    (300, 4, 2, 16),
    (1, 8, 1, 4),
    (129, 32, 1, 2),
    (2600, 16, 1, 5),
    (4096, 4, 1, 8),
    (700, 8, 8, 3),
    (900, 2, 2, 6),
    (1500, 4, 2, 7),
    (640, 1, 1, 4),
]


@pytest.mark.parametrize("N,H_q,H_kv,k", BWD_SHAPES)
def test_backward_matches_oracle(msa, N, H_q, H_kv, k):
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1700 + N, needles=1 if N >= 2000 else 0,
                              device=DEV)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, 128), k, 128)
    dO, o, lse, grads = _run(msa, inp, torch.from_numpy(bi).to(DEV), seed=N)
    torch.cuda.synchronize()
    ref = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, 128)
    check_grads(grads, ref, f"N={N} H_q={H_q} H_kv={H_kv} k={k}")


def test_backward_arbitrary_block_sets(msa):
    N, H_q, H_kv, k = 1500, 8, 2, 5
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1801, device=DEV)
    g = np.random.default_rng(8)
    B = (N + 127) // 128
    bi = np.full((N, H_kv, k), -1, dtype=np.int32)
    for i in range(N):
        for r in range(H_kv):
            c = g.choice(B, size=g.integers(0, k + 1), replace=False)
            bi[i, r, :len(c)] = c
    bi[9] = -1
    dO, o, lse, grads = _run(msa, inp, torch.from_numpy(bi).to(DEV), seed=3)
    torch.cuda.synchronize()
    ref = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, 128)
    assert torch.all(grads[0][9] == 0)
    check_grads(grads, ref, "arbitrary sets")


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_backward_end_to_end(msa, mode):
    N, H_q, H_kv, k = 3000, 16, 2, 8
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1802, mode=mode, needles=2, device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    dO, o, lse, grads = _run(msa, inp, bi, seed=4)
    torch.cuda.synchronize()
    ref = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi.cpu().numpy(), 128)
    check_grads(grads, ref, f"e2e {mode}")


def test_backward_windows_and_reruns(msa):
    """dq is bitwise reproducible across reruns and window sizes: every dQ row is one
    query's own sum.  dk and dv sum each list's rows in (query, slot) order, so a
    rerun with the same workspace reproduces them bitwise; another window size
    groups the per-window sums differently and changes them at fp32 rounding only."""
    N, H_q, H_kv, k = 2500, 8, 2, 6
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1803, needles=2, device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    dO, o, lse, g1 = _run(msa, inp, bi, seed=5)
    g3 = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi)
    wmin = msa.msa_sparse_attn_bwd_workspace(N, H_q, H_kv, k, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    g2 = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi, workspace=ws)
    g4 = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g3[0]) and torch.equal(g1[0], g2[0]), "dq"
    for name, a, b in zip(("dk", "dv"), g1[1:], g3[1:]):
        assert torch.equal(a, b), f"{name} rerun"
    for name, a, b in zip(("dk", "dv"), g2[1:], g4[1:]):
        assert torch.equal(a, b), f"{name} rerun, min workspace"
    for name, x, y in zip(("dk", "dv"), g1[1:], g2[1:]):
        rel = ((x - y).abs().max() / y.abs().max().clamp(min=1.0)).item()
        assert rel <= 1e-5, (name, rel)
    ref = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi.cpu().numpy(), 128)
    check_grads(g2, ref, "min workspace")
