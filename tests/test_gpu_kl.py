"""GPU parity of the KL alignment pass (Eq. 9-10) against the oracle.

The GPU pass takes the main branch's emitted lse (from msa_sparse_attn_fwd on the
GPU); the oracle computes everything itself in fp64 from the same bf16 inputs.
Tolerances (derived in the design notes): kl within 5e-4 + 2e-3 |kl|, lse_idx
within 1e-3, loss within 5e-4 + 1e-3 |loss|.
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


def _check_kl(kl, lse_idx, loss, kl_ref, li_ref, what):
    kl, lse_idx = kl.cpu().double().numpy(), lse_idx.cpu().double().numpy()
    fin = np.isfinite(li_ref)
    assert np.array_equal(np.isfinite(lse_idx), fin), what
    assert np.all(lse_idx[~fin] == -np.inf) and np.all(kl[~fin] == 0), what
    err = np.abs(kl - kl_ref)
    assert np.all(err <= 5e-4 + 2e-3 * np.abs(kl_ref)), (what, err.max())
    assert np.abs(lse_idx[fin] - li_ref[fin]).max(initial=0) <= 1e-3, what
    ref_loss = kl_ref.mean()
    assert abs(float(loss.item()) - ref_loss) <= 5e-4 + 1e-3 * abs(ref_loss), (what, float(loss.item()), ref_loss)
    # the loss is the mean of the kl the pass returned (fixed-order fp64 sum)
    assert abs(float(loss.item()) - kl.mean()) <= 1e-6 * max(1.0, abs(kl.mean())), what


KL_SHAPES = [  # N, H_q, H_kv, k
    (4096, 4, 1, 8),
    (1000, 16, 2, 4),
    (700, 8, 8, 3),
    (300, 4, 2, 16),
    (1, 8, 1, 4),
    (129, 32, 1, 2),
    (2600, 16, 1, 5),
    (3000, 8, 1, 16),
    (900, 2, 2, 6),
    (1500, 4, 2, 7),
    (512, 64, 2, 4),
]


@pytest.mark.parametrize("N,H_q,H_kv,k", KL_SHAPES)
def test_sparse_kl_on_oracle_selection(msa, N, H_q, H_kv, k):
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1100 + N, needles=1 if N >= 2000 else 0,
                              device=DEV)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, 128), k, 128)
    bi_d = torch.from_numpy(bi).to(DEV)
    _, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi_d)
    kl, lse_idx, loss = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi_d, lse)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, 128)
    _check_kl(kl, lse_idx, loss, kl_ref, li_ref, f"N={N} H_q={H_q} H_kv={H_kv} k={k}")


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_sparse_kl_end_to_end(msa, mode):
    """Selection, attention and KL all on the GPU (the oracle on the GPU's selection)."""
    N, H_q, H_kv, k = 3000, 16, 2, 8
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1201, mode=mode, needles=2, device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    _, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    kl, lse_idx, loss = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi.cpu().numpy(), 128)
    _check_kl(kl, lse_idx, loss, kl_ref, li_ref, f"e2e {mode}")


def test_sparse_kl_arbitrary_block_sets(msa):
    """-1 entries, future blocks and empty rows (kl 0, lse_idx -inf)."""
    N, H_q, H_kv, k = 1500, 8, 2, 5
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1202, device=DEV)
    g = np.random.default_rng(5)
    B = (N + 127) // 128
    bi = np.full((N, H_kv, k), -1, dtype=np.int32)
    for i in range(N):
        for r in range(H_kv):
            c = g.choice(B, size=g.integers(0, k + 1), replace=False)
            bi[i, r, :len(c)] = c
    bi[7] = -1
    bi_d = torch.from_numpy(bi).to(DEV)
    _, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi_d)
    kl, lse_idx, loss = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi_d, lse)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, 128)
    assert np.all(np.isinf(li_ref[7]))
    _check_kl(kl, lse_idx, loss, kl_ref, li_ref, "arbitrary sets")


def test_sparse_kl_windows_and_reruns_are_bitwise_identical(msa):
    N, H_q, H_kv, k = 2500, 8, 2, 6
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1203, needles=2, device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    _, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    r1 = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse)
    wmin = msa.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, k, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    r2 = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, workspace=ws)
    r3 = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse)
    torch.cuda.synchronize()
    for a, b in ((r1, r2), (r1, r3)):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_sparse_kl_empty(msa):
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    qi = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    ki = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    bi = torch.empty((0, 2, 4), dtype=torch.int32, device=DEV)
    lse = torch.empty((0, 8), dtype=torch.float32, device=DEV)
    kl, li, loss = msa.msa_sparse_kl_fwd(q, kv, qi, ki, bi, lse)
    assert kl.shape == (0, 2) and li.shape == (0, 2)


def _check_lse_idx(got, li_ref, what, tol=1e-3):
    got = got.cpu().double().numpy()
    fin = np.isfinite(li_ref)
    assert np.array_equal(np.isfinite(got), fin), what
    assert np.all(got[~fin] == -np.inf), what
    assert np.abs(got[fin] - li_ref[fin]).max(initial=0) <= tol, (what, np.abs(got[fin] - li_ref[fin]).max())


@pytest.mark.parametrize("N,H_q,H_kv,k,B_k", [s + (128,) for s in KL_SHAPES[:8]] + [(2600, 16, 2, 8, 64),
                                                                                     (700, 8, 1, 16, 64)])
def test_forward_emits_lse_idx(msa, N, H_q, H_kv, k, B_k):
    """LSE_idx from the forward (msa_sparse_attn_fwd_lse_idx) against the oracle's, and
    the forward's o / lse bit-identical to the plain forward."""
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1300 + N, needles=1 if N >= 2000 else 0,
                              device=DEV, B_k=B_k)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=B_k)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=B_k)
    o2, lse2, li = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi, B_k=B_k)
    _, li_kl, _ = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, B_k=B_k)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    _, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi.cpu().numpy(), B_k)
    _check_lse_idx(li, li_ref, f"N={N} H_q={H_q} H_kv={H_kv} k={k} B_k={B_k}")
    _check_lse_idx(li, li_kl.cpu().double().numpy(), "against the KL pass", tol=1e-5)


def test_forward_lse_idx_arbitrary_block_sets_and_windows(msa):
    """-1 entries, future blocks and empty rows (-inf), and the minimum workspace's
    query windows giving the same bits."""
    N, H_q, H_kv, k = 1500, 8, 2, 5
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1302, device=DEV)
    g = np.random.default_rng(6)
    B = (N + 127) // 128
    bi = np.full((N, H_kv, k), -1, dtype=np.int32)
    for i in range(N):
        for r in range(H_kv):
            c = g.choice(B, size=g.integers(0, k + 1), replace=False)
            bi[i, r, :len(c)] = c
    bi[7] = -1
    bi_d = torch.from_numpy(bi).to(DEV)
    _, _, li = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi_d)
    wmin = msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    _, _, li2 = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi_d, workspace=ws)
    torch.cuda.synchronize()
    _, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, 128)
    assert np.all(np.isinf(li_ref[7]))
    _check_lse_idx(li, li_ref, "arbitrary sets")
    assert torch.equal(li, li2)


@pytest.mark.parametrize("N,H_q,H_kv,k,B_k", [s + (128,) for s in KL_SHAPES] + [(2600, 16, 2, 8, 64),
                                                                                (700, 8, 1, 16, 64)])
def test_kl_from_forward_lse_idx(msa, N, H_q, H_kv, k, B_k):
    """The KL value with LSE_idx given (from the forward) against the oracle, and
    within fp32 rounding of the pass that computes LSE_idx itself."""
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1400 + N, needles=1 if N >= 2000 else 0,
                              device=DEV, B_k=B_k)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=B_k)
    _, lse, li = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi, B_k=B_k)
    kl, loss = msa.msa_sparse_kl_fwd_from_lse_idx(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, li, B_k=B_k)
    kl2, _, loss2 = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, B_k=B_k)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi.cpu().numpy(), B_k)
    _check_kl(kl, li, loss, kl_ref, li_ref, f"from lse_idx N={N} H_q={H_q} H_kv={H_kv} k={k} B_k={B_k}")
    d = (kl.double() - kl2.double()).abs()
    assert float(d.max()) <= 1e-4 + 1e-4 * float(kl2.double().abs().max())


def test_kl_from_lse_idx_arbitrary_block_sets(msa):
    """-1 entries, future blocks and empty rows: kl 0 where LSE_idx is -inf."""
    N, H_q, H_kv, k = 1500, 8, 2, 5
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1402, device=DEV)
    g = np.random.default_rng(7)
    B = (N + 127) // 128
    bi = np.full((N, H_kv, k), -1, dtype=np.int32)
    for i in range(N):
        for r in range(H_kv):
            c = g.choice(B, size=g.integers(0, k + 1), replace=False)
            bi[i, r, :len(c)] = c
    bi[7] = -1
    bi_d = torch.from_numpy(bi).to(DEV)
    _, lse, li = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi_d)
    kl, loss = msa.msa_sparse_kl_fwd_from_lse_idx(inp.q, inp.k, inp.q_idx, inp.k_idx, bi_d, lse, li)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, 128)
    _check_kl(kl, li, loss, kl_ref, li_ref, "from lse_idx, arbitrary sets")
