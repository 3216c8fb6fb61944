"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's formula: each compares it with a closed
form, an invariant, a special case that reduces to a textbook routine, a
brute-force enumeration on a tiny input, or a hand-derived golden value.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


# --- Eq. 4: block partition ---------------------------------------------------------------

def test_partition_counts_match_workloads():
    # Block counts printed for the workloads: 32 / 256 / 1024 / 8192 blocks.
    for name, B in (("c0", 32), ("c1", 256), ("c2", 1024), ("c4", 8192)):
        c = synth.CONFIGS[name]
        assert oracle.num_blocks(c.N, c.B_k) == B == c.B
    assert oracle.num_blocks(129, 128) == 2
    assert oracle.num_blocks(128, 128) == 1
    assert oracle.num_blocks(1, 128) == 1


# --- Eq. 6: index scores and causal block max-pool ----------------------------------------

def test_block_scores_one_hot_closed_form():
    """K_idx[j] = c_j e_0, Q_idx[i, r] = a_r e_0  =>  S_ij = a_r c_j / sqrt(d_idx)."""
    N, H_kv, d_idx, B_k = 11, 2, 64, 4
    c = [0.5, -1.0, 2.0, 0.25, -3.0, 1.5, 0.75, -0.5, 4.0, 1.0, -2.5]
    a = [1.5, -2.0]
    k_idx = torch.zeros(N, d_idx)
    k_idx[:, 0] = torch.tensor(c)
    q_idx = torch.zeros(N, H_kv, d_idx)
    for r in range(H_kv):
        q_idx[:, r, 0] = a[r]
    M = oracle.block_scores(bf16(q_idx), bf16(k_idx), B_k)
    B = 3
    assert M.shape == (N, H_kv, B)
    for i in range(N):
        for r in range(H_kv):
            for b in range(B):
                visible = [j for j in range(b * B_k, min((b + 1) * B_k, N)) if j <= i]
                if not visible:
                    assert M[i, r, b] == -math.inf
                else:
                    assert M[i, r, b] == max(a[r] * c[j] for j in visible) / 8.0


def test_block_scores_scale_does_not_change_ranking():
    """Multiplying every index key by 2 doubles M exactly (power-of-two scaling)."""
    q = rand_bf16((40, 2, 64), 1)
    kk = rand_bf16((40, 64), 2)
    M1 = oracle.block_scores(q, kk, 8)
    M2 = oracle.block_scores(q, (kk.float() * 2).to(torch.bfloat16), 8)
    fin = np.isfinite(M1)
    assert np.array_equal(np.isfinite(M2), fin)
    np.testing.assert_array_equal(M2[fin], 2 * M1[fin])


# --- Eq. 7: Top-k with the forced local block ---------------------------------------------

def _golden_topk_cases():
    cases = []
    with open(os.path.join(GOLDEN, "topk_rules.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, params, mvals, exp = [p.strip() for p in line.split("|")]
            i, B_k, k = map(int, params.split())
            M = [float(x) for x in mvals.split()]
            cases.append((name, i, B_k, k, M, [int(x) for x in exp.split()]))
    return cases


@pytest.mark.parametrize("case", _golden_topk_cases(), ids=lambda c: c[0])
def test_topk_golden(case):
    name, i, B_k, k, M, expected = case
    Marr = np.array(M, dtype=np.float64).reshape(1, 1, -1)
    got = oracle.topk(Marr, k, B_k, rows=[i])
    assert got[0, 0].tolist() == expected


def _brute_topk(Mrow, i, B_k, k):
    bl = i // B_k
    if bl + 1 <= k:
        chosen = list(range(bl + 1))
    else:
        order = sorted(range(bl), key=lambda b: (-Mrow[b], b))
        chosen = sorted(order[:k - 1] + [bl])
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_full_sort(seed):
    """Brute force: sort every causal block by (score desc, index asc); ties are frequent."""
    rng = np.random.default_rng(seed)
    N, H_kv, B_k = 90, 3, 4
    B = oracle.num_blocks(N, B_k)
    M = rng.integers(-3, 4, size=(N, H_kv, B)).astype(np.float64) * 0.5  # many exact ties
    for k in (1, 2, 5, 8, 23, 30):
        got = oracle.topk(M, k, B_k)
        for i in range(N):
            for r in range(H_kv):
                assert got[i, r].tolist() == _brute_topk(M[i, r], i, B_k, k), (k, i, r)


def test_local_block_always_selected_and_exp_free():
    inp = synth.small_prefill(N=700, H_q=4, H_kv=2, k=4, seed=5, B_k=32)
    M = oracle.block_scores(inp.q_idx, inp.k_idx, 32)
    bi = oracle.topk(M, 4, 32)
    for i in range(700):
        for r in range(2):
            assert i // 32 in bi[i, r]
            row = [b for b in bi[i, r] if b >= 0]
            assert row == sorted(row) and len(set(row)) == len(row)
            assert max(row) == i // 32
    # Exp-free selection: softmax over the causal blocks is order-preserving, so
    # selecting on exp(M) / sum exp(M) gives the same blocks.
    P = np.exp(M - np.nanmax(np.where(np.isfinite(M), M, np.nan), axis=2, keepdims=True))
    P = P / P.sum(axis=2, keepdims=True)
    np.testing.assert_array_equal(oracle.topk(P, 4, 32), bi)


def test_fewer_than_k_blocks_padding():
    inp = synth.small_prefill(N=300, H_q=2, H_kv=1, k=8, seed=9, B_k=64)
    M = oracle.block_scores(inp.q_idx, inp.k_idx, 64)
    bi = oracle.topk(M, 8, 64)
    for i in range(300):
        bl = i // 64
        assert bi[i, 0].tolist() == list(range(bl + 1)) + [-1] * (8 - bl - 1)


# --- Eq. 8: attention over the chosen blocks ---------------------------------------------

def _dense_causal_gqa(q, k, v, scale):
    """Textbook causal GQA (Eq. 1) in float64 with torch: adjacent heads share a KV head."""
    qd, kd, vd = q.double(), k.double(), v.double()
    N, H_q, _ = qd.shape
    G = H_q // kd.shape[1]
    kr = kd.repeat_interleave(G, dim=1)
    vr = vd.repeat_interleave(G, dim=1)
    s = torch.einsum("ihd,jhd->hij", qd, kr) * scale
    mask = torch.triu(torch.ones(N, N, dtype=torch.bool), diagonal=1)
    s = s.masked_fill(mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("hij,jhd->ihd", p, vr)
    return o.numpy(), lse.T.numpy()


@pytest.mark.parametrize("N,H_q,H_kv,B_k,d_h", [(37, 4, 2, 8, 16), (64, 6, 3, 16, 32), (50, 8, 1, 4, 8)])
def test_k_covering_all_blocks_is_dense_gqa(N, H_q, H_kv, B_k, d_h):
    q = rand_bf16((N, H_q, d_h), 11)
    k = rand_bf16((N, H_kv, d_h), 12)
    v = rand_bf16((N, H_kv, d_h), 13)
    q_idx = rand_bf16((N, H_kv, 16), 14)
    k_idx = rand_bf16((N, 16), 15)
    B = oracle.num_blocks(N, B_k)
    M = oracle.block_scores(q_idx, k_idx, B_k)
    bi = oracle.topk(M, B, B_k)  # k = B: every causal block
    scale = 1.0 / math.sqrt(d_h)
    o, lse = oracle.sparse_attn(q, k, v, bi, B_k, scale)
    o_ref, lse_ref = _dense_causal_gqa(q, k, v, scale)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    """With V = 1 the output is the sum of the softmax weights."""
    inp = synth.small_prefill(N=500, H_q=4, H_kv=2, k=3, seed=21, B_k=32, d_h=32)
    v = torch.ones_like(inp.v)
    M = oracle.block_scores(inp.q_idx, inp.k_idx, 32)
    bi = oracle.topk(M, 3, 32)
    o, _ = oracle.sparse_attn(inp.q, inp.k, v, bi, 32)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-12)


def test_uniform_scores_closed_form():
    """q = 0: every score is 0, so lse = ln|T| and o is the mean of V over T."""
    N, H_q, H_kv, d_h, B_k = 45, 2, 1, 8, 8
    q = torch.zeros(N, H_q, d_h, dtype=torch.bfloat16)
    k = rand_bf16((N, H_kv, d_h), 31)
    v = rand_bf16((N, H_kv, d_h), 32)
    rows = [3, 17, 44, 40]
    sets = [[0, -1, -1], [0, 2, -1], [1, 3, 5], [5, 0, 2]]
    bi = np.array(sets, dtype=np.int32).reshape(4, 1, 3)
    o, lse = oracle.sparse_attn(q, k, v, bi, B_k, rows=rows)
    vd = v.double().numpy()
    for n, i in enumerate(rows):
        T = [j for j in range(N) if j <= i and (j // B_k) in sets[n]]
        for h in range(H_q):
            assert lse[n, h] == pytest.approx(math.log(len(T)), abs=1e-12)
            np.testing.assert_allclose(o[n, h], vd[T, 0].mean(0), atol=1e-12)


def test_lse_merge_of_disjoint_partials():
    """Two-phase combine identity: attention over A u B equals the LSE merge of A and B."""
    inp = synth.small_prefill(N=600, H_q=4, H_kv=2, k=6, seed=41, B_k=32, d_h=32)
    rows = [599, 450, 333, 100]
    A = np.array([[0, 3, 7, -1], [1, 2, 5, 9], [2, 4, -1, -1], [0, 1, -1, -1]], np.int32)
    Bs = np.array([[9, 12, 18, -1], [11, 13, 14, -1], [6, 8, 10, -1], [3, -1, -1, -1]], np.int32)
    A = np.repeat(A[:, None, :], 2, axis=1)
    Bs = np.repeat(Bs[:, None, :], 2, axis=1)
    U = np.concatenate([A, Bs], axis=2)
    oA, lA = oracle.sparse_attn(inp.q, inp.k, inp.v, A, 32, rows=rows)
    oB, lB = oracle.sparse_attn(inp.q, inp.k, inp.v, Bs, 32, rows=rows)
    oU, lU = oracle.sparse_attn(inp.q, inp.k, inp.v, U, 32, rows=rows)
    l = np.logaddexp(lA, lB)
    o = np.exp(lA - l)[..., None] * oA + np.exp(lB - l)[..., None] * oB
    np.testing.assert_allclose(lU, l, atol=1e-12)
    np.testing.assert_allclose(oU, o, atol=1e-12)


def test_block_order_and_empty_sets():
    inp = synth.small_prefill(N=300, H_q=2, H_kv=1, k=4, seed=51, B_k=16, d_h=16)
    rows = [299, 150]
    bi = np.array([[[0, 5, 9, 18]], [[1, 2, 9, -1]]], np.int32)
    perm = bi[:, :, ::-1].copy()
    o1, l1 = oracle.sparse_attn(inp.q, inp.k, inp.v, bi, 16, rows=rows)
    o2, l2 = oracle.sparse_attn(inp.q, inp.k, inp.v, perm, 16, rows=rows)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    # A set holding only future blocks (or nothing) has no visible token.
    empty = np.array([[[-1, -1, -1, -1]], [[10, 12, -1, -1]]], np.int32)
    o3, l3 = oracle.sparse_attn(inp.q, inp.k, inp.v, empty, 16, rows=rows)
    assert np.all(l3 == -np.inf) and np.all(o3 == 0)


# --- Decode --------------------------------------------------------------------------------

def test_decode_equals_last_prefill_row():
    lengths = [130, 64, 257]
    d = synth.make_decode(synth.DecodeConfig("t", batch=3, H_q=4, H_kv=2, k=3, len_lo_blocks=1,
                                             len_hi_blocks=1, B_k=32, d_h=32, d_idx=16, seed=7),
                          lengths=lengths)
    bi, o, lse, M = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, 3, 32,
                                  want_scores=True)
    cu = d.cu_seqlens.tolist()
    for s, L in enumerate(lengths):
        sl = slice(cu[s], cu[s + 1])
        q_idx = d.k_idx_cache.new_zeros((L, 2, 16))
        q_idx[L - 1] = d.q_idx[s]
        q = d.k_cache.new_zeros((L, 4, 32))
        q[L - 1] = d.q[s]
        Mp = oracle.block_scores(q_idx, d.k_idx_cache[sl], 32, rows=[L - 1])
        bp = oracle.topk(Mp, 3, 32, rows=[L - 1])
        op, lp = oracle.sparse_attn(q, d.k_cache[sl], d.v_cache[sl], bp, 32, rows=[L - 1])
        B = Mp.shape[2]
        np.testing.assert_array_equal(M[s, :, :B], Mp[0])
        np.testing.assert_array_equal(bi[s], bp[0])
        np.testing.assert_array_equal(o[s], op[0])
        np.testing.assert_array_equal(lse[s], lp[0])


# --- Eq. 12: FLOP accounting used by the benchmark ----------------------------------------

def test_eq12_ratio_matches_printed_28_4():
    import bench
    with open(os.path.join(GOLDEN, "eq12_flops.txt")) as f:
        lines = [l for l in f if l.strip() and not l.startswith("#")]
    for line in lines:
        params, printed, exact = [p.strip() for p in line.split("|")]
        N, H_q, H_kv, d_h, d_idx, B_k, k = map(int, params.split())
        num = bench.flops_gqa_eq12(N, H_q, d_h)
        den = bench.flops_msa_eq12(N, H_q, H_kv, d_h, d_idx, B_k, k)
        assert Fraction(num, den) == Fraction(exact)
        assert round(num / den, 1) == float(printed)


def test_decode_attn_on_given_selection_equals_decode():
    lengths = [300, 1000]
    d = synth.make_decode(synth.DecodeConfig("t", batch=2, H_q=4, H_kv=2, k=3, len_lo_blocks=1,
                                             len_hi_blocks=1, seed=9), lengths=lengths)
    bi, o, lse = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, 3, 128)
    o2, l2 = oracle.decode_attn(d.q, d.k_cache, d.v_cache, d.cu_seqlens, bi, 128)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)


# --- Packed sequences --------------------------------------------------------------------

def test_varlen_first_sequence_equals_causal_prefix():
    # Causality makes the rows of the first packed sequence a prefix problem: the
    # unpacked oracle over the concatenation gives them the same selection and output
    # when the first sequence ends on a block boundary.  Other sequences must differ
    # from the concatenated run (they may not see earlier sequences).
    lengths = [256, 300, 0, 77]
    p = synth.packed_prefill(lengths, H_q=4, H_kv=2, k=3, seed=21)
    bi = oracle.index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, 3, 128)
    o, lse = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, 128)
    T = sum(lengths)
    M_all = oracle.block_scores(p.q_idx, p.k_idx, 128)
    bi_all = oracle.topk(M_all, 3, 128)
    np.testing.assert_array_equal(bi[:256], bi_all[:256])
    o_all, l_all = oracle.sparse_attn(p.q, p.k, p.v, bi_all[:256], 128, rows=range(256))
    np.testing.assert_array_equal(o[:256], o_all)
    np.testing.assert_array_equal(lse[:256], l_all)
    # Second sequence: its local block numbering restarts at 0.
    pos = np.arange(300)
    assert np.all((bi[256:556] == (pos // 128)[:, None, None]).any(axis=2))
    # Sequence 3 (77 tokens, one block): everything selects block 0 and pads.
    assert np.all(bi[556:, :, 0] == 0) and np.all(bi[556:, :, 1:] == -1)
    assert bi.shape == (T, 2, 3)


def test_varlen_sequence_is_independent_of_neighbours():
    # Replacing every other sequence's tokens leaves a sequence's results unchanged.
    lengths = [200, 333, 129]
    a = synth.packed_prefill(lengths, H_q=4, H_kv=2, k=2, seed=5)
    b = synth.packed_prefill(lengths, H_q=4, H_kv=2, k=2, seed=5)
    for name in ("q", "k", "v", "q_idx", "k_idx"):
        t = getattr(b, name)
        t[:200] = -t[:200]
        t[533:] = 0.5 * t[533:]
    ra = oracle.index_topk_varlen(a.q_idx, a.k_idx, a.cu_seqlens, 2, 128)
    rb = oracle.index_topk_varlen(b.q_idx, b.k_idx, b.cu_seqlens, 2, 128)
    np.testing.assert_array_equal(ra[200:533], rb[200:533])
    oa, la = oracle.sparse_attn_varlen(a.q, a.k, a.v, ra, a.cu_seqlens, 128)
    ob, lb = oracle.sparse_attn_varlen(b.q, b.k, b.v, rb, b.cu_seqlens, 128)
    np.testing.assert_array_equal(oa[200:533], ob[200:533])
    np.testing.assert_array_equal(la[200:533], lb[200:533])
    assert not np.array_equal(oa[:200], ob[:200])


# --- Eq. 9-10: KL alignment ---------------------------------------------------------------

def _bf(a):
    return torch.tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def test_kl_zero_when_index_scores_equal_main_scores():
    # q and k live in the first 64 dims, the index inputs are those same 64 dims and
    # the main scale is 1/sqrt(64): every index score equals every main score, and
    # the two heads of the group are identical, so the teacher equals the index
    # distribution and KL = 0; the index log partition is then the main lse.
    N, d = 700, 64
    g = torch.Generator().manual_seed(31)
    q0 = torch.randn(N, 1, d, generator=g)
    k0 = torch.randn(N, 1, d, generator=g)
    q = torch.zeros(N, 2, 128)
    q[:, 0, :d] = q0[:, 0]
    q[:, 1, :d] = q0[:, 0]
    k = torch.zeros(N, 1, 128)
    k[:, 0, :d] = k0[:, 0]
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    q_idx, k_idx = q0.to(torch.bfloat16), k0[:, 0].to(torch.bfloat16)
    bi = oracle.topk(oracle.block_scores(q_idx, k_idx, 128), 3, 128)
    kl, lse_idx = oracle.sparse_kl(q, k, q_idx, k_idx, bi, 128, scale=0.125)
    assert np.max(np.abs(kl)) < 1e-12
    _, lse = oracle.sparse_attn(q, k, k, bi, 128, scale=0.125)
    np.testing.assert_allclose(lse_idx[:, 0], lse[:, 0], rtol=0, atol=1e-12)


def test_kl_closed_form_mean_of_two_heads():
    # Uniform index scores (k_idx = 0): P_idx = 1/n.  Main scores take two levels:
    # head h scores alpha_h on the first m tokens and 0 elsewhere (scale 1), so each
    # head's softmax and their mean have closed forms, and so has the KL.
    N, n, m = 256, 256, 32
    alphas = (1.0, 2.0)
    q = np.zeros((N, 2, 128), np.float32)
    k = np.zeros((N, 1, 128), np.float32)
    q[:, 0, 0], q[:, 1, 0] = alphas
    k[:m, 0, 0] = 1.0
    q_idx = np.ones((N, 1, 64), np.float32)
    k_idx = np.zeros((N, 64), np.float32)
    bi = np.array([[[0, 1]]], np.int32)
    kl, lse_idx = oracle.sparse_kl(_bf(q), _bf(k), _bf(q_idx), _bf(k_idx), bi, 128, scale=1.0, rows=[N - 1])
    pa = sum(math.exp(a) / (m * math.exp(a) + n - m) for a in alphas) / 2
    pb = sum(1.0 / (m * math.exp(a) + n - m) for a in alphas) / 2
    want = m * pa * math.log(n * pa) + (n - m) * pb * math.log(n * pb)
    assert abs(kl[0, 0] - want) < 1e-12
    assert abs(lse_idx[0, 0] - math.log(n)) < 1e-12


def test_kl_token_set_is_causal_and_selected():
    # With all scores zero both distributions are uniform over the selected causal
    # tokens: KL = 0 and the index log partition is log |T|.
    N = 300
    z3 = _bf(np.zeros((N, 1, 128)))
    q_idx, k_idx = _bf(np.zeros((N, 1, 64))), _bf(np.zeros((N, 64)))
    rows = [200, 200, 200, 5, 299]
    bi = np.array([[[0, 1, -1]], [[1, 7, -1]], [[2, 0, -1]], [[-1, -1, -1]], [[2, 1, 0]]], np.int32)
    kl, lse_idx = oracle.sparse_kl(z3, z3, q_idx, k_idx, bi, 128, rows=rows)
    sizes = [201, 73, 128, 0, 300]
    for t, n in enumerate(sizes):
        if n == 0:
            assert kl[t, 0] == 0 and lse_idx[t, 0] == -np.inf
        else:
            assert abs(kl[t, 0]) < 1e-12
            assert abs(lse_idx[t, 0] - math.log(n)) < 1e-12


def test_kl_is_nonnegative_and_groups_are_separate():
    inp = synth.small_prefill(N=900, H_q=8, H_kv=2, k=3, seed=17)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, 128), 3, 128)
    kl, lse_idx = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, 128)
    assert np.all(kl >= -1e-12) and np.all(np.isfinite(lse_idx))
    assert kl[1:].mean() > 0.05  # unrelated distributions differ
    # Group 1 alone (its heads, its KV head, its index query) gives the same numbers.
    kl1, li1 = oracle.sparse_kl(inp.q[:, 4:], inp.k[:, 1:], inp.q_idx[:, 1:], inp.k_idx, bi[:, 1:], 128)
    np.testing.assert_array_equal(kl1[:, 0], kl[:, 1])
    np.testing.assert_array_equal(li1[:, 0], lse_idx[:, 1])


# --- Paged FP8 decode ------------------------------------------------------------------------

def test_fp8_e4m3_decoding():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()  # the library's own decoding
    got = np.array([oracle.fp8_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    np.testing.assert_array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    # format definition: 1.0, the largest finite 448, the smallest subnormal 2^-9,
    # the smallest normal 2^-6, and the sign bit
    assert (got[0x38], got[0x7E], got[0x01], got[0x08], got[0xB8]) == (1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0)


def _exact_fp8_decode_case(lengths, seed):
    """A decode case whose bf16 K/V hold exactly FP8-representable values, with the
    paged FP8 copy of it (scales 1)."""
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=4, H_kv=2, k=3, len_lo_blocks=1, len_hi_blocks=1,
                             seed=seed)
    d = synth.make_decode(cfg, lengths=lengths)
    for t in (d.k_cache, d.v_cache):
        t.copy_(t.float().to(torch.float8_e4m3fn).float().to(torch.bfloat16))
    return cfg, d


def _paged_copy(d, B_k, perm_seed, k_div=1.0, v_div=1.0):
    nblk = [(L + B_k - 1) // B_k for L in d.lengths]
    P = sum(nblk) + 2
    perm = np.random.default_rng(perm_seed).permutation(P)
    H_kv, d_h = d.k_cache.shape[1], d.k_cache.shape[2]
    kp = torch.zeros((P, B_k, H_kv, d_h), dtype=torch.uint8)
    vp = torch.zeros_like(kp)
    kip = torch.zeros((P, B_k, d.k_idx_cache.shape[1]), dtype=torch.bfloat16)
    table = np.full((len(d.lengths), max(nblk)), -1, np.int32)
    cu = d.cu_seqlens.tolist()
    kq = (d.k_cache.float() / k_div).to(torch.float8_e4m3fn).view(torch.uint8)
    vq = (d.v_cache.float() / v_div).to(torch.float8_e4m3fn).view(torch.uint8)
    n = 0
    for s, L in enumerate(d.lengths):
        for b in range(nblk[s]):
            p = int(perm[n])
            n += 1
            table[s, b] = p
            t0, t1 = cu[s] + b * B_k, min(cu[s] + (b + 1) * B_k, cu[s + 1])
            kp[p, :t1 - t0], vp[p, :t1 - t0] = kq[t0:t1], vq[t0:t1]
            kip[p, :t1 - t0] = d.k_idx_cache[t0:t1]
    return kp, vp, kip, table


def test_paged_fp8_decode_equals_contiguous_decode():
    # Exactly representable K/V, scales 1, pages in a shuffled order: the paged FP8
    # decode must reproduce the contiguous bf16 decode bit for bit.
    lengths = [130, 64, 257, 1]
    cfg, d = _exact_fp8_decode_case(lengths, 41)
    kp, vp, kip, table = _paged_copy(d, 128, 5)
    ref = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, 3, 128, want_scores=True)
    got = oracle.decode_paged(d.q, d.q_idx, kp, vp, 1.0, 1.0, kip, table, lengths, 3, 128, want_scores=True)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


def test_paged_fp8_scales_multiply_keys_and_values():
    # Codes of 2K and 4V with k_scale 1/2 and v_scale 1/4 describe the same K and V
    # (scaling up by powers of two keeps every value exact).
    lengths = [300, 129]
    cfg, d = _exact_fp8_decode_case(lengths, 43)
    kp, vp, kip, table = _paged_copy(d, 128, 6, k_div=0.5, v_div=0.25)
    ref = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, 3, 128)
    got = oracle.decode_paged(d.q, d.q_idx, kp, vp, 0.5, 0.25, kip, table, lengths, 3, 128)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)


# --- Backward of Eq. 8 -----------------------------------------------------------------------

def _masked_attention_autograd(q, k, v, dO, bi, B_k, scale):
    """Eq. 8 as dense attention with the selection as a mask, differentiated by torch's
    autograd in fp64 (an independent implementation of the same gradients)."""
    N, H_q, d_h = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    qd = q.double().clone().requires_grad_(True)
    kd = k.double().clone().requires_grad_(True)
    vd = v.double().clone().requires_grad_(True)
    i = torch.arange(N).view(N, 1)
    j = torch.arange(N).view(1, N)
    outs = []
    for h in range(H_q):
        r = h // G
        sel = torch.from_numpy(bi[:, r, :].astype(np.int64))  # [N, kk]
        chosen = torch.zeros(N, (N + B_k - 1) // B_k + 1, dtype=torch.bool)
        chosen.scatter_(1, torch.where(sel >= 0, sel, chosen.shape[1] - 1), True)
        chosen[:, -1] = False
        mask = chosen[:, (j // B_k).view(-1)].view(N, N) & (j <= i)
        s = (qd[:, h] @ kd[:, r].T) * scale
        s = s.masked_fill(~mask, float("-inf"))
        p = torch.softmax(s, dim=1)
        p = torch.nan_to_num(p, nan=0.0)
        outs.append(p @ vd[:, r])
    o = torch.stack(outs, dim=1)
    (o * dO.double()).sum().backward()
    return qd.grad.numpy(), kd.grad.numpy(), vd.grad.numpy()


@pytest.mark.parametrize("N,H_q,H_kv,k,B_k", [(300, 4, 2, 2, 64), (260, 2, 1, 3, 128), (129, 4, 4, 1, 32)])
def test_attention_backward_matches_autograd(N, H_q, H_kv, k, B_k):
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=60 + N, B_k=B_k)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, B_k), k, B_k)
    bi[7] = -1  # a row with no token: no gradient
    g = torch.Generator().manual_seed(N)
    dO = torch.randn(N, H_q, 128, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    got = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, B_k)
    ref = _masked_attention_autograd(inp.q, inp.k, inp.v, dO, bi, B_k, scale)
    for a, b, name in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11, err_msg=name)


def test_attention_backward_finite_differences():
    # Directional derivatives of L = <dO, o> (the forward oracle) against the gradients.
    N, H_q, H_kv, k, B_k = 40, 2, 1, 2, 16
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=71, B_k=B_k, d_h=128)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, B_k), k, B_k)
    g = torch.Generator().manual_seed(5)
    dO = torch.randn(N, H_q, 128, generator=g).to(torch.bfloat16)
    dq, dk, dv = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, B_k)
    dOd = dO.double().numpy()

    def loss(q, kk, v):
        o, _ = oracle.sparse_attn(q, kk, v, bi, B_k)
        return float((o * dOd).sum())

    # Inputs are bf16: perturb along directions of exactly representable steps and
    # compare with the exact central difference of a quadratic fit (eps small).
    rng = np.random.default_rng(1)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        base = getattr(inp, name).float()
        direction = torch.from_numpy(rng.choice([-1.0, 1.0], size=tuple(base.shape)).astype(np.float32))
        eps = 2.0 ** -6
        args_p = {n: getattr(inp, n) for n in ("q", "k", "v")}
        args_m = dict(args_p)
        args_p[name] = (base + eps * direction).to(torch.bfloat16)
        args_m[name] = (base - eps * direction).to(torch.bfloat16)
        # the perturbation must be exact in bf16 for the difference to mean anything
        step = (args_p[name].double() - args_m[name].double()) / 2
        fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / 2
        lin = float((grad * step.numpy()).sum())
        assert abs(fd - lin) <= 2e-3 * max(1.0, abs(lin)), (name, fd, lin)


@pytest.mark.parametrize("N,H_q,H_kv,k,B_k", [(300, 4, 2, 2, 64), (700, 8, 2, 3, 128)])
def test_restricted_backward_matches_autograd(N, H_q, H_kv, k, B_k):
    """dq on chosen rows and dk, dv of one key block (the checks used at full size)
    against torch fp64 autograd of the dense masked attention, with arbitrary
    selections (-1, repeats of nothing, future blocks) on some rows."""
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=80 + N, B_k=B_k)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, B_k), k, B_k)
    bi[5] = -1
    bi[N - 3, 0, 0] = (N - 1) // B_k  # a block reaching past the row (causal: no tokens)
    g = torch.Generator().manual_seed(N + 1)
    dO = torch.randn(N, H_q, 128, generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(128)
    ref_dq, ref_dk, ref_dv = _masked_attention_autograd(inp.q, inp.k, inp.v, dO, bi, B_k, scale)
    rows = np.array([0, 5, 7, B_k - 1, B_k, N // 2, N - 3, N - 1])
    nb = (N + B_k - 1) // B_k
    for kb, r in ((0, 0), (nb // 2, H_kv - 1), (nb - 1, 0)):
        dq, (dk, dv) = oracle.sparse_attn_bwd_part(inp.q, inp.k, inp.v, dO, bi, B_k, rows=rows, key_block=kb, group=r)
        np.testing.assert_allclose(dq, ref_dq[rows], rtol=1e-9, atol=1e-11, err_msg="dq rows")
        j0, j1 = kb * B_k, min(N, (kb + 1) * B_k)
        np.testing.assert_allclose(dk[:j1 - j0], ref_dk[j0:j1, r], rtol=1e-9, atol=1e-11, err_msg=f"dk block {kb}")
        np.testing.assert_allclose(dv[:j1 - j0], ref_dv[j0:j1, r], rtol=1e-9, atol=1e-11, err_msg=f"dv block {kb}")
        assert np.all(dk[j1 - j0:] == 0) and np.all(dv[j1 - j0:] == 0)


def test_restricted_backward_equals_full_oracle():
    N, H_q, H_kv, k, B_k = 1000, 4, 2, 4, 128
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=91, B_k=B_k, needles=1)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, B_k), k, B_k)
    g = torch.Generator().manual_seed(92)
    dO = torch.randn(N, H_q, 128, generator=g).to(torch.bfloat16)
    dq_f, dk_f, dv_f = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, B_k)
    rows = np.arange(0, N, 37)
    dq, (dk, dv) = oracle.sparse_attn_bwd_part(inp.q, inp.k, inp.v, dO, bi, B_k, rows=rows, key_block=3, group=1)
    np.testing.assert_allclose(dq, dq_f[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, dk_f[384:512, 1], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dv, dv_f[384:512, 1], rtol=1e-9, atol=1e-12)
