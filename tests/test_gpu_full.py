"""GPU parity at the full workload sizes (32K, 128K and 1M prefill, 128K with B_k = 64,
a packed batch of 128K tokens; 64-sequence decode, contiguous and paged FP8; the KL
pass and the backward at 128K),
in the launch configuration the benchmark times, on sampled rows the oracle computes
one by one.  The sample holds rows with fewer than k causal blocks, uniform rows, the
last rows of the sequence and rows right after needle blocks."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_attn, check_block_idx

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def sample_rows(cfg, needles, n_uniform, seed):
    g = np.random.default_rng(seed)
    N, B_k, k = cfg.N, cfg.B_k, cfg.k
    rows = set(range(0, min(N, k * B_k), 37))                      # fewer than k causal blocks
    rows |= set(g.choice(N, size=n_uniform, replace=False).tolist())  # uniform
    rows |= set(range(max(0, N - 24), N))                          # last rows
    for b in needles[0][:4] if needles and needles[0] else []:
        rows |= {min(N - 1, (b + 1) * B_k), min(N - 1, (b + 1) * B_k + 77)}
    return np.array(sorted(rows), dtype=np.int64)


def _run_prefill(msa, name, mode, n_uniform):
    cfg = synth.CONFIGS[name]
    print(f"[full] {name} {mode}: generating inputs", flush=True)
    inp = synth.make_prefill(cfg, mode, device=DEV)
    k = cfg.k
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=cfg.B_k)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=cfg.B_k)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, inp.needles, n_uniform, cfg.seed)
    print(f"[full] {name} {mode}: oracle on {len(rows)} rows", flush=True)
    ridx = torch.from_numpy(rows).to(DEV)
    bi_s = bi[ridx].cpu().numpy()
    M = oracle.block_scores(inp.q_idx.cpu(), inp.k_idx.cpu(), cfg.B_k, rows=rows)
    tie = check_block_idx(bi_s, M, rows, k, cfg.B_k)
    # Main branch alone, at full size, on the GPU's own selection.
    q_h, k_h, v_h = inp.q.cpu(), inp.k.cpu(), inp.v.cpu()
    o_ref, lse_ref = oracle.sparse_attn(q_h, k_h, v_h, bi_s, cfg.B_k, rows=rows)
    stats = check_attn(o[ridx].cpu().numpy(), lse[ridx].cpu().numpy(), o_ref, lse_ref, f"{name} {mode}")
    # Rows away from near ties use exactly the oracle's selection.
    exact = oracle.topk(M, k, cfg.B_k, rows=rows)
    np.testing.assert_array_equal(bi_s[~tie], exact[~tie])
    print(f"[full] {name} {mode}: {len(rows)} rows, {int(tie.sum())} near-tie rows, {stats}", flush=True)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_32k(msa, mode):
    _run_prefill(msa, "c1", mode, n_uniform=512)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_128k(msa, mode):
    _run_prefill(msa, "c2", mode, n_uniform=256)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_1m(msa, mode):
    _run_prefill(msa, "c4", mode, n_uniform=48)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_128k_bk64(msa, mode):
    _run_prefill(msa, "c2_bk64", mode, n_uniform=128)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_packed_batch_128k(msa, mode):
    """The packed variable-length batch the benchmark times (9 sequences, 131072
    tokens), checked per sequence on sampled rows."""
    vcfg = synth.VARLEN_CONFIGS["c2_varlen"]
    lengths = synth.varlen_lengths(vcfg)
    print(f"[full] {vcfg.name} {mode}: generating {len(lengths)} sequences", flush=True)
    p = synth.packed_prefill(lengths, vcfg.H_q, vcfg.H_kv, vcfg.k, vcfg.seed, mode, device=DEV)
    k, B_k = vcfg.k, vcfg.B_k
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k, B_k=B_k)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, B_k=B_k)
    torch.cuda.synchronize()
    cu = p.cu_seqlens.cpu().tolist()
    for s, L in enumerate(lengths):
        a = cu[s]
        scfg = synth.PrefillConfig(f"seq{s}", N=L, H_q=vcfg.H_q, H_kv=vcfg.H_kv, k=k, B_k=B_k)
        rows = sample_rows(scfg, None, min(24, L), vcfg.seed + s)
        ridx = torch.from_numpy(rows + a).to(DEV)
        bi_s = bi[ridx].cpu().numpy()
        sl = slice(a, a + L)
        M = oracle.block_scores(p.q_idx[sl].cpu(), p.k_idx[sl].cpu(), B_k, rows=rows)
        tie = check_block_idx(bi_s, M, rows, k, B_k)
        o_ref, lse_ref = oracle.sparse_attn(p.q[sl].cpu(), p.k[sl].cpu(), p.v[sl].cpu(), bi_s, B_k, rows=rows)
        stats = check_attn(o[ridx].cpu().numpy(), lse[ridx].cpu().numpy(), o_ref, lse_ref,
                           f"{vcfg.name} {mode} sequence {s}")
        exact = oracle.topk(M, k, B_k, rows=rows)
        np.testing.assert_array_equal(bi_s[~tie], exact[~tie])
        print(f"[full] {vcfg.name} {mode} sequence {s} (L={L}): {len(rows)} rows, {stats}", flush=True)


@pytest.mark.parametrize("name", ["c3", "c3_128k"])
@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_decode_64_sequences(msa, name, mode):
    cfg = synth.CONFIGS[name]
    print(f"[full] {name} {mode}: generating caches", flush=True)
    d = synth.make_decode(cfg, mode, device=DEV)
    max_len = max(d.lengths)
    bi, o, lse = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, cfg.k)
    torch.cuda.synchronize()
    print(f"[full] {name} {mode}: oracle on all {cfg.batch} sequences", flush=True)
    h = lambda t: t.cpu()
    bi_ref, o_ref, lse_ref, M = oracle.decode(h(d.q), h(d.q_idx), h(d.k_cache), h(d.v_cache), h(d.k_idx_cache),
                                              d.cu_seqlens, cfg.k, cfg.B_k, want_scores=True)
    bi_g = bi.cpu().numpy()
    tie = check_block_idx(bi_g, M, np.array(d.lengths) - 1, cfg.k, cfg.B_k)
    np.testing.assert_array_equal(bi_g[~tie], bi_ref[~tie])
    if tie.any():  # compare attention on the GPU's own selection
        o_ref, lse_ref = oracle.decode_attn(h(d.q), h(d.k_cache), h(d.v_cache), d.cu_seqlens, bi_g, cfg.B_k)
    stats = check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"{name} {mode}")
    print(f"[full] {name} {mode}: {int(tie.sum())} near-tie rows, {stats}", flush=True)


def _prefill_128k(msa, mode="literal"):
    cfg = synth.CONFIGS["c2"]
    print(f"[full] c2 {mode}: generating inputs", flush=True)
    inp = synth.make_prefill(cfg, mode, device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, cfg.k, B_k=cfg.B_k)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=cfg.B_k)
    return cfg, inp, bi, o, lse


def test_sparse_kl_128k(msa):
    """Eq. 9-10 at 128K with the default workspace, on sampled rows of the GPU's own
    selection; the loss is the mean of the returned per-row KL over all rows."""
    cfg, inp, bi, _, lse = _prefill_128k(msa)
    kl, lse_idx, loss = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, B_k=cfg.B_k)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, inp.needles, 64, cfg.seed + 7)
    ridx = torch.from_numpy(rows).to(DEV)
    print(f"[full] c2 KL: oracle on {len(rows)} rows", flush=True)
    kl_ref, li_ref = oracle.sparse_kl(inp.q.cpu(), inp.k.cpu(), inp.q_idx.cpu(), inp.k_idx.cpu(),
                                      bi[ridx].cpu().numpy(), cfg.B_k, rows=rows)
    kl_s, li_s = kl[ridx].cpu().double().numpy(), lse_idx[ridx].cpu().double().numpy()
    assert np.all(np.isfinite(li_ref)) and np.all(np.isfinite(li_s))
    err = np.abs(kl_s - kl_ref)
    assert np.all(err <= 5e-4 + 2e-3 * np.abs(kl_ref)), err.max()
    assert np.abs(li_s - li_ref).max() <= 1e-3
    kl_all = kl.double()
    assert bool(torch.isfinite(kl_all).all()) and float(kl_all.min()) >= -1e-4
    assert abs(float(loss.item()) - float(kl_all.mean())) <= 1e-6 * max(1.0, abs(float(kl_all.mean())))
    print(f"[full] c2 KL: max err {err.max():.2e}, loss {float(loss.item()):.6f}", flush=True)
    # LSE_idx emitted by the forward itself: the same values on the sampled rows, and
    # everywhere within fp32 rounding of the KL pass's.
    _, _, li_fwd = msa.msa_sparse_attn_fwd_lse_idx(inp.q, inp.k, inp.v, inp.q_idx, inp.k_idx, bi, B_k=cfg.B_k)
    torch.cuda.synchronize()
    li_f = li_fwd[ridx].cpu().double().numpy()
    assert np.abs(li_f - li_ref).max() <= 1e-3
    assert float((li_fwd.double() - lse_idx.double()).abs().max()) <= 1e-4
    print(f"[full] c2 forward LSE_idx: max err {np.abs(li_f - li_ref).max():.2e}", flush=True)
    # The KL value from that LSE_idx.
    kl2, loss2 = msa.msa_sparse_kl_fwd_from_lse_idx(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, li_fwd,
                                                    B_k=cfg.B_k)
    torch.cuda.synchronize()
    kl2_s = kl2[ridx].cpu().double().numpy()
    err2 = np.abs(kl2_s - kl_ref)
    assert np.all(err2 <= 5e-4 + 2e-3 * np.abs(kl_ref)), err2.max()
    assert abs(float(loss2.item()) - float(loss.item())) <= 1e-4 * max(1.0, abs(float(loss.item())))
    print(f"[full] c2 KL from the forward's LSE_idx: max err {err2.max():.2e}", flush=True)


def test_backward_128k(msa):
    """Gradients of Eq. 8 at 128K with the default workspace (query windows).
    dQ of the first 1024 rows: those rows see only keys < 1024, so the oracle on that
    prefix gives their exact gradient.  dK, dV over all tokens: for each KV head r,
    sum_t dK[t, r] = 0 (every row of dS sums to 0) and sum_t dV[t, r] = the sum of dO
    over the rows of r's heads (every row of P sums to 1).  The GPU rounds P and dS to
    bf16 (relative 2^-9) before its matrix products; those errors change sign from
    row to row, so each identity is asserted to 2^-9 of the sum of the magnitudes it
    adds up."""
    from tests.test_gpu_backward import check_grads
    cfg, inp, bi, o, lse = _prefill_128k(msa)
    g = torch.Generator(device=DEV).manual_seed(cfg.seed + 11)
    dO = torch.randn(inp.q.shape, generator=g, device=DEV).to(torch.bfloat16)
    dq, dk, dv = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi, B_k=cfg.B_k)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    P0 = 1024
    print(f"[full] c2 backward: oracle on the first {P0} rows", flush=True)
    ref = oracle.sparse_attn_bwd(inp.q[:P0].cpu(), inp.k[:P0].cpu(), inp.v[:P0].cpu(), dO[:P0].cpu(),
                                 bi[:P0].cpu().numpy(), cfg.B_k)
    check_grads((dq[:P0],), (ref[0],), "c2 backward dq, first rows")
    G = cfg.H_q // cfg.H_kv
    dk_sum, dk_mag = dk.double().sum(0), dk.double().abs().sum(0)
    dv_sum = dv.double().sum(0)
    do_sum = dO.double().view(cfg.N, cfg.H_kv, G, -1).sum((0, 2))
    do_mag = dO.double().abs().view(cfg.N, cfg.H_kv, G, -1).sum((0, 2))
    rk = float((dk_sum.abs() / dk_mag).max())
    rv = float(((dv_sum - do_sum).abs() / do_mag).max())
    print(f"[full] c2 backward: |sum dK| / sum |dK| <= {rk:.2e}, |sum dV - sum dO| / sum |dO| <= {rv:.2e}",
          flush=True)
    assert rk <= 2.0 ** -9 and rv <= 2.0 ** -9
    # Element-wise at full size: dQ on sampled rows past the first window (rows right
    # after needle blocks, uniform rows, the last rows), and dK, dV of whole key blocks
    # of one KV head, each the sum over every row that selected the block: the last
    # block, a block of median fan-in and a needle block (the sink block, selected by
    # almost every row, costs the oracle too much and is left to the identities above).
    rows = sample_rows(cfg, inp.needles, 24, cfg.seed + 13)
    rows = rows[rows >= P0]
    nb = (cfg.N + cfg.B_k - 1) // cfg.B_k
    picks = []
    for r in (0, cfg.H_kv - 1):
        sel = bi[:, r, :]
        fan = torch.bincount(sel[sel >= 0].long(), minlength=nb).cpu().numpy()
        if r == 0:
            picks.append((nb - 1, r, int(fan[nb - 1])))
            nd = [b for b in (inp.needles[r] if inp.needles else []) if fan[b] <= 32768]
            if nd:
                b = max(nd, key=lambda b: fan[b])
                picks.append((b, r, int(fan[b])))
        else:
            inner = np.arange(1, nb - 1)
            b = int(inner[np.argsort(fan[inner], kind="stable")[len(inner) // 2]])
            picks.append((b, r, int(fan[b])))
    q_h, k_h, v_h, g_h, bi_h = inp.q.cpu(), inp.k.cpu(), inp.v.cpu(), dO.cpu(), bi.cpu().numpy()
    ridx = torch.from_numpy(rows).to(DEV)
    for n, (kb, r, f) in enumerate(picks):
        print(f"[full] c2 backward: oracle on {len(rows) if n == 0 else 0} rows and key block {kb} of "
              f"KV head {r} (fan-in {f} rows)", flush=True)
        dq_ref, (dk_ref, dv_ref) = oracle.sparse_attn_bwd_part(q_h, k_h, v_h, g_h, bi_h, cfg.B_k,
                                                               rows=rows if n == 0 else (), key_block=kb, group=r)
        j0, j1 = kb * cfg.B_k, min(cfg.N, (kb + 1) * cfg.B_k)
        got_kv = (dk[j0:j1, r], dv[j0:j1, r])
        ref_kv = (dk_ref[:j1 - j0], dv_ref[:j1 - j0])
        if n == 0:
            st = check_grads((dq[ridx],) + got_kv, (dq_ref,) + ref_kv, f"c2 backward, block {kb}",
                             floor=1e-6)
        else:
            st = check_grads((None,) + got_kv, (None,) + ref_kv, f"c2 backward, block {kb}",
                             floor=1e-6)
        print(f"[full] c2 backward: block {kb}: {st}", flush=True)


def test_decode_paged_64_sequences(msa):
    """The paged FP8 decode at the benchmark's size (64 sequences of 128K tokens, pages
    in random order), every sequence against the oracle on the same FP8 codes."""
    cfg = synth.CONFIGS["c3_128k"]
    print("[full] c3_128k paged: generating caches", flush=True)
    p = synth.make_decode_paged(cfg, "literal", device=DEV)
    bi, o, lse = msa.msa_decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages,
                                      p.block_table, p.seqlens, max(p.lengths), cfg.k, B_k=cfg.B_k)
    torch.cuda.synchronize()
    print("[full] c3_128k paged: oracle on all sequences", flush=True)
    h = lambda t: t.cpu()
    bi_ref, o_ref, lse_ref, M = oracle.decode_paged(h(p.q), h(p.q_idx), h(p.k_pages), h(p.v_pages), p.k_scale,
                                                    p.v_scale, h(p.kidx_pages), p.block_table, p.seqlens, cfg.k,
                                                    cfg.B_k, want_scores=True)
    bi_g = bi.cpu().numpy()
    tie = check_block_idx(bi_g, M, np.array(p.lengths) - 1, cfg.k, cfg.B_k)
    np.testing.assert_array_equal(bi_g[~tie], bi_ref[~tie])
    if tie.any():
        _, o_ref, lse_ref = oracle.decode_paged(h(p.q), h(p.q_idx), h(p.k_pages), h(p.v_pages), p.k_scale,
                                                p.v_scale, h(p.kidx_pages), p.block_table, p.seqlens, cfg.k,
                                                cfg.B_k, block_idx=bi_g)
    stats = check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "c3_128k paged")
    print(f"[full] c3_128k paged: {int(tie.sum())} near-tie rows, {stats}", flush=True)
