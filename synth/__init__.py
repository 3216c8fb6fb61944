"""Seeded synthetic inputs for the MSA forward path.

This module only draws numbers and places them in the layouts the library
takes; it holds none of the method's arithmetic (no scores, no pooling, no
selection, no softmax).  Both the oracle side and the GPU side of a test are
fed from here: the GPU gets the tensors, the oracle gets host copies of the
very same bf16 bytes, so the two never have to agree on a random generator.

Workload shapes follow the pages' setting (MiniMax Sparse Attention, section
"Computational Complexity" / Table 1 / "1M context" results: B_k = 128,
k = 16, d_h = 128, contexts from 32K to 1M) and the five workloads named for
this path.  Two input modes exist:

* ``literal``: every tensor N(0,1); an attention-sink direction ``u`` is added
  to all index queries and twice to the index keys of block 0; needle blocks
  get ``2 * normalize(mean_i Q_idx[i, r])`` added to their index keys.
* ``structured``: the learned selection pattern the pages visualise (sink
  column, local diagonal, group-specific long-range stripes): index queries get
  ``4 (u + w_r)``, block 0's index keys get ``16 u`` and the needle blocks of
  group r get ``16 w_r``, with ``w_r`` orthonormal to ``u`` and each other.

Tensor ids seed independent streams: Q=1, K=2, V=3, Q_idx=4, K_idx=5, u=6,
w=7, needles=8, lengths=9.  Config ids 0..4 use seed 1000 + id.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

T_Q, T_K, T_V, T_QIDX, T_KIDX, T_U, T_W, T_NEEDLE, T_LEN = 1, 2, 3, 4, 5, 6, 7, 8, 9

# Elements drawn per randn call when filling very large tensors (keeps the
# fp32 temporary at 1 GiB).
_CHUNK = 1 << 28


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    N: int
    H_q: int
    H_kv: int
    k: int
    d_h: int = 128
    d_idx: int = 64
    B_k: int = 128
    needles: int = 0            # needle blocks per group
    needle_dist: str = "uniform"  # "uniform" or "loguniform"
    seed: int = 1000

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def B(self) -> int:
        return (self.N + self.B_k - 1) // self.B_k


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    H_q: int
    H_kv: int
    k: int
    len_lo_blocks: int          # lengths are B_k * U{lo..hi}
    len_hi_blocks: int
    d_h: int = 128
    d_idx: int = 64
    B_k: int = 128
    seed: int = 1003

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv


CONFIGS = {
    "c0": PrefillConfig("c0", N=4096, H_q=4, H_kv=1, k=8, seed=1000),
    "c1": PrefillConfig("c1", N=32768, H_q=32, H_kv=4, k=16, needles=4, seed=1001),
    "c2": PrefillConfig("c2", N=131072, H_q=64, H_kv=8, k=16, needles=8, seed=1002),
    "c3": DecodeConfig("c3", batch=64, H_q=64, H_kv=8, k=16, len_lo_blocks=256, len_hi_blocks=1024, seed=1003),
    "c3_128k": DecodeConfig("c3_128k", batch=64, H_q=64, H_kv=8, k=16, len_lo_blocks=1024, len_hi_blocks=1024, seed=1003),
    "c4": PrefillConfig("c4", N=1048576, H_q=64, H_kv=8, k=16, needles=32, needle_dist="loguniform", seed=1004),
    # 128K with blocks of 64 keys and k = 32: the same 2048 attended keys per query.
    "c2_bk64": PrefillConfig("c2_bk64", N=131072, H_q=64, H_kv=8, k=32, B_k=64, needles=8, seed=1005),
}


@dataclass(frozen=True)
class VarlenConfig:
    """A packed batch of about ``total`` tokens: lengths B_k * U{lo..hi} drawn from the
    lengths stream until the total is reached (the last one cut to fit)."""
    name: str
    total: int
    H_q: int
    H_kv: int
    k: int
    len_lo_blocks: int
    len_hi_blocks: int
    B_k: int = 128
    seed: int = 1006


VARLEN_CONFIGS = {
    "c2_varlen": VarlenConfig("c2_varlen", total=131072, H_q=64, H_kv=8, k=16, len_lo_blocks=8,
                              len_hi_blocks=256),
}


def varlen_lengths(cfg: VarlenConfig):
    g = _gen(cfg.seed, T_LEN, "cpu")
    out, t = [], 0
    while t < cfg.total:
        L = int(torch.randint(cfg.len_lo_blocks, cfg.len_hi_blocks + 1, (1,), generator=g)) * cfg.B_k
        L = min(L, cfg.total - t)
        out.append(L)
        t += L
    return out


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + tensor_id * 7919)
    return g


def _randn_bf16(shape, seed: int, tensor_id: int, device) -> torch.Tensor:
    """N(0,1) drawn in fp32 and rounded to nearest-even bf16, filled in chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    g = _gen(seed, tensor_id, device)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        flat[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return out


def directions(seed: int, H_kv: int, d_idx: int):
    """Unit vector u and H_kv unit vectors w_r, all mutually orthonormal (fp32, CPU)."""
    g = _gen(seed, T_U, "cpu")
    raw = torch.randn(H_kv + 1, d_idx, generator=g, dtype=torch.float64)
    basis = []
    for v in raw:
        for b in basis:
            v = v - (v @ b) * b
        basis.append(v / v.norm())
    u = basis[0].float()
    w = torch.stack(basis[1:]).float()
    return u, w


def needle_blocks(cfg: PrefillConfig):
    """Needle block ids per group, drawn without replacement over all groups, never block 0."""
    if cfg.needles == 0:
        return [[] for _ in range(cfg.H_kv)]
    g = _gen(cfg.seed, T_NEEDLE, "cpu")
    total = cfg.needles * cfg.H_kv
    B = cfg.B
    if total > B - 1:
        raise ValueError("more needle blocks than non-sink blocks")
    chosen: list[int] = []
    seen = set()
    while len(chosen) < total:
        x = torch.rand(1, generator=g, dtype=torch.float64).item()
        if cfg.needle_dist == "loguniform":
            b = int(math.floor(math.exp(x * math.log(B))))
        else:
            b = 1 + int(math.floor(x * (B - 1)))
        b = min(max(b, 1), B - 1)
        if b in seen:
            continue
        seen.add(b)
        chosen.append(b)
    return [chosen[r * cfg.needles:(r + 1) * cfg.needles] for r in range(cfg.H_kv)]


def _add_bf16(t: torch.Tensor, delta: torch.Tensor) -> None:
    """t += delta, computed in fp32 and rounded back to bf16, in place."""
    t.copy_((t.float() + delta).to(torch.bfloat16))


@dataclass
class PrefillInputs:
    cfg: PrefillConfig
    mode: str
    q: torch.Tensor        # [N, H_q, d_h] bf16
    k: torch.Tensor        # [N, H_kv, d_h] bf16
    v: torch.Tensor        # [N, H_kv, d_h] bf16
    q_idx: torch.Tensor    # [N, H_kv, d_idx] bf16
    k_idx: torch.Tensor    # [N, d_idx] bf16
    needles: list = field(default_factory=list)


def make_prefill(cfg: PrefillConfig, mode: str = "literal", device="cpu", main_branch: bool = True) -> PrefillInputs:
    """All prefill inputs for ``cfg`` on ``device``.  ``main_branch=False`` skips Q/K/V."""
    if mode not in ("literal", "structured"):
        raise ValueError(mode)
    N, s = cfg.N, cfg.seed
    if main_branch:
        q = _randn_bf16((N, cfg.H_q, cfg.d_h), s, T_Q, device)
        k = _randn_bf16((N, cfg.H_kv, cfg.d_h), s, T_K, device)
        v = _randn_bf16((N, cfg.H_kv, cfg.d_h), s, T_V, device)
    else:
        q = k = v = None
    q_idx = _randn_bf16((N, cfg.H_kv, cfg.d_idx), s, T_QIDX, device)
    k_idx = _randn_bf16((N, cfg.d_idx), s, T_KIDX, device)
    u, w = directions(s, cfg.H_kv, cfg.d_idx)
    u, w = u.to(device), w.to(device)
    nb = needle_blocks(cfg)
    B_k = cfg.B_k
    if mode == "literal":
        for i0 in range(0, N, 1 << 16):
            i1 = min(N, i0 + (1 << 16))
            _add_bf16(q_idx[i0:i1], u)
        _add_bf16(k_idx[0:min(B_k, N)], 2.0 * u)
        for r in range(cfg.H_kv):
            if not nb[r]:
                continue
            mean = torch.zeros(cfg.d_idx, dtype=torch.float64, device=device)
            for i0 in range(0, N, 1 << 16):
                mean += q_idx[i0:i0 + (1 << 16), r].double().sum(0)
            d_hat = (mean / mean.norm()).float()
            for b in nb[r]:
                _add_bf16(k_idx[b * B_k:min(N, (b + 1) * B_k)], 2.0 * d_hat)
    else:
        shift = 4.0 * (u[None, :] + w)            # [H_kv, d_idx]
        for i0 in range(0, N, 1 << 16):
            i1 = min(N, i0 + (1 << 16))
            _add_bf16(q_idx[i0:i1], shift[None])
        _add_bf16(k_idx[0:min(B_k, N)], 16.0 * u)
        for r in range(cfg.H_kv):
            for b in nb[r]:
                _add_bf16(k_idx[b * B_k:min(N, (b + 1) * B_k)], 16.0 * w[r])
    return PrefillInputs(cfg, mode, q, k, v, q_idx, k_idx, nb)


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    mode: str
    lengths: list
    cu_seqlens: torch.Tensor  # [batch + 1] int64
    q: torch.Tensor           # [batch, H_q, d_h]
    q_idx: torch.Tensor       # [batch, H_kv, d_idx]
    k_cache: torch.Tensor     # [T, H_kv, d_h]
    v_cache: torch.Tensor     # [T, H_kv, d_h]
    k_idx_cache: torch.Tensor  # [T, d_idx]


def decode_lengths(cfg: DecodeConfig):
    g = _gen(cfg.seed, T_LEN, "cpu")
    nblk = torch.randint(cfg.len_lo_blocks, cfg.len_hi_blocks + 1, (cfg.batch,), generator=g)
    return [int(x) * cfg.B_k for x in nblk]


def make_decode(cfg: DecodeConfig, mode: str = "literal", device="cpu", lengths=None) -> DecodeInputs:
    """Packed varlen caches; the new token of each sequence is its last cache entry."""
    if mode not in ("literal", "structured"):
        raise ValueError(mode)
    lengths = list(lengths) if lengths is not None else decode_lengths(cfg)
    b = len(lengths)
    cu = torch.zeros(b + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    T = int(cu[-1])
    s = cfg.seed
    q = _randn_bf16((b, cfg.H_q, cfg.d_h), s, T_Q, device)
    k_cache = _randn_bf16((T, cfg.H_kv, cfg.d_h), s, T_K, device)
    v_cache = _randn_bf16((T, cfg.H_kv, cfg.d_h), s, T_V, device)
    q_idx = _randn_bf16((b, cfg.H_kv, cfg.d_idx), s, T_QIDX, device)
    k_idx = _randn_bf16((T, cfg.d_idx), s, T_KIDX, device)
    u, w = directions(s, cfg.H_kv, cfg.d_idx)
    u, w = u.to(device), w.to(device)
    if mode == "literal":
        _add_bf16(q_idx, u)
        sink = 2.0 * u
    else:
        _add_bf16(q_idx, 4.0 * (u[None, None, :] + w[None]))
        sink = 16.0 * u
    for si in range(b):
        j0 = int(cu[si])
        _add_bf16(k_idx[j0:j0 + min(cfg.B_k, lengths[si])], sink)
    return DecodeInputs(cfg, mode, lengths, cu.to(device), q, q_idx, k_cache, v_cache, k_idx)


def small_prefill(N: int, H_q: int, H_kv: int, k: int, seed: int, mode: str = "literal",
                  B_k: int = 128, d_h: int = 128, d_idx: int = 64, needles: int = 0, device="cpu") -> PrefillInputs:
    """A small custom-shaped prefill case (parity tests over ragged shapes)."""
    cfg = PrefillConfig(f"small_N{N}", N=N, H_q=H_q, H_kv=H_kv, k=k, d_h=d_h, d_idx=d_idx, B_k=B_k,
                        needles=needles, seed=seed)
    return make_prefill(cfg, mode, device)


@dataclass
class PackedPrefillInputs:
    lengths: list
    cu_seqlens: torch.Tensor  # [batch + 1] int64 (on ``device``)
    q: torch.Tensor           # [T, H_q, d_h] bf16
    k: torch.Tensor           # [T, H_kv, d_h] bf16
    v: torch.Tensor           # [T, H_kv, d_h] bf16
    q_idx: torch.Tensor       # [T, H_kv, d_idx] bf16
    k_idx: torch.Tensor       # [T, d_idx] bf16


def packed_prefill(lengths, H_q: int, H_kv: int, k: int, seed: int, mode: str = "literal", needles: int = 1,
                   device="cpu") -> PackedPrefillInputs:
    """Packed variable-length prefill: sequence s is ``small_prefill`` of its own length
    with seed ``seed + s`` (its own sink block and needles), concatenated on the
    token axis."""
    parts = []
    for s, L in enumerate(lengths):
        if L == 0:
            continue
        fits = (int(L) + 127) // 128 - 1 >= needles * H_kv
        parts.append(small_prefill(int(L), H_q, H_kv, k, seed + s, mode, needles=needles if fits else 0,
                                   device=device))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(torch.tensor(list(lengths), dtype=torch.int64), 0)

    def cat(name, shape_tail):
        ts = [getattr(p, name) for p in parts]
        return torch.cat(ts) if ts else torch.empty((0, *shape_tail), dtype=torch.bfloat16, device=device)

    return PackedPrefillInputs(list(lengths), cu.to(device), cat("q", (H_q, 128)), cat("k", (H_kv, 128)),
                               cat("v", (H_kv, 128)), cat("q_idx", (H_kv, 64)), cat("k_idx", (64,)))


T_PAGE = 10  # tensor id of the page permutation


@dataclass
class PagedDecodeInputs:
    lengths: list
    seqlens: torch.Tensor      # [batch] int64
    block_table: torch.Tensor  # [batch, max_blocks] int32 (unused entries -1)
    q: torch.Tensor            # [batch, H_q, d_h] bf16
    q_idx: torch.Tensor        # [batch, H_kv, d_idx] bf16
    k_pages: torch.Tensor      # [P, B_k, H_kv, d_h] uint8 (FP8 E4M3 codes)
    v_pages: torch.Tensor      # [P, B_k, H_kv, d_h] uint8
    kidx_pages: torch.Tensor   # [P, B_k, d_idx] bf16
    k_scale: float
    v_scale: float
    contiguous: DecodeInputs   # the bf16 caches the pages were made from


def quantize_fp8(x: torch.Tensor):
    """Per-tensor scale amax / 448 and the OCP E4M3 codes (torch's round-to-nearest)."""
    amax = float(x.float().abs().max()) if x.numel() else 1.0
    scale = amax / 448.0 if amax > 0 else 1.0
    codes = (x.float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_decode_paged(cfg: DecodeConfig, mode: str = "literal", device="cpu", lengths=None,
                      spare_pages: int = 3, unit_scale: bool = False) -> PagedDecodeInputs:
    """The decode inputs of ``make_decode`` moved into a paged cache: K/V quantised to
    FP8 E4M3 with per-tensor scales, index keys kept bf16, pages of B_k tokens placed
    in a seeded random order (plus a few unused pages).  ``unit_scale``: the
    contiguous K/V are first rounded to FP8 values themselves and the scales are 1,
    so that both caches hold the same numbers."""
    d = make_decode(cfg, mode, device=device, lengths=lengths)
    if unit_scale:
        for t in (d.k_cache, d.v_cache):
            t.copy_(t.float().to(torch.float8_e4m3fn).float().to(torch.bfloat16))
    B_k = cfg.B_k
    nblk = [(L + B_k - 1) // B_k for L in d.lengths]
    P = sum(nblk) + spare_pages
    perm = torch.randperm(P, generator=_gen(cfg.seed, T_PAGE, "cpu"))
    max_blocks = max(nblk) if nblk else 1
    table = torch.full((len(d.lengths), max_blocks), -1, dtype=torch.int32)
    if unit_scale:
        kq, k_scale = d.k_cache.float().to(torch.float8_e4m3fn).view(torch.uint8), 1.0
        vq, v_scale = d.v_cache.float().to(torch.float8_e4m3fn).view(torch.uint8), 1.0
    else:
        kq, k_scale = quantize_fp8(d.k_cache)
        vq, v_scale = quantize_fp8(d.v_cache)
    k_pages = torch.zeros((P, B_k, cfg.H_kv, cfg.d_h), dtype=torch.uint8, device=device)
    v_pages = torch.zeros_like(k_pages)
    kidx_pages = torch.zeros((P, B_k, cfg.d_idx), dtype=torch.bfloat16, device=device)
    cu = d.cu_seqlens.tolist()
    nxt = 0
    for s, L in enumerate(d.lengths):
        ids = perm[nxt:nxt + nblk[s]]
        nxt += nblk[s]
        table[s, :nblk[s]] = ids.to(torch.int32)
        full = L // B_k  # whole pages in one indexed copy, then the partial last page
        if full:
            idx = ids[:full].to(device)
            t0 = cu[s]
            k_pages[idx] = kq[t0:t0 + full * B_k].view(full, B_k, cfg.H_kv, cfg.d_h)
            v_pages[idx] = vq[t0:t0 + full * B_k].view(full, B_k, cfg.H_kv, cfg.d_h)
            kidx_pages[idx] = d.k_idx_cache[t0:t0 + full * B_k].view(full, B_k, cfg.d_idx)
        if L % B_k:
            p = int(ids[full])
            t0, t1 = cu[s] + full * B_k, cu[s + 1]
            k_pages[p, :t1 - t0] = kq[t0:t1]
            v_pages[p, :t1 - t0] = vq[t0:t1]
            kidx_pages[p, :t1 - t0] = d.k_idx_cache[t0:t1]
    seqlens = torch.tensor(d.lengths, dtype=torch.int64, device=device)
    return PagedDecodeInputs(list(d.lengths), seqlens, table.to(device), d.q, d.q_idx, k_pages, v_pages,
                             kidx_pages, k_scale, v_scale, d)
