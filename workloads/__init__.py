"""Seeded synthetic inputs for the fine-grained-scaled FP8 GEMM and its M-grouped forms.

This module is shared by the CPU oracle's tests and by the HIP path's tests and bench.
It holds none of the GEMM's arithmetic: only random draws (numpy ``default_rng``), the
per-segment amax/448 FP8 cast that the DeepGEMM pages leave to the caller (pt.news.hada.io
page, "Interface GEMM e restrições de layout": casting to FP8 and transposition are the
user's job), and the assembly of the documented memory layouts.

Layouts produced (all row-major numpy arrays, bytes for e4m3):
  A    uint8 [M, K]            e4m3 bits, K contiguous ("not transposed")
  sfa  float32 [K/128, ld]     one FP32 scale per 1x128 row segment, stored MN-major
                               ("transposed" LHS scale), ld = ceil(M/4)*4
  B    uint8 [N, K]            e4m3 bits (B.T is column-major)
  sfb  float32 [ceil(N/128), K/128]   one FP32 scale per 128x128 block
  C    float32 [M, N] or None
Grouped forms add a leading group axis to B/sfb (and to A/sfa for the masked layout).

Quantisation recipe (input preparation, not a parity question: both sides read the same
bytes): scale = max(amax, 1e-4) / 448 over the segment/block, q = clip(x / scale, +-448)
rounded to nearest-even e4m3 (OCP E4M3FN) by torch's float8_e4m3fn cast.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F            # OCP E4M3FN NaN bit pattern (S.1111.111)
BF16_SENTINEL = 0x7FC1     # a bf16 NaN payload never produced by a rounding; marks "untouched"
BLOCK = 128                # K block / B block edge / contiguous-layout M alignment
AMAX_FLOOR = 1e-4


def sf_aligned(m: int) -> int:
    """Leading dimension of the MN-major A-scale array: rows padded to 4 floats (16 bytes)."""
    return (m + 3) // 4 * 4


def to_e4m3_bits(y: np.ndarray) -> np.ndarray:
    """Round float32 values already inside [-448, 448] to e4m3 bit patterns (uint8)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _cast(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    y = np.clip(x / scale, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return to_e4m3_bits(y)


def _scale_of(amax: np.ndarray, pow2: bool) -> np.ndarray:
    """Scale for a block with absolute maximum ``amax``: amax/448, or (``pow2``, for UE8M0
    scales) the next power of two at or above it, so the cast never saturates."""
    s = np.maximum(amax, AMAX_FLOOR) / E4M3_MAX
    if pow2:
        s = np.exp2(np.ceil(np.log2(s)))
    return s.astype(np.float32)


def quantize_rows(x: np.ndarray, seg_mult: Optional[np.ndarray] = None, pow2: bool = False):
    """1x128 row-segment cast. x: float32 [M, K] -> (bits uint8 [M, K], scales float32 [M, K/128]).

    ``seg_mult`` (float32 [M, K/128]) multiplies each segment before the cast (stress inputs);
    ``pow2`` rounds every scale up to a power of two (UE8M0-representable).
    """
    m, k = x.shape
    assert k % BLOCK == 0
    kb = k // BLOCK
    xs = x.reshape(m, kb, BLOCK)
    if seg_mult is not None:
        xs = xs * seg_mult[:, :, None].astype(np.float32)
    amax = np.abs(xs).max(axis=2)
    scale = _scale_of(amax, pow2)
    bits = _cast(xs, scale[:, :, None]).reshape(m, k)
    return bits, scale


def quantize_blocks(x: np.ndarray, blk_mult: Optional[np.ndarray] = None, pow2: bool = False):
    """128x128 block cast. x: float32 [N, K] -> (bits uint8 [N, K], scales float32 [ceil(N/128), K/128]).

    The last block row may be partial (N % 128 != 0): its amax is over the rows that exist.
    """
    n, k = x.shape
    assert k % BLOCK == 0
    kb = k // BLOCK
    nb = (n + BLOCK - 1) // BLOCK
    bits = np.empty((n, k), dtype=np.uint8)
    scale = np.empty((nb, kb), dtype=np.float32)
    for i in range(nb):
        rows = x[i * BLOCK:(i + 1) * BLOCK].reshape(-1, kb, BLOCK)
        if blk_mult is not None:
            rows = rows * blk_mult[i][None, :, None].astype(np.float32)
        amax = np.abs(rows).max(axis=(0, 2))
        s = _scale_of(amax, pow2)
        scale[i] = s
        bits[i * BLOCK:(i + 1) * BLOCK] = _cast(rows, s[None, :, None]).reshape(-1, k)
    return bits, scale


def mn_major(scales_mk: np.ndarray, ld: Optional[int] = None) -> np.ndarray:
    """[M, K/128] row scales -> MN-major [K/128, ld] (zero in the padding columns)."""
    m, kb = scales_mk.shape
    ld = sf_aligned(m) if ld is None else ld
    out = np.zeros((kb, ld), dtype=np.float32)
    out[:, :m] = scales_mk.T
    return out


def pack_ue8m0(scales: np.ndarray, axis: int) -> np.ndarray:
    """Power-of-two FP32 scales -> packed UE8M0: along ``axis`` (the K-block axis), K blocks
    4q .. 4q+3 become the bytes 0..3 (least significant first) of int32 number q; a byte is
    the biased exponent e with scale 2^(e-127), NaN scales become 0xFF, and the bytes past the
    last K block hold 127 (scale 1).  Zero scales (padding columns of MN-major arrays) also
    become 127."""
    s = np.moveaxis(np.asarray(scales, dtype=np.float32), axis, -1)
    kb = s.shape[-1]
    kq = (kb + 3) // 4
    e = np.full(s.shape[:-1] + (kq * 4,), 127, dtype=np.uint8)
    with np.errstate(divide="ignore", invalid="ignore"):
        m, ex = np.frexp(s.astype(np.float64))
    ok = np.isfinite(s) & (s > 0)
    assert np.all(m[ok] == 0.5), "UE8M0 scales must be powers of two"
    e[..., :kb] = np.where(np.isnan(s), 255, np.where(ok, ex - 1 + 127, 127)).astype(np.uint8)
    packed = e.reshape(s.shape[:-1] + (kq, 4)).copy().view("<u4")[..., 0].astype(np.uint32)
    return np.moveaxis(packed.view(np.int32), -1, axis).copy()


def _pow2_mult(rng: np.random.Generator, shape) -> np.ndarray:
    return np.exp2(rng.integers(-8, 9, size=shape)).astype(np.float32)


@dataclasses.dataclass
class Dense:
    a: np.ndarray
    sfa: np.ndarray          # [K/128, ld]
    b: np.ndarray
    sfb: np.ndarray
    c: Optional[np.ndarray]
    m: int
    n: int
    k: int


def make_dense(m: int, n: int, k: int, seed: int = 0, with_c: bool = False,
               c_std: float = 0.1, stress: bool = False, ue8m0: bool = False) -> Dense:
    """Dense problem; draw order A, B, C, then (stress) segment and block multipliers.

    ``ue8m0``: power-of-two scales, returned packed (``pack_ue8m0``): ``sfa`` int32
    [ceil(K/512), ld] and ``sfb`` int32 [ceil(N/128), ceil(K/512)].
    """
    rng = np.random.default_rng(seed)
    xa = rng.standard_normal((m, k), dtype=np.float32)
    xb = rng.standard_normal((n, k), dtype=np.float32)
    c = (rng.standard_normal((m, n), dtype=np.float32) * np.float32(c_std)) if with_c else None
    seg = blk = None
    if stress:
        seg = _pow2_mult(rng, (m, k // BLOCK))
        blk = _pow2_mult(rng, ((n + BLOCK - 1) // BLOCK, k // BLOCK))
    a, sa = quantize_rows(xa, seg, pow2=ue8m0)
    b, sb = quantize_blocks(xb, blk, pow2=ue8m0)
    sfa = mn_major(sa)
    if ue8m0:
        sfa, sb = pack_ue8m0(sfa, 0), pack_ue8m0(sb, 1)
    return Dense(a=a, sfa=sfa, b=b, sfb=sb, c=c, m=m, n=n, k=k)


def stored_layout(p: "Dense", layout: str) -> "Dense":
    """The same problem with A and B stored as ``layout`` ("nt", "nn", "tn" or "tt"; first
    letter A: "n" = [M, K], "t" = [K, M]; second letter B: "t" = [N, K], "n" = [K, N]).  The
    scales keep their layouts."""
    a = p.a if layout[0] == "n" else np.ascontiguousarray(p.a.T)
    b = p.b if layout[1] == "t" else np.ascontiguousarray(p.b.T)
    return dataclasses.replace(p, a=a, b=b)


@dataclasses.dataclass
class Contiguous:
    a: np.ndarray            # [M_total, K]
    sfa: np.ndarray          # [K/128, ld >= M_total]
    b: np.ndarray            # [G, N, K]
    sfb: np.ndarray          # [G, ceil(N/128), K/128]
    m_indices: np.ndarray    # int32 [M_total], -1 on padding rows
    counts: np.ndarray       # valid rows per group
    m_total: int
    n: int
    k: int
    num_groups: int


def make_contiguous(num_groups: int, total_rows: int, n: int, k: int, seed: int = 0,
                    counts=None, stress: bool = False, pad_nan: bool = False,
                    ue8m0: bool = False) -> Contiguous:
    """Contiguous M-grouped layout.

    Draw order: the ``total_rows`` valid token rows of A, then B for every group, then the
    routing p ~ Dirichlet(1), counts ~ Multinomial(total_rows, p) (unless ``counts`` is given),
    then (stress) multipliers. Rows are placed group after group; each group's segment is
    padded with rows of index -1 to a multiple of 128. Padding rows of A hold 0 (or the e4m3
    NaN pattern when ``pad_nan``) and scale 1 (NaN when ``pad_nan``).
    """
    rng = np.random.default_rng(seed)
    xa = rng.standard_normal((total_rows, k), dtype=np.float32)
    xb = rng.standard_normal((num_groups, n, k), dtype=np.float32)
    if counts is None:
        p = rng.dirichlet(np.ones(num_groups))
        counts = rng.multinomial(total_rows, p)
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.sum() == total_rows
    seg = blk = None
    nb = (n + BLOCK - 1) // BLOCK
    if stress:
        seg = _pow2_mult(rng, (total_rows, k // BLOCK))
        # a distinct power-of-two magnitude per group, so a misrouted row is a >= 2x error
        gmag = np.exp2(np.arange(num_groups) % 5 - 2).astype(np.float32)
        blk = _pow2_mult(rng, (num_groups, nb, k // BLOCK)) * gmag[:, None, None]
    qa, sa = quantize_rows(xa, seg, pow2=ue8m0)
    padded = (counts + BLOCK - 1) // BLOCK * BLOCK
    m_total = int(padded.sum())
    a = np.full((m_total, k), E4M3_NAN if pad_nan else 0, dtype=np.uint8)
    sa_full = np.full((m_total, k // BLOCK), np.nan if pad_nan else 1.0, dtype=np.float32)
    m_indices = np.full(m_total, -1, dtype=np.int32)
    src = dst = 0
    for g in range(num_groups):
        cnt = int(counts[g])
        a[dst:dst + cnt] = qa[src:src + cnt]
        sa_full[dst:dst + cnt] = sa[src:src + cnt]
        m_indices[dst:dst + cnt] = g
        src += cnt
        dst += int(padded[g])
    b = np.empty((num_groups, n, k), dtype=np.uint8)
    sfb = np.empty((num_groups, nb, k // BLOCK), dtype=np.float32)
    for g in range(num_groups):
        b[g], sfb[g] = quantize_blocks(xb[g], None if blk is None else blk[g], pow2=ue8m0)
    sfa = mn_major(sa_full)
    if ue8m0:
        sfa, sfb = pack_ue8m0(sfa, 0), pack_ue8m0(sfb, 2)
    return Contiguous(a=a, sfa=sfa, b=b, sfb=sfb, m_indices=m_indices,
                      counts=counts, m_total=m_total, n=n, k=k, num_groups=num_groups)


@dataclasses.dataclass
class Masked:
    a: np.ndarray            # [G, M_max, K]
    sfa: np.ndarray          # [G, K/128, ld >= M_max]
    b: np.ndarray            # [G, N, K]
    sfb: np.ndarray          # [G, ceil(N/128), K/128]
    masked_m: np.ndarray     # int32 [G]
    num_groups: int
    m_max: int
    n: int
    k: int


# ---------------------------------------------------------------------------------------------
# K-grouped form (MoE weight gradient, pt.news.hada.io, "GEMM denso e grouped": grouping on the
# K axis with M and N fixed).  Both operands are token-major ("T"/"N" of the TN layout): A is
# stored [K_total, M] and B [K_total, N], K being the tokens, concatenated group after group,
# each group's run padded with zero tokens to a multiple of 128.  Both are cast per 128 tokens
# of one column (a 128x1 block along K), the granularity the two-level accumulation needs when
# K is the token axis.


def quantize_kblocks(x: np.ndarray, mult: Optional[np.ndarray] = None):
    """128x1 cast along the leading (K) axis: x float32 [K, C] -> (bits uint8 [K, C],
    scales float32 [K/128, C]); ``mult`` [K/128, C] multiplies each block first (stress)."""
    k, cols = x.shape
    assert k % BLOCK == 0
    xs = x.reshape(k // BLOCK, BLOCK, cols)
    if mult is not None:
        xs = xs * mult[:, None, :].astype(np.float32)
    scale = _scale_of(np.abs(xs).max(axis=1), False)
    bits = _cast(xs, scale[:, None, :]).reshape(k, cols)
    return bits, scale


@dataclasses.dataclass
class KGrouped:
    a: np.ndarray            # uint8 [K_total, M]  (M contiguous)
    sfa: np.ndarray          # float32 [K_total/128, M]
    b: np.ndarray            # uint8 [K_total, N]  (N contiguous)
    sfb: np.ndarray          # float32 [K_total/128, N]
    ks: np.ndarray           # int32 [G]: the K extent of each group, multiples of 128 (0 allowed)
    counts: np.ndarray       # real tokens per group (the rest of its extent is zero padding)
    c: Optional[np.ndarray]  # float32 [G, M, N] or None
    num_groups: int
    m: int
    n: int
    k_total: int


def make_k_grouped(num_groups: int, total_tokens: int, m: int, n: int, seed: int = 0,
                   counts=None, with_c: bool = False, c_std: float = 0.1,
                   stress: bool = False) -> KGrouped:
    """K-grouped TN layout.  Draw order: the ``total_tokens`` token rows of A [T, M], those of
    B [T, N], the routing p ~ Dirichlet(1) and counts ~ Multinomial(T, p) (unless ``counts`` is
    given), C [G, M, N], then (stress) per-block multipliers 2^U{-8..8}.  Group g's tokens
    follow group g-1's; its extent is its count rounded up to a multiple of 128, with zero
    tokens (e4m3 0) in the padding."""
    rng = np.random.default_rng(seed)
    xa = rng.standard_normal((total_tokens, m), dtype=np.float32)
    xb = rng.standard_normal((total_tokens, n), dtype=np.float32)
    if counts is None:
        p = rng.dirichlet(np.ones(num_groups))
        counts = rng.multinomial(total_tokens, p)
    counts = np.asarray(counts, dtype=np.int64)
    assert counts.sum() == total_tokens
    c = None
    if with_c:
        c = rng.standard_normal((num_groups, m, n), dtype=np.float32) * np.float32(c_std)
    ks = (counts + BLOCK - 1) // BLOCK * BLOCK
    k_total = int(ks.sum())
    pa = np.zeros((k_total, m), dtype=np.float32)
    pb = np.zeros((k_total, n), dtype=np.float32)
    src = dst = 0
    for g in range(num_groups):
        cnt = int(counts[g])
        pa[dst:dst + cnt] = xa[src:src + cnt]
        pb[dst:dst + cnt] = xb[src:src + cnt]
        src += cnt
        dst += int(ks[g])
    del xa, xb
    ma = mb = None
    if stress:
        ma = _pow2_mult(rng, (k_total // BLOCK, m))
        mb = _pow2_mult(rng, (k_total // BLOCK, n))
    a, sfa = quantize_kblocks(pa, ma)
    del pa
    b, sfb = quantize_kblocks(pb, mb)
    return KGrouped(a=a, sfa=sfa, b=b, sfb=sfb, ks=ks.astype(np.int32), counts=counts, c=c,
                    num_groups=num_groups, m=m, n=n, k_total=k_total)


# ---------------------------------------------------------------------------------------------
# Input of the activation step between an expert's two GEMMs: the first GEMM's bf16 output
# X [M, 2I] (gate columns first, then up).


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (no NaN in the input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def make_swiglu_input(m: int, i: int, seed: int = 0, outliers: bool = True) -> np.ndarray:
    """bf16 bits [M, 2I]: N(0, 2) activations; with ``outliers``, one row segment in 64 scaled
    by 2^U{-6..6} (so segments' amax spans a wide range) and a few all-zero segments."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, 2 * i), dtype=np.float32) * np.float32(2.0)
    if outliers:
        segs = x.reshape(m, 2 * i // 128, 128)
        pick = rng.random(segs.shape[:2]) < 1 / 64
        mult = np.exp2(rng.integers(-6, 7, size=segs.shape[:2])).astype(np.float32)
        segs *= np.where(pick, mult, np.float32(1.0))[:, :, None]
        zero = rng.random(segs.shape[:2]) < 1 / 256
        segs *= np.where(zero, np.float32(0.0), np.float32(1.0))[:, :, None]
        x = segs.reshape(m, 2 * i)
    return f32_to_bf16_bits(x)


def masked_counts(num_groups: int, m_max: int, seed: int, replay: Optional[int] = None) -> np.ndarray:
    """masked_m ~ U{0..m_max} per group (inclusive). Replay r draws from default_rng((seed, r))."""
    rng = np.random.default_rng(seed if replay is None else (seed, replay))
    return rng.integers(0, m_max + 1, size=num_groups).astype(np.int32)


def make_masked(num_groups: int, m_max: int, n: int, k: int, seed: int = 0,
                masked_m=None, stress: bool = False, tail_nan: bool = False,
                ue8m0: bool = False) -> Masked:
    """Masked M-grouped layout. Draw order: A [G, M_max, K], B [G, N, K], masked_m, (stress).

    Every row of A is drawn; rows at or beyond masked_m[g] are ignored by the method and are
    replaced by the e4m3 NaN pattern (scale NaN) when ``tail_nan``.
    """
    rng = np.random.default_rng(seed)
    xa = rng.standard_normal((num_groups, m_max, k), dtype=np.float32)
    xb = rng.standard_normal((num_groups, n, k), dtype=np.float32)
    mm = rng.integers(0, m_max + 1, size=num_groups).astype(np.int32)
    if masked_m is not None:
        mm = np.asarray(masked_m, dtype=np.int32)
    nb = (n + BLOCK - 1) // BLOCK
    seg = blk = None
    if stress:
        seg = _pow2_mult(rng, (num_groups, m_max, k // BLOCK))
        gmag = np.exp2(np.arange(num_groups) % 5 - 2).astype(np.float32)
        blk = _pow2_mult(rng, (num_groups, nb, k // BLOCK)) * gmag[:, None, None]
    ld = sf_aligned(m_max)
    a = np.empty((num_groups, m_max, k), dtype=np.uint8)
    sfa = np.zeros((num_groups, k // BLOCK, ld), dtype=np.float32)
    b = np.empty((num_groups, n, k), dtype=np.uint8)
    sfb = np.empty((num_groups, nb, k // BLOCK), dtype=np.float32)
    for g in range(num_groups):
        a[g], sa = quantize_rows(xa[g], None if seg is None else seg[g], pow2=ue8m0)
        sfa[g] = mn_major(sa, ld)
        b[g], sfb[g] = quantize_blocks(xb[g], None if blk is None else blk[g], pow2=ue8m0)
        if tail_nan:
            lim = min(max(int(mm[g]), 0), m_max)
            a[g, lim:] = E4M3_NAN
            sfa[g, :, lim:m_max] = np.nan
    if ue8m0:
        sfa, sfb = pack_ue8m0(sfa, 1), pack_ue8m0(sfb, 2)
    return Masked(a=a, sfa=sfa, b=b, sfb=sfb, masked_m=mm, num_groups=num_groups,
                  m_max=m_max, n=n, k=k)


@dataclasses.dataclass
class MoEBlock:
    up: Contiguous           # first GEMM: B [G, 2I, K], gate rows first (n = 2I)
    b2: np.ndarray           # second GEMM's B [G, N2, I] e4m3
    sfb2: np.ndarray         # [G, ceil(N2/128), I/128]
    n2: int


def make_moe_block(num_groups: int, total_rows: int, n: int, k: int, n2: int, seed: int = 0,
                   counts=None) -> MoEBlock:
    """The two GEMMs of an MoE block's experts on the contiguous layout: the first as
    make_contiguous (n = 2I output columns, gate then up), then the second GEMM's weights,
    N(0,1) drawn [G, n2, I] from a generator seeded (seed, 2), each cast per 128x128 block."""
    up = make_contiguous(num_groups, total_rows, n, k, seed=seed, counts=counts)
    rng = np.random.default_rng((seed, 2))
    i = n // 2
    x2 = rng.standard_normal((num_groups, n2, i), dtype=np.float32)
    b2 = np.empty((num_groups, n2, i), dtype=np.uint8)
    sfb2 = np.empty((num_groups, (n2 + BLOCK - 1) // BLOCK, i // BLOCK), dtype=np.float32)
    for g in range(num_groups):
        b2[g], sfb2[g] = quantize_blocks(x2[g])
    return MoEBlock(up=up, b2=b2, sfb2=sfb2, n2=n2)


# The five workloads the library is measured and checked on (sizes from the method's
# DeepSeek-V3/R1 inference shapes: hidden 7168, MoE intermediate 2048/4096, 2112-wide
# low-rank projections).
CONFIGS = {
    "dense_small": dict(kind="dense", m=128, n=256, k=512, with_c=False),
    "dense_prefill": dict(kind="dense", m=4096, n=7168, k=2048, with_c=True),
    "dense_skinny": dict(kind="dense", m=64, n=2112, k=7168, with_c=False),
    "moe_contiguous": dict(kind="contiguous", num_groups=8, total_rows=32768, n=4096, k=7168),
    "moe_masked": dict(kind="masked", num_groups=16, m_max=256, n=7168, k=2048),
    # weight gradient of moe_contiguous's experts: dW[g] (4096 x 7168) over each expert's tokens
    "moe_wgrad": dict(kind="k_grouped", num_groups=8, total_tokens=32768, m=4096, n=7168),
    # SwiGLU + 1x128 FP8 cast of moe_contiguous's 32768 routed rows, expert width I = 2048
    "moe_swiglu_quant": dict(kind="swiglu", m=32768, i=2048),
    # the experts of an MoE block on moe_contiguous's routing: hidden 7168 -> 2 x 2048 (gate,
    # up) -> SwiGLU and the 1x128 cast -> 7168
    "moe_block": dict(kind="moe_block", num_groups=8, total_rows=32768, n=4096, k=7168,
                      n2=7168),
}


def make_config(name: str, seed: int = 0, **overrides):
    """One of CONFIGS; ``ue8m0=True`` gives the same shapes with packed UE8M0 scales."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "dense":
        return make_dense(seed=seed, **cfg)
    if kind == "contiguous":
        return make_contiguous(seed=seed, **cfg)
    if kind == "k_grouped":
        return make_k_grouped(seed=seed, **cfg)
    if kind == "swiglu":
        return make_swiglu_input(seed=seed, **cfg)
    if kind == "moe_block":
        return make_moe_block(seed=seed, **cfg)
    return make_masked(seed=seed, **cfg)
