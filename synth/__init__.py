"""Seeded synthetic inputs for block-sparse attention.

This module only draws numbers and lays them out.  It holds none of the
method's arithmetic (no pooling, scoring, selection, layout or softmax), so
that both the CPU oracle and the GPU path can consume the very same tensors
without sharing any code that computes results.

Every tensor is drawn in float32 from numpy ``Generator(PCG64)`` sub-streams
of one ``SeedSequence`` per workload and then rounded to bfloat16 with
round-to-nearest-even.  bfloat16 tensors are carried as ``uint16`` bit
patterns; ``bf16_to_f32`` widens them exactly.

Workloads (shapes from the source pages; structure terms are this module's
own recipe, chosen so that locality or content structure is real):

* ``C1`` tiny content-driven case: 64 text + 448 image tokens, block 64.
* ``C2`` single-stream DiT at FLUX.1 1024x1024 (4096 image + 512 text
  tokens, "UNet -> DiT" token-count table), arrow layout with per-head
  modes full / arrow(w=1) / skip.
* ``C3`` content-driven multimodal DiT at N = 256 + 4096, head dim 64,
  block 64 (block-sparse DiT write-up, sections 2.2 and 3.2).
* ``C4`` FLUX.1 2048x2048 (16384 image + 512 text tokens), arrow layout,
  window 8 blocks on every head.
* ``C5`` 64k-token bidirectional diffusion LM (SparseD notes: block 128,
  rho = 30 %, isolated prefill / generation selection).  Each head's
  structure (a diagonal band, 16 column-spike keys, or both) is strong
  enough to dominate the N(0, 1) noise over 64k keys, as the head-specific
  patterns the notes describe do: the top 30 % of key blocks hold ~0.99 of
  a band or spike head's attention and ~0.89 of a mixed head's (with the
  band at amplitude 0.75 and spikes at 0.6 they held ~0.35, little more
  than a uniform map).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

# Head modes.  The numeric codes are part of the C ABI.
HEAD_FULL = 0
HEAD_ARROW = 1
HEAD_SKIP = 2

# Scoring modes.  The numeric codes are part of the C ABI.
SCORE_MEANPOOL_PROJ = 0
SCORE_EXACT_AVGPOOL = 1


# --------------------------------------------------------------------------
# bfloat16 bit helpers (data format only)
# --------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bfloat16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    block: int
    text_len: int
    layout: str                     # "select", "arrow" or "neighborhood"
    seed: int
    score_mode: int = SCORE_MEANPOOL_PROJ
    r: int = 32                     # projection width (meanpool mode)
    groups: Tuple[Tuple[int, int, int], ...] = ()   # (col_begin, col_end, k)
    arrow_counts: Tuple[int, int, int] = (0, 0, 0)  # (#arrow, #full, #skip) heads
    arrow_window: int = 0
    nb_grid: Tuple[int, int] = (0, 0)      # neighbourhood: image grid (rows, cols)
    nb_tile: Tuple[int, int] = (0, 0)      # tile (rows, cols), one block each
    nb_window: Tuple[int, int] = (0, 0)
    nb_stride: Tuple[int, int] = (1, 1)
    structure: str = "none"
    description: str = ""

    @property
    def n_blocks(self) -> int:
        return -(-self.N // self.block)

    @property
    def text_blocks(self) -> int:
        # a block that holds any text token counts as a text block
        return -(-self.text_len // self.block)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "C1": Workload(
        name="C1", B=1, H=2, N=512, D=64, block=64, text_len=64, layout="select",
        seed=1, score_mode=SCORE_MEANPOOL_PROJ, r=32, groups=((0, 8, 4),),
        structure="iid",
        description="tiny content-driven: 64 text + 448 image tokens, top-4 of 8 key blocks"),
    "C2": Workload(
        name="C2", B=1, H=24, N=4608, D=128, block=128, text_len=512, layout="arrow",
        seed=2, arrow_counts=(12, 8, 4), arrow_window=1, structure="pos2d",
        description="single-stream DiT, FLUX.1 1024^2: 512 text + 64x64 image, "
                    "12 arrow(w=1) / 8 full / 4 skip heads"),
    "C3": Workload(
        name="C3", B=2, H=16, N=4352, D=64, block=64, text_len=256, layout="select",
        seed=3, score_mode=SCORE_MEANPOOL_PROJ, r=32, groups=((4, 68, 16),),
        structure="lowrank",
        description="content-driven multimodal DiT: 256 text + 4096 image, "
                    "top-25% image key blocks"),
    "C4": Workload(
        name="C4", B=1, H=24, N=16896, D=128, block=128, text_len=512, layout="arrow",
        seed=4, arrow_counts=(24, 0, 0), arrow_window=8, structure="pos2d",
        description="2K MMDiT, FLUX.1 2048^2: 512 text + 128x128 image, arrow w=8 all heads"),
    "C5": Workload(
        name="C5", B=1, H=32, N=65536, D=128, block=128, text_len=0, layout="select",
        seed=5, score_mode=SCORE_EXACT_AVGPOOL, groups=((0, 480, 144), (480, 512, 10)),
        structure="dlm",
        description="64k bidirectional diffusion LM: exact avgpool scores, "
                    "top-30% prefill and generation columns"),
    # 2-D neighbourhood attention (GNA) on the FLUX.1 2048^2 shape: window
    # side a quarter of the 128 x 128 latent grid, 8 x 16 tiles of one block
    "G1": Workload(
        name="G1", B=1, H=24, N=16896, D=128, block=128, text_len=512, layout="neighborhood",
        seed=6, nb_grid=(128, 128), nb_tile=(8, 16), nb_window=(32, 32), nb_stride=(1, 1),
        structure="pos2d",
        description="2K MMDiT, FLUX.1 2048^2: 512 text + 128x128 image, 2-D neighbourhood window "
                    "32x32 (GNA), 8x16 tiles"),
}


# --------------------------------------------------------------------------
# Structure terms (this module's own recipe)
# --------------------------------------------------------------------------
def _pos2d(rng: np.random.Generator, n_img: int, D: int, amp: float) -> np.ndarray:
    """Smooth 2-D positional embedding on a square row-major image grid.

    D/4 frequencies with wavelengths log-spaced in [4, R]; each frequency
    contributes (sin, cos) of the row and of the column with seeded phases.
    The dot product of two embeddings is a sum of cosines of the row and
    column offsets, peaked at zero offset with value amp^2 * D / 2.
    """
    R = int(round(math.sqrt(n_img)))
    assert R * R == n_img, "image tokens must form a square grid"
    nf = D // 4
    lam = np.geomspace(4.0, max(float(R), 4.0), nf)
    om = 2.0 * np.pi / lam
    ph_r = rng.uniform(0, 2 * np.pi, nf)
    ph_c = rng.uniform(0, 2 * np.pi, nf)
    idx = np.arange(n_img)
    rr = (idx // R).astype(np.float64)[:, None]
    cc = (idx % R).astype(np.float64)[:, None]
    e = np.empty((n_img, D), dtype=np.float64)
    e[:, 0::4] = np.sin(om * rr + ph_r)
    e[:, 1::4] = np.cos(om * rr + ph_r)
    e[:, 2::4] = np.sin(om * cc + ph_c)
    e[:, 3::4] = np.cos(om * cc + ph_c)
    return (amp * e).astype(np.float32)


def _pos1d(rng: np.random.Generator, N: int, D: int, amp: float,
           lam_lo: float, lam_hi: float) -> np.ndarray:
    """Smooth 1-D positional embedding (a diagonal band in the logits)."""
    nf = D // 2
    lam = np.geomspace(lam_lo, lam_hi, nf)
    om = 2.0 * np.pi / lam
    ph = rng.uniform(0, 2 * np.pi, nf)
    t = np.arange(N, dtype=np.float64)[:, None]
    e = np.empty((N, D), dtype=np.float32)
    e[:, 0::2] = np.sin(om * t + ph)
    e[:, 1::2] = np.cos(om * t + ph)
    e *= amp
    return e


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# --------------------------------------------------------------------------
# Workload generator
# --------------------------------------------------------------------------
def make_inputs(wl: Workload, seed: Optional[int] = None) -> dict:
    """Draw every input of a workload.

    Returns a dict with
      q, k, v        uint16 bf16 bits, shape [B, H, N, D]
      w              float32 [D, r] projection (meanpool selection only)
      head_modes     int8 [H]   (arrow layout only)
      head_windows   int32 [H]  (arrow layout only)
      o_cache        uint16 bf16 [B, H, N, D] (when some head is SKIP)
      lse_cache      float32 [B, H, N]        (when some head is SKIP)
    """
    seed = wl.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_w, s_mode, s_cache, s_struct, s_extra = ss.spawn(8)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    shape = (B, H, N, D)
    rq, rk, rv = (np.random.Generator(np.random.PCG64(s)) for s in (s_q, s_k, s_v))
    rs = np.random.Generator(np.random.PCG64(s_struct))

    q = _normal(rq, shape)
    k = _normal(rk, shape)
    v = _normal(rv, shape)

    if wl.structure == "pos2d":
        n_img = N - wl.text_len
        for h in range(H):
            e = _pos2d(rs, n_img, D, amp=0.75)
            q[:, h, wl.text_len:, :] += e
            k[:, h, wl.text_len:, :] += e
    elif wl.structure == "lowrank":
        for b in range(B):
            for h in range(H):
                L = _normal(rs, (N, 8))
                R = _normal(rs, (8, D), scale=1.0 / math.sqrt(8.0))
                c = L @ R
                q[b, h] += c
                k[b, h] += c
    elif wl.structure == "dlm":
        # per-head type: 0 band, 1 column spikes, 2 mixed (counts 11/11/10 at H=32)
        n_band = int(round(H * 11 / 32))
        n_col = int(round(H * 11 / 32))
        types = np.array([0] * n_band + [1] * n_col + [2] * (H - n_band - n_col))
        types = types[rs.permutation(H)]
        for h in range(H):
            t = int(types[h])
            wb = 1.0 if t == 0 else (0.0 if t == 1 else 1.0 / math.sqrt(2.0))
            wc = 1.0 if t == 1 else (0.0 if t == 0 else 1.0 / math.sqrt(2.0))
            # band: +12.7 on the scaled logit at zero offset (amp^2 D / 2 / sqrt(D));
            # spikes: +16.3 on the 16 spike keys (scale^2 D / sqrt(D))
            if wb > 0:
                e = _pos1d(rs, N, D, amp=1.5 * wb, lam_lo=64.0, lam_hi=8192.0)
                q[:, h] += e
                k[:, h] += e
            if wc > 0:
                u = _normal(rs, (D,), scale=1.2 * wc)
                pos = rs.choice(N, size=min(16, N), replace=False)
                q[:, h] += u
                k[:, h, pos, :] += u
    elif wl.structure in ("iid", "none"):
        pass
    else:
        raise ValueError(f"unknown structure {wl.structure!r}")

    out = {"q": f32_to_bf16(q), "k": f32_to_bf16(k), "v": f32_to_bf16(v)}
    del q, k, v

    if wl.layout == "select" and wl.score_mode == SCORE_MEANPOOL_PROJ:
        rw = np.random.Generator(np.random.PCG64(s_w))
        out["w"] = _normal(rw, (D, wl.r), scale=1.0 / math.sqrt(D))

    if wl.layout == "arrow":
        n_arrow, n_full, n_skip = wl.arrow_counts
        assert n_arrow + n_full + n_skip == H
        modes = np.array([HEAD_ARROW] * n_arrow + [HEAD_FULL] * n_full
                         + [HEAD_SKIP] * n_skip, dtype=np.int8)
        rm = np.random.Generator(np.random.PCG64(s_mode))
        modes = modes[rm.permutation(H)]
        out["head_modes"] = modes
        out["head_windows"] = np.full(H, wl.arrow_window, dtype=np.int32)
        if n_skip > 0:
            rc = np.random.Generator(np.random.PCG64(s_cache))
            out["o_cache"] = f32_to_bf16(_normal(rc, shape))
            out["lse_cache"] = (_normal(rc, (B, H, N)) + np.float32(math.log(N))).astype(np.float32)
    return out


# --------------------------------------------------------------------------
# Small random cases for property and parity tests
# --------------------------------------------------------------------------
def random_qkv(B: int, H: int, N: int, D: int, seed: int, scale: float = 1.0):
    """Three bf16 tensors [B, H, N, D] with N(0, scale^2) entries."""
    ss = np.random.SeedSequence(seed)
    out = []
    for s in ss.spawn(3):
        r = np.random.Generator(np.random.PCG64(s))
        out.append(f32_to_bf16(_normal(r, (B, H, N, D), scale=scale)))
    return tuple(out)


def random_block_lists(B: int, H: int, nB: int, seed: int,
                       density: float = 0.3, empty_rows: int = 1,
                       full_rows: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """A random CSR block list: per (b, h, query block) row an ascending set of
    key blocks.  Some rows are forced empty and some full, to cover both edges."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    rows = B * H * nB
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    cols = []
    special = r.permutation(rows)
    empty = set(special[:empty_rows].tolist())
    full = set(special[empty_rows:empty_rows + full_rows].tolist())
    for x in range(rows):
        if x in empty:
            sel = np.zeros(0, dtype=np.int32)
        elif x in full:
            sel = np.arange(nB, dtype=np.int32)
        else:
            m = r.random(nB) < density
            if not m.any():
                m[r.integers(nB)] = True
            sel = np.nonzero(m)[0].astype(np.int32)
        cols.append(sel)
        row_ptr[x + 1] = row_ptr[x] + len(sel)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int32)
    return row_ptr, col_idx.astype(np.int32)


def block_lists_with_counts(B: int, H: int, nB: int, groups: Sequence[Tuple[int, int, int]],
                            text_blocks: int, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    """A random CSR with the shape of a group-budgeted selection: rows of text
    query blocks are dense; every other row holds the text columns plus k_g
    distinct random columns from each group range.  Used where a selection of
    the true size is needed without running any scoring."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    rows = B * H * nB
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    cols = []
    for x in range(rows):
        i = x % nB
        if i < text_blocks:
            sel = np.arange(nB, dtype=np.int32)
        else:
            m = np.zeros(nB, dtype=bool)
            m[:text_blocks] = True
            for (c0, c1, kk) in groups:
                m[c0 + r.choice(c1 - c0, size=kk, replace=False)] = True
            sel = np.nonzero(m)[0].astype(np.int32)
        cols.append(sel)
        row_ptr[x + 1] = row_ptr[x] + len(sel)
    return row_ptr, np.concatenate(cols).astype(np.int32)


def random_scores(B: int, H: int, nB: int, seed: int, tie_levels: int = 0) -> np.ndarray:
    """float32 score matrices [B, H, nB, nB].  With tie_levels > 0 the values are
    drawn from that many distinct levels, so exact ties are common."""
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    if tie_levels > 0:
        lv = r.standard_normal(tie_levels).astype(np.float32)
        return lv[r.integers(0, tie_levels, size=(B, H, nB, nB))]
    return r.standard_normal((B, H, nB, nB)).astype(np.float32)
