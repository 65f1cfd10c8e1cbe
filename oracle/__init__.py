"""fp64 CPU oracle for block-sparse attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The GPU library never imports, links or calls
it, and this package never imports the GPU library.

The arithmetic lives in ``bsa_oracle.c`` (plain C, fp64, OpenMP over
independent outputs); this module only marshals numpy arrays.  The shared
library is compiled with gcc on first use (or by ``build()``).

Every function follows the definitions stated in ``bsa_oracle.c``:
  pool_mean               mean of each block's rows
  scores_meanpool_proj    S_ij = (W^T qbar_i) . (W^T kbar_j)
  score_grad              its vector-Jacobian product: dW, dqbar, dkbar for
                          an upstream gradient dS
  scores_exact_avgpool    S_ij = block-average of softmax(scale * Q K^T)
  select_rows / select    text rows dense, text columns forced, top-k per
                          column group with lower-index tie-break
  arrow                   closed-form arrow / full / skip layout
  forward                 dense softmax restricted to the kept blocks
  quantize_fp8 / forward_fp8   E4M3 codes with max-abs scales; the forward
                          on the dequantised inputs
  na_start / forward_neighborhood / tile_permutation / neighborhood_layout
                          2-D neighbourhood (GNA) attention on the latent
                          grid: window start, the masked forward, tile-major
                          token order, block layout with full / partial flags
  forward_f64 / backward  the forward on fp64 inputs and its gradient
                          (dQ, dK, dV of the kept-block softmax)
  backward_dq_rows        dQ of selected query rows (full-size checks)
  forward_neighborhood_f64 / backward_neighborhood
                          the same under the 2-D neighbourhood token mask
  output_rse              per-head relative squared error of an output
  mask_jaccard            per-head Jaccard similarity of two block masks
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

HEAD_FULL, HEAD_ARROW, HEAD_SKIP = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, -O2, OpenMP).  Returns the .so path."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_pool_mean.argtypes = [P, I, I, I, I, I, P]
        lib.oracle_pool_mean.restype = ctypes.c_int
        lib.oracle_scores_meanpool_proj.argtypes = [P, P, I, I, I, I, I, P, I, P]
        lib.oracle_scores_meanpool_proj.restype = ctypes.c_int
        D_ = ctypes.c_double
        lib.oracle_forward_neighborhood_f64.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, D_, P, P]
        lib.oracle_forward_neighborhood_f64.restype = ctypes.c_int
        lib.oracle_forward_neighborhood_f64_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, D_, P, I, P, P]
        lib.oracle_forward_neighborhood_f64_rows.restype = ctypes.c_int
        lib.oracle_backward_neighborhood_f64.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, D_, P, P, P]
        lib.oracle_backward_neighborhood_f64.restype = ctypes.c_int
        lib.oracle_backward_dq_rows.argtypes = [P, P, P, P, I, I, I, I, I, P, P, D_, P, I, P]
        lib.oracle_backward_dq_rows.restype = ctypes.c_int
        lib.oracle_backward_neighborhood_dq_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I, I, I, I, D_, P, I,
                                                             P]
        lib.oracle_backward_neighborhood_dq_rows.restype = ctypes.c_int
        lib.oracle_score_grad.argtypes = [P, P, I, I, I, I, I, P, I, P, P, P, P]
        lib.oracle_score_grad.restype = ctypes.c_int
        lib.oracle_scores_exact_avgpool.argtypes = [P, P, I, I, I, I, I, D, P, I, P]
        lib.oracle_scores_exact_avgpool.restype = ctypes.c_int
        lib.oracle_select_rows.argtypes = [P, P, I, I, I, P, I, P, P, I]
        lib.oracle_select_rows.restype = ctypes.c_int64
        lib.oracle_arrow.argtypes = [I, I, I, I, P, P, P, P, I]
        lib.oracle_arrow.restype = ctypes.c_int64
        lib.oracle_forward.argtypes = [P, P, P, I, I, I, I, I, P, P, P, P, P, D, P, I, P, P]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_e4m3_encode_array.argtypes = [P, I, P]
        lib.oracle_e4m3_encode_array.restype = None
        lib.oracle_e4m3_decode_array.argtypes = [P, I, P]
        lib.oracle_e4m3_decode_array.restype = None
        lib.oracle_quantize_fp8.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, P]
        lib.oracle_na_start.argtypes = [I, I, I, I]
        lib.oracle_na_start.restype = I
        lib.oracle_forward_neighborhood.argtypes = [P, P, P, I, I, I, I, I, I, I, I, I, I, I, D, P, I, P, P]
        lib.oracle_tile_permutation.argtypes = [I, I, I, I, I, P]
        lib.oracle_neighborhood_layout.argtypes = [I, I, I, I, I, I, I, I, I, P, P, P, I]
        lib.oracle_forward_f64.argtypes = [P, P, P, I, I, I, I, I, P, P, D, P, P]
        lib.oracle_backward_f64.argtypes = [P, P, P, P, I, I, I, I, I, P, P, D, P, P, P]
        lib.oracle_forward_fp8.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P, D, P, I, P, P]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 tensors are passed as uint16 bit patterns"
    return a


def _check(rc: int, what: str):
    if rc < 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def n_blocks(N: int, block: int) -> int:
    return -(-N // block)


def threads() -> int:
    return int(_load().oracle_threads())


def pool_mean(x: np.ndarray, block: int) -> np.ndarray:
    """[B,H,N,D] bf16 bits -> fp64 [B,H,nB,D] block means."""
    x = _u16(x)
    B, H, N, D = x.shape
    out = np.empty((B, H, n_blocks(N, block), D), dtype=np.float64)
    _check(_load().oracle_pool_mean(_ptr(x), B, H, N, D, block, _ptr(out)), "pool_mean")
    return out


def scores_meanpool_proj(q: np.ndarray, k: np.ndarray, block: int, w: np.ndarray) -> np.ndarray:
    """fp64 S [B,H,nB,nB] from mean-pooled, projected blocks."""
    q, k = _u16(q), _u16(k)
    w = np.ascontiguousarray(w, dtype=np.float32)
    B, H, N, D = q.shape
    assert k.shape == q.shape and w.shape[0] == D
    nB = n_blocks(N, block)
    S = np.empty((B, H, nB, nB), dtype=np.float64)
    _check(_load().oracle_scores_meanpool_proj(_ptr(q), _ptr(k), B, H, N, D, block,
                                               _ptr(w), w.shape[1], _ptr(S)), "scores_meanpool_proj")
    return S


def score_grad(q: np.ndarray, k: np.ndarray, block: int, w: np.ndarray,
               dS: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradient of L with dL/dS = dS through S = scores_meanpool_proj(q, k,
    block, w): returns fp64 (dW [D, r], dqbar [B,H,nB,D], dkbar [B,H,nB,D])."""
    q, k = _u16(q), _u16(k)
    w = np.ascontiguousarray(w, dtype=np.float32)
    B, H, N, D = q.shape
    r = w.shape[1]
    nB = n_blocks(N, block)
    assert k.shape == q.shape and w.shape[0] == D
    dS = np.ascontiguousarray(dS, dtype=np.float64)
    assert dS.shape == (B, H, nB, nB)
    dW = np.empty((D, r), dtype=np.float64)
    dq = np.empty((B, H, nB, D), dtype=np.float64)
    dk = np.empty((B, H, nB, D), dtype=np.float64)
    _check(_load().oracle_score_grad(_ptr(q), _ptr(k), B, H, N, D, block, _ptr(w), r, _ptr(dS),
                                     _ptr(dW), _ptr(dq), _ptr(dk)), "score_grad")
    return dW, dq, dk


def scores_exact_avgpool(q: np.ndarray, k: np.ndarray, block: int, scale: Optional[float] = None,
                         rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 block-averaged softmax attention.  With rows=None returns
    [B,H,nB,nB]; otherwise [len(rows), nB] for the listed flat rows
    (b*H + h)*nB + i."""
    q, k = _u16(q), _u16(k)
    B, H, N, D = q.shape
    nB = n_blocks(N, block)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    lib = _load()
    if rows is None:
        S = np.empty((B, H, nB, nB), dtype=np.float64)
        _check(lib.oracle_scores_exact_avgpool(_ptr(q), _ptr(k), B, H, N, D, block, scale,
                                               None, 0, _ptr(S)), "scores_exact_avgpool")
        return S
    r = np.ascontiguousarray(rows, dtype=np.int64)
    S = np.empty((len(r), nB), dtype=np.float64)
    _check(lib.oracle_scores_exact_avgpool(_ptr(q), _ptr(k), B, H, N, D, block, scale,
                                           _ptr(r), len(r), _ptr(S)), "scores_exact_avgpool")
    return S


def _groups_arr(groups) -> np.ndarray:
    g = np.ascontiguousarray(np.array(groups, dtype=np.int32).reshape(-1, 3))
    return g


def select_rows(S_rows: np.ndarray, qblock: Sequence[int], text_blocks: int,
                groups) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k selection for a list of rows.  S_rows [n, nB] (any float dtype,
    widened to fp64 exactly), qblock[n] = each row's query-block index."""
    S_rows = np.ascontiguousarray(S_rows, dtype=np.float64)
    n, nB = S_rows.shape
    qb = np.ascontiguousarray(qblock, dtype=np.int32)
    g = _groups_arr(groups)
    cap = n * nB
    row_ptr = np.zeros(n + 1, dtype=np.int32)
    col_idx = np.zeros(max(cap, 1), dtype=np.int32)
    nnz = _load().oracle_select_rows(_ptr(S_rows), _ptr(qb), n, nB, text_blocks, _ptr(g),
                                     len(g), _ptr(row_ptr), _ptr(col_idx), cap)
    _check(nnz, "select_rows")
    return row_ptr, col_idx[:nnz].copy()


def select(S: np.ndarray, text_blocks: int, groups) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k selection over a full [B,H,nB,nB] score tensor -> CSR over (b,h,i)."""
    B, H, nB, nB2 = S.shape
    assert nB == nB2
    qb = np.tile(np.arange(nB, dtype=np.int32), B * H)
    return select_rows(S.reshape(B * H * nB, nB), qb, text_blocks, groups)


def arrow(B: int, H: int, nB: int, text_blocks: int, modes: np.ndarray,
          windows: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Arrow / full / skip layout as CSR over (b,h,i)."""
    modes = np.ascontiguousarray(modes, dtype=np.int8)
    windows = np.ascontiguousarray(windows, dtype=np.int32)
    lib = _load()
    row_ptr = np.zeros(B * H * nB + 1, dtype=np.int32)
    nnz = lib.oracle_arrow(B, H, nB, text_blocks, _ptr(modes), _ptr(windows), _ptr(row_ptr),
                           None, 0)
    _check(nnz, "arrow")
    col_idx = np.zeros(max(nnz, 1), dtype=np.int32)
    nnz2 = lib.oracle_arrow(B, H, nB, text_blocks, _ptr(modes), _ptr(windows), _ptr(row_ptr),
                            _ptr(col_idx), nnz)
    _check(nnz2, "arrow")
    return row_ptr, col_idx[:nnz].copy()


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int,
            row_ptr: np.ndarray, col_idx: np.ndarray, modes: Optional[np.ndarray] = None,
            o_cache: Optional[np.ndarray] = None, lse_cache: Optional[np.ndarray] = None,
            scale: Optional[float] = None,
            rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Dense softmax over the kept blocks.  rows=None -> O [B,H,N,D], LSE
    [B,H,N]; otherwise O [n, D], LSE [n] for flat token rows (b*H + h)*N + t."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    if col_idx.size == 0:
        col_idx = np.zeros(1, dtype=np.int32)
    assert row_ptr.shape[0] == B * H * n_blocks(N, block) + 1
    modes_a = None if modes is None else np.ascontiguousarray(modes, dtype=np.int8)
    oc = None if o_cache is None else _u16(o_cache)
    lc = None if lse_cache is None else np.ascontiguousarray(lse_cache, dtype=np.float32)
    lib = _load()
    if rows is None:
        O = np.empty((B, H, N, D), dtype=np.float64)
        L = np.empty((B, H, N), dtype=np.float64)
        rc = lib.oracle_forward(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, block, _ptr(row_ptr),
                                _ptr(col_idx), _ptr(modes_a), _ptr(oc), _ptr(lc), scale,
                                None, 0, _ptr(O), _ptr(L))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        O = np.empty((len(r), D), dtype=np.float64)
        L = np.empty((len(r),), dtype=np.float64)
        rc = lib.oracle_forward(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, block, _ptr(row_ptr),
                                _ptr(col_idx), _ptr(modes_a), _ptr(oc), _ptr(lc), scale,
                                _ptr(r), len(r), _ptr(O), _ptr(L))
    _check(rc, "forward")
    return O, L


# ---------------------------------------------------------------------------
# FP8 (OCP E4M3) quantisation and the forward on the quantised inputs
# ---------------------------------------------------------------------------
def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) of float32 values, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
    return out


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """Values (float64) of OCP E4M3 codes."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def quantize_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """(q8 [B,H,N,D], q_scale [B,H,N], k8 [B,H,N,D], k_scale [B,H,ceil(N/64)],
    v8 [B,H,N,D], v_scale [B,H,D]): per-token Q, per-64-key-tile K and
    per-channel V max-abs scaling to E4M3 (codes decided in fp32)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, D = q.shape
    NT = (N + 63) // 64
    q8 = np.empty((B, H, N, D), np.uint8); k8 = np.empty_like(q8); v8 = np.empty_like(q8)
    qs = np.empty((B, H, N), np.float32); ks = np.empty((B, H, NT), np.float32)
    vs = np.empty((B, H, D), np.float32)
    _check(_load().oracle_quantize_fp8(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, _ptr(q8), _ptr(qs),
                                       _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs)), "quantize_fp8")
    return q8, qs, k8, ks, v8, vs


def forward_fp8(q8, q_scale, k8, k_scale, v8, v_scale, block: int, row_ptr, col_idx,
                scale: Optional[float] = None, rows: Optional[Sequence[int]] = None):
    """The block-sparse forward on the dequantised inputs (see quantize_fp8)."""
    q8 = np.ascontiguousarray(q8, np.uint8); k8 = np.ascontiguousarray(k8, np.uint8)
    v8 = np.ascontiguousarray(v8, np.uint8)
    qs = np.ascontiguousarray(q_scale, np.float32); ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    B, H, N, D = q8.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    if col_idx.size == 0:
        col_idx = np.zeros(1, dtype=np.int32)
    lib = _load()
    if rows is None:
        O = np.empty((B, H, N, D), np.float64); L = np.empty((B, H, N), np.float64)
        rc = lib.oracle_forward_fp8(_ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs), B, H, N, D,
                                    block, _ptr(row_ptr), _ptr(col_idx), scale, None, 0, _ptr(O), _ptr(L))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        O = np.empty((len(r), D), np.float64); L = np.empty((len(r),), np.float64)
        rc = lib.oracle_forward_fp8(_ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs), B, H, N, D,
                                    block, _ptr(row_ptr), _ptr(col_idx), scale, _ptr(r), len(r), _ptr(O),
                                    _ptr(L))
    _check(rc, "forward_fp8")
    return O, L


# ---------------------------------------------------------------------------
# Diagnostics of sparse against full attention and of mask reuse
# ---------------------------------------------------------------------------
def output_rse(y_test: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-(b, h) relative squared error of an attention output against a
    reference (DiTFastAttnV2, "Headwise Arrow Attention", single-layer RSE):

        RSE = sum (y_test - y_ref)^2 / sum (y_ref - mean(y_ref))^2

    over the head's N x D elements, mean over the same elements.  Inputs are
    [B, H, N, D] (bf16 bit patterns as uint16, or floats); returns fp64
    [B, H].  A reference with no spread gives +inf (0/0 gives 0)."""
    t = _widen(y_test)
    r = _widen(y_ref)
    B, H = r.shape[:2]
    out = np.empty((B, H), np.float64)
    for b in range(B):
        for h in range(H):
            ref = r[b, h].reshape(-1)
            num = float(np.sum((t[b, h].reshape(-1) - ref) ** 2))
            den = float(np.sum((ref - ref.mean()) ** 2))
            out[b, h] = (0.0 if num == 0.0 else math.inf) if den == 0.0 else num / den
    return out


def mask_jaccard(B: int, H: int, n_blocks: int, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b) -> np.ndarray:
    """Per-(b, h) Jaccard similarity |A & B| / |A | B| of two block masks
    given as CSR over rows (b*H + h)*nB + i (SparseD, "sparse reuse": the
    stability of the reused mask against each step's own selection).
    Entries outside [0, nB) are ignored; repeated entries count once; two
    empty masks have similarity 1."""
    out = np.empty((B, H), np.float64)
    for b in range(B):
        for h in range(H):
            inter = union = 0
            for i in range(n_blocks):
                r = (b * H + h) * n_blocks + i
                a = {int(j) for j in col_idx_a[row_ptr_a[r]:row_ptr_a[r + 1]] if 0 <= j < n_blocks}
                c = {int(j) for j in col_idx_b[row_ptr_b[r]:row_ptr_b[r + 1]] if 0 <= j < n_blocks}
                inter += len(a & c)
                union += len(a | c)
            out[b, h] = 1.0 if union == 0 else inter / union
    return out


def _widen(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# 2-D neighbourhood attention (GNA)
# ---------------------------------------------------------------------------
def na_start(i: int, L: int, k: int, s: int) -> int:
    """First position of the window of position i on an axis of length L
    (window k, stride s)."""
    return int(_load().oracle_na_start(i, L, k, s))


def forward_neighborhood(q, k, v, text_len: int, grid: Tuple[int, int], window: Tuple[int, int],
                         stride: Tuple[int, int] = (1, 1), scale: Optional[float] = None,
                         rows: Optional[Sequence[int]] = None):
    """Softmax attention under the 2-D neighbourhood mask, natural token order
    (text tokens, then the image grid row-major)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    (R, C), (kh, kw), (sh, sw) = grid, window, stride
    lib = _load()
    if rows is None:
        O = np.empty((B, H, N, D), np.float64); L = np.empty((B, H, N), np.float64)
        rc = lib.oracle_forward_neighborhood(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, text_len, R, C, kh, kw, sh, sw,
                                             scale, None, 0, _ptr(O), _ptr(L))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        O = np.empty((len(r), D), np.float64); L = np.empty((len(r),), np.float64)
        rc = lib.oracle_forward_neighborhood(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, text_len, R, C, kh, kw, sh, sw,
                                             scale, _ptr(r), len(r), _ptr(O), _ptr(L))
    _check(rc, "forward_neighborhood")
    return O, L


def tile_permutation(text_len: int, grid: Tuple[int, int], tile: Tuple[int, int]) -> np.ndarray:
    """perm[p] = natural index of the token at tile-major position p."""
    (R, C), (th, tw) = grid, tile
    perm = np.empty(text_len + R * C, np.int64)
    _check(_load().oracle_tile_permutation(text_len, R, C, th, tw, _ptr(perm)), "tile_permutation")
    return perm


def neighborhood_layout(text_len: int, grid: Tuple[int, int], tile: Tuple[int, int], window: Tuple[int, int],
                        stride: Tuple[int, int] = (1, 1)):
    """Block layout of one head in tile-major order: (row_ptr, col_idx, flags),
    flag 0 = every (query, key) pair of the block pair kept, 1 = some."""
    (R, C), (th, tw), (kh, kw), (sh, sw) = grid, tile, window, stride
    nB = (text_len + R * C) // (th * tw)
    row_ptr = np.empty(nB + 1, np.int32)
    col_idx = np.empty(nB * nB, np.int32)
    flags = np.empty(nB * nB, np.uint8)
    _check(_load().oracle_neighborhood_layout(text_len, R, C, th, tw, kh, kw, sh, sw, _ptr(row_ptr), _ptr(col_idx),
                                              _ptr(flags), nB * nB), "neighborhood_layout")
    n = int(row_ptr[-1])
    return row_ptr, col_idx[:n].copy(), flags[:n].copy()


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(_widen(a))
    return np.ascontiguousarray(a, dtype=np.float64)


def _csr(row_ptr, col_idx):
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    if ci.size == 0:
        ci = np.zeros(1, dtype=np.int32)
    return rp, ci


def forward_f64(q, k, v, block: int, row_ptr, col_idx, scale: Optional[float] = None):
    """The block-sparse forward on fp64 (or bf16-bit) inputs: (O, LSE) in fp64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rp, ci = _csr(row_ptr, col_idx)
    O = np.empty((B, H, N, D), np.float64); L = np.empty((B, H, N), np.float64)
    _check(_load().oracle_forward_f64(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, block, _ptr(rp), _ptr(ci), scale,
                                      _ptr(O), _ptr(L)), "forward_f64")
    return O, L


def backward(q, k, v, dO, block: int, row_ptr, col_idx, scale: Optional[float] = None):
    """(dQ, dK, dV) in fp64 of the block-sparse forward at (q, k, v) for the
    output gradient dO (fp64 or bf16-bit inputs)."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rp, ci = _csr(row_ptr, col_idx)
    dQ = np.empty_like(q); dK = np.empty_like(q); dV = np.empty_like(q)
    _check(_load().oracle_backward_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), B, H, N, D, block, _ptr(rp), _ptr(ci),
                                       scale, _ptr(dQ), _ptr(dK), _ptr(dV)), "backward")
    return dQ, dK, dV


def backward_dq_rows(q, k, v, dO, block: int, row_ptr, col_idx, rows, scale: Optional[float] = None):
    """dQ (fp64, [len(rows), D]) of the flat query rows `rows` (indices into
    [B*H*N]) of the block-sparse forward's gradient."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    rp, ci = _csr(row_ptr, col_idx)
    r = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(r), D), np.float64)
    _check(_load().oracle_backward_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), B, H, N, D, block, _ptr(rp),
                                           _ptr(ci), scale, _ptr(r), len(r), _ptr(out)), "backward_dq_rows")
    return out


def forward_neighborhood_f64(q, k, v, text_len: int, grid: Tuple[int, int], window: Tuple[int, int],
                             stride: Tuple[int, int] = (1, 1), scale: Optional[float] = None,
                             rows: Optional[Sequence[int]] = None):
    """The neighbourhood forward on fp64 (or bf16-bit) inputs, natural token
    order: (O, LSE) in fp64; with `rows`, only those flat query rows
    ((b*H + h)*N + t): O [len(rows), D], LSE [len(rows)]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    (R, C), (kh, kw), (sh, sw) = grid, window, stride
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        O = np.empty((len(r), D), np.float64); L = np.empty((len(r),), np.float64)
        _check(_load().oracle_forward_neighborhood_f64_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, text_len, R, C,
                                                            kh, kw, sh, sw, scale, _ptr(r), len(r), _ptr(O),
                                                            _ptr(L)), "forward_neighborhood_f64 rows")
        return O, L
    O = np.empty((B, H, N, D), np.float64); L = np.empty((B, H, N), np.float64)
    _check(_load().oracle_forward_neighborhood_f64(_ptr(q), _ptr(k), _ptr(v), B, H, N, D, text_len, R, C, kh, kw,
                                                   sh, sw, scale, _ptr(O), _ptr(L)), "forward_neighborhood_f64")
    return O, L


def backward_neighborhood(q, k, v, dO, text_len: int, grid: Tuple[int, int], window: Tuple[int, int],
                          stride: Tuple[int, int] = (1, 1), scale: Optional[float] = None):
    """(dQ, dK, dV) in fp64 of the neighbourhood forward (natural token order)
    for the output gradient dO (fp64 or bf16-bit inputs)."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    (R, C), (kh, kw), (sh, sw) = grid, window, stride
    dQ = np.empty_like(q); dK = np.empty_like(q); dV = np.empty_like(q)
    _check(_load().oracle_backward_neighborhood_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), B, H, N, D, text_len, R, C,
                                                    kh, kw, sh, sw, scale, _ptr(dQ), _ptr(dK), _ptr(dV)),
           "backward_neighborhood")
    return dQ, dK, dV


def backward_neighborhood_dq_rows(q, k, v, dO, text_len: int, grid: Tuple[int, int], window: Tuple[int, int],
                                  stride: Tuple[int, int], rows, scale: Optional[float] = None):
    """dQ (fp64, [len(rows), D]) of the flat natural-order query rows `rows`
    of the neighbourhood backward."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    B, H, N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    (R, C), (kh, kw), (sh, sw) = grid, window, stride
    r = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(r), D), np.float64)
    _check(_load().oracle_backward_neighborhood_dq_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), B, H, N, D, text_len,
                                                        R, C, kh, kw, sh, sw, scale, _ptr(r), len(r), _ptr(out)),
           "backward_neighborhood_dq_rows")
    return out
