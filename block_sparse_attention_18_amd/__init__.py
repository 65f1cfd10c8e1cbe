"""Block-sparse attention forward for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/bsa.h``.  Every
step of the path runs in the HIP kernels of ``libbsa.so``; this module only
marshals torch tensors (device memory, current stream) into the C calls and
allocates outputs and workspaces when the caller does not pass them.  If the
library is not built, every call raises: there is no fallback.

The four calls mirror the C ABI:

  pool_scores          block score matrix (mean-pool + projection, or the
                       block average of exact softmax attention)
  select_topk          CSR block list: text rows / columns dense, top-k per
                       column group
  build_arrow_layout   CSR block list of the arrow / full / skip layout
  forward              online-softmax attention over the CSR block list,
                       returning O (bf16) and LSE (fp32, natural log)
  backward             dQ, dK, dV of that forward

and the FP8 (E4M3) mode of the forward:

  quantize_fp8         E4M3 codes and scales of Q, K, V
  forward_fp8          the forward on those codes (FP8 matrix cores)

2-D neighbourhood (GNA) attention on the latent grid:

  permute_tokens             natural <-> tile-major token order
  build_neighborhood_layout  block list + full / partial flag per entry
  forward_neighborhood       the forward, masking partial tiles per token

diagnostics of sparse against full attention, and the step schedule of a
mask that is selected once and reused:

  output_rse           per-head relative squared error of an output
  mask_jaccard         per-head Jaccard similarity of two block masks
  ReuseSchedule        full / select / sparse action of each step
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

HEAD_FULL, HEAD_ARROW, HEAD_SKIP = 0, 1, 2
SCORE_MEANPOOL_PROJ, SCORE_EXACT_AVGPOOL = 0, 1

STATUS = {0: "BSA_OK", 1: "BSA_ERR_INVALID_ARG", 2: "BSA_ERR_UNSUPPORTED",
          3: "BSA_ERR_CAPACITY", 4: "BSA_ERR_WORKSPACE", 5: "BSA_ERR_HIP"}


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class BsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("N", ctypes.c_int64), ("D", ctypes.c_int64),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_n", ctypes.c_int64)]


class BsaSplit(ctypes.Structure):
    _fields_ = [("chunk_blocks", ctypes.c_int32), ("max_chunks", ctypes.c_int32),
                ("max_split_rows", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class BsaGroup(ctypes.Structure):
    _fields_ = [("col_begin", ctypes.c_int32), ("col_end", ctypes.c_int32),
                ("k", ctypes.c_int32)]


class BsaFp8Qkv(ctypes.Structure):
    _fields_ = [("q8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("k8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v8t", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("N", ctypes.c_int64), ("D", ctypes.c_int64)]


class BsaNeighborhood(ctypes.Structure):
    _fields_ = [("text_len", ctypes.c_int64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32),
                ("window_rows", ctypes.c_int32), ("window_cols", ctypes.c_int32),
                ("stride_rows", ctypes.c_int32), ("stride_cols", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libbsa.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run `python -m block_sparse_attention_18_amd.build`")
        lib = ctypes.CDLL(p)
        V, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        F = ctypes.c_float
        TP = ctypes.POINTER(BsaTensor)
        GP = ctypes.POINTER(BsaGroup)
        sig = {
            "bsa_pool_scores_workspace_size": (SZ, [I64, I64, I64, I64, I32, I32, I32]),
            "bsa_pool_scores": (I32, [TP, TP, I32, I32, V, I32, F, V, V, SZ, V]),
            "bsa_pool_scores_noalloc": (I32, [TP, TP, I32, I32, V, I32, F, V, V]),
            "bsa_select_meanpool_workspace_size": (SZ, [I64, I64, I64, I32, I32]),
            "bsa_select_meanpool": (I32, [TP, TP, I32, V, I32, I32, GP, I32, V, V, V, I64, V, SZ, V]),
            "bsa_score_grad_workspace_size": (SZ, [I64, I64, I64, I64, I32, I32]),
            "bsa_score_grad": (I32, [TP, TP, I32, V, I32, V, V, V, V, V, SZ, V]),
            "bsa_select_capacity": (I64, [I64, I64, I32, I32, GP, I32]),
            "bsa_select_workspace_size": (SZ, [I64, I64, I32]),
            "bsa_select_topk": (I32, [V, I64, I64, I32, I32, GP, I32, V, V, I64, V, SZ, V]),
            "bsa_arrow_capacity": (I64, [I64, I64, I64, I32, I64, V, V]),
            "bsa_build_arrow_layout": (I32, [I64, I64, I64, I32, I64, V, V, V, V, I64, V]),
            "bsa_forward": (I32, [TP, TP, TP, I32, V, V, V, TP, V, F, TP, V,
                                  ctypes.POINTER(BsaSplit), V]),
            "bsa_forward_split_workspace_size": (SZ, [I64, I64, I64, I64, I32, I32, I64]),
            "bsa_split_policy_arrow": (I32, [I64, I64, I64, I32, I64, V, V, ctypes.POINTER(BsaSplit)]),
            "bsa_split_policy_select": (I32, [I64, I64, I32, I32, GP, I32, I32, ctypes.POINTER(BsaSplit)]),
            "bsa_split_policy_neighborhood": (I32, [I64, I64, I32, ctypes.POINTER(BsaNeighborhood),
                                                    ctypes.POINTER(BsaSplit)]),
            "bsa_quantize_fp8_workspace_size": (SZ, [I64, I64, I64, I64]),
            "bsa_quantize_fp8": (I32, [TP, TP, TP, ctypes.POINTER(BsaFp8Qkv), V, SZ, V]),
            "bsa_forward_fp8": (I32, [ctypes.POINTER(BsaFp8Qkv), I32, V, V, V, TP, V, F, TP, V,
                                      ctypes.POINTER(BsaSplit), V]),
            "bsa_forward_fp8_neighborhood": (I32, [ctypes.POINTER(BsaFp8Qkv), I32, V, V, V,
                                                   ctypes.POINTER(BsaNeighborhood), F, TP, V, V]),
            "bsa_forward_fp8_neighborhood_natural": (I32, [ctypes.POINTER(BsaFp8Qkv), I32, V, V, V,
                                                           ctypes.POINTER(BsaNeighborhood), F, TP, V, V]),
            "bsa_quantize_fp8_neighborhood": (I32, [TP, TP, TP, I32, ctypes.POINTER(BsaNeighborhood),
                                                    ctypes.POINTER(BsaFp8Qkv), V, SZ, V]),
            "bsa_output_rse_workspace_size": (SZ, [I64, I64, I64, I64]),
            "bsa_output_rse": (I32, [TP, TP, V, V, SZ, V]),
            "bsa_mask_jaccard": (I32, [I64, I64, I32, V, V, V, V, V, V]),
            "bsa_permute_tokens": (I32, [TP, TP, V, V, I32, ctypes.POINTER(BsaNeighborhood), I32, V]),
            "bsa_neighborhood_capacity": (I64, [I64, I64, I32, ctypes.POINTER(BsaNeighborhood)]),
            "bsa_build_neighborhood_layout": (I32, [I64, I64, I32, ctypes.POINTER(BsaNeighborhood), V, V, V, I64,
                                                    V]),
            "bsa_forward_neighborhood": (I32, [TP, TP, TP, I32, V, V, V, ctypes.POINTER(BsaNeighborhood), F, TP, V,
                                               ctypes.POINTER(BsaSplit), V]),
            "bsa_forward_neighborhood_natural": (I32, [TP, TP, TP, I32, V, V, V, ctypes.POINTER(BsaNeighborhood), F, TP, V,
                                               ctypes.POINTER(BsaSplit), V]),
            "bsa_backward_workspace_size": (SZ, [I64, I64, I64]),
            "bsa_backward": (I32, [TP, TP, TP, TP, TP, I32, V, V, V, F, TP, TP, TP, V, SZ, V]),
            "bsa_backward_neighborhood": (I32, [TP, TP, TP, TP, TP, I32, V, V, V, ctypes.POINTER(BsaNeighborhood), V, F,
                                                TP, TP, TP, V, SZ, V]),
            "bsa_backward_neighborhood_natural": (I32, [TP, TP, TP, TP, TP, I32, V, V, V,
                                                        ctypes.POINTER(BsaNeighborhood), V, F, TP, TP, TP, V, SZ, V]),
            "bsa_reuse_full_steps": (I32, [I32, ctypes.c_double]),
            "bsa_reuse_step_action": (I32, [I32, ctypes.c_double, I32]),
            "bsa_status_string": (ctypes.c_char_p, [I32]),
            "bsa_last_error": (ctypes.c_char_p, []),
            "bsa_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        msg = load().bsa_last_error().decode(errors="replace")
        raise BsaError(status, msg)


def _desc(t: Optional[torch.Tensor], name: str) -> Optional[BsaTensor]:
    if t is None:
        return None
    if t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{name}: expected a bfloat16 [B, H, N, D] tensor with D contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    B, H, N, D = t.shape
    sb, sh, sn, _ = t.stride()
    return BsaTensor(t.data_ptr(), B, H, N, D, sb, sh, sn)


def _ref(d: Optional[BsaTensor]):
    return None if d is None else ctypes.byref(d)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _groups(groups) -> Tuple[ctypes.Array, int]:
    gl = [tuple(int(v) for v in g) for g in groups]
    arr = (BsaGroup * max(len(gl), 1))(*[BsaGroup(*g) for g in gl])
    return arr, len(gl)


def n_blocks(N: int, block: int) -> int:
    return -(-N // block)


# ---------------------------------------------------------------------------
def pool_scores_workspace_size(B, H, N, D, block, mode=SCORE_MEANPOOL_PROJ, r=32) -> int:
    return int(load().bsa_pool_scores_workspace_size(B, H, N, D, block, mode, r))


def pool_scores(q: torch.Tensor, k: torch.Tensor, block: int, mode: int = SCORE_MEANPOOL_PROJ,
                w: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block scores S [B, H, nB, nB] (fp32).  MEANPOOL_PROJ needs w [D, r]
    (fp32, contiguous); EXACT_AVGPOOL uses `scale` (default 1/sqrt(D))."""
    lib = load()
    B, H, N, D = q.shape
    nB = n_blocks(N, block)
    r = 0
    if mode == SCORE_MEANPOOL_PROJ:
        if w is None or w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
            raise ValueError("w must be a contiguous fp32 [D, r] device tensor")
        r = int(w.shape[1])
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.float32, device=q.device)
    ws_need = pool_scores_workspace_size(B, H, N, D, block, mode, r)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 16), dtype=torch.uint8, device=q.device)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    _check(lib.bsa_pool_scores(ctypes.byref(dq), ctypes.byref(dk), block, mode, _ptr(w), r,
                               float(scale or 0.0), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out


def pool_scores_noalloc(q: torch.Tensor, k: torch.Tensor, block: int, mode: int = SCORE_MEANPOOL_PROJ,
                        w: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """pool_scores through bsa_pool_scores_noalloc: the library's static
    per-device scratch replaces the workspace (for callers that cannot
    allocate; pass `out` to allocate nothing here either)."""
    lib = load()
    B, H, N, D = q.shape
    nB = n_blocks(N, block)
    r = 0
    if mode == SCORE_MEANPOOL_PROJ:
        if w is None or w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
            raise ValueError("w must be a contiguous fp32 [D, r] device tensor")
        r = int(w.shape[1])
    if out is None:
        out = torch.empty((B, H, nB, nB), dtype=torch.float32, device=q.device)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    _check(lib.bsa_pool_scores_noalloc(ctypes.byref(dq), ctypes.byref(dk), block, mode, _ptr(w), r,
                                       float(scale or 0.0), _ptr(out), _stream(q.device)))
    return out


def score_grad_workspace_size(B, H, N, D, block, r) -> int:
    return int(load().bsa_score_grad_workspace_size(B, H, N, D, block, r))


def score_grad(q: torch.Tensor, k: torch.Tensor, block: int, w: torch.Tensor, dscores: torch.Tensor,
               dw: Optional[torch.Tensor] = None, dq_pool: Optional[torch.Tensor] = None,
               dk_pool: Optional[torch.Tensor] = None, pooled: bool = True,
               workspace: Optional[torch.Tensor] = None):
    """Gradient of the MEANPOOL_PROJ score for the upstream gradient dscores
    = dL/dS [B, H, nB, nB] (fp32): returns (dW [D, r], dL/dqbar, dL/dkbar
    [B, H, nB, D]); the pooled gradients are None with pooled=False."""
    lib = load()
    B, H, N, D = q.shape
    nB = n_blocks(N, block)
    if w is None or w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous fp32 [D, r] device tensor")
    r = int(w.shape[1])
    if (dscores.dtype != torch.float32 or not dscores.is_contiguous()
            or tuple(dscores.shape) != (B, H, nB, nB)):
        raise ValueError("dscores must be a contiguous fp32 [B, H, nB, nB] device tensor")
    if dw is None:
        dw = torch.empty((D, r), dtype=torch.float32, device=q.device)
    if pooled:
        if dq_pool is None:
            dq_pool = torch.empty((B, H, nB, D), dtype=torch.float32, device=q.device)
        if dk_pool is None:
            dk_pool = torch.empty((B, H, nB, D), dtype=torch.float32, device=q.device)
    for name, t, shape in (("dw", dw, (D, r)), ("dq_pool", dq_pool, (B, H, nB, D)),
                           ("dk_pool", dk_pool, (B, H, nB, D))):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != shape):
            raise ValueError(f"{name} must be a contiguous fp32 {list(shape)} device tensor")
    if workspace is None:
        workspace = torch.empty(max(score_grad_workspace_size(B, H, N, D, block, r), 16), dtype=torch.uint8,
                                device=q.device)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    _check(lib.bsa_score_grad(ctypes.byref(dq), ctypes.byref(dk), block, _ptr(w), r, _ptr(dscores), _ptr(dw),
                              _ptr(dq_pool), _ptr(dk_pool), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(q.device)))
    return dw, dq_pool, dk_pool


def select_capacity(B, H, nB, text_blocks, groups) -> int:
    arr, ng = _groups(groups)
    return int(load().bsa_select_capacity(B, H, nB, text_blocks, arr, ng))


def select_topk(scores: torch.Tensor, text_blocks: int, groups: Sequence[Tuple[int, int, int]],
                row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """CSR block list from fp32 scores [B, H, nB, nB].  col_idx is sized to the
    capacity bound; the entries in use are col_idx[:row_ptr[-1]]."""
    lib = load()
    if scores.dtype != torch.float32 or not scores.is_contiguous() or scores.dim() != 4:
        raise ValueError("scores must be a contiguous fp32 [B, H, nB, nB] device tensor")
    B, H, nB, _ = scores.shape
    arr, ng = _groups(groups)
    cap = int(lib.bsa_select_capacity(B, H, nB, text_blocks, arr, ng))
    dev = scores.device
    if row_ptr is None:
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        ws = int(lib.bsa_select_workspace_size(B, H, nB))
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev)
    _check(lib.bsa_select_topk(_ptr(scores), B, H, nB, text_blocks, arr, ng, _ptr(row_ptr),
                               _ptr(col_idx), col_idx.numel(), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(dev)))
    return row_ptr, col_idx


MPS_MAX_BLOCKS, MPS_MAX_PROJ = 256, 4096


def select_meanpool_applies(nB: int, r: int, text_blocks: int, groups) -> bool:
    """Whether bsa_select_meanpool takes this shape: nB <= 256, nB * r4 <= 4096
    (r4 = r rounded up to a multiple of 4), the groups with k > 0 pairwise
    disjoint and clear of the text columns."""
    if nB > MPS_MAX_BLOCKS or nB * ((r + 3) // 4 * 4) > MPS_MAX_PROJ or not 1 <= r <= 64:
        return False
    live = sorted((int(g[0]), int(g[1])) for g in groups if int(g[2]) > 0)
    if any(c0 < text_blocks for (c0, _) in live):
        return False
    return all(b0 >= a1 for (_, a1), (b0, _) in zip(live, live[1:]))


def select_meanpool_workspace(B: int, H: int, N: int, block: int, r: int, device) -> torch.Tensor:
    """A workspace for select_meanpool (the projected blocks)."""
    n = int(load().bsa_select_meanpool_workspace_size(B, H, N, block, r))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def select_meanpool(q: torch.Tensor, k: torch.Tensor, block: int, w: torch.Tensor, text_blocks: int,
                    groups: Sequence[Tuple[int, int, int]], scores: Optional[torch.Tensor] = None,
                    row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Mean-pool scores and top-k selection in one call (bsa_select_meanpool):
    returns the CSR (row_ptr, col_idx); the scores go to `scores` when given
    (fp32 [B, H, nB, nB]).  A missing workspace is allocated here."""
    lib = load()
    B, H, N, D = q.shape
    nB = n_blocks(N, block)
    if w is None or w.dtype != torch.float32 or not w.is_contiguous() or w.dim() != 2:
        raise ValueError("w must be a contiguous fp32 [D, r] device tensor")
    r = int(w.shape[1])
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()
                               or tuple(scores.shape) != (B, H, nB, nB)):
        raise ValueError("scores must be a contiguous fp32 [B, H, nB, nB] device tensor")
    arr, ng = _groups(groups)
    cap = int(lib.bsa_select_capacity(B, H, nB, text_blocks, arr, ng))
    dev = q.device
    if row_ptr is None:
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = select_meanpool_workspace(B, H, N, block, r, dev)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    _check(lib.bsa_select_meanpool(ctypes.byref(dq), ctypes.byref(dk), block, _ptr(w), r, text_blocks, arr, ng,
                                   _ptr(scores), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(dev)))
    return row_ptr, col_idx


def _host_i8(x, H) -> ctypes.Array:
    vals = [int(v) for v in x]
    if len(vals) != H:
        raise ValueError("head array length must equal H")
    return (ctypes.c_int8 * H)(*vals)


def _host_i32(x, H) -> ctypes.Array:
    vals = [int(v) for v in x]
    if len(vals) != H:
        raise ValueError("head array length must equal H")
    return (ctypes.c_int32 * H)(*vals)


def arrow_capacity(B, H, N, block, text_len, head_modes, head_windows) -> int:
    m, w = _host_i8(head_modes, H), _host_i32(head_windows, H)
    return int(load().bsa_arrow_capacity(B, H, N, block, text_len, m, w))


def build_arrow_layout(B: int, H: int, N: int, block: int, text_len: int, head_modes,
                       head_windows, device=None,
                       row_ptr: Optional[torch.Tensor] = None,
                       col_idx: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """CSR block list of the arrow layout (exactly sized)."""
    lib = load()
    dev = torch.device(device) if device is not None else torch.device("cuda")
    m, w = _host_i8(head_modes, H), _host_i32(head_windows, H)
    cap = int(lib.bsa_arrow_capacity(B, H, N, block, text_len, m, w))
    if cap < 0:
        _check(lib.bsa_build_arrow_layout(B, H, N, block, text_len, m, w, None, None, 0, None))
    nB = n_blocks(N, block)
    if row_ptr is None:
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check(lib.bsa_build_arrow_layout(B, H, N, block, text_len, m, w, _ptr(row_ptr), _ptr(col_idx),
                                      col_idx.numel(), _stream(dev)))
    return row_ptr, col_idx[:cap] if cap > 0 else col_idx[:0]


def split_workspace_size(B, H, N, D, block, max_chunks, max_split_rows) -> int:
    return int(load().bsa_forward_split_workspace_size(B, H, N, D, block, max_chunks, max_split_rows))


def _split_dict(status: int, sp: "BsaSplit") -> Optional[dict]:
    if status < 0:
        raise ValueError("invalid arguments to the split policy")
    if status == 0:
        return None
    return {"chunk_blocks": int(sp.chunk_blocks), "max_chunks": int(sp.max_chunks),
            "max_split_rows": int(sp.max_split_rows)}


def arrow_split_policy(B: int, H: int, N: int, block: int, text_len: int, head_modes, head_windows):
    """Long-row split for an arrow layout (bsa_split_policy_arrow), or None when
    every row should run whole."""
    sp = BsaSplit()
    st = load().bsa_split_policy_arrow(B, H, N, block, text_len, _host_i8(head_modes, H),
                                       _host_i32(head_windows, H), ctypes.byref(sp))
    return _split_dict(st, sp)


def select_split_policy(B: int, H: int, nB: int, text_blocks: int, groups, block: int = 128):
    """Long-row split for a top-k selection (bsa_split_policy_select), or None."""
    arr, ng = _groups(groups)
    sp = BsaSplit()
    st = load().bsa_split_policy_select(B, H, nB, text_blocks, arr, ng, block, ctypes.byref(sp))
    return _split_dict(st, sp)


def neighborhood_split_policy(B: int, H: int, nb: "BsaNeighborhood", block: int):
    """Long-row split for a neighbourhood layout (bsa_split_policy_neighborhood), or None."""
    sp = BsaSplit()
    st = load().bsa_split_policy_neighborhood(B, H, block, ctypes.byref(nb), ctypes.byref(sp))
    return _split_dict(st, sp)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int,
            row_ptr: torch.Tensor, col_idx: torch.Tensor, head_modes=None,
            o_cache: Optional[torch.Tensor] = None, lse_cache: Optional[torch.Tensor] = None,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, return_lse: bool = True,
            split: Optional[dict] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse attention forward.  Returns (O bf16 [B,H,N,D], LSE fp32 [B,H,N]).

    split: None, or {"chunk_blocks", "max_chunks", "max_split_rows"[, "workspace"]}
    to cut long rows over several workgroups (see arrow_split_policy /
    select_split_policy).  A missing workspace is allocated here.

    The LSE of a SKIP head is copied from lse_cache; without lse_cache the C
    ABI leaves it untouched, so an LSE tensor allocated here holds NaN for
    those heads (a caller-given lse keeps its contents there)."""
    lib = load()
    B, H, N, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    modes = None if head_modes is None else _host_i8(head_modes, H)
    if lse is None and return_lse:
        if modes is not None and lse_cache is None and any(m == HEAD_SKIP for m in modes):
            lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
        else:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if lse_cache is not None and (lse_cache.dtype != torch.float32 or not lse_cache.is_contiguous()):
        raise ValueError("lse_cache must be a contiguous fp32 [B, H, N] tensor")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if col_idx.numel() == 0:
        # a block list with no entries: the kernels never read col_idx, but the
        # C ABI wants a valid pointer
        col_idx = torch.zeros(1, dtype=torch.int32, device=row_ptr.device)
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    dc = _desc(o_cache, "o_cache")
    sp = None
    if split is not None:
        ws = split.get("workspace")
        if ws is None:
            need = split_workspace_size(B, H, N, D, block, split["max_chunks"], split["max_split_rows"])
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            split["workspace"] = ws
        sp = BsaSplit(int(split["chunk_blocks"]), int(split["max_chunks"]), int(split["max_split_rows"]),
                      ws.data_ptr(), ws.numel() * ws.element_size())
    _check(lib.bsa_forward(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), block,
                           _ptr(row_ptr), _ptr(col_idx), modes, _ref(dc), _ptr(lse_cache),
                           float(scale or 0.0), ctypes.byref(do), _ptr(lse),
                           None if sp is None else ctypes.byref(sp), _stream(q.device)))
    return out, lse


class Fp8QKV:
    """E4M3 codes and scales of Q, K, V (the layout of bsa_quantize_fp8):
    q8 / k8 uint8 [B,H,N,D], q_scale fp32 [B,H,N], k_scale fp32 [B,H,ceil(N/64)],
    v8t uint8 [B,H,D,64*ceil(N/64)] (V transposed, keys permuted inside each
    64-key group), v_scale fp32 [B,H,D]."""

    def __init__(self, B: int, H: int, N: int, D: int, device):
        NT = (N + 63) // 64
        u8 = dict(dtype=torch.uint8, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        self.shape = (B, H, N, D)
        self.q8 = torch.empty((B, H, N, D), **u8)
        self.q_scale = torch.empty((B, H, N), **f32)
        self.k8 = torch.empty((B, H, N, D), **u8)
        self.k_scale = torch.empty((B, H, NT), **f32)
        self.v8t = torch.empty((B, H, D, 64 * NT), **u8)
        self.v_scale = torch.empty((B, H, D), **f32)

    def desc(self) -> BsaFp8Qkv:
        arrays = (self.q8, self.q_scale, self.k8, self.k_scale, self.v8t, self.v_scale)
        for a in arrays:
            if not a.is_cuda or not a.is_contiguous():
                raise ValueError("fp8 operands must be contiguous device tensors")
        return BsaFp8Qkv(*[a.data_ptr() for a in arrays], *self.shape)


def v8t_key_column(key: int) -> int:
    """Column of V^T (inside the padded array) that holds key `key`."""
    t, k = divmod(key, 64)
    a, g, h, e = k >> 5, (k >> 3) & 3, (k >> 2) & 1, k & 3
    return 64 * t + 32 * h + 16 * a + 4 * g + e


def quantize_fp8_workspace_size(B, H, N, D) -> int:
    return int(load().bsa_quantize_fp8_workspace_size(B, H, N, D))


def quantize_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[Fp8QKV] = None,
                 workspace: Optional[torch.Tensor] = None, nb: Optional["BsaNeighborhood"] = None) -> Fp8QKV:
    """E4M3 codes with max-abs scales: per token for Q, per 64-key tile for K,
    per channel for V.  With a neighbourhood geometry `nb`, Q, K, V are in
    natural order and the codes come out in its tile-major order
    (bsa_quantize_fp8_neighborhood)."""
    lib = load()
    B, H, N, D = q.shape
    if out is None:
        out = Fp8QKV(B, H, N, D, q.device)
    if workspace is None:
        workspace = torch.empty(max(quantize_fp8_workspace_size(B, H, N, D), 16), dtype=torch.uint8,
                                device=q.device)
    dq, dk, dv = _desc(q, "q"), _desc(k, "k"), _desc(v, "v")
    d8 = out.desc()
    if nb is None:
        _check(lib.bsa_quantize_fp8(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(d8),
                                    _ptr(workspace), workspace.numel(), _stream(q.device)))
    else:
        _check(lib.bsa_quantize_fp8_neighborhood(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                                 nb.tile_rows * nb.tile_cols, ctypes.byref(nb), ctypes.byref(d8),
                                                 _ptr(workspace), workspace.numel(), _stream(q.device)))
    return out


def forward_fp8(qkv: Fp8QKV, block: int, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, return_lse: bool = True, head_modes=None,
                o_cache: Optional[torch.Tensor] = None, lse_cache: Optional[torch.Tensor] = None,
                split: Optional[dict] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Block-sparse attention forward on E4M3 operands.  Returns (O bf16, LSE fp32).
    head_modes / o_cache / lse_cache / split as for forward()."""
    lib = load()
    B, H, N, D = qkv.shape
    dev = qkv.q8.device
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    modes = None if head_modes is None else _host_i8(head_modes, H)
    if lse is None and return_lse:
        if modes is not None and lse_cache is None and any(m == HEAD_SKIP for m in modes):
            lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
        else:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if lse_cache is not None and (lse_cache.dtype != torch.float32 or not lse_cache.is_contiguous()):
        raise ValueError("lse_cache must be a contiguous fp32 [B, H, N] tensor")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if col_idx.numel() == 0:
        col_idx = torch.zeros(1, dtype=torch.int32, device=row_ptr.device)
    d8, do, dc = qkv.desc(), _desc(out, "out"), _desc(o_cache, "o_cache")
    sp = None
    if split is not None:
        ws = split.get("workspace")
        if ws is None:
            need = split_workspace_size(B, H, N, D, block, split["max_chunks"], split["max_split_rows"])
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            split["workspace"] = ws
        sp = BsaSplit(int(split["chunk_blocks"]), int(split["max_chunks"]), int(split["max_split_rows"]),
                      ws.data_ptr(), ws.numel() * ws.element_size())
    _check(lib.bsa_forward_fp8(ctypes.byref(d8), block, _ptr(row_ptr), _ptr(col_idx), modes, _ref(dc),
                               _ptr(lse_cache), float(scale or 0.0), ctypes.byref(do), _ptr(lse),
                               None if sp is None else ctypes.byref(sp), _stream(dev)))
    return out, lse


def forward_fp8_neighborhood(qkv: Fp8QKV, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                             entry_flags: torch.Tensor, nb: "BsaNeighborhood", scale: Optional[float] = None,
                             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                             return_lse: bool = True, natural: bool = False
                             ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """FP8 forward of 2-D neighbourhood attention on E4M3 operands in
    tile-major order.  Returns (O bf16, LSE fp32), in tile-major order, or in
    natural order with natural=True (bsa_forward_fp8_neighborhood_natural)."""
    lib = load()
    B, H, N, D = qkv.shape
    dev = qkv.q8.device
    block = nb.tile_rows * nb.tile_cols
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx), ("entry_flags", entry_flags)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    d8, do = qkv.desc(), _desc(out, "out")
    fn = lib.bsa_forward_fp8_neighborhood_natural if natural else lib.bsa_forward_fp8_neighborhood
    _check(fn(ctypes.byref(d8), block, _ptr(row_ptr), _ptr(col_idx), _ptr(entry_flags), ctypes.byref(nb),
              float(scale or 0.0), ctypes.byref(do), _ptr(lse), _stream(dev)))
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dO: torch.Tensor, block: int,
             row_ptr: torch.Tensor, col_idx: torch.Tensor, lse: torch.Tensor, scale: Optional[float] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """(dQ, dK, dV) bf16 of the block-sparse forward, given its output O and
    LSE and the output gradient dO."""
    lib = load()
    B, H, N, D = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if col_idx.numel() == 0:
        col_idx = torch.zeros(1, dtype=torch.int32, device=row_ptr.device)
    if workspace is None:
        workspace = torch.empty(max(int(lib.bsa_backward_workspace_size(B, H, N)), 16), dtype=torch.uint8,
                                device=q.device)
    ds = [_desc(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"), (dq, "dq"), (dk, "dk"),
                                   (dv, "dv"))]
    _check(lib.bsa_backward(*[ctypes.byref(d) for d in ds[:5]], block, _ptr(row_ptr), _ptr(col_idx), _ptr(lse),
                            float(scale or 0.0), *[ctypes.byref(d) for d in ds[5:]], _ptr(workspace),
                            workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def neighborhood(text_len: int, grid: Tuple[int, int], tile: Tuple[int, int], window: Tuple[int, int],
                 stride: Tuple[int, int] = (1, 1)) -> BsaNeighborhood:
    """Geometry of 2-D neighbourhood attention: text_len text tokens, then a
    grid = (rows, cols) image in row-major order, cut into tile = (tile_rows,
    tile_cols) tiles of one block each; window and stride per axis."""
    return BsaNeighborhood(int(text_len), int(grid[0]), int(grid[1]), int(tile[0]), int(tile[1]),
                           int(window[0]), int(window[1]), int(stride[0]), int(stride[1]))


def permute_tokens(x: torch.Tensor, nb: BsaNeighborhood, inverse: bool = False,
                   lse: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   lse_out: Optional[torch.Tensor] = None):
    """Natural -> tile-major token order (inverse: back).  Returns out, or
    (out, lse_out) when lse is given."""
    lib = load()
    if out is None:
        out = torch.empty_like(x)
    if lse is not None and lse_out is None:
        lse_out = torch.empty_like(lse)
    for name, t in (("lse", lse), ("lse_out", lse_out)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 [B, H, N] tensor")
    block = nb.tile_rows * nb.tile_cols
    di, do = _desc(x, "in"), _desc(out, "out")
    _check(lib.bsa_permute_tokens(ctypes.byref(di), ctypes.byref(do), _ptr(lse), _ptr(lse_out), block,
                                  ctypes.byref(nb), 1 if inverse else 0, _stream(x.device)))
    return out if lse is None else (out, lse_out)


def neighborhood_capacity(B: int, H: int, nb: BsaNeighborhood) -> int:
    return int(load().bsa_neighborhood_capacity(B, H, nb.tile_rows * nb.tile_cols, ctypes.byref(nb)))


def build_neighborhood_layout(B: int, H: int, nb: BsaNeighborhood, device=None,
                              row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None,
                              flags: Optional[torch.Tensor] = None):
    """(row_ptr, col_idx, entry_flags) int32 device tensors of the tile-major
    block list; flag 1 marks a partially covered key tile."""
    lib = load()
    dev = device or (row_ptr.device if row_ptr is not None else torch.device("cuda"))
    cap = neighborhood_capacity(B, H, nb)
    block = nb.tile_rows * nb.tile_cols
    if cap < 0:
        _check(lib.bsa_build_neighborhood_layout(B, H, block, ctypes.byref(nb), None, None, None, 0, None))
    nB = (nb.text_len + nb.rows * nb.cols) // block
    if row_ptr is None:
        row_ptr = torch.empty(B * H * nB + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if flags is None:
        flags = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if min(col_idx.numel(), flags.numel()) < cap or row_ptr.numel() < B * H * nB + 1:
        raise ValueError("layout buffers too small")
    _check(lib.bsa_build_neighborhood_layout(B, H, block, ctypes.byref(nb), _ptr(row_ptr), _ptr(col_idx),
                                             _ptr(flags), min(col_idx.numel(), flags.numel()), _stream(dev)))
    return row_ptr, col_idx, flags


def forward_neighborhood(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: torch.Tensor,
                         col_idx: torch.Tensor, entry_flags: torch.Tensor, nb: BsaNeighborhood,
                         scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                         split: Optional[dict] = None, natural: bool = False):
    """Block-sparse forward on tile-major Q, K, V, masking the partially
    covered key tiles per token.  Returns (O, LSE) in tile-major order; with
    natural=True, Q, K, V and the returned O, LSE are in natural order (the
    kernel gathers the tiles itself)."""
    lib = load()
    B, H, N, D = q.shape
    block = nb.tile_rows * nb.tile_cols
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx), ("entry_flags", entry_flags)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    sp = None
    if split is not None:
        ws = split.get("workspace")
        if ws is None:
            need = split_workspace_size(B, H, N, D, block, split["max_chunks"], split["max_split_rows"])
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
            split["workspace"] = ws
        sp = BsaSplit(int(split["chunk_blocks"]), int(split["max_chunks"]), int(split["max_split_rows"]),
                      ws.data_ptr(), ws.numel() * ws.element_size())
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    fn = lib.bsa_forward_neighborhood_natural if natural else lib.bsa_forward_neighborhood
    _check(fn(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), block, _ptr(row_ptr),
                                        _ptr(col_idx), _ptr(entry_flags), ctypes.byref(nb), float(scale or 0.0),
                                        ctypes.byref(do), _ptr(lse), None if sp is None else ctypes.byref(sp),
                                        _stream(q.device)))
    return out, lse


def backward_neighborhood(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dO: torch.Tensor,
                          row_ptr: torch.Tensor, col_idx: torch.Tensor, entry_flags: torch.Tensor,
                          nb: BsaNeighborhood, lse: torch.Tensor, scale: Optional[float] = None,
                          dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                          dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          natural: bool = False):
    """(dQ, dK, dV) bf16 in tile-major order of forward_neighborhood, given its
    tile-major output O and LSE and the tile-major output gradient dO; with
    natural=True every tensor is in natural token order
    (bsa_backward_neighborhood_natural)."""
    lib = load()
    B, H, N, D = q.shape
    block = nb.tile_rows * nb.tile_cols
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx), ("entry_flags", entry_flags)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if workspace is None:
        workspace = torch.empty(max(int(lib.bsa_backward_workspace_size(B, H, N)), 16), dtype=torch.uint8,
                                device=q.device)
    ds = [_desc(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dO, "dO"), (dq, "dq"), (dk, "dk"),
                                   (dv, "dv"))]
    fn = lib.bsa_backward_neighborhood_natural if natural else lib.bsa_backward_neighborhood
    _check(fn(*[ctypes.byref(d) for d in ds[:5]], block, _ptr(row_ptr), _ptr(col_idx), _ptr(entry_flags),
              ctypes.byref(nb), _ptr(lse), float(scale or 0.0), *[ctypes.byref(d) for d in ds[5:]],
              _ptr(workspace), workspace.numel(), _stream(q.device)))
    return dq, dk, dv


def output_rse(test: torch.Tensor, ref: torch.Tensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head sum (test - ref)^2 / sum (ref - mean ref)^2 over each head's
    N x D elements; fp64 [B, H] on the device."""
    lib = load()
    B, H, N, D = ref.shape
    if out is None:
        out = torch.empty((B, H), dtype=torch.float64, device=ref.device)
    if out.dtype != torch.float64 or not out.is_contiguous() or out.numel() < B * H:
        raise ValueError("out must be a contiguous fp64 tensor of B*H elements")
    if workspace is None:
        need = int(lib.bsa_output_rse_workspace_size(B, H, N, D))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=ref.device)
    dt, dr = _desc(test, "test"), _desc(ref, "ref")
    _check(lib.bsa_output_rse(ctypes.byref(dt), ctypes.byref(dr), _ptr(out), _ptr(workspace),
                              workspace.numel(), _stream(ref.device)))
    return out


def mask_jaccard(B: int, H: int, n_blocks: int, row_ptr_a: torch.Tensor, col_idx_a: torch.Tensor,
                 row_ptr_b: torch.Tensor, col_idx_b: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head Jaccard similarity of two CSR block masks; fp64 [B, H]."""
    lib = load()
    dev = row_ptr_a.device
    if out is None:
        out = torch.empty((B, H), dtype=torch.float64, device=dev)
    if out.dtype != torch.float64 or not out.is_contiguous() or out.numel() < B * H:
        raise ValueError("out must be a contiguous fp64 tensor of B*H elements")
    arrs = []
    for name, t in (("row_ptr_a", row_ptr_a), ("col_idx_a", col_idx_a), ("row_ptr_b", row_ptr_b),
                    ("col_idx_b", col_idx_b)):
        if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
        arrs.append(t if t.numel() else torch.zeros(1, dtype=torch.int32, device=dev))
    _check(lib.bsa_mask_jaccard(B, H, n_blocks, *[_ptr(a) for a in arrs], _ptr(out), _stream(dev)))
    return out


class ReuseSchedule:
    """Which attention each of T denoising steps runs when a block mask is
    selected once and reused (SparseD, "skipping sparse" and "sparse
    reuse"): steps 0 .. n_full-1 run full attention, n_full = floor(T *
    skip); step n_full selects the mask (exact avgpool scores and isolated
    top-k) and runs sparse attention with it; every later step reuses it.
    The schedule comes from bsa_reuse_full_steps / bsa_reuse_step_action."""

    FULL, SELECT, SPARSE = "full", "select", "sparse"
    _ACTIONS = (FULL, SELECT, SPARSE)

    def __init__(self, steps: int, skip: float = 0.2):
        if not (1 <= steps < 2 ** 31) or not (0.0 <= skip <= 1.0):
            raise ValueError("1 <= steps < 2^31 and 0 <= skip <= 1 required")
        self.steps = int(steps)
        self.skip = float(skip)
        self.n_full = int(load().bsa_reuse_full_steps(self.steps, self.skip))
        if self.n_full < 0:
            raise ValueError("bsa_reuse_full_steps rejected the schedule")

    def action(self, step: int) -> str:
        if not 0 <= step < self.steps:
            raise IndexError(step)
        a = load().bsa_reuse_step_action(self.steps, self.skip, int(step))
        if a < 0:
            raise ValueError("bsa_reuse_step_action rejected the step")
        return self._ACTIONS[a]

    def counts(self) -> dict:
        n_sel = 1 if self.n_full < self.steps else 0
        return {self.FULL: self.n_full, self.SELECT: n_sel,
                self.SPARSE: self.steps - self.n_full - n_sel}

    def amortised_speedup(self, t_full: float, t_select: float, t_sparse: float) -> float:
        """Time of T full steps over the time of this schedule, given the time
        of a full step, of the selection (scores + top-k) and of a sparse step."""
        c = self.counts()
        t = c[self.FULL] * t_full + c[self.SELECT] * (t_select + t_sparse) + c[self.SPARSE] * t_sparse
        return self.steps * t_full / t


def version() -> str:
    return load().bsa_version().decode()
