"""C ABI checks that need no GPU: the library loads, exports every function
include/bsa.h declares, and rejects bad arguments before enqueuing anything.

Device pointers passed here are fake (never dereferenced): every call below
must fail in host-side validation, which runs before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_18_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bsa.LIB_PATH),
                                reason="libbsa.so not built (run __graft_entry__.build())")

FAKE = 0x7F0000000000      # 16-byte aligned, never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_are_exported():
    lib = ctypes.CDLL(bsa.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 11
    for n in ["bsa_pool_scores", "bsa_select_topk", "bsa_build_arrow_layout", "bsa_forward"]:
        assert n in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in bsa.h but not exported"


def test_status_strings_and_version():
    lib = bsa.load()
    for code, name in bsa.STATUS.items():
        assert lib.bsa_status_string(code).decode() == name
    assert lib.bsa_status_string(99).decode() == "BSA_ERR_UNKNOWN"
    assert "gfx950" in bsa.version()


def _t(B=1, H=2, N=256, D=64, data=FAKE, sb=None, sh=None, sn=None):
    sn = D if sn is None else sn
    sh = N * sn if sh is None else sh
    sb = H * sh if sb is None else sb
    return bsa.BsaTensor(data, B, H, N, D, sb, sh, sn)


def _fwd(q=None, k=None, v=None, o=None, block=64, rp=FAKE, ci=FAKE, modes=None, oc=None,
         scale=0.0, split=None):
    lib = bsa.load()
    q = q or _t()
    k = k or _t()
    v = v or _t()
    o = o or _t()
    ref = lambda d: None if d is None else ctypes.byref(d)
    return lib.bsa_forward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), block,
                           ctypes.c_void_p(rp) if rp else None, ctypes.c_void_p(ci) if ci else None,
                           modes, ref(oc), None, scale, ctypes.byref(o), None,
                           None if split is None else ctypes.byref(split), None)


def _err():
    return bsa.load().bsa_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=_t(data=0)), 1, "null data"),
    (dict(q=_t(D=96)), 2, "head dim"),
    (dict(k=_t(N=128)), 1, "shapes differ"),
    (dict(q=_t(data=FAKE + 8)), 1, "aligned"),
    (dict(v=_t(sn=60)), 1, "strides"),
    (dict(o=_t(sh=-64)), 1, "strides"),
    (dict(block=32), 2, "block size"),
    # one head's rows span 4 GiB: beyond the kernels' 32-bit buffer range
    (dict(q=_t(N=1 << 24, D=128)), 2, "4 GiB"),
    (dict(k=_t(N=(1 << 19) + 8, D=128, sn=128 * 32)), 2, "4 GiB"),
    (dict(rp=0), 1, "row_ptr"),
    (dict(scale=float("nan")), 1, "NaN"),
])
def test_forward_validation(kw, code, msg):
    assert _fwd(**kw) == code
    assert msg in _err()


def test_forward_skip_requires_cache_and_known_modes():
    modes = (ctypes.c_int8 * 2)(bsa.HEAD_FULL, bsa.HEAD_SKIP)
    assert _fwd(modes=modes) == 1 and "o_cache" in _err()
    assert _fwd(modes=modes, oc=_t(N=128)) == 1 and "o_cache" in _err()
    bad = (ctypes.c_int8 * 2)(0, 7)
    assert _fwd(modes=bad) == 1 and "unknown mode" in _err()


def test_forward_split_validation_and_workspace_size():
    lib = bsa.load()
    # 1 x 2 heads x 4 query blocks = 8 rows; 3 split rows of 4 chunks
    need = lib.bsa_forward_split_workspace_size(1, 2, 256, 64, 64, 4, 3)
    items = 8 + 3 * 3
    slot_floats = 64 * 64 + 2 * 64
    up = lambda x: (x + 255) // 256 * 256
    assert need == 256 + up(items * 16) + up(3 * 8) + 3 * 4 * slot_floats * 4
    # the split-row pool is capped at the number of rows
    assert lib.bsa_forward_split_workspace_size(1, 2, 256, 64, 64, 4, 100) == \
        lib.bsa_forward_split_workspace_size(1, 2, 256, 64, 64, 4, 8)
    assert lib.bsa_forward_split_workspace_size(1, 2, 256, 64, 64, 1, 3) == 0
    mk = lambda cb=8, mc=4, msr=3, ws=FAKE, wsb=1 << 30: bsa.BsaSplit(cb, mc, msr, ws, wsb)
    assert _fwd(split=mk(cb=0)) == 1 and "split" in _err()
    assert _fwd(split=mk(mc=1)) == 1
    assert _fwd(split=mk(mc=65)) == 1
    assert _fwd(split=mk(msr=0)) == 1
    assert _fwd(split=mk(wsb=need - 1)) == 4 and "split workspace" in _err()
    assert _fwd(split=mk(ws=0)) == 4
    assert _fwd(split=mk(ws=FAKE + 4)) == 4


def test_split_policies():
    # 2K MMDiT arrow, w = 8: text rows (132 blocks) are shorter than the average
    # work per workgroup slot, so splitting does not pay
    modes = [bsa.HEAD_ARROW] * 24
    assert bsa.arrow_split_policy(1, 24, 16896, 128, 512, modes, [8] * 24) is None
    # w = 0: the text rows dominate; they are cut into 4 chunks of <= 33 blocks
    plan = bsa.arrow_split_policy(1, 24, 16896, 128, 512, modes, [0] * 24)
    assert plan == {"chunk_blocks": 33, "max_chunks": 4, "max_split_rows": 96}
    # FLUX 1024^2 mix (12 arrow w=1 / 8 full / 4 skip): the full heads' and the
    # text rows (36 blocks) against 7-block arrow rows leave a tail; they are
    # cut into 4 chunks of <= 9 blocks
    modes2 = [1] * 12 + [0] * 8 + [2] * 4
    plan2 = bsa.arrow_split_policy(1, 24, 4608, 128, 512, modes2, [1] * 24)
    assert plan2 == {"chunk_blocks": 9, "max_chunks": 4, "max_split_rows": 8 * 36 + 12 * 4}
    # the content-driven DiT (block 64): the plan and combine cost more than
    # the tail of its text rows
    assert bsa.select_split_policy(2, 16, 68, 4, ((4, 68, 16),), block=64) is None
    # with a single long head among many windowed ones the split pays
    modes3 = [0] + [1] * 63
    plan3 = bsa.arrow_split_policy(1, 64, 4608, 128, 512, modes3, [0] * 64)
    assert plan3 is not None and plan3["max_split_rows"] == 36 + 63 * 4
    # uniform rows: nothing to split
    assert bsa.select_split_policy(1, 32, 512, 0, ((0, 480, 144), (480, 512, 10))) is None
    # invalid arguments raise
    with pytest.raises(ValueError):
        bsa.arrow_split_policy(1, 2, 512, 96, 0, [1, 1], [1, 1])


def test_pool_scores_validation():
    lib = bsa.load()
    q, k = _t(), _t()
    call = lambda mode=0, w=FAKE, r=32, ws=FAKE, wsb=1 << 20, block=64, scores=FAKE: lib.bsa_pool_scores(
        ctypes.byref(q), ctypes.byref(k), block, mode, ctypes.c_void_p(w) if w else None, r, 0.0,
        ctypes.c_void_p(scores) if scores else None, ctypes.c_void_p(ws) if ws else None, wsb, None)
    assert call(mode=5) == 2
    assert call(w=0) == 1 and "projection" in _err()
    assert call(r=0) == 1 and call(r=65) == 1
    assert call(wsb=16) == 4 and "workspace" in _err()
    assert call(ws=0) == 4
    assert call(block=96) == 2
    assert call(scores=0) == 1
    # exact mode needs at least one scratch slot: nB * block floats
    assert call(mode=1, wsb=4 * 64 * 4 - 4) == 4
    need = lib.bsa_pool_scores_workspace_size(1, 2, 256, 64, 64, 0, 32)
    assert need == 2 * 1 * 2 * 4 * 32 * 4
    need_exact = lib.bsa_pool_scores_workspace_size(1, 2, 256, 64, 64, 1, 0)
    assert need_exact == (1 * 2 * 4) * 4 * 64 * 4


def test_score_grad_validation_and_workspace():
    lib = bsa.load()
    q, k = _t(), _t()
    P = lambda x: ctypes.c_void_p(x) if x else None
    call = lambda w=FAKE, r=32, ds=FAKE, dw=FAKE, ws=FAKE, wsb=1 << 20, block=64, kk=k: lib.bsa_score_grad(
        ctypes.byref(q), ctypes.byref(kk), block, P(w), r, P(ds), P(dw), None, None, P(ws), wsb, None)
    assert call(w=0) == 1 and call(ds=0) == 1 and call(dw=0) == 1
    assert call(r=0) == 1 and call(r=65) == 1
    assert call(block=96) == 2
    assert call(wsb=64) == 4 and "workspace" in _err()
    assert call(ws=0) == 4 and call(ws=FAKE + 8) == 4
    k2 = _t(N=128)
    assert call(kk=k2) == 1 and "shapes differ" in _err()
    # proj, means, g (per block and side) and a partial dW per chunk of 16
    # blocks of a head, each 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256
    rows = 1 * 2 * 4
    assert lib.bsa_score_grad_workspace_size(1, 2, 256, 64, 64, 32) == \
        up(2 * rows * 32 * 4) + up(2 * rows * 64 * 4) + up(2 * rows * 32 * 4) + up(2 * 1 * 64 * 32 * 4)
    rows = 1 * 2 * 17                               # 17 blocks: two chunks per head
    assert lib.bsa_score_grad_workspace_size(1, 2, 17 * 64, 128, 64, 8) == \
        up(2 * rows * 8 * 4) + up(2 * rows * 128 * 4) + up(2 * rows * 8 * 4) + up(2 * 2 * 128 * 8 * 4)
    assert lib.bsa_score_grad_workspace_size(1, 2, 256, 64, 64, 0) == 0
    assert lib.bsa_score_grad_workspace_size(1, 2, 256, 64, 96, 32) == 0


def test_select_validation_and_capacity():
    lib = bsa.load()
    G = bsa.BsaGroup
    g = (G * 2)(G(0, 480, 144), G(480, 512, 10))
    cap = lib.bsa_select_capacity(1, 32, 512, 0, g, 2)
    assert cap == 32 * 512 * 154
    g1 = (G * 1)(G(0, 8, 4))
    # text rows dense, other rows at most text + k
    assert lib.bsa_select_capacity(1, 2, 8, 1, g1, 1) == 2 * (8 + 7 * 5)
    assert lib.bsa_select_workspace_size(1, 2, 40) == 2 * 40 * 2 * 4
    call = lambda nb=8, tb=1, grp=g1, ng=1, cap=10 ** 6, ws=FAKE, wsb=1 << 20: lib.bsa_select_topk(
        ctypes.c_void_p(FAKE), 1, 2, nb, tb, grp, ng, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        cap, ctypes.c_void_p(ws) if ws else None, wsb, None)
    assert call(nb=2000) == 2
    assert call(tb=9) == 1
    assert call(grp=(G * 1)(G(0, 9, 4))) == 1 and "group" in _err()
    assert call(grp=(G * 1)(G(2, 6, 5))) == 1
    assert call(grp=(G * 1)(G(5, 5, 0))) == 1
    assert call(cap=2 * (8 + 7 * 5) - 1) == 3 and "capacity" in _err()
    assert call(wsb=8) == 4
    assert call(ng=9) == 2


def _arrow_count(nB, tb, w):
    n = nB - tb
    if w >= n - 1:
        return nB * nB
    return tb * nB + n * tb + n * (2 * w + 1) - w * (w + 1)


def test_arrow_validation_and_capacity():
    lib = bsa.load()
    H = 3
    modes = (ctypes.c_int8 * H)(bsa.HEAD_ARROW, bsa.HEAD_FULL, bsa.HEAD_SKIP)
    wins = (ctypes.c_int32 * H)(8, 0, 0)
    cap = lib.bsa_arrow_capacity(2, H, 16896, 128, 512, modes, wins)
    assert cap == 2 * (_arrow_count(132, 4, 8) + 132 * 132)
    # ragged text: 300 text tokens with block 128 -> 3 text blocks
    cap2 = lib.bsa_arrow_capacity(1, 1, 4396, 128, 300, (ctypes.c_int8 * 1)(1), (ctypes.c_int32 * 1)(2))
    assert cap2 == _arrow_count(35, 3, 2)
    call = lambda B=1, N=1024, block=128, tl=0, m=modes, w=wins, cap=10 ** 7, rp=FAKE: \
        lib.bsa_build_arrow_layout(B, H, N, block, tl, m, w, ctypes.c_void_p(rp) if rp else None,
                                   ctypes.c_void_p(FAKE), cap, None)
    assert call(block=32) == 2
    assert call(tl=2000) == 1
    assert call(m=(ctypes.c_int8 * H)(1, 4, 0)) == 1
    assert call(w=(ctypes.c_int32 * H)(-1, 0, 0)) == 1
    assert call(cap=5) == 3
    assert call(rp=0) == 1
    assert call(B=0) == 1
    many = (ctypes.c_int8 * 300)(*([0] * 300))
    wm = (ctypes.c_int32 * 300)(*([0] * 300))
    assert lib.bsa_build_arrow_layout(1, 300, 1024, 128, 0, many, wm, ctypes.c_void_p(FAKE),
                                      ctypes.c_void_p(FAKE), 10 ** 7, None) == 2


def _fp8(B=1, H=2, N=256, D=64, base=FAKE):
    return bsa.BsaFp8Qkv(base, base + 0x100000, base + 0x200000, base + 0x300000, base + 0x400000,
                         base + 0x500000, B, H, N, D)


def test_fp8_workspace_and_quantize_validation():
    lib = bsa.load()
    up = lambda x: (x + 255) // 256 * 256
    # reciprocal channel scales, then channel maxima of 256-key chunks
    assert lib.bsa_quantize_fp8_workspace_size(1, 2, 600, 64) == up(2 * 64 * 4) + 2 * 3 * 64 * 4
    assert lib.bsa_quantize_fp8_workspace_size(1, 2, 600, 96) == 0
    need = lib.bsa_quantize_fp8_workspace_size(1, 2, 256, 64)
    call = lambda out=None, ws=FAKE, wsb=need, q=None: lib.bsa_quantize_fp8(
        ctypes.byref(q or _t()), ctypes.byref(_t()), ctypes.byref(_t()),
        None if out is False else ctypes.byref(out or _fp8()),
        ctypes.c_void_p(ws) if ws else None, wsb, None)
    assert call(out=False) == 1 and "null descriptor" in _err()
    assert call(out=_fp8(N=128)) == 1 and "shape" in _err()
    assert call(out=_fp8(base=FAKE + 4)) == 1 and "aligned" in _err()
    assert call(wsb=need - 1) == 4 and "workspace" in _err()
    assert call(ws=0) == 4
    assert call(q=_t(D=128)) == 1
    bad = _fp8()
    bad.k_scale = None
    assert call(out=bad) == 1 and "null array" in _err()


def test_fp8_forward_validation():
    lib = bsa.load()
    call = lambda inp=None, block=64, rp=FAKE, ci=FAKE, scale=0.0, o=None, modes=None, oc=None, split=None: \
        lib.bsa_forward_fp8(ctypes.byref(inp or _fp8()), block, ctypes.c_void_p(rp) if rp else None,
                            ctypes.c_void_p(ci) if ci else None, modes, None if oc is None else ctypes.byref(oc),
                            None, scale, ctypes.byref(o or _t()), None,
                            None if split is None else ctypes.byref(split), None)
    assert call(block=32) == 2 and "block size" in _err()
    assert call(inp=_fp8(D=96), o=_t(D=96)) == 2
    assert call(o=_t(N=128)) == 1 and "shape" in _err()
    assert call(rp=0) == 1 and "row_ptr" in _err()
    assert call(scale=float("nan")) == 1 and "NaN" in _err()
    assert call(inp=_fp8(N=(1 << 24) + 1), o=_t(N=(1 << 24) + 1)) == 2 and "2^24" in _err()
    skip = (ctypes.c_int8 * 2)(bsa.HEAD_FULL, bsa.HEAD_SKIP)
    assert call(modes=skip) == 1 and "o_cache" in _err()             # a SKIP head needs the cache
    bad = (ctypes.c_int8 * 2)(bsa.HEAD_FULL, 7)
    assert call(modes=bad, oc=_t()) == 1 and "mode" in _err()
    assert call(split=bsa.BsaSplit(0, 4, 8, FAKE, 1 << 30)) == 1 and "split" in _err()
    assert call(split=bsa.BsaSplit(2, 4, 8, FAKE, 16)) == 4 and "workspace" in _err()


def test_diagnostics_validation_and_workspace():
    lib = bsa.load()
    # per-chunk partial sums: 3 doubles per chunk, ~64 K elements per chunk
    assert lib.bsa_output_rse_workspace_size(1, 2, 4096, 128) == 2 * 8 * 3 * 8
    assert lib.bsa_output_rse_workspace_size(1, 2, 10, 64) == 2 * 1 * 3 * 8
    assert lib.bsa_output_rse_workspace_size(1, 2, 10, 96) == 0
    need = lib.bsa_output_rse_workspace_size(1, 2, 256, 64)
    call = lambda t=None, r=None, out=FAKE, ws=FAKE, wsb=need: lib.bsa_output_rse(
        ctypes.byref(t or _t()), ctypes.byref(r or _t()), ctypes.c_void_p(out) if out else None,
        ctypes.c_void_p(ws) if ws else None, wsb, None)
    assert call(r=_t(N=128)) == 1 and "shapes differ" in _err()
    assert call(out=0) == 1
    assert call(wsb=need - 1) == 4 and "workspace" in _err()
    assert call(t=_t(D=96)) == 2
    jac = lambda B=1, H=2, nb=8, rp=FAKE, out=FAKE: lib.bsa_mask_jaccard(
        B, H, nb, ctypes.c_void_p(rp) if rp else None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(out) if out else None, None)
    assert jac(nb=0) == 1
    assert jac(rp=0) == 1 and "null" in _err()
    assert jac(out=0) == 1
    assert jac(nb=70000) == 2


@pytest.mark.parametrize("T,grid,tile,window,stride", [
    (512, (128, 128), (8, 16), (32, 32), (1, 1)),
    (128, (32, 64), (8, 16), (9, 17), (3, 4)),
    (0, (16, 32), (4, 16), (16, 32), (16, 32)),
    (64, (24, 40), (8, 8), (8, 16), (8, 16)),
])
def test_neighborhood_capacity_matches_oracle_layout(T, grid, tile, window, stride):
    """The host's closed-form entry count of the neighbourhood layout equals the
    nnz of the oracle's brute-force layout."""
    import oracle
    lib = bsa.load()
    nb = bsa.neighborhood(T, grid, tile, window, stride)
    rp, ci, fl = oracle.neighborhood_layout(T, grid, tile, window, stride)
    block = tile[0] * tile[1]
    assert lib.bsa_neighborhood_capacity(2, 3, block, ctypes.byref(nb)) == 6 * int(rp[-1])


def test_neighborhood_validation():
    lib = bsa.load()
    cap = lambda **kw: lib.bsa_neighborhood_capacity(1, 1, 128, ctypes.byref(bsa.neighborhood(
        kw.get("T", 512), kw.get("grid", (128, 128)), kw.get("tile", (8, 16)), kw.get("window", (32, 32)),
        kw.get("stride", (1, 1)))))
    assert cap() > 0
    assert cap(tile=(8, 8)) == -1            # 64 tokens: not the block
    assert cap(tile=(16, 8), grid=(128, 120)) > 0   # any grid of whole tiles
    assert cap(tile=(4, 32), grid=(128, 112)) == -1   # grid not a whole number of tiles
    assert cap(T=500) == -1                  # text not a whole number of blocks
    assert cap(window=(0, 32)) == -1 and cap(window=(129, 32)) == -1
    assert cap(stride=(0, 1)) == -1
    nb = bsa.neighborhood(512, (128, 128), (8, 16), (32, 32))
    t = lambda N=16896: _t(B=1, H=2, N=N, D=128, data=FAKE)
    fwd = lambda N=16896, fl=FAKE: lib.bsa_forward_neighborhood(
        ctypes.byref(t(N)), ctypes.byref(t(N)), ctypes.byref(t(N)), 128, ctypes.c_void_p(FAKE),
        ctypes.c_void_p(FAKE), ctypes.c_void_p(fl) if fl else None, ctypes.byref(nb), 0.0, ctypes.byref(t(N)),
        None, None, None)
    assert fwd(N=16895) == 1 and "N" in _err()
    assert fwd(fl=0) == 1 and "entry_flags" in _err()
    perm = lambda inp, outp, inv=0: lib.bsa_permute_tokens(ctypes.byref(inp), ctypes.byref(outp), None, None, 128,
                                                            ctypes.byref(nb), inv, None)
    assert perm(t(), t()) == 1 and "in place" in _err()
    lay = lambda capacity: lib.bsa_build_neighborhood_layout(1, 2, 128, ctypes.byref(nb), ctypes.c_void_p(FAKE),
                                                             ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                                             capacity, None)
    need = lib.bsa_neighborhood_capacity(1, 2, 128, ctypes.byref(nb))
    assert lay(need - 1) == 3
    # FP8 with natural-order inputs and outputs: the geometry is checked
    # against the tensors before anything else runs
    ws = lib.bsa_quantize_fp8_workspace_size(1, 2, 16896, 128)
    quant = lambda N=16896, block=128: lib.bsa_quantize_fp8_neighborhood(
        ctypes.byref(t(N)), ctypes.byref(t(N)), ctypes.byref(t(N)), block, ctypes.byref(nb),
        ctypes.byref(_fp8(B=1, H=2, N=N, D=128)), ctypes.c_void_p(FAKE), ws, None)
    assert quant(N=16895) == 1 and "N" in _err()
    assert quant(block=64) == 1 and "tile_rows" in _err()
    fwd8 = lambda N=16896, fl=FAKE: lib.bsa_forward_fp8_neighborhood_natural(
        ctypes.byref(_fp8(B=1, H=2, N=N, D=128)), 128, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        ctypes.c_void_p(fl) if fl else None, ctypes.byref(nb), 0.0, ctypes.byref(t(N)), None, None)
    assert fwd8(N=16895) == 1 and "N" in _err()
    assert fwd8(fl=0) == 1 and "entry_flags" in _err()
    bwd = lambda N=16896, fl=FAKE: lib.bsa_backward_neighborhood_natural(
        *[ctypes.byref(t(N)) for _ in range(5)], 128, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        ctypes.c_void_p(fl) if fl else None, ctypes.byref(nb), ctypes.c_void_p(FAKE), 0.0,
        *[ctypes.byref(t(N)) for _ in range(3)], ctypes.c_void_p(FAKE), 1 << 30, None)
    assert bwd(N=16895) == 1 and "N" in _err()
    assert bwd(fl=0) == 1 and "entry_flags" in _err()


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa._desc(q, "q")
    with pytest.raises(ValueError):
        bsa._desc(torch.zeros(1, 1, 64, 64), "q")


def test_neighborhood_split_policy_from_the_geometry():
    # the 2-D neighbourhood workload (512 text tokens, 128 x 128 grid, 8 x 16
    # tiles, 32 x 32 window): at strides 1 and 16 the windowed rows are long
    # enough that the 132-block text rows fit the average load; at stride 32
    # the windows shrink to whole tiles and the text rows are cut into 4
    for stride, want in (((1, 1), None), ((16, 16), None),
                         ((32, 32), {"chunk_blocks": 33, "max_chunks": 4, "max_split_rows": 96})):
        nb = bsa.neighborhood(512, (128, 128), (8, 16), (32, 32), stride)
        assert bsa.neighborhood_split_policy(1, 24, nb, 128) == want
    with pytest.raises(ValueError):          # tile of 128 tokens against block 64
        bsa.neighborhood_split_policy(1, 24, bsa.neighborhood(512, (128, 128), (8, 16), (32, 32)), 64)


@pytest.mark.parametrize("mode,N,D,block,r", [
    (0, 65536, 128, 64, 64),         # projections: 2 * 4 * 32 * 1024 * 64 * 4 bytes > 32 MiB
    (1, 1 << 24, 64, 128, 0),        # one exact-score slot: 131072 * 128 * 4 bytes > 32 MiB
])
def test_pool_scores_noalloc_rejects_requests_beyond_its_scratch(mode, N, D, block, r):
    """Checked before the scratch is resolved or anything is enqueued, so no
    GPU is needed."""
    lib = bsa.load()
    q = _t(B=4, H=32, N=N, D=D)
    k = _t(B=4, H=32, N=N, D=D)
    st = lib.bsa_pool_scores_noalloc(ctypes.byref(q), ctypes.byref(k), block, mode,
                                     ctypes.c_void_p(FAKE) if r else None, r, 0.0,
                                     ctypes.c_void_p(FAKE), None)
    assert st == 4
    assert "scratch" in _err()


@pytest.mark.parametrize("N,block,r,tb,groups,code,msg", [
    (512, 64, 32, 1, [(0, 8, 4)], 2, "text columns"),            # a group over the text column
    (4352, 64, 32, 4, [(4, 60, 8), (50, 68, 2)], 2, "disjoint"),   # overlapping groups
    (300 * 64, 64, 8, 0, [(0, 300, 10)], 2, "at most 256"),        # more blocks than the fused kernel holds
    (4352, 64, 64, 4, [(4, 68, 16)], 2, "at most"),                # nB * r above 4096
    (220 * 64, 64, 18, 4, [(4, 220, 16)], 2, "at most"),           # nB * r <= 4096, r padded to 20 is not
    (4352, 64, 32, 4, [(4, 68, 70)], 1, "invalid"),                # k above the group's width
])
def test_select_meanpool_validation(N, block, r, tb, groups, code, msg):
    lib = bsa.load()
    q, k = _t(N=N, D=64), _t(N=N, D=64)
    arr = (bsa.BsaGroup * len(groups))(*[bsa.BsaGroup(*g) for g in groups])
    st = lib.bsa_select_meanpool(ctypes.byref(q), ctypes.byref(k), block, ctypes.c_void_p(FAKE), r, tb, arr,
                                 len(groups), None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 1 << 30,
                                 ctypes.c_void_p(FAKE), 1 << 30, None)
    assert st == code
    assert msg in _err()


def test_select_meanpool_applies_mirrors_the_abi_limits():
    assert bsa.select_meanpool_applies(68, 32, 4, [(4, 68, 16)])
    assert bsa.select_meanpool_applies(70, 32, 4, [(4, 60, 14), (60, 70, 3), (0, 70, 0)])
    assert not bsa.select_meanpool_applies(8, 32, 1, [(0, 8, 4)])
    assert not bsa.select_meanpool_applies(68, 32, 4, [(4, 60, 8), (50, 68, 2)])
    assert not bsa.select_meanpool_applies(257, 8, 0, [(0, 257, 10)])
    assert not bsa.select_meanpool_applies(68, 64, 4, [(4, 68, 16)])
    assert bsa.select_meanpool_applies(256, 13, 2, [(2, 200, 50), (200, 256, 9)])   # r padded to 16: 4096
    assert not bsa.select_meanpool_applies(220, 18, 4, [(4, 220, 16)])               # r padded to 20: 4400
