"""Host-side checks of the C ABI: the library loads, exports every entry point
include/dcoco.h declares, answers workspace queries and rejects bad arguments
before launching anything.  No GPU needed: every call here returns before the
library touches the HIP runtime."""
import ctypes
import os
import re

import pytest

from helpers import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "dcoco.h")


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dcoco_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    import draft_block_contextual_amd as dc
    names = _declared_functions()
    assert set(names) == set(dc.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    import draft_block_contextual_amd as dc
    assert lib.dcoco_abi_version() == 108
    assert dc.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert dc.status_string(code) not in ("ok", "unknown status")
    assert dc.status_string(7) == "unknown status"


def _dims(**kw):
    import draft_block_contextual_amd as dc
    base = dict(n_blocks=32, B=16, K=16, V=151936, d_hidden=4096, d_embed=4096, d_proj=256,
                d_z=256, d_pair=256, d_mlp=512, dtype="bf16", ln_eps=1e-5)
    base.update(kw)
    return dc.Dims(**base)


def _query_topk(lib, dims):
    cd = dims.c()
    n = ctypes.c_size_t(0)
    rc = lib.dcoco_topk(ctypes.byref(cd), None, None, None, None, ctypes.byref(n), None)
    return rc, n.value


def _query_block(lib, dims):
    import draft_block_contextual_amd as dc
    cd = dims.c()
    cw = dc.CWeights()
    n = ctypes.c_size_t(0)
    rc = lib.dcoco_correct_block(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None,
                                 ctypes.byref(n), None, None, None, None, None, None)
    return rc, n.value


def test_workspace_queries(lib):
    rc, n = _query_topk(lib, _dims())
    assert rc == 0 and n > 0
    rc, n = _query_block(lib, _dims())
    assert rc == 0 and n >= 16 * 2 ** 20
    rc, n2 = _query_block(lib, _dims(n_blocks=4))
    assert rc == 0 and 0 < n2 < n


@pytest.mark.parametrize("kw,code", [
    (dict(n_blocks=0), -1), (dict(B=0), -1), (dict(K=0), -1), (dict(K=20, V=10), -1),
    (dict(ln_eps=0.0), -1), (dict(ln_eps=float("nan")), -1), (dict(ln_eps=-1.0), -1),
    (dict(K=65), -2), (dict(d_proj=48), -2), (dict(d_proj=0), -1), (dict(d_mlp=-32), -1),
    (dict(d_z=4096), -2), (dict(d_hidden=100), -2),
])
def test_invalid_dims_rejected(lib, kw, code):
    rc, _ = _query_block(lib, _dims(**kw))
    assert rc == code


def test_bad_dtype_rejected(lib):
    d = _dims()
    cd = d.c()
    cd.dtype = 7
    n = ctypes.c_size_t(0)
    assert lib.dcoco_topk(ctypes.byref(cd), None, None, None, None, ctypes.byref(n), None) == -1


def test_workspace_and_pointer_checks(lib):
    import draft_block_contextual_amd as dc
    d = _dims()
    cd = d.c()
    rc, need = _query_topk(lib, d)
    fake = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced: checks fail first
    small = ctypes.c_size_t(need - 256)
    assert lib.dcoco_topk(ctypes.byref(cd), fake, fake, fake, fake, ctypes.byref(small), None) == -3
    ok = ctypes.c_size_t(need)
    mis = ctypes.c_void_p((1 << 20) + 128)
    assert lib.dcoco_topk(ctypes.byref(cd), fake, fake, fake, mis, ctypes.byref(ok), None) == -3
    # null or misaligned data pointers
    assert lib.dcoco_topk(ctypes.byref(cd), None, fake, fake, fake, ctypes.byref(ok), None) == -1
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert lib.dcoco_topk(ctypes.byref(cd), odd, fake, fake, fake, ctypes.byref(ok), None) == -1
    # a missing workspace_bytes pointer
    assert lib.dcoco_topk(ctypes.byref(cd), fake, fake, fake, None, None, None) == -1
    # missing weights in the full path
    rc, need_b = _query_block(lib, d)
    cw = dc.CWeights()
    nb = ctypes.c_size_t(need_b)
    assert lib.dcoco_correct_block(ctypes.byref(cd), ctypes.byref(cw), fake, fake, fake, fake,
                                   ctypes.byref(nb), fake, None, None, None, None, None) == -1
    # select: null outputs
    assert lib.dcoco_select(ctypes.byref(cd), fake, fake, fake, None, None, None) == -1


@pytest.mark.parametrize("n_blocks,K,V,segments", [
    (1, 16, 151936, 8), (1, 64, 151936, 8), (2, 16, 151936, 8), (1, 16, 40000, 8), (1, 16, 20000, 4),
    (1, 16, 5000, 1), (4, 16, 151936, 1), (32, 16, 151936, 1)])
def test_topk_workspace_holds_the_row_segments(lib, n_blocks, K, V, segments):
    # bf16 calls of at most 32 rows cut each row into column segments (at
    # most 256 workgroups in all, at most 8 per row, each segment at least
    # 4096 columns) and keep each segment's K composites (8 bytes) for the merge;
    # more rows, or rows too short to cut, need no workspace beyond the minimum
    rows = n_blocks * 16
    rc, n = _query_topk(lib, _dims(n_blocks=n_blocks, K=K, V=V))
    assert rc == 0
    if segments > 1:
        assert n >= rows * segments * K * 8
        assert n < rows * segments * K * 8 + 4096
    else:
        assert n <= 4096


def test_vocab_limits_for_topk(lib):
    # bf16 rows: one workgroup per row, any vocabulary up to 2^30
    rc, n = _query_topk(lib, _dims(K=64, V=600000))
    assert rc == 0 and n >= 256
    assert _query_topk(lib, _dims(K=64, V=(1 << 30) + 1))[0] == -2
    # fp32 rows: the chunk merge holds at most 2048 candidates
    rc, _ = _query_topk(lib, _dims(K=64, V=600000, dtype="f32"))
    assert rc == -2


def test_btable_queries(lib):
    import draft_block_contextual_amd as dc
    d = _dims()
    cd = d.c()
    cw = dc.CWeights()
    n = ctypes.c_size_t(0)
    assert lib.dcoco_build_btable(ctypes.byref(cd), ctypes.byref(cw), None, None, None, ctypes.byref(n), None) == 0
    assert n.value >= 4 * 8192 * 256 * 4
    n2 = ctypes.c_size_t(0)
    assert lib.dcoco_correct_block_btable(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None,
                                          ctypes.byref(n2), None, None, None, None, None, None) == 0
    rc, n_full = _query_block(lib, d)
    assert rc == 0 and 0 < n2.value < n_full          # no buffers for the gathered projection
    # fp32 storage has no table path; wide projections do (the GEMM gathers the table rows)
    cdx = _dims(dtype="f32").c()
    assert lib.dcoco_build_btable(ctypes.byref(cdx), ctypes.byref(cw), None, None, None,
                                  ctypes.byref(n), None) == -2
    assert lib.dcoco_correct_block_btable(ctypes.byref(cdx), ctypes.byref(cw), None, None, None, None,
                                          ctypes.byref(n2), None, None, None, None, None, None) == -2
    for r in (512, 2048):
        cdx = _dims(d_proj=r).c()
        assert lib.dcoco_build_btable(ctypes.byref(cdx), ctypes.byref(cw), None, None, None,
                                      ctypes.byref(n), None) == 0
        assert n.value >= 4 * 8192 * r * 4
        assert lib.dcoco_correct_block_btable(ctypes.byref(cdx), ctypes.byref(cw), None, None, None, None,
                                              ctypes.byref(n2), None, None, None, None, None, None) == 0


def test_select_path_argument_checks(lib):
    # every case returns before a launch: the rule, lambda and shape checks
    # come first, and the fake pointers are never dereferenced
    fake = ctypes.c_void_p(1 << 20)
    cd = _dims(n_blocks=2, B=16, K=16).c()

    def call(rule, lam, dims=cd, S=fake):
        return lib.dcoco_select_path(ctypes.byref(dims), S, fake, fake, rule, lam, None, fake, None)

    assert call(3, 1.0) == -1                    # unknown rule
    assert call(-1, 1.0) == -1
    for lam in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert call(2, lam) == -1, lam           # a discount lies in (0, 1]
    assert call(2, 0.75, S=None) == -1           # B > 1 needs scores
    big = _dims(n_blocks=2, B=4097, K=2).c()
    assert call(1, 1.0, dims=big) == -2          # too many slots for the back-pointer buffer
    wide = _dims(n_blocks=2, B=300, K=64).c()
    assert call(2, 0.5, dims=wide) == -2         # B*K > 16384
    assert call(1, 1.0, dims=_dims(n_blocks=2, B=16, K=65).c()) == -2   # K > 64


def test_training_argument_checks(lib):
    import draft_block_contextual_amd as dc
    fake = ctypes.c_void_p(1 << 20)
    cd = _dims(n_blocks=2).c()
    for rho in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.dcoco_loss(ctypes.byref(cd), fake, fake, fake, rho, fake, fake, fake, None) == -1
    assert lib.dcoco_loss(ctypes.byref(cd), fake, fake, fake, 4.0, None, fake, fake, None) == -1
    assert lib.dcoco_loss(ctypes.byref(cd), None, fake, fake, 4.0, fake, fake, fake, None) == -1
    # backward: size query, then missing gradient buffers
    cw = dc.CWeights()
    g = dc.CMlpGrads()
    n = ctypes.c_size_t(0)
    assert lib.dcoco_score_backward(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None, None, None,
                                    ctypes.byref(g), None, ctypes.byref(n), None) == 0
    # A and B, their gradients, the pair term and the split partials
    assert n.value >= 2 * 2 * 16 * 16 * 512 * 4 * 2
    cw.W1 = cw.w2 = 1 << 20
    nb = ctypes.c_size_t(n.value)
    assert lib.dcoco_score_backward(ctypes.byref(cd), ctypes.byref(cw), fake, fake, fake, fake, None, None,
                                    ctypes.byref(g), fake, ctypes.byref(nb), None) == -1
    small = ctypes.c_size_t(n.value - 256)
    assert lib.dcoco_score_backward(ctypes.byref(cd), ctypes.byref(cw), fake, fake, fake, fake, None, None,
                                    ctypes.byref(g), fake, ctypes.byref(small), None) == -3


def test_represent_backward_argument_checks(lib):
    import draft_block_contextual_amd as dc
    fake = ctypes.c_void_p(1 << 20)
    cw = dc.CWeights()
    g = dc.CRepGrads()
    n = ctypes.c_size_t(0)

    def call(dims, h=None, E=None, ids=None, dz=None, ds=None, grads=g, ws=None, nb=n):
        return lib.dcoco_represent_backward(ctypes.byref(dims.c()), ctypes.byref(cw), h, E, ids, dz, ds,
                                            ctypes.byref(grads), None, ws, ctypes.byref(nb), None)

    d = _dims(n_blocks=2)
    assert call(d) == 0
    # per candidate row: dz W_f (2 r fp32), dx_e (r fp32), [b | g] (2 r bf16)
    RK = 2 * 16 * 16
    assert n.value >= RK * 256 * (8 + 4 + 4)
    assert call(_dims(n_blocks=2, dtype="f32")) == -2          # bf16 storage only
    assert call(_dims(n_blocks=2, d_proj=48)) == -2
    # weights, gradient buffers and inputs are checked before any launch
    need = n.value
    nb = ctypes.c_size_t(need)
    assert call(d, fake, fake, fake, fake, fake, ws=fake, nb=nb) == -1          # no weights
    cw.P_e = cw.P_h = cw.W_f = cw.W_pair = 1 << 20
    assert call(d, fake, fake, fake, fake, fake, ws=fake, nb=nb) == -1          # no gradient buffers
    g.dP_e = g.dP_h = g.dW_f = g.dW_pair = 1 << 20
    assert call(d, fake, fake, fake, fake, None, ws=fake, nb=nb) == -1          # B > 1 needs ds
    assert call(d, None, fake, fake, fake, fake, ws=fake, nb=nb) == -1          # no h
    small = ctypes.c_size_t(need - 256)
    assert call(d, fake, fake, fake, fake, fake, ws=fake, nb=small) == -3


def _query_score(lib, dims):
    import draft_block_contextual_amd as dc
    cd = dims.c()
    cw = dc.CWeights()
    n = ctypes.c_size_t(0)
    rc = lib.dcoco_score(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None, None, ctypes.byref(n), None)
    return rc, n.value


@pytest.mark.parametrize("n_blocks,B,K,H,on_chip", [
    (256, 16, 4, 64, True),      # five pairs per scoring workgroup: the pair term formed in the scoring launch
    (32, 16, 16, 512, True),     # the 32-stream shape (five pairs per workgroup)
    (8, 64, 8, 512, False),      # six pairs per workgroup: the pair term from its own product
    (2, 5, 32, 320, True),       # K > 16: one pair per workgroup
])
def test_score_workspace_drops_the_pair_term_buffer_when_formed_on_chip(lib, n_blocks, B, K, H, on_chip):
    # bf16 scoring on the slab path needs the bf16 split of s and the per-slab
    # pair sums, plus the fp32 pair term [3, P, H] only when the scoring launch
    # does not form it (each piece rounded up to 256 bytes)
    def up(x):
        return (x + 255) // 256 * 256
    d = _dims(n_blocks=n_blocks, B=B, K=K, d_mlp=H, d_z=64, d_pair=64, d_proj=64, d_hidden=64, d_embed=64, V=3001)
    rc, n = _query_score(lib, d)
    assert rc == 0
    P = n_blocks * (B - 1)
    nslab = (H + 63) // 64
    need = up(3 * P * 64 * 2) + up(4 * nslab * P * K * K)
    if not on_chip:
        need += up(4 * 3 * P * H)
    assert n == need
