"""Python binding of libdcoco, the MI355X (gfx950) DCOCO corrector hot path.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/dcoco.h.  torch supplies device memory and the current
HIP stream.  Importing this package does not need a GPU; the first call that
launches work does.  If libdcoco.so has not been built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdcoco.so")

DCOCO_OK = 0
DCOCO_ERR_INVALID_ARG = -1
DCOCO_ERR_UNSUPPORTED = -2
DCOCO_ERR_WORKSPACE = -3
DCOCO_ERR_HIP = -4
DTYPE_CODE = {"f32": 0, "bf16": 1}

# every entry point include/dcoco.h declares
EXPORTS = ["dcoco_topk", "dcoco_represent", "dcoco_score", "dcoco_select", "dcoco_select_path",
           "dcoco_lm_head_topk", "dcoco_loss", "dcoco_score_backward", "dcoco_represent_backward",
           "dcoco_correct_block", "dcoco_correct_block_static", "dcoco_build_btable",
           "dcoco_correct_block_btable", "dcoco_static_scratch_bytes", "dcoco_status_string", "dcoco_abi_version"]


class DcocoError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class CDims(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("B", ctypes.c_int32), ("K", ctypes.c_int32),
                ("V", ctypes.c_int32), ("d_hidden", ctypes.c_int32), ("d_embed", ctypes.c_int32),
                ("d_proj", ctypes.c_int32), ("d_z", ctypes.c_int32), ("d_pair", ctypes.c_int32),
                ("d_mlp", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class CMlpGrads(ctypes.Structure):
    _fields_ = [("dW1", ctypes.c_void_p), ("db1", ctypes.c_void_p), ("dw2", ctypes.c_void_p),
                ("db2", ctypes.c_void_p)]


class CRepGrads(ctypes.Structure):
    _fields_ = [("dP_e", ctypes.c_void_p), ("dP_h", ctypes.c_void_p), ("dW_f", ctypes.c_void_p),
                ("dW_pair", ctypes.c_void_p)]


class CWeights(ctypes.Structure):
    _fields_ = [("P_e", ctypes.c_void_p), ("P_h", ctypes.c_void_p), ("W_f", ctypes.c_void_p),
                ("W_pair", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("b2", ctypes.c_float)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdcoco.so (built by draft_block_contextual_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m draft_block_contextual_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
    pd, pw = ctypes.POINTER(CDims), ctypes.POINTER(CWeights)
    lib.dcoco_topk.argtypes = [pd, vp, vp, vp, vp, sz, vp]
    lib.dcoco_represent.argtypes = [pd, pw, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dcoco_score.argtypes = [pd, pw, vp, vp, vp, vp, vp, sz, vp]
    lib.dcoco_select.argtypes = [pd, vp, vp, vp, vp, vp, vp]
    lib.dcoco_select_path.argtypes = [pd, vp, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp]
    lib.dcoco_loss.argtypes = [pd, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp]
    lib.dcoco_lm_head_topk.argtypes = [pd, vp, vp, vp, vp, vp, sz, vp]
    lib.dcoco_score_backward.argtypes = [pd, pw, vp, vp, vp, vp, vp, vp, ctypes.POINTER(CMlpGrads), vp, sz, vp]
    lib.dcoco_represent_backward.argtypes = [pd, pw, vp, vp, vp, vp, vp, ctypes.POINTER(CRepGrads), vp, vp, sz, vp]
    lib.dcoco_correct_block.argtypes = [pd, pw, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp]
    lib.dcoco_correct_block_static.argtypes = [pd, pw, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dcoco_static_scratch_bytes.argtypes = []
    lib.dcoco_static_scratch_bytes.restype = ctypes.c_size_t
    lib.dcoco_build_btable.argtypes = [pd, pw, vp, vp, vp, sz, vp]
    lib.dcoco_correct_block_btable.argtypes = [pd, pw, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp]
    for f in ["dcoco_topk", "dcoco_represent", "dcoco_score", "dcoco_select", "dcoco_select_path",
              "dcoco_lm_head_topk", "dcoco_loss", "dcoco_score_backward", "dcoco_represent_backward",
              "dcoco_correct_block", "dcoco_correct_block_static", "dcoco_build_btable",
              "dcoco_correct_block_btable"]:
        getattr(lib, f).restype = ctypes.c_int
    lib.dcoco_status_string.argtypes = [ctypes.c_int]
    lib.dcoco_status_string.restype = ctypes.c_char_p
    lib.dcoco_abi_version.argtypes = []
    lib.dcoco_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dcoco_status_string(status).decode()


@dataclasses.dataclass
class Dims:
    n_blocks: int
    B: int
    K: int
    V: int
    d_hidden: int
    d_embed: int
    d_proj: int
    d_z: int
    d_pair: int
    d_mlp: int
    dtype: str = "bf16"
    ln_eps: float = 1e-5

    def c(self) -> CDims:
        return CDims(self.n_blocks, self.B, self.K, self.V, self.d_hidden, self.d_embed, self.d_proj,
                     self.d_z, self.d_pair, self.d_mlp, DTYPE_CODE[self.dtype], self.ln_eps)

    @classmethod
    def from_synth(cls, D) -> "Dims":
        return cls(D.n_blocks, D.B, D.K, D.V, D.d, D.e, D.r, D.r_z, D.r_s, D.H, D.dtype, D.ln_eps)


@dataclasses.dataclass
class Weights:
    P_e: object
    P_h: object
    W_f: object
    W_pair: object
    W1: object
    b1: object
    w2: object
    b2: float

    def c(self) -> CWeights:
        return CWeights(_ptr(self.P_e), _ptr(self.P_h), _ptr(self.W_f), _ptr(self.W_pair),
                        _ptr(self.W1), _ptr(self.b1), _ptr(self.w2), float(self.b2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _resolve(stream):
    """The torch stream a call runs on: the one given, else the current one."""
    import torch
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_resolve(stream).cuda_stream)


def _on(stream):
    """Allocate under the stream the kernels run on, so that the caching
    allocator hands a freed block to other work only after that stream's work
    (the outputs and workspaces made here are used on that stream only)."""
    import torch
    return torch.cuda.stream(_resolve(stream))


def _check(fn: str, rc: int):
    if rc != DCOCO_OK:
        raise DcocoError(fn, rc, status_string(rc))


def _torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


# One cached workspace per (device, stream), allocated on that stream: a
# replaced buffer is released to the caching allocator on the stream that
# used it, so it is reused only after that stream's queued work.
_ws_cache: dict = {}
_WS_STREAMS = 8


def _workspace(nbytes: int, device, workspace=None, stream=None):
    import torch
    if workspace is not None:
        return workspace
    st = _resolve(stream)
    key = (str(device), st.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        _ws_cache.pop(key, None)
        if len(_ws_cache) >= _WS_STREAMS:
            _ws_cache.pop(next(iter(_ws_cache)))
        with torch.cuda.stream(st):
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _empty(stream, *shape_args, **kw):
    """torch.empty allocated under the call's stream (see _on); with no stream
    given the call runs on the current stream, where torch allocates anyway."""
    import torch
    if stream is None:
        return torch.empty(*shape_args, **kw)
    with torch.cuda.stream(stream):
        return torch.empty(*shape_args, **kw)


def _query(fn, *args) -> int:
    n = ctypes.c_size_t(0)
    _check(fn.__name__, fn(*args, None, ctypes.byref(n), None))
    return n.value


def topk(dims: Dims, logits, cand_ids=None, cand_logits=None, workspace=None, stream=None):
    """dcoco_topk: logits [N*B, V] -> (cand_ids [N*B, K] int32, cand_logits [N*B, K] fp32)."""
    import torch
    lib = load()
    cd = dims.c()
    R = dims.n_blocks * dims.B
    dev = logits.device
    if cand_ids is None:
        cand_ids = _empty(stream, (R, dims.K), dtype=torch.int32, device=dev)
    if cand_logits is None:
        cand_logits = _empty(stream, (R, dims.K), dtype=torch.float32, device=dev)
    need = _query(lib.dcoco_topk, ctypes.byref(cd), _ptr(logits), _ptr(cand_ids), _ptr(cand_logits))
    ws = _workspace(need, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_topk", lib.dcoco_topk(ctypes.byref(cd), _ptr(logits), _ptr(cand_ids), _ptr(cand_logits),
                                        _ptr(ws), ctypes.byref(n), _stream(stream)))
    return cand_ids, cand_logits


def represent(dims: Dims, w: Weights, h, E, cand_ids, z=None, s=None, workspace=None, stream=None):
    """dcoco_represent -> (z [N,B,K,d_z] dtype, s [N,B-1,d_pair] fp32)."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = h.device
    if z is None:
        z = _empty(stream, (dims.n_blocks, dims.B, dims.K, dims.d_z), dtype=_torch_dtype(dims.dtype), device=dev)
    if s is None:
        s = _empty(stream, (dims.n_blocks, max(dims.B - 1, 1), dims.d_pair), dtype=torch.float32, device=dev)
    args = (ctypes.byref(cd), ctypes.byref(cw), _ptr(h), _ptr(E), _ptr(cand_ids), _ptr(z), _ptr(s))
    need = _query(lib.dcoco_represent, *args)
    ws = _workspace(need, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_represent", lib.dcoco_represent(*args, _ptr(ws), ctypes.byref(n), _stream(stream)))
    return z, s[:, :dims.B - 1]


def score(dims: Dims, w: Weights, z, s, cand_logits, S=None, workspace=None, stream=None):
    """dcoco_score -> S [N, B-1, K, K] fp32."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = z.device
    if S is None:
        S = _empty(stream, (dims.n_blocks, max(dims.B - 1, 1), dims.K, dims.K), dtype=torch.float32, device=dev)
    args = (ctypes.byref(cd), ctypes.byref(cw), _ptr(z), _ptr(s), _ptr(cand_logits), _ptr(S))
    need = _query(lib.dcoco_score, *args)
    ws = _workspace(need, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_score", lib.dcoco_score(*args, _ptr(ws), ctypes.byref(n), _stream(stream)))
    return S[:, :dims.B - 1]


def select(dims: Dims, S, cand_logits, cand_ids, sel_idx=None, sel_tok=None, stream=None):
    """dcoco_select -> (sel_idx [N, B] int32, sel_tok [N, B] int32)."""
    import torch
    lib = load()
    cd = dims.c()
    dev = cand_logits.device
    if sel_idx is None:
        sel_idx = _empty(stream, (dims.n_blocks, dims.B), dtype=torch.int32, device=dev)
    if sel_tok is None:
        sel_tok = _empty(stream, (dims.n_blocks, dims.B), dtype=torch.int32, device=dev)
    _check("dcoco_select", lib.dcoco_select(ctypes.byref(cd), _ptr(S), _ptr(cand_logits), _ptr(cand_ids),
                                            _ptr(sel_idx), _ptr(sel_tok), _stream(stream)))
    return sel_idx, sel_tok


PATH_RULES = {"greedy": 0, "global_sum": 1, "discount": 2}


def select_path(dims: Dims, S, cand_logits, cand_ids, rule: str = "greedy", lam: float = 1.0,
                sel_idx=None, sel_tok=None, stream=None):
    """dcoco_select_path -> (sel_idx [N, B] int32, sel_tok [N, B] int32).
    rule: "greedy", "global_sum" or "discount" (weight lam^(j-1) on slot j)."""
    import torch
    lib = load()
    cd = dims.c()
    dev = cand_logits.device
    if sel_idx is None:
        sel_idx = _empty(stream, (dims.n_blocks, dims.B), dtype=torch.int32, device=dev)
    if sel_tok is None:
        sel_tok = _empty(stream, (dims.n_blocks, dims.B), dtype=torch.int32, device=dev)
    _check("dcoco_select_path", lib.dcoco_select_path(ctypes.byref(cd), _ptr(S), _ptr(cand_logits),
                                                      _ptr(cand_ids), PATH_RULES[rule], float(lam),
                                                      _ptr(sel_idx), _ptr(sel_tok), _stream(stream)))
    return sel_idx, sel_tok


def lm_head_topk(dims: Dims, hd, W_lm, cand_ids=None, cand_logits=None, workspace=None, stream=None):
    """dcoco_lm_head_topk -> (cand_ids [N*B, K] int32, cand_logits [N*B, K] fp32)."""
    import torch
    lib = load()
    cd = dims.c()
    dev = hd.device
    R = dims.n_blocks * dims.B
    if cand_ids is None:
        cand_ids = _empty(stream, (R, dims.K), dtype=torch.int32, device=dev)
    if cand_logits is None:
        cand_logits = _empty(stream, (R, dims.K), dtype=torch.float32, device=dev)
    n = ctypes.c_size_t(0)
    _check("dcoco_lm_head_topk", lib.dcoco_lm_head_topk(ctypes.byref(cd), None, None, None, None, None,
                                                        ctypes.byref(n), None))
    ws = _workspace(n.value, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_lm_head_topk", lib.dcoco_lm_head_topk(ctypes.byref(cd), _ptr(hd), _ptr(W_lm), _ptr(cand_ids),
                                                        _ptr(cand_logits), _ptr(ws), ctypes.byref(n),
                                                        _stream(stream)))
    return cand_ids, cand_logits


def loss(dims: Dims, S, cand_ids, target_tok, rho: float = 4.0, stream=None):
    """dcoco_loss -> (loss [1], pair_loss [N, B-1], dS [N, B-1, K, K]), fp32."""
    import torch
    lib = load()
    cd = dims.c()
    dev = cand_ids.device
    Bm1 = max(dims.B - 1, 1)
    # one buffer for the scalar (a 16-byte slot), the pair terms and dS
    n_pair = dims.n_blocks * Bm1
    off = 4 + (n_pair + 3) // 4 * 4          # dS starts 16-byte aligned
    buf = _empty(stream, off + n_pair * dims.K * dims.K, dtype=torch.float32, device=dev)
    out = buf[:4]
    pair = buf[4:4 + n_pair].view(dims.n_blocks, Bm1)
    dS = buf[off:].view(dims.n_blocks, Bm1, dims.K, dims.K)
    _check("dcoco_loss", lib.dcoco_loss(ctypes.byref(cd), _ptr(S), _ptr(cand_ids), _ptr(target_tok),
                                        float(rho), _ptr(out), _ptr(pair), _ptr(dS), _stream(stream)))
    return out[:1], pair[:, :dims.B - 1], dS[:, :dims.B - 1]


def score_backward(dims: Dims, w: Weights, z, s, dS, workspace=None, stream=None) -> dict:
    """dcoco_score_backward -> dict of fp32 gradients: dz, ds, d_cand_logits,
    dW1, db1, dw2, db2."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = z.device
    N, B, K = dims.n_blocks, dims.B, dims.K
    H, rz, rs = dims.d_mlp, dims.d_z, dims.d_pair
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dz": _empty(stream, (N, B, K, rz), **f32), "ds": _empty(stream, (N, max(B - 1, 1), rs), **f32),
           "d_cand_logits": _empty(stream, (N, B, K), **f32), "dW1": _empty(stream, (H, 2 * rz + rs), **f32),
           "db1": _empty(stream, H, **f32), "dw2": _empty(stream, H, **f32), "db2": _empty(stream, 4, **f32)}
    g = CMlpGrads(out["dW1"].data_ptr(), out["db1"].data_ptr(), out["dw2"].data_ptr(), out["db2"].data_ptr())
    n = ctypes.c_size_t(0)
    _check("dcoco_score_backward", lib.dcoco_score_backward(ctypes.byref(cd), ctypes.byref(cw), None, None, None,
                                                            None, None, None, ctypes.byref(g), None,
                                                            ctypes.byref(n), None))
    ws = _workspace(n.value, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_score_backward",
           lib.dcoco_score_backward(ctypes.byref(cd), ctypes.byref(cw), _ptr(z), _ptr(s), _ptr(dS),
                                    _ptr(out["dz"]), _ptr(out["ds"]) if B > 1 else None,
                                    _ptr(out["d_cand_logits"]), ctypes.byref(g), _ptr(ws), ctypes.byref(n),
                                    _stream(stream)))
    out["ds"] = out["ds"][:, :B - 1]
    out["db2"] = out["db2"][:1]
    return out


def represent_backward(dims: Dims, w: Weights, h, E, cand_ids, dz, ds, want_dh: bool = True, workspace=None,
                       stream=None) -> dict:
    """dcoco_represent_backward -> dict of fp32 gradients: dP_e, dP_h, dW_f,
    dW_pair and (want_dh) dh."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = h.device
    N, B = dims.n_blocks, dims.B
    r, rs = dims.d_proj, dims.d_pair
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dP_e": _empty(stream, (r, dims.d_embed), **f32), "dP_h": _empty(stream, (r, dims.d_hidden), **f32),
           "dW_f": _empty(stream, (dims.d_z, 2 * r), **f32), "dW_pair": _empty(stream, (rs, 2 * dims.d_hidden), **f32)}
    if want_dh:
        out["dh"] = _empty(stream, (N, B, dims.d_hidden), **f32)
    g = CRepGrads(out["dP_e"].data_ptr(), out["dP_h"].data_ptr(), out["dW_f"].data_ptr(), out["dW_pair"].data_ptr())
    n = ctypes.c_size_t(0)
    _check("dcoco_represent_backward",
           lib.dcoco_represent_backward(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None, None,
                                        ctypes.byref(g), None, None, ctypes.byref(n), None))
    ws = _workspace(n.value, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_represent_backward",
           lib.dcoco_represent_backward(ctypes.byref(cd), ctypes.byref(cw), _ptr(h), _ptr(E), _ptr(cand_ids),
                                        _ptr(dz), _ptr(ds) if B > 1 else None, ctypes.byref(g),
                                        _ptr(out["dh"]) if want_dh else None, _ptr(ws), ctypes.byref(n),
                                        _stream(stream)))
    return out


def correct_block_workspace_bytes(dims: Dims, w: Weights, btable: bool = False) -> int:
    lib = load()
    cd, cw = dims.c(), w.c()
    n = ctypes.c_size_t(0)
    fn = lib.dcoco_correct_block_btable if btable else lib.dcoco_correct_block
    _check(fn.__name__, fn(ctypes.byref(cd), ctypes.byref(cw), None, None, None, None, ctypes.byref(n),
                           None, None, None, None, None, None))
    return n.value


def build_btable(dims: Dims, w: Weights, E, table=None, workspace=None, stream=None):
    """dcoco_build_btable: the [V, d_proj] bf16 table of LN(P_e E_v)."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = E.device
    if table is None:
        table = _empty(stream, (dims.V, dims.d_proj), dtype=torch.bfloat16, device=dev)
    args = (ctypes.byref(cd), ctypes.byref(cw), _ptr(E), _ptr(table))
    need = _query(lib.dcoco_build_btable, *args)
    ws = _workspace(need, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    _check("dcoco_build_btable", lib.dcoco_build_btable(*args, _ptr(ws), ctypes.byref(n), _stream(stream)))
    return table


def correct_block(dims: Dims, w: Weights, logits, h, E, sel_tok=None, sel_idx=None, S=None,
                  cand_ids=None, cand_logits=None, want_all: bool = False, workspace=None, stream=None,
                  btable=None):
    """dcoco_correct_block (dcoco_correct_block_btable when btable, a table from
    build_btable, is given; E is then not used).  Returns a dict with sel_tok
    (and, when asked for or passed in, sel_idx, S, cand_ids, cand_logits)."""
    import torch
    lib = load()
    cd, cw = dims.c(), w.c()
    dev = logits.device
    N, B, K = dims.n_blocks, dims.B, dims.K
    if sel_tok is None:
        sel_tok = _empty(stream, (N, B), dtype=torch.int32, device=dev)
    if want_all:
        if sel_idx is None:
            sel_idx = _empty(stream, (N, B), dtype=torch.int32, device=dev)
        if S is None:
            S = _empty(stream, (N, max(B - 1, 1), K, K), dtype=torch.float32, device=dev)
        if cand_ids is None:
            cand_ids = _empty(stream, (N, B, K), dtype=torch.int32, device=dev)
        if cand_logits is None:
            cand_logits = _empty(stream, (N, B, K), dtype=torch.float32, device=dev)
    need = correct_block_workspace_bytes(dims, w, btable is not None)
    ws = _workspace(need, dev, workspace, stream)
    n = ctypes.c_size_t(ws.numel())
    fn = lib.dcoco_correct_block if btable is None else lib.dcoco_correct_block_btable
    src = E if btable is None else btable
    _check(fn.__name__, fn(
        ctypes.byref(cd), ctypes.byref(cw), _ptr(logits), _ptr(h), _ptr(src), _ptr(ws), ctypes.byref(n),
        _ptr(sel_tok), _ptr(sel_idx), _ptr(S), _ptr(cand_ids), _ptr(cand_logits), _stream(stream)))
    out = {"sel_tok": sel_tok}
    if sel_idx is not None:
        out["sel_idx"] = sel_idx
    if S is not None:
        out["S"] = S[:, :B - 1]
    if cand_ids is not None:
        out["cand_ids"] = cand_ids
    if cand_logits is not None:
        out["cand_logits"] = cand_logits
    return out


def static_scratch_bytes() -> int:
    """Size of the library's static per-GPU scratch buffer (dcoco_correct_block_static)."""
    return int(load().dcoco_static_scratch_bytes())


def correct_block_static(dims: Dims, w: Weights, logits, h, E, sel_tok, sel_idx=None, S=None, cand_ids=None,
                         cand_logits=None, stream=None):
    """dcoco_correct_block_static: the whole path with the intermediates in the
    library's static scratch buffer.  Allocates nothing: every output is the
    caller's (sel_tok required; the others may be None).  Calls that overlap
    on one GPU race on the shared buffer."""
    lib = load()
    cd, cw = dims.c(), w.c()
    _check("dcoco_correct_block_static", lib.dcoco_correct_block_static(
        ctypes.byref(cd), ctypes.byref(cw), _ptr(logits), _ptr(h), _ptr(E), _ptr(sel_tok), _ptr(sel_idx), _ptr(S),
        _ptr(cand_ids), _ptr(cand_logits), _stream(stream)))
