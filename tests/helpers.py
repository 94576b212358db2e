"""Shared test plumbing: synthetic inputs to device tensors, library loading,
and the comparison rules for the HIP path against the CPU oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

# S tolerances: 3e-2 absolute on the bf16-MFMA path; 1e-4 relative (to
# max(1, |S|)) on the fp32 path.
S_ABS_BF16 = 3e-2
S_REL_F32 = 1e-4
# selected tokens must agree wherever the oracle's best-vs-second margin
# exceeds this
PATH_MARGIN = 0.1


def ensure_built():
    import draft_block_contextual_amd as dc
    if not os.path.exists(dc.LIB_PATH):
        from draft_block_contextual_amd import build
        build.build()
    return dc.load()


def to_dev(a, dtype: str, device="cuda"):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def device_inputs(inp: dict, device="cuda"):
    """Upload one synth input set; returns (Dims, Weights, logits, h, E)."""
    import draft_block_contextual_amd as dc
    D = inp["dims"]
    dt = D.dtype
    dims = dc.Dims.from_synth(D)
    w = dc.Weights(P_e=to_dev(inp["P_e"], dt, device), P_h=to_dev(inp["P_h"], dt, device),
                   W_f=to_dev(inp["W_f"], dt, device), W_pair=to_dev(inp["W_pair"], dt, device),
                   W1=to_dev(inp["W1"], dt, device), b1=to_dev(inp["b1"], dt, device),
                   w2=to_dev(inp["w2"], dt, device), b2=inp["b2"])
    logits = to_dev(inp["logits"].reshape(D.n_blocks * D.B, D.V), dt, device)
    h = to_dev(inp["h"], dt, device)
    E = to_dev(inp["E"], dt, device)
    return dims, w, logits, h, E


def s_tolerance_ok(S_gpu: np.ndarray, S_ref: np.ndarray, dtype: str):
    diff = np.abs(S_gpu.astype(np.float64) - S_ref)
    if dtype == "bf16":
        bound = np.full_like(S_ref, S_ABS_BF16)
    else:
        bound = S_REL_F32 * np.maximum(1.0, np.abs(S_ref))
    bad = ~(diff <= bound)
    return not bad.any(), float(np.nanmax(diff)) if diff.size else 0.0, int(bad.sum())


def lockstep_path_check(S_gpu, S_ref, cand_vals, sel_gpu, sel_ref):
    """Walk the GPU and oracle paths in lockstep.  At each step where both
    paths share the predecessor, the chosen successor must agree whenever the
    oracle's best-vs-second margin on that row exceeds PATH_MARGIN.  A block
    is compared until its paths part at a low-margin step (later rows are
    conditioned on different predecessors).  Returns (ok, steps_compared,
    steps_total, first failure or None)."""
    N, B = sel_ref.shape
    compared = 0
    total = 0
    for n in range(N):
        if sel_gpu[n, 0] != sel_ref[n, 0]:
            return False, compared, total, (n, 0)
        for p in range(B - 1):
            total += 1
            k = sel_ref[n, p]
            row = S_ref[n, p, k]
            srt = np.sort(row[~np.isnan(row)])[::-1]
            margin = srt[0] - srt[1] if len(srt) > 1 else np.inf
            same = sel_gpu[n, p + 1] == sel_ref[n, p + 1]
            compared += 1
            if not same:
                if margin > PATH_MARGIN:
                    return False, compared, total, (n, p + 1, float(margin))
                break
    return True, compared, total, None
