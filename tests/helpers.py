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


def score_magnitude(z, s, cand_vals, W1, b1, w2, b2):
    """M[n, p, a, b]: the size of what an evaluation of S_p(a, b) adds up,
    |l| + |b2| + sum_h |w2_h| (|SiLU(u_h)| + |SiLU'(u_h)| sum_j |W1[h, j] x_j|)
    with x = [z_{p,a}; z_{p+1,b}; s_p] and u = W1 x + b1 (float64).  A first-
    order rounding analysis of any fp32 evaluation bounds its error by
    n 2^-24 M, n = 2 r_z + r_s + H (the lengths of the two sums)."""
    z = np.asarray(z, np.float64)
    N, B, K, rz = z.shape
    W1 = np.asarray(W1, np.float64)
    Wa, Wb, Ws = W1[:, :rz], W1[:, rz:2 * rz], W1[:, 2 * rz:]
    M = np.empty((N, B - 1, K, K))
    for n in range(N):
        for p in range(B - 1):
            A, Bv, C = z[n, p] @ Wa.T, z[n, p + 1] @ Wb.T, s[n, p] @ Ws.T + b1
            aA, aB, aC = np.abs(z[n, p]) @ np.abs(Wa).T, np.abs(z[n, p + 1]) @ np.abs(Wb).T, np.abs(s[n, p]) @ np.abs(Ws).T
            u = A[:, None, :] + Bv[None, :, :] + C
            with np.errstate(over="ignore"):
                sig = 1.0 / (1.0 + np.exp(-u))
            dsilu = sig * (1.0 + u * (1.0 - sig))
            absx = aA[:, None, :] + aB[None, :, :] + aC
            M[n, p] = (np.abs(cand_vals[n, p + 1])[None, :] + abs(b2)
                       + (np.abs(w2) * (np.abs(u * sig) + np.abs(dsilu) * absx)).sum(-1))
    return M


def s_tolerance_cancelling(S_gpu, S_ref, M, n_terms, frac=0.99):
    """fp32 scores whose terms cancel far below their magnitude M: every
    element within max(1e-4 max(1, |S|), n_terms 2^-24 M), and at least `frac`
    of them within 1e-4 max(1, |S|).  Returns (ok, worst, count outside the
    relative bar, count outside both)."""
    diff = np.abs(S_gpu.astype(np.float64) - S_ref)
    rel = S_REL_F32 * np.maximum(1.0, np.abs(S_ref))
    cond = n_terms * 2.0 ** -24 * M
    out_rel = ~(diff <= rel)
    out_all = ~(diff <= np.maximum(rel, cond))
    ok = (not out_all.any()) and out_rel.mean() <= 1.0 - frac
    return ok, float(np.nanmax(diff)), int(out_rel.sum()), int(out_all.sum())


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
