"""Plain CPU oracle of the DCOCO contextual-corrector hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (``draft_block_contextual_amd``) and never imports it.

Everything is computed in NumPy float64 from the stored input values, step by
step in the order the pages give, with no blocking, fusion or re-association
beyond what a step's own definition states.  Sources, cited by page title and
section:

[P1]  Two Delta, "Two Delta makes NVIDIA Nemotron 3.5 Super even faster with
      DCOCO" (twodelta.com/blog/dcoco), section "How DCOCO works" and its
      parts "Keep the leading candidates", "Score neighboring candidates in
      parallel", "Select using the realized token identities", and section
      "How we train the corrector".
[P2]  Review of arXiv 2610.12570, "Contextual Correction of Parallel Drafts
      for Speculative Decoding" (jaehun.me/posts/paper-2610-12570), section
      "New approach: DCOCO": part 1 "learned corrector on the block grid"
      (paper Sec. 3.2), part 2 "prefix-first greedy selection" (paper
      Sec. 3.3), section "How it works: a concrete example" (paper Fig. 2),
      section "Path selection and ablation" (paper Sec. 4.3, Tab. 3), and
      part 3 "training: supervised by the verifier's prefix only" (paper
      Sec. 3.2, App. A).

Readings taken where the pages are silent (each is listed with its reason in
the design notes):
  * top-K order: value descending, NaN below every number, -0 equal to +0,
    equal values broken by the lower vocabulary id;
  * LayerNorm: non-affine, biased variance, eps = dims.ln_eps (1e-5);
  * the fusion f is linear without bias: z = W_f [b; g];
  * the MLP is Linear(2 r_z + r_s -> H) with bias b1, SiLU, Linear(H -> 1)
    with bias b2, fed the concatenation [z_{p,a}; z_{p+1,b}; s_p]; the draft
    logit enters only as the additive term l_{p+1}(b);
  * projections P_e, P_h, W_f and W_pair carry no bias; s_p is not normalised;
  * walk argmax: the lowest index among maxima, NaN never wins (index 0 if a
    whole row is NaN);
  * LM head: logits rounded to bf16 (the stored drafter logit) before the
    top-K, which follows the top-K order above;
  * training loss: joint softmax over the K^2 scores of a pair, pair p
    weighted by exp(-(p-1)/rho), masked unless both target tokens are among
    the candidates, summed over pairs and averaged over blocks;
  * whole-path rules: the path score is l_1(k_1) plus the transition scores
    along the path, slot j weighted by lam^(j-1) (lam = 1: Global-Sum); the
    first slot is free; NaN terms count as -inf; ties go to the
    lexicographically smallest path;
  * bf16 contract: inputs and weights are bf16 values; g, b and z are rounded
    to bf16 (nearest, ties to even) where they are produced; s, the MLP and S
    stay unrounded.  In "f32" mode nothing is rounded.

Pins: every function here is checked by ``tests/test_oracle_pins.py``
against closed forms, special cases of the pages, invariants, brute force or
library routines it does not itself call.  No function is left unpinned.
"""
from __future__ import annotations

import math
import numpy as np

__all__ = [
    "to_f64", "round_bf16", "top_k", "layer_norm", "slot_context",
    "candidate_embedding", "fuse", "pair_state", "silu", "transition_scores",
    "greedy_walk", "best_path", "corrector_loss", "score_backward", "represent_backward", "lm_head_logits", "lm_head_topk",
    "correct_block",
]


# ---------------------------------------------------------------- storage ---

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values as float64.  bf16 values arrive as uint16 bit patterns:
    the bits are the upper half of a binary32 with the same value."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_QUANTUM = 2.0 ** -133          # spacing of bf16 subnormals


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits: a value m * 2**ex with 0.5 <= |m| < 1 is
    rounded to a multiple of 2**(ex - 8) (never finer than the subnormal
    spacing 2**-133).  np.round rounds halves to even.  Results beyond the
    largest finite bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0)
    _, ex = np.frexp(x[fin])
    q = np.maximum(np.ldexp(1.0, ex - 8), _BF16_MIN_QUANTUM)
    y = np.round(x[fin] / q) * q
    big = np.abs(y) > _BF16_MAX
    y[big] = np.copysign(np.inf, y[big])
    out[fin] = y
    return out


# ------------------------------------------------------------------ top-K ---

def top_k(logits: np.ndarray, K: int):
    """Keep the K leading candidates of every slot ([P1] "Keep the leading
    candidates"; [P2] part 1, paper Sec. 3.2: c_{i,k} is the id of slot i's
    k-th candidate and l_i(k) its raw draft logit).

    logits: float64 [R, V].  Returns ids int64 [R, K] and the logits l_i(k)
    float64 [R, K] (passed through unchanged), ordered by value descending,
    NaN after every number, ties to the lower id.
    """
    logits = np.asarray(logits, dtype=np.float64)
    R, V = logits.shape
    assert 1 <= K <= V
    ids = np.empty((R, K), np.int64)
    vals = np.empty((R, K), np.float64)
    col = np.arange(V)
    for i in range(R):
        row = logits[i]
        nan = np.isnan(row)
        v = np.where(nan, 0.0, row)
        # np.lexsort sorts by its last key first: non-NaN before NaN, then
        # larger values first, then lower ids.  -0.0 and +0.0 compare equal.
        order = np.lexsort((col, -v, nan))[:K]
        ids[i] = order
        vals[i] = row[order]
    return ids, vals


# ----------------------------------------------------------- LayerNorm ------

def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """Non-affine LayerNorm over the last axis ([P2] part 1, paper Sec. 3.2:
    no learned scale or shift, because hidden states and token embeddings
    differ in scale by over two orders of magnitude).
    (x - mean) / sqrt(var + eps), var = mean of squared deviations."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


# ------------------------------------------------------- representations ---

def slot_context(h: np.ndarray, P_h: np.ndarray, eps: float, bf16: bool) -> np.ndarray:
    """g_i = LN(P_h h_i): the slot's hidden state projected into the compact
    space and normalised ([P1] "Score neighboring candidates in parallel";
    [P2] part 1, paper Sec. 3.2).  h [..., d], P_h [r, d] -> g [..., r]."""
    g = layer_norm(np.asarray(h) @ np.asarray(P_h).T, eps)
    return round_bf16(g) if bf16 else g


def candidate_embedding(E: np.ndarray, ids: np.ndarray, P_e: np.ndarray, eps: float,
                        bf16: bool) -> np.ndarray:
    """b_{i,k} = LN(P_e E[c_{i,k}]): the candidate's row of the frozen token
    embedding table, projected and normalised ([P1] "Score neighboring
    candidates in parallel"; [P2] part 1, paper Sec. 3.2).
    E [V, e] (any float array or a callable mapping ids to rows), ids [...],
    P_e [r, e] -> b [..., r]."""
    rows = E(ids) if callable(E) else np.asarray(E)[ids]
    b = layer_norm(np.asarray(rows, dtype=np.float64) @ np.asarray(P_e).T, eps)
    return round_bf16(b) if bf16 else b


def fuse(b: np.ndarray, g: np.ndarray, W_f: np.ndarray, bf16: bool) -> np.ndarray:
    """z_{i,k} = f(b_{i,k}, g_i) = W_f [b_{i,k}; g_i]: concatenate the
    candidate part and the slot part and fuse them ([P1] "Score neighboring
    candidates in parallel"; [P2] part 1, paper Sec. 3.2).
    b [N, B, K, r], g [N, B, r], W_f [r_z, 2r] -> z [N, B, K, r_z]."""
    b = np.asarray(b, np.float64)
    g = np.asarray(g, np.float64)
    gb = np.broadcast_to(g[:, :, None, :], b.shape)
    cat = np.concatenate([b, gb], axis=-1)
    z = cat @ np.asarray(W_f, np.float64).T
    return round_bf16(z) if bf16 else z


def pair_state(h: np.ndarray, W_pair: np.ndarray) -> np.ndarray:
    """s_p = W_pair [h_p; h_{p+1}] for p = 1..B-1: one state per pair of
    neighbouring slots, shared by all K^2 transitions between them ([P1]
    "Score neighboring candidates in parallel"; [P2] part 1, paper Sec. 3.2).
    h [N, B, d], W_pair [r_s, 2d] -> s [N, B-1, r_s]."""
    h = np.asarray(h, np.float64)
    cat = np.concatenate([h[:, :-1, :], h[:, 1:, :]], axis=-1)
    return cat @ np.asarray(W_pair, np.float64).T


def silu(u: np.ndarray) -> np.ndarray:
    """SiLU(u) = u / (1 + exp(-u))."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def transition_scores(z: np.ndarray, s: np.ndarray, cand_vals: np.ndarray,
                      W1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: float) -> np.ndarray:
    """S_p(a, b) = l_{p+1}(b) + Delta_theta(z_{p,a}, z_{p+1,b}, s_p) for every
    pair of neighbouring slots and every candidate pair (a, b) ([P1] "Score
    neighboring candidates in parallel": the first term is the later slot's
    draft logit, the second the learned correction; [P2] part 1, paper
    Sec. 3.2: Delta_theta is one shared two-layer MLP and all (B-1)K^2 scores
    are formed before any selection).

    Delta_theta(x) = w2 . SiLU(W1 x + b1) + b2 with x = [z_{p,a}; z_{p+1,b}; s_p].
    z [N, B, K, r_z], s [N, B-1, r_s], cand_vals [N, B, K] -> S [N, B-1, K, K]
    (float64, unnormalised).
    """
    z = np.asarray(z, np.float64)
    s = np.asarray(s, np.float64)
    W1 = np.asarray(W1, np.float64)
    b1 = np.asarray(b1, np.float64)
    w2 = np.asarray(w2, np.float64)
    N, B, K, rz = z.shape
    S = np.empty((N, max(B - 1, 0), K, K), np.float64)
    for n in range(N):
        for p in range(B - 1):
            za = np.broadcast_to(z[n, p][:, None, :], (K, K, rz))      # predecessor a
            zb = np.broadcast_to(z[n, p + 1][None, :, :], (K, K, rz))  # successor b
            sp = np.broadcast_to(s[n, p][None, None, :], (K, K, s.shape[-1]))
            x = np.concatenate([za, zb, sp], axis=-1)
            delta = silu(x @ W1.T + b1) @ w2 + b2
            S[n, p] = cand_vals[n, p + 1][None, :] + delta
    return S


# ------------------------------------------------------------------- walk ---

def _argmax_lowest(row) -> int:
    """Index of the largest entry; the lowest index among equal maxima; NaN
    never wins; 0 when every entry is NaN."""
    best = -1
    best_v = 0.0
    for j, v in enumerate(row):
        v = float(v)
        if math.isnan(v):
            continue
        if best < 0 or v > best_v:
            best, best_v = j, v
    return max(best, 0)


def greedy_walk(S: np.ndarray, cand_vals: np.ndarray, cand_ids: np.ndarray):
    """Prefix-first greedy selection ([P1] "Select using the realized token
    identities"; [P2] part 2, paper Sec. 3.3): the first slot keeps the
    drafter's own first choice, k_1 = argmax_k l_1(k); every later slot takes
    the successor with the highest score given the candidate actually chosen
    just before it, k_{p+1} = argmax_b S_p(k_p, b); the proposed token is
    y_p = c_{p, k_p}.  No look-ahead.

    S [N, B-1, K, K], cand_vals [N, B, K], cand_ids [N, B, K] ->
    sel_idx [N, B], sel_tok [N, B] (int64) and the number of score/logit
    entries read per block (K + (B-1) K: the walk is O(BK)).
    """
    N, B, K = cand_vals.shape
    sel_idx = np.zeros((N, B), np.int64)
    sel_tok = np.zeros((N, B), np.int64)
    reads = np.zeros(N, np.int64)
    for n in range(N):
        k = _argmax_lowest(cand_vals[n, 0])
        reads[n] += K
        sel_idx[n, 0] = k
        for p in range(B - 1):
            row = S[n, p, k]
            reads[n] += len(row)
            k = _argmax_lowest(row)
            sel_idx[n, p + 1] = k
        sel_tok[n] = cand_ids[n, np.arange(B), sel_idx[n]]
    return sel_idx, sel_tok, reads


# ---------------------------------------------------- drafter LM head ---

def lm_head_logits(hd: np.ndarray, W_lm: np.ndarray, dtype: str, rows=None, v_chunk: int = 16384) -> np.ndarray:
    """The drafter's logits from its LM head: l_i(v) = W_lm[v] . hd_i, stored
    as the drafter stores logits (rounded to bf16 in the bf16 contract).

    hd [R, d], W_lm [V, d] (stored values) -> [R or len(rows), V] float64.
    The vocabulary is processed in chunks only to bound memory; each logit is
    one plain dot product.
    """
    h = to_f64(hd if rows is None else hd[np.asarray(rows)], dtype)
    V = W_lm.shape[0]
    logits = np.empty((h.shape[0], V), np.float64)
    for v0 in range(0, V, v_chunk):
        v1 = min(V, v0 + v_chunk)
        logits[:, v0:v1] = h @ to_f64(W_lm[v0:v1], dtype).T
    if dtype == "bf16":
        logits = round_bf16(logits)
    return logits


def lm_head_topk(hd: np.ndarray, W_lm: np.ndarray, K: int, dtype: str, rows=None, v_chunk: int = 16384):
    """The drafter's candidates straight from its LM head ([P1] "Keep the
    leading candidates"): top_k of lm_head_logits.  -> ids, vals."""
    return top_k(lm_head_logits(hd, W_lm, dtype, rows, v_chunk), K)


# ------------------------------------------------------------ training ---

def corrector_loss(S: np.ndarray, cand_ids: np.ndarray, target_tok: np.ndarray, rho: float) -> dict:
    """The corrector's training loss and its gradient with respect to the
    scores ([P1] "How we train the corrector"; [P2] part 3, paper Sec. 3.2
    and App. A).  The label of pair p is the pair of target tokens of slots
    p and p+1, (a*_p, b*_p) = their positions in the two slots' candidate
    lists; m_p = 1 only when both are present.  Each active pair contributes
    the cross-entropy of a softmax taken jointly over its K^2 scores, weighted
    by an exponential decay over the pair's position.  The pages lose the
    formula; the reading taken:

        L = (1/N) sum_n sum_{p=1..B-1} m_{n,p} exp(-(p-1)/rho) CE_{n,p},
        CE = log sum_{a,b} exp(S_p(a, b)) - S_p(a*, b*),

    and dL/dS_p(a, b) = (1/N) m w_p (softmax(S_p)(a, b) - [(a, b) = (a*, b*)]).

    S [N, B-1, K, K], cand_ids [N, B, K], target_tok [N, B] -> dict with
    loss (float), pair_loss [N, B-1] (m w CE / N), mask, a_star, b_star
    [N, B-1] (-1 where absent) and dS [N, B-1, K, K] (float64).
    """
    S = np.asarray(S, np.float64)
    N, Bm1, K, _ = S.shape
    pos = np.full((N, Bm1 + 1), -1, np.int64)
    for n in range(N):
        for i in range(Bm1 + 1):
            hit = np.nonzero(np.asarray(cand_ids[n, i]) == target_tok[n, i])[0]
            if len(hit):
                pos[n, i] = hit[0]
    a_star, b_star = pos[:, :-1], pos[:, 1:]
    mask = (a_star >= 0) & (b_star >= 0)
    w = np.exp(-np.arange(Bm1, dtype=np.float64) / rho)
    pair_loss = np.zeros((N, Bm1))
    dS = np.zeros_like(S)
    for n in range(N):
        for p in range(Bm1):
            if not mask[n, p]:
                continue
            flat = S[n, p].reshape(-1)
            top = flat.max()
            e = np.exp(flat - top)
            lse = top + np.log(e.sum())
            label = a_star[n, p] * K + b_star[n, p]
            coef = w[p] / N
            pair_loss[n, p] = coef * (lse - flat[label])
            g = e / e.sum()
            g[label] -= 1.0
            dS[n, p] = (coef * g).reshape(K, K)
    return {"loss": float(pair_loss.sum()), "pair_loss": pair_loss, "mask": mask,
            "a_star": np.where(mask, a_star, -1), "b_star": np.where(mask, b_star, -1), "dS": dS}


def score_backward(z: np.ndarray, s: np.ndarray, W1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
                   dS: np.ndarray) -> dict:
    """Gradients of a loss through the transition scores, given G = dL/dS
    (the backward of transition_scores; [P2] part 1, paper Sec. 3.2: one
    shared MLP over x = [z_{p,a}; z_{p+1,b}; s_p]).  With u = W1 x + b1:

        dL/dw2 = sum G SiLU(u),  dL/db2 = sum G,
        dL/du = G w2 SiLU'(u),   SiLU'(u) = sig(u) (1 + u (1 - sig(u))),
        dL/dW1 = sum dL/du x^T,  dL/db1 = sum dL/du,  dL/dx = W1^T dL/du,

    dL/dx split back into its three parts and added into dz_{p,a},
    dz_{p+1,b} and ds_p; the draft logit term gives dL/dl_{p+1}(b) =
    sum_a G(a, b).  Sums run over every pair and candidate pair.  The bf16
    rounding of z in the forward pass is taken as the identity.

    z [N, B, K, r_z], s [N, B-1, r_s], dS [N, B-1, K, K] -> dict of float64
    dz, ds, dW1, db1, dw2, db2, d_cand_vals.
    """
    z = np.asarray(z, np.float64)
    s = np.asarray(s, np.float64)
    W1 = np.asarray(W1, np.float64)
    b1 = np.asarray(b1, np.float64)
    w2 = np.asarray(w2, np.float64)
    G = np.asarray(dS, np.float64)
    N, B, K, rz = z.shape
    rs = s.shape[-1]
    out = {"dz": np.zeros_like(z), "ds": np.zeros((N, max(B - 1, 0), rs)), "dW1": np.zeros_like(W1),
           "db1": np.zeros_like(b1), "dw2": np.zeros_like(w2), "db2": 0.0,
           "d_cand_vals": np.zeros((N, B, K))}
    for n in range(N):
        for p in range(B - 1):
            za = np.broadcast_to(z[n, p][:, None, :], (K, K, rz))
            zb = np.broadcast_to(z[n, p + 1][None, :, :], (K, K, rz))
            sp = np.broadcast_to(s[n, p][None, None, :], (K, K, rs))
            x = np.concatenate([za, zb, sp], axis=-1).reshape(K * K, -1)
            u = x @ W1.T + b1
            with np.errstate(over="ignore"):
                sig = 1.0 / (1.0 + np.exp(-u))
            g = G[n, p].reshape(K * K)
            out["dw2"] += (g[:, None] * (u * sig)).sum(axis=0)
            out["db2"] += g.sum()
            du = g[:, None] * w2[None, :] * sig * (1.0 + u * (1.0 - sig))
            out["dW1"] += du.T @ x
            out["db1"] += du.sum(axis=0)
            dx = (du @ W1).reshape(K, K, -1)
            out["dz"][n, p] += dx[:, :, :rz].sum(axis=1)
            out["dz"][n, p + 1] += dx[:, :, rz:2 * rz].sum(axis=0)
            out["ds"][n, p] += dx[:, :, 2 * rz:].sum(axis=(0, 1))
            out["d_cand_vals"][n, p + 1] += G[n, p].sum(axis=0)
    return out


def represent_backward(h: np.ndarray, E_rows: np.ndarray, P_e: np.ndarray, P_h: np.ndarray, W_f: np.ndarray,
                       W_pair: np.ndarray, dz: np.ndarray, ds: np.ndarray, eps: float, bf16: bool) -> dict:
    """Gradients of a loss through the representations, given dL/dz and
    dL/ds (the backward of slot_context, candidate_embedding, fuse and
    pair_state; [P2] part 1, paper Sec. 3.2).  Step by step, in the forward's
    notation:

        z = W_f [b; g]        dW_f = sum dz [b; g]^T,  db = W_fb^T dz,
                              dg_i = W_fg^T sum_k dz_{i,k}
        b = LN(x_e), g = LN(x_h), y = LN(x) with sigma = sqrt(var + eps):
                              dx = (dy - mean(dy) - y mean(dy y)) / sigma
        x_e = P_e E[c]        dP_e = sum dx_e E[c]^T
        x_h = P_h h           dP_h = sum dx_h h^T,  dh += P_h^T dx_h
        s_p = W_pair [h_p; h_{p+1}]
                              dW_pair = sum ds_p [h_p; h_{p+1}]^T,
                              dh_p += W_L^T ds_p,  dh_{p+1} += W_R^T ds_p

    The bf16 roundings of b and g count as the identity; dW_f takes the
    rounded b and g the forward multiplied by.  E is frozen (no gradient).
    h [N, B, d], E_rows [N, B, K, e] (the gathered rows), dz [N, B, K, r_z],
    ds [N, B-1, r_s] -> dict of float64 dP_e, dP_h, dW_f, dW_pair, dh.
    """
    h = np.asarray(h, np.float64)
    Er = np.asarray(E_rows, np.float64)
    P_e = np.asarray(P_e, np.float64)
    P_h = np.asarray(P_h, np.float64)
    W_f = np.asarray(W_f, np.float64)
    W_pair = np.asarray(W_pair, np.float64)
    dz = np.asarray(dz, np.float64)
    ds = np.asarray(ds, np.float64)
    N, B, K, e = Er.shape
    d = h.shape[-1]
    r = P_e.shape[0]

    def ln_fwd(x):
        mu = x.mean(axis=-1, keepdims=True)
        sig = np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
        return (x - mu) / sig, sig

    def ln_bwd(dy, y, sig):
        return (dy - dy.mean(axis=-1, keepdims=True) - y * (dy * y).mean(axis=-1, keepdims=True)) / sig

    x_e = Er @ P_e.T                              # [N, B, K, r]
    y_e, sig_e = ln_fwd(x_e)
    x_h = h @ P_h.T                               # [N, B, r]
    y_h, sig_h = ln_fwd(x_h)
    b = round_bf16(y_e) if bf16 else y_e
    g = round_bf16(y_h) if bf16 else y_h
    W_fb, W_fg = W_f[:, :r], W_f[:, r:]
    dzs = dz.sum(axis=2)                          # [N, B, r_z]
    dW_f = np.concatenate([np.einsum("nbkz,nbkr->zr", dz, b), np.einsum("nbz,nbr->zr", dzs, g)], axis=1)
    db = dz @ W_fb                                # [N, B, K, r]
    dg = dzs @ W_fg                               # [N, B, r]
    dx_e = ln_bwd(db, y_e, sig_e)
    dx_h = ln_bwd(dg, y_h, sig_h)
    dP_e = np.einsum("nbkr,nbke->re", dx_e, Er)
    dP_h = np.einsum("nbr,nbd->rd", dx_h, h)
    dh = dx_h @ P_h
    W_L, W_R = W_pair[:, :d], W_pair[:, d:]
    dW_pair = np.concatenate([np.einsum("nps,npd->sd", ds, h[:, :-1]), np.einsum("nps,npd->sd", ds, h[:, 1:])],
                             axis=1)
    dh[:, :-1] += ds @ W_L
    dh[:, 1:] += ds @ W_R
    return {"dP_e": dP_e, "dP_h": dP_h, "dW_f": dW_f, "dW_pair": dW_pair, "dh": dh}


# ---------------------------------------------------- whole-path rules ---

def best_path(S: np.ndarray, cand_vals: np.ndarray, cand_ids: np.ndarray, lam: float):
    """The two whole-path rules the P2 review compares with the greedy walk on
    the same score grid ([P2] section "Path selection and ablation", paper
    Sec. 4.3 and Tab. 3; the objective is the one [P2] part 2 sets the greedy
    rule against): choose the candidate path k_1..k_B that maximises the
    weighted total score

        J(k) = sum_{j=1..B} lam^(j-1) * sigma_j,
        sigma_1 = l_1(k_1),   sigma_j = S_{j-1}(k_{j-1}, k_j)  (j >= 2).

    lam = 1 is Global-Sum (the plain total); 0 < lam < 1 is the geometric
    discount (the pages evaluate lam = 0.75).  The first slot is free, as a
    total over the path implies.  A NaN term counts as -inf; among paths of
    equal J the lexicographically smallest (k_1, ..., k_B) wins.

    The maximum over all K^B paths is taken by dynamic programming over the
    chain: V_B = 0 and, from the back, V_j(a) = max_b [lam^j S_j(a,b) +
    V_{j+1}(b)] is the best weighted score of the slots after j given
    k_j = a.  Then k_1 = argmax_a [l_1(a) + V_1(a)] and k_{j+1} = argmax_b
    [lam^j S_j(k_j, b) + V_{j+1}(b)], each the lowest index among maxima,
    which walks the lexicographically smallest optimal path.

    S [N, B-1, K, K], cand_vals [N, B, K], cand_ids [N, B, K] ->
    sel_idx [N, B], sel_tok [N, B] (int64) and J of the chosen path [N].
    """
    if not lam > 0:
        raise ValueError("lam must be positive")
    N, B, K = cand_vals.shape
    w = float(lam) ** np.arange(B, dtype=np.float64)     # weight of slot j (0-based)
    sel_idx = np.zeros((N, B), np.int64)
    sel_tok = np.zeros((N, B), np.int64)
    best = np.zeros(N)

    def no_nan(x):
        return np.where(np.isnan(x), -np.inf, x)

    for n in range(N):
        V = [None] * B
        V[B - 1] = np.zeros(K)
        for p in range(B - 2, -1, -1):        # pair p joins slots p and p+1
            V[p] = no_nan(w[p + 1] * S[n, p].astype(np.float64) + V[p + 1][None, :]).max(axis=1)
        first = no_nan(w[0] * cand_vals[n, 0].astype(np.float64) + V[0])
        k = int(np.argmax(first))            # first occurrence: the lowest index
        best[n] = first[k]
        sel_idx[n, 0] = k
        for p in range(B - 1):
            row = no_nan(w[p + 1] * S[n, p, k].astype(np.float64) + V[p + 1])
            k = int(np.argmax(row))
            sel_idx[n, p + 1] = k
        sel_tok[n] = cand_ids[n, np.arange(B), sel_idx[n]]
    return sel_idx, sel_tok, best


# ------------------------------------------------------------- the block ---

def correct_block(inp: dict, blocks=None) -> dict:
    """Run the whole hot path on stored inputs (the dict ``synth.make_inputs``
    returns: arrays of bf16 bits or float32 plus "dims").

    ``blocks`` optionally selects a subset of the N blocks (streams); blocks
    are independent, so a subset gives exactly those blocks' results.
    Returns every intermediate (float64) and the selection.
    """
    D = inp["dims"]
    dt = D.dtype
    bf = dt == "bf16"
    blocks = np.arange(D.n_blocks) if blocks is None else np.asarray(blocks)
    Nsel = len(blocks)
    logits = inp["logits"][blocks]
    h = to_f64(inp["h"][blocks], dt)
    E_store = inp["E"]

    def E_rows(ids):
        return to_f64(E_store[ids], dt)

    P_e = to_f64(inp["P_e"], dt)
    P_h = to_f64(inp["P_h"], dt)
    W_f = to_f64(inp["W_f"], dt)
    W_pair = to_f64(inp["W_pair"], dt)
    W1 = to_f64(inp["W1"], dt)
    b1 = to_f64(inp["b1"], dt)
    w2 = to_f64(inp["w2"], dt)
    b2 = float(inp["b2"])

    lg = to_f64(logits.reshape(Nsel * D.B, D.V), dt)
    ids, vals = top_k(lg, D.K)
    ids = ids.reshape(Nsel, D.B, D.K)
    vals = vals.reshape(Nsel, D.B, D.K)
    g = slot_context(h, P_h, D.ln_eps, bf)
    b = candidate_embedding(E_rows, ids, P_e, D.ln_eps, bf)
    z = fuse(b, g, W_f, bf)
    s = pair_state(h, W_pair)
    S = transition_scores(z, s, vals, W1, b1, w2, b2)
    sel_idx, sel_tok, reads = greedy_walk(S, vals, ids)
    return {"cand_ids": ids, "cand_vals": vals, "g": g, "b": b, "z": z, "s": s,
            "S": S, "sel_idx": sel_idx, "sel_tok": sel_tok, "reads": reads,
            "blocks": blocks}
