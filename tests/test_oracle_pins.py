"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every oracle function is checked here against something other than itself:
the pages' worked example, the special cases the pages state (a zeroed MLP
output layer reproduces the drafter), closed forms, invariants, algebraic
identities computed another way, brute force on tiny inputs, and library
routines the oracle does not call.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import dcoco_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_conversion():
    # torch's float32 -> bfloat16 cast rounds to nearest, ties to even.
    g = _rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 3,
        (g.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        g.standard_normal(2000).astype(np.float32) * 1e30,
        np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38, 1e-45], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_round_bf16_ties_and_overflow():
    one = 1.0
    assert O.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0                 # tie -> even
    assert O.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == one + 2 ** -6   # tie -> even
    assert O.round_bf16(np.array([one + 2 ** -8 + 2 ** -30]))[0] == one + 2 ** -7
    assert O.round_bf16(np.array([2.0 ** 128]))[0] == math.inf
    assert O.round_bf16(np.array([-(2.0 - 2 ** -9) * 2.0 ** 127]))[0] == -math.inf
    assert O.round_bf16(np.array([2.0 ** -134]))[0] == 0.0                   # tie -> even (0)
    assert O.round_bf16(np.array([3 * 2.0 ** -134]))[0] == 2 * 2.0 ** -133


# ------------------------------------------------------------------ top-K

def _brute_topk(row, K):
    """K rounds of a plain scan: take the largest remaining value, NaN only
    after every number, the lowest id among equals."""
    taken = set()
    out = []
    for _ in range(K):
        best = None
        for j, v in enumerate(row):
            if j in taken:
                continue
            if best is None:
                best = j
                continue
            bv = row[best]
            if math.isnan(bv) and not math.isnan(v):
                best = j
            elif not math.isnan(v) and not math.isnan(bv) and v > bv:
                best = j
        taken.add(best)
        out.append(best)
    return out


def test_topk_brute_force_tie_heavy_rows():
    g = _rng(2)
    rows = []
    for t in range(60):
        V = int(g.integers(5, 40))
        kind = t % 6
        if kind == 0:
            row = np.full(V, 1.5)
        elif kind == 1:
            row = g.choice([-1.0, 0.0, 2.0, 2.5], size=V)
        elif kind == 2:
            row = g.choice([0.0, -0.0, 1.0, -np.inf], size=V)
        elif kind == 3:
            row = g.standard_normal(V)
            row[g.integers(0, V, 3)] = np.nan
        elif kind == 4:
            row = g.choice([np.inf, -np.inf, np.nan, 0.0], size=V)
        else:
            row = np.round(g.standard_normal(V) * 2) / 2
        rows.append(row)
    for row in rows:
        for K in sorted({1, 2, min(5, len(row)), len(row)}):
            ids, vals = O.top_k(row[None, :], K)
            assert list(ids[0]) == _brute_topk(list(row), K)
            np.testing.assert_array_equal(vals[0], row[ids[0]])


def test_topk_planted_peaks_closed_form():
    # The generator plants P distinct peaks far above the background, so the
    # top-P of every row is the planted ids ordered by planted value.
    for name in ["small_bf16", "k64_small"]:
        cfg = synth.get_config(name)
        inp = synth.make_inputs(cfg, with_E=False)
        D = inp["dims"]
        lg = O.to_f64(inp["logits"].reshape(-1, D.V), D.dtype)
        ids, vals = O.top_k(lg, cfg.n_peaks)
        for n in range(D.n_blocks):
            pid, pv = synth.planted_peaks(cfg, n)
            np.testing.assert_array_equal(ids.reshape(D.n_blocks, D.B, -1)[n], pid)
            np.testing.assert_array_equal(vals.reshape(D.n_blocks, D.B, -1)[n], pv)


# -------------------------------------------------------------- LayerNorm

def test_layer_norm_invariants():
    g = _rng(3)
    x = g.standard_normal((50, 64)) * 7 + 3
    eps = 1e-5
    y = O.layer_norm(x, eps)
    v = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose((y ** 2).mean(axis=1), v / (v + eps), rtol=1e-12)


def test_layer_norm_closed_form():
    # x = (a+t, a-t): mean a, biased variance t^2, so LN = (+-t)/sqrt(t^2+eps)
    for a, t, eps in [(3.0, 2.0, 1e-5), (-1.0, 1e-3, 1e-5), (0.0, 5.0, 0.5)]:
        y = O.layer_norm(np.array([[a + t, a - t]]), eps)
        ref = t / math.sqrt(t * t + eps)
        np.testing.assert_allclose(y[0], [ref, -ref], rtol=1e-10)


def test_layer_norm_scale_gap():
    # Hidden states sit two orders of magnitude above embeddings; the
    # non-affine LN removes the scale: LN(c x) = LN(x) up to the eps term,
    # exactly LN_{eps/c^2}(x).
    g = _rng(4)
    x = g.standard_normal((8, 256)) * 0.02
    c = 30.0 / 0.02
    np.testing.assert_allclose(O.layer_norm(c * x, 1e-5), O.layer_norm(x, 1e-5 / c ** 2),
                               rtol=1e-12, atol=1e-12)


# -------------------------------------------------------- representations

def _sel_matrix(rows, cols, perm):
    M = np.zeros((rows, cols))
    M[np.arange(rows), perm[:rows]] = 1.0
    return M


def test_slot_context_projection_selects():
    g = _rng(5)
    d, r = 48, 16
    perm = g.permutation(d)
    P_h = _sel_matrix(r, d, perm)
    h = g.standard_normal((2, 3, d)) * 30
    got = O.slot_context(h, P_h, 1e-5, bf16=False)
    sel = h[..., perm[:r]]
    mu = sel.mean(-1, keepdims=True)
    var = ((sel - mu) ** 2).mean(-1, keepdims=True)
    np.testing.assert_allclose(got, (sel - mu) / np.sqrt(var + 1e-5), rtol=1e-12)
    # bf16 mode rounds the result
    gb = O.slot_context(h, P_h, 1e-5, bf16=True)
    ref = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.max(np.abs(gb - got)) <= 2 ** -8 * np.max(np.abs(got))
    # values that are exact in float32 round identically through torch
    np.testing.assert_array_equal(O.round_bf16(got.astype(np.float32).astype(np.float64)), ref)


def test_candidate_embedding_gathers_the_right_rows():
    V, e, r = 50, 24, 8
    E = np.arange(V)[:, None] * 1.0 + np.arange(e)[None, :] * np.arange(V)[:, None] * 0.01
    perm = _rng(6).permutation(e)
    P_e = _sel_matrix(r, e, perm)
    ids = np.array([[[3, 17, 42], [0, 49, 8]]])
    got = O.candidate_embedding(E, ids, P_e, 1e-5, bf16=False)
    for idx in np.ndindex(ids.shape):
        v = ids[idx]
        pre = v + perm[:r] * v * 0.01
        mu = pre.mean()
        ref = (pre - mu) / math.sqrt(((pre - mu) ** 2).mean() + 1e-5)
        np.testing.assert_allclose(got[idx], ref, rtol=1e-12, atol=1e-15)


def test_fuse_concatenation_order():
    g = _rng(7)
    N, B, K, r = 2, 3, 4, 5
    b = g.standard_normal((N, B, K, r))
    gg = g.standard_normal((N, B, r))
    I = np.eye(r)
    Z = np.zeros((r, r))
    np.testing.assert_array_equal(O.fuse(b, gg, np.hstack([I, Z]), False), b)
    np.testing.assert_array_equal(O.fuse(b, gg, np.hstack([Z, I]), False),
                                  np.broadcast_to(gg[:, :, None, :], b.shape))
    # a permutation of the concatenation, wider output: z_j = [b; g]_{perm[j]}
    perm = g.permutation(2 * r)
    Wp = _sel_matrix(2 * r, 2 * r, perm)
    cat = np.concatenate([b, np.broadcast_to(gg[:, :, None, :], b.shape)], -1)
    np.testing.assert_array_equal(O.fuse(b, gg, Wp, False), cat[..., perm])


def test_pair_state_neighbours():
    g = _rng(8)
    N, B, d = 2, 5, 6
    h = g.standard_normal((N, B, d))
    I = np.eye(d)
    Z = np.zeros((d, d))
    np.testing.assert_array_equal(O.pair_state(h, np.hstack([I, Z])), h[:, :-1])
    np.testing.assert_array_equal(O.pair_state(h, np.hstack([Z, I])), h[:, 1:])
    W = g.standard_normal((3, 2 * d))
    np.testing.assert_allclose(O.pair_state(h, W),
                               h[:, :-1] @ W[:, :d].T + h[:, 1:] @ W[:, d:].T, rtol=1e-12)


# ------------------------------------------------------- transition scores

def _small_grid(seed, N=2, B=4, K=3, rz=5, rs=4, H=6):
    g = _rng(seed)
    z = g.standard_normal((N, B, K, rz))
    s = g.standard_normal((N, B - 1, rs)) * 3
    vals = g.standard_normal((N, B, K))
    W1 = g.standard_normal((H, 2 * rz + rs)) * 0.5
    b1 = g.standard_normal(H) * 0.1
    w2 = g.standard_normal(H)
    b2 = 0.37
    return z, s, vals, W1, b1, w2, b2


def test_zero_output_layer_reproduces_draft_logits():
    # Zero-initialised output layer: Delta = 0, so S_p(a, b) = l_{p+1}(b)
    # exactly, for every predecessor a.
    z, s, vals, W1, b1, w2, b2 = _small_grid(9)
    S = O.transition_scores(z, s, vals, W1, b1, np.zeros_like(w2), 0.0)
    N, Bm1, K, _ = S.shape
    for n in range(N):
        for p in range(Bm1):
            for a in range(K):
                np.testing.assert_array_equal(S[n, p, a], vals[n, p + 1])


def test_single_unit_mlp_closed_form():
    # H = 1, w2 = 1, b1 = b2 = 0 and W1 a one-hot selector: Delta is SiLU of
    # one chosen input coordinate.  SiLU via scipy's expit (not used by the oracle).
    z, s, vals, _, _, _, _ = _small_grid(10)
    rz, rs = z.shape[-1], s.shape[-1]
    N, B, K, _ = z.shape

    def ref_silu(u):
        return u * scipy.special.expit(u)

    for block, j in [("a", 2), ("b", 4), ("s", 1)]:
        W1 = np.zeros((1, 2 * rz + rs))
        col = {"a": j, "b": rz + j, "s": 2 * rz + j}[block]
        W1[0, col] = 1.0
        S = O.transition_scores(z, s, vals, W1, np.zeros(1), np.ones(1), 0.0)
        for n, p, a, b in itertools.product(range(N), range(B - 1), range(K), range(K)):
            if block == "a":
                u = z[n, p, a, j]
            elif block == "b":
                u = z[n, p + 1, b, j]
            else:
                u = s[n, p, j]
            assert S[n, p, a, b] == pytest.approx(vals[n, p + 1, b] + ref_silu(u), rel=1e-13, abs=1e-13)


def test_factored_mlp_identity():
    # W1 [z_a; z_b; s] = W1a z_a + W1b z_b + W1s s: compute Delta the factored
    # way and compare with the concatenated definition.
    z, s, vals, W1, b1, w2, b2 = _small_grid(11, N=2, B=5, K=4, rz=7, rs=3, H=9)
    rz = z.shape[-1]
    S = O.transition_scores(z, s, vals, W1, b1, w2, b2)
    A = z @ W1[:, :rz].T
    Bm = z @ W1[:, rz:2 * rz].T
    C = s @ W1[:, 2 * rz:].T + b1
    N, B, K, _ = z.shape
    for n in range(N):
        for p in range(B - 1):
            u = A[n, p][:, None, :] + Bm[n, p + 1][None, :, :] + C[n, p][None, None, :]
            d = (u * scipy.special.expit(u)) @ w2 + b2
            np.testing.assert_allclose(S[n, p], vals[n, p + 1][None, :] + d, rtol=1e-12, atol=1e-12)


def test_predecessor_blind_rows_equal():
    z, s, vals, W1, b1, w2, b2 = _small_grid(12)
    rz = z.shape[-1]
    W1 = W1.copy()
    W1[:, :rz] = 0.0
    S = O.transition_scores(z, s, vals, W1, b1, w2, b2)
    for a in range(1, S.shape[2]):
        np.testing.assert_array_equal(S[:, :, a, :], S[:, :, 0, :])


def test_zeroed_candidate_states_follow_drafter():
    # '-cand state' ablation: z = 0 makes Delta independent of (a, b), so the
    # walk returns each slot's own top candidate.
    z, s, vals, W1, b1, w2, b2 = _small_grid(13)
    S = O.transition_scores(np.zeros_like(z), s, vals, W1, b1, w2, b2)
    ids = np.arange(vals.size).reshape(vals.shape)
    sel, _, _ = O.greedy_walk(S, vals, ids)
    np.testing.assert_array_equal(sel, vals.argmax(axis=-1))


# ------------------------------------------------------------------- walk

def _lex_best(S, vals):
    """Brute force over all K^(B-1) continuations: the path whose sequence
    (S_1(k1,k2), -k2, S_2(k2,k3), -k3, ...) is lexicographically largest, with
    k1 the drafter's first choice."""
    Bm1, K, _ = S.shape
    k1 = int(np.argmax(vals[0]))
    best, best_key = None, None
    for rest in itertools.product(range(K), repeat=Bm1):
        path = (k1,) + rest
        key = []
        for p in range(Bm1):
            key += [S[p, path[p], path[p + 1]], -path[p + 1]]
        if best_key is None or key > best_key:
            best, best_key = path, key
    return list(best)


def test_walk_brute_force_lexicographic():
    g = _rng(14)
    for t in range(200):
        B = int(g.integers(2, 6))
        K = int(g.integers(1, 5))
        S = np.round(g.standard_normal((1, B - 1, K, K)) * 2) / 2   # many ties
        vals = np.sort(g.standard_normal((1, B, K)))[..., ::-1].copy()
        ids = g.integers(0, 1000, (1, B, K))
        sel, tok, reads = O.greedy_walk(S, vals, ids)
        assert list(sel[0]) == _lex_best(S[0], vals[0])
        np.testing.assert_array_equal(tok[0], ids[0, np.arange(B), sel[0]])
        assert reads[0] == K + (B - 1) * K


def test_walk_reads_only_the_realised_rows():
    # O(BK): poisoning every row except the one the walk reads changes nothing.
    g = _rng(15)
    N, B, K = 3, 6, 5
    S = g.standard_normal((N, B - 1, K, K))
    vals = np.sort(g.standard_normal((N, B, K)))[..., ::-1].copy()
    ids = g.integers(0, 100, (N, B, K))
    sel, tok, reads = O.greedy_walk(S, vals, ids)
    P = np.full_like(S, np.nan)
    for n in range(N):
        for p in range(B - 1):
            P[n, p, sel[n, p]] = S[n, p, sel[n, p]]
    sel2, tok2, _ = O.greedy_walk(P, vals, ids)
    np.testing.assert_array_equal(sel, sel2)
    np.testing.assert_array_equal(reads, K + (B - 1) * K)


def test_walk_nan_never_wins():
    S = np.array([[[[np.nan, 1.0, 1.0], [0, 0, 0], [0, 0, 0]],
                   [[np.nan, np.nan, np.nan], [0, 0, 0], [0, 0, 0]]]])
    vals = np.array([[[5.0, 4.0, 3.0], [0, 0, 0], [0, 0, 0]]])
    ids = np.arange(9).reshape(1, 3, 3)
    sel, _, _ = O.greedy_walk(S, vals, ids)
    # step 1 row [nan, 1, 1] -> 1 (lowest among maxima); step 2 row 1 = [0,0,0] -> 0
    assert list(sel[0]) == [0, 1, 0]
    S[0, 1, 1] = np.nan
    sel, _, _ = O.greedy_walk(S, vals, ids)
    assert list(sel[0]) == [0, 1, 0]     # all-NaN row -> index 0


def _worked():
    with open(os.path.join(GOLD, "worked_example.json")) as f:
        return json.load(f)


def _worked_S(logits, plants):
    ell = np.array(logits)
    B, K = ell.shape
    S = np.zeros((1, B - 1, K, K))
    for p in range(B - 1):
        S[0, p] = ell[p + 1][None, :]
    for p, a, b, v in plants:
        S[0, p, a, b] += v
    return S, ell[None]


def test_worked_example_walk():
    W = _worked()
    for name, rd in W["readings"].items():
        for case in rd["cases"]:
            S, vals = _worked_S(rd["logits"], case.get("plants", []))
            ids = np.arange(W["B"] * W["K"]).reshape(1, W["B"], W["K"])
            sel, tok, reads = O.greedy_walk(S, vals, ids)
            assert list(sel[0]) == case["path"], (name, case)
            words = [W["tokens"][p][k] for p, k in enumerate(sel[0])]
            assert " ".join(words) == case["text"]
            assert reads[0] == W["K"] + (W["B"] - 1) * W["K"]


def _worked_inputs(logits):
    """The worked example through the whole path: a 12-word vocabulary (word
    w of slot p, candidate j has id 3p + j), off-shortlist logits -10,
    zeroed MLP output layer, small random other weights."""
    W = _worked()
    B, K = W["B"], W["K"]
    V, d, e, r, H = 12, 32, 32, 32, 32
    g = _rng(16)
    lg = np.full((1, B, V), -10.0, np.float32)
    for p in range(B):
        for j in range(K):
            lg[0, p, 3 * p + j] = logits[p][j]
    D = synth.Dims(1, B, K, V, d, e, r, r, r, H, "f32")
    return {"dims": D, "logits": lg,
            "h": (g.standard_normal((1, B, d)) * 30).astype(np.float32),
            "E": (g.standard_normal((V, e)) * 0.02).astype(np.float32),
            "P_e": g.standard_normal((r, e)).astype(np.float32) * 0.1,
            "P_h": g.standard_normal((r, d)).astype(np.float32) * 0.1,
            "W_f": g.standard_normal((r, 2 * r)).astype(np.float32) * 0.1,
            "W_pair": g.standard_normal((r, 2 * d)).astype(np.float32) * 0.1,
            "W1": g.standard_normal((H, 3 * r)).astype(np.float32) * 0.1,
            "b1": np.zeros(H, np.float32), "w2": np.zeros(H, np.float32), "b2": 0.0}


def test_worked_example_end_to_end_zero_delta():
    W = _worked()
    for name in ["W-lit", "W-rank"]:
        rd = W["readings"][name]
        inp = _worked_inputs(rd["logits"])
        out = O.correct_block(inp)
        case = [c for c in rd["cases"] if c["delta"] == "zero"][0]
        words = []
        for p, tok in enumerate(out["sel_tok"][0]):
            words.append(W["tokens"][p][int(tok) - 3 * p])
        assert " ".join(words) == case["text"]


def test_tiny_zero_config_reproduces_drafter_argmax():
    inp = synth.make_inputs("tiny_zero")
    out = O.correct_block(inp)
    D = inp["dims"]
    lg = inp["logits"].astype(np.float64)
    np.testing.assert_array_equal(out["sel_idx"], 0)
    np.testing.assert_array_equal(out["sel_tok"], lg.argmax(axis=-1))
    for p in range(D.B - 1):
        for a in range(D.K):
            np.testing.assert_array_equal(out["S"][:, p, a, :], out["cand_vals"][:, p + 1, :])


# ------------------------------------------------------- whole-path rules

def _brute_best_path(S, vals, lam):
    """Every one of the K^B paths scored left to right; the first maximum in
    itertools.product order is the lexicographically smallest one."""
    B, K = vals.shape
    best, arg = None, None
    for path in itertools.product(range(K), repeat=B):
        terms = [vals[0, path[0]]] + [S[p, path[p], path[p + 1]] for p in range(B - 1)]
        J = 0.0
        for j, t in enumerate(terms):
            t = -math.inf if math.isnan(t) else float(t)
            J = J + lam ** j * t
        if math.isnan(J):
            J = -math.inf
        if best is None or J > best:
            best, arg = J, path
    return np.array(arg), best


@pytest.mark.parametrize("lam", [1.0, 0.75, 0.5])
def test_best_path_brute_force(lam):
    # small integers and dyadic weights: every total is exact in float64, so
    # ties are real ties and both orders of summation agree bit for bit
    g = _rng(31)
    for trial in range(60):
        B = int(g.integers(1, 6))
        K = int(g.integers(1, 5))
        vals = g.integers(-3, 4, size=(1, B, K)).astype(np.float64)
        S = g.integers(-3, 4, size=(1, max(B - 1, 0), K, K)).astype(np.float64)
        if trial % 5 == 0 and B > 1:
            S[0, 0, 0, :] = np.nan            # a NaN row
        if trial % 7 == 0 and B > 1:
            S[0, -1, :, 0] = -np.inf
        ids = g.integers(0, 1000, size=(1, B, K))
        sel, tok, J = O.best_path(S, vals, ids, lam)
        ref, Jref = _brute_best_path(S[0], vals[0], lam)
        assert sel[0].tolist() == ref.tolist(), (trial, B, K)
        assert J[0] == Jref
        assert tok[0].tolist() == ids[0, np.arange(B), ref].tolist()


def test_best_path_departs_from_greedy_by_hand():
    # l_1 = (1, 0); S_1 rows: from candidate 0 (0, 0), from candidate 1 (5, 4).
    # Greedy keeps k_1 = 0 and takes the lower of the tied successors: (0, 0).
    # Global-Sum: (1, 0) scores 0 + 5 = 5 against 1 + 0 = 1 for (0, 0).
    # Discount 0.75: (1, 0) scores 0 + 0.75*5 = 3.75 > 1.  Discount 0.1:
    # 0 + 0.1*5 = 0.5 < 1 + 0.1*0 = 1, so (0, 0) again.
    vals = np.array([[[1.0, 0.0], [0.0, 0.0]]])
    S = np.array([[[[0.0, 0.0], [5.0, 4.0]]]])
    ids = np.array([[[10, 11], [20, 21]]])
    gsel, _, _ = O.greedy_walk(S, vals, ids)
    assert gsel[0].tolist() == [0, 0]
    for lam, want, J in ((1.0, [1, 0], 5.0), (0.75, [1, 0], 3.75), (0.1, [0, 0], 1.0)):
        sel, tok, best = O.best_path(S, vals, ids, lam)
        assert sel[0].tolist() == want
        assert best[0] == pytest.approx(J, abs=1e-15)
        assert tok[0].tolist() == [ids[0, 0, want[0]], ids[0, 1, want[1]]]


def test_best_path_tiny_discount_is_greedy():
    # lam -> 0 orders paths lexicographically by (l_1(k_1), S_1(k_1, k_2), ...):
    # exactly the prefix-first greedy walk when no step has a near-tie
    g = _rng(32)
    N, B, K = 6, 9, 7
    vals = g.standard_normal((N, B, K))
    S = g.standard_normal((N, B - 1, K, K)) * 3
    ids = g.integers(0, 50000, size=(N, B, K))
    gsel, gtok, _ = O.greedy_walk(S, vals, ids)
    sel, tok, _ = O.best_path(S, vals, ids, 1e-9)
    assert np.array_equal(sel, gsel) and np.array_equal(tok, gtok)


@pytest.mark.parametrize("lam", [1.0, 0.75])
def test_best_path_zero_correction_is_drafter_argmax(lam):
    # with Delta = 0, S_p(a, b) = l_{p+1}(b): the weighted total splits into
    # independent per-slot terms, so the best path is each slot's own argmax
    g = _rng(33)
    N, B, K = 4, 6, 5
    vals = g.standard_normal((N, B, K))
    S = np.broadcast_to(vals[:, 1:, None, :], (N, B - 1, K, K)).copy()
    ids = g.integers(0, 50000, size=(N, B, K))
    sel, _, J = O.best_path(S, vals, ids, lam)
    assert np.array_equal(sel, vals.argmax(axis=2))
    w = lam ** np.arange(B)
    assert np.allclose(J, (vals.max(axis=2) * w).sum(axis=1), rtol=0, atol=1e-12)


# --------------------------------------------------------------- training

def _loss_case(seed, N=3, B=6, K=4, absent=True):
    g = _rng(seed)
    S = g.standard_normal((N, B - 1, K, K)) * 2
    ids = np.stack([np.stack([g.permutation(1000)[:K] for _ in range(B)]) for _ in range(N)])
    tgt = np.empty((N, B), np.int64)
    for n in range(N):
        for i in range(B):
            tgt[n, i] = ids[n, i, g.integers(0, K)]
    if absent:
        tgt[0, 2] = 5000                       # not among slot 2's candidates
    return S, ids, tgt


def test_loss_against_torch_cross_entropy():
    # torch's own cross-entropy and autograd, float64, as an independent route
    S, ids, tgt = _loss_case(51)
    rho = 4.0
    out = O.corrector_loss(S, ids, tgt, rho)
    N, Bm1, K, _ = S.shape
    St = torch.tensor(S, dtype=torch.float64, requires_grad=True)
    labels = torch.zeros((N, Bm1), dtype=torch.long)
    coef = torch.zeros((N, Bm1), dtype=torch.float64)
    for n in range(N):
        for p in range(Bm1):
            a = list(ids[n, p]).index(tgt[n, p]) if tgt[n, p] in ids[n, p] else None
            b = list(ids[n, p + 1]).index(tgt[n, p + 1]) if tgt[n, p + 1] in ids[n, p + 1] else None
            if a is not None and b is not None:
                labels[n, p] = a * K + b
                coef[n, p] = math.exp(-p / rho) / N
    ce = torch.nn.functional.cross_entropy(St.reshape(N * Bm1, K * K), labels.reshape(-1), reduction="none")
    L = (ce.reshape(N, Bm1) * coef).sum()
    L.backward()
    assert out["loss"] == pytest.approx(L.item(), rel=1e-13)
    np.testing.assert_allclose(out["dS"], St.grad.numpy(), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(out["mask"], (coef > 0).numpy())
    # slot 2 has no target among its candidates: pairs 1 and 2 are dropped
    assert not out["mask"][0, 1] and not out["mask"][0, 2]
    assert np.all(out["dS"][0, 1] == 0) and np.all(out["dS"][0, 2] == 0)


def test_loss_closed_forms():
    # equal scores: the joint softmax is uniform, CE = log K^2 for every pair
    N, B, K = 2, 4, 3
    ids = np.arange(N * B * K).reshape(N, B, K)
    tgt = ids[:, :, 1]
    out = O.corrector_loss(np.full((N, B - 1, K, K), 0.7), ids, tgt, 4.0)
    w = np.exp(-np.arange(B - 1) / 4.0)
    assert out["loss"] == pytest.approx(math.log(K * K) * w.sum(), rel=1e-14)
    # each active pair's gradient sums to zero (softmax minus a one-hot)
    S, ids, tgt = _loss_case(52)
    out = O.corrector_loss(S, ids, tgt, 4.0)
    np.testing.assert_allclose(out["dS"].sum(axis=(2, 3)), 0.0, atol=1e-15)
    # one candidate per slot: the softmax is certain, no loss and no gradient
    S1 = _rng(53).standard_normal((2, 3, 1, 1))
    ids1 = np.arange(8).reshape(2, 4, 1)
    out = O.corrector_loss(S1, ids1, ids1[:, :, 0], 4.0)
    assert out["loss"] == 0.0 and np.all(out["dS"] == 0)
    # a dominant label score: CE -> log(1 + (K^2 - 1) e^-D)
    S2 = np.zeros((1, 1, 2, 2))
    S2[0, 0, 1, 0] = 30.0
    ids2 = np.array([[[7, 8], [9, 10]]])
    out = O.corrector_loss(S2, ids2, np.array([[8, 9]]), 4.0)
    assert out["loss"] == pytest.approx(math.log1p(3 * math.exp(-30.0)), rel=1e-12)


def _bwd_case(seed):
    g = _rng(seed)
    N, B, K, rz, rs, H = 2, 3, 2, 3, 2, 4
    z = g.standard_normal((N, B, K, rz))
    s = g.standard_normal((N, B - 1, rs))
    W1 = g.standard_normal((H, 2 * rz + rs)) * 0.7
    b1 = g.standard_normal(H) * 0.3
    w2 = g.standard_normal(H)
    b2 = 0.2
    vals = g.standard_normal((N, B, K))
    G = g.standard_normal((N, B - 1, K, K))
    return z, s, W1, b1, w2, b2, vals, G


def test_score_backward_finite_differences():
    # f(theta) = sum G * S(theta) with the (separately pinned) forward; every
    # gradient entry against a central difference
    z, s, W1, b1, w2, b2, vals, G = _bwd_case(54)
    out = O.score_backward(z, s, W1, b1, w2, G)

    def f(z=z, s=s, W1=W1, b1=b1, w2=w2, b2=b2, vals=vals):
        return float((G * O.transition_scores(z, s, vals, W1, b1, w2, b2)).sum())

    eps = 1e-6
    for name, arr in (("dz", z), ("ds", s), ("dW1", W1), ("db1", b1), ("dw2", w2), ("d_cand_vals", vals)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hi, lo = arr.copy(), arr.copy()
            hi[idx] += eps
            lo[idx] -= eps
            key = {"dz": "z", "ds": "s", "dW1": "W1", "db1": "b1", "dw2": "w2", "d_cand_vals": "vals"}[name]
            num[idx] = (f(**{key: hi}) - f(**{key: lo})) / (2 * eps)
        np.testing.assert_allclose(out[name], num, rtol=1e-6, atol=1e-8, err_msg=name)
    num_b2 = (f(b2=b2 + eps) - f(b2=b2 - eps)) / (2 * eps)
    assert out["db2"] == pytest.approx(num_b2, rel=1e-8)


def test_score_backward_against_torch_autograd():
    # a larger case through torch's autograd (float64, torch's own SiLU)
    g = _rng(55)
    N, B, K, rz, rs, H = 2, 5, 4, 8, 6, 16
    z = g.standard_normal((N, B, K, rz))
    s = g.standard_normal((N, B - 1, rs)) * 3
    W1 = g.standard_normal((H, 2 * rz + rs)) * 0.4
    b1 = g.standard_normal(H) * 0.3
    w2 = g.standard_normal(H)
    G = g.standard_normal((N, B - 1, K, K))
    out = O.score_backward(z, s, W1, b1, w2, G)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(z=z, s=s, W1=W1, b1=b1, w2=w2).items()}
    b2 = torch.tensor(0.0, dtype=torch.float64, requires_grad=True)
    vals = torch.zeros((N, B, K), dtype=torch.float64, requires_grad=True)
    za = t["z"][:, :-1, :, None, :].expand(N, B - 1, K, K, rz)
    zb = t["z"][:, 1:, None, :, :].expand(N, B - 1, K, K, rz)
    sp = t["s"][:, :, None, None, :].expand(N, B - 1, K, K, rs)
    x = torch.cat([za, zb, sp], dim=-1)
    delta = torch.nn.functional.silu(x @ t["W1"].T + t["b1"]) @ t["w2"] + b2
    S = vals[:, 1:, None, :] + delta
    (torch.tensor(G) * S).sum().backward()
    for name, key in (("dz", "z"), ("ds", "s"), ("dW1", "W1"), ("db1", "b1"), ("dw2", "w2")):
        np.testing.assert_allclose(out[name], t[key].grad.numpy(), rtol=1e-12, atol=1e-12, err_msg=name)
    assert out["db2"] == pytest.approx(b2.grad.item(), rel=1e-12)
    np.testing.assert_allclose(out["d_cand_vals"], vals.grad.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------- drafter LM head

def test_lm_head_one_hot_rows_closed_form():
    # a head whose row v is c_v times a unit vector e_{j(v)}: the logit is
    # bf16(c_v * hd_i[j(v)]) element by element, so the head's orientation
    # (rows = vocabulary) and the bf16 rounding of the logits are both pinned
    g = _rng(71)
    R, d, V, K = 5, 24, 300, 9
    hd = synth.f32_to_bf16_bits(g.standard_normal((R, d)).astype(np.float32) * 3)
    j = g.integers(0, d, V)
    c = synth.f32_to_bf16_bits(g.standard_normal(V).astype(np.float32))
    W = np.zeros((V, d), np.uint16)
    W[np.arange(V), j] = c
    h = synth.bf16_bits_to_f32(hd).astype(np.float64)
    want = O.round_bf16(h[:, j] * synth.bf16_bits_to_f32(c).astype(np.float64)[None, :])
    np.testing.assert_array_equal(O.lm_head_logits(hd, W, "bf16"), want)
    ids, vals = O.lm_head_topk(hd, W, K, "bf16")
    rids, rvals = O.top_k(want, K)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(vals, rvals)
    # a head stored transposed would not even have the right shape here: V != d
    assert O.lm_head_logits(hd, W, "bf16").shape == (R, V)


def test_lm_head_chunking_and_row_subsets():
    g = _rng(72)
    R, d, V = 6, 32, 1001
    hd = synth.f32_to_bf16_bits(g.standard_normal((R, d)).astype(np.float32))
    W = synth.f32_to_bf16_bits(g.standard_normal((V, d)).astype(np.float32) * 0.3)
    full = O.lm_head_logits(hd, W, "bf16")
    np.testing.assert_array_equal(O.lm_head_logits(hd, W, "bf16", v_chunk=7), full)
    np.testing.assert_array_equal(O.lm_head_logits(hd, W, "bf16", rows=[4, 1]), full[[4, 1]])
    # rounding only in the bf16 contract: fp32 storage keeps the exact sums
    hf = synth.bf16_bits_to_f32(hd)
    Wf = synth.bf16_bits_to_f32(W)
    np.testing.assert_allclose(O.lm_head_logits(hf, Wf, "f32"), hf.astype(np.float64) @ Wf.T.astype(np.float64),
                               rtol=1e-15, atol=0)


def _rep_case(seed, N=2, B=3, K=2, d=6, e=5, r=4, rz=3, rs=3):
    g = _rng(seed)
    h = g.standard_normal((N, B, d)) * 2
    Er = g.standard_normal((N, B, K, e)) * 0.5
    P_e = g.standard_normal((r, e))
    P_h = g.standard_normal((r, d)) * 0.5
    W_f = g.standard_normal((rz, 2 * r))
    W_pair = g.standard_normal((rs, 2 * d))
    dz = g.standard_normal((N, B, K, rz))
    ds = g.standard_normal((N, B - 1, rs))
    return h, Er, P_e, P_h, W_f, W_pair, dz, ds


def test_represent_backward_finite_differences():
    # f = sum dz * z + sum ds * s through the (separately pinned) forward
    # functions in fp32 storage mode; every gradient entry against a central
    # difference
    h, Er, P_e, P_h, W_f, W_pair, dz, ds = _rep_case(81)
    eps = 1e-5
    out = O.represent_backward(h, Er, P_e, P_h, W_f, W_pair, dz, ds, eps, bf16=False)
    N, B, K, e = Er.shape
    ids = np.arange(N * B * K).reshape(N, B, K)
    Etab = Er.reshape(N * B * K, e)

    def f(h=h, P_e=P_e, P_h=P_h, W_f=W_f, W_pair=W_pair):
        b = O.candidate_embedding(Etab, ids, P_e, eps, bf16=False)
        g = O.slot_context(h, P_h, eps, bf16=False)
        z = O.fuse(b, g, W_f, bf16=False)
        s = O.pair_state(h, W_pair)
        return float((dz * z).sum() + (ds * s).sum())

    step = 1e-6
    for name, key, arr in (("dP_e", "P_e", P_e), ("dP_h", "P_h", P_h), ("dW_f", "W_f", W_f),
                           ("dW_pair", "W_pair", W_pair), ("dh", "h", h)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            hi, lo = arr.copy(), arr.copy()
            hi[idx] += step
            lo[idx] -= step
            num[idx] = (f(**{key: hi}) - f(**{key: lo})) / (2 * step)
        np.testing.assert_allclose(out[name], num, rtol=1e-5, atol=1e-7, err_msg=name)


def test_represent_backward_torch_autograd_straight_through():
    # bf16 mode: torch's own layer_norm and autograd, with each bf16 rounding
    # written as x + (round(x) - x).detach() (identity in the backward)
    h, Er, P_e, P_h, W_f, W_pair, dz, ds = _rep_case(82, N=2, B=4, K=3, d=16, e=12, r=8, rz=6, rs=5)
    eps = 1e-5
    out = O.represent_backward(h, Er, P_e, P_h, W_f, W_pair, dz, ds, eps, bf16=True)
    T = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
         for k, v in dict(h=h, P_e=P_e, P_h=P_h, W_f=W_f, W_pair=W_pair).items()}

    def rnd(x):
        q = x.detach().to(torch.float32).to(torch.bfloat16).to(torch.float64)
        return x + (q - x).detach()

    r = P_e.shape[0]
    d = h.shape[-1]
    Ert = torch.tensor(Er, dtype=torch.float64)
    b = rnd(torch.nn.functional.layer_norm(Ert @ T["P_e"].T, (r,), eps=eps))
    g = rnd(torch.nn.functional.layer_norm(T["h"] @ T["P_h"].T, (r,), eps=eps))
    z = torch.cat([b, g[:, :, None, :].expand_as(b)], dim=-1) @ T["W_f"].T
    s = torch.cat([T["h"][:, :-1], T["h"][:, 1:]], dim=-1) @ T["W_pair"].T
    ((torch.tensor(dz) * z).sum() + (torch.tensor(ds) * s).sum()).backward()
    for name, key in (("dP_e", "P_e"), ("dP_h", "P_h"), ("dW_f", "W_f"), ("dW_pair", "W_pair"), ("dh", "h")):
        np.testing.assert_allclose(out[name], T[key].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
    assert d > 0
