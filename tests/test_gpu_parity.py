"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: top-K ids and selected paths bit-exact; S within 3e-2 absolute on the
bf16 path and 1e-4 relative on the fp32 path; end-to-end tokens identical
wherever the oracle's best-vs-second margin exceeds 0.1.  Full-size shapes are
run in the same launch configuration the benchmark times and compared on
sampled blocks (blocks are independent).
"""
import functools
import json
import os

import numpy as np
import pytest

import synth
from helpers import (device_inputs, ensure_built, lockstep_path_check, s_tolerance_ok, to_dev,
                     PATH_MARGIN)
from oracle import dcoco_oracle as O

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    print(f"device: {torch.cuda.get_device_name(0)}", flush=True)


def _np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.cpu().numpy()


@functools.lru_cache(maxsize=4)
def _inputs(name, n_blocks=None):
    return synth.make_inputs(name, n_blocks=n_blocks)


@functools.lru_cache(maxsize=8)
def _oracle(name, blocks=None):
    inp = _inputs(name)
    return O.correct_block(inp, blocks=None if blocks is None else list(blocks))


SMALL = ["tiny", "tiny_zero", "tiny_bias", "small_bf16", "small_f32", "mid_bf16", "mid_f32",
         "k64_small", "k32_small", "widez_bf16", "tall_bf16", "b1_bf16", "k1_bf16", "wide_max",
         "chunks_bf16", "chunks_ragged", "chunks_five", "chunks_long"]


def _run_block(name):
    import draft_block_contextual_amd as dc
    import torch
    inp = _inputs(name)
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    return inp, {k: _np(v) for k, v in out.items()}


# ------------------------------------------------------------------ top-K

@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_f32", "mid_bf16", "k64_small", "k32_small"])
def test_topk_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case topk {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    dims = dc.Dims.from_synth(D)
    logits = to_dev(inp["logits"].reshape(-1, D.V), D.dtype)
    ids, vals = dc.topk(dims, logits)
    torch.cuda.synchronize()
    ref = _oracle(name)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["cand_ids"].reshape(-1, D.K))
    np.testing.assert_array_equal(vals.cpu().numpy().astype(np.float64), ref["cand_vals"].reshape(-1, D.K))


def _special_rows(V, dtype, seed):
    g = np.random.default_rng(seed)
    rows = [
        np.full(V, 1.5),                                    # all equal
        g.choice([-1.0, 0.0, 2.0, 2.5], size=V),            # few distinct values
        g.choice([0.0, -0.0, 1.0, -np.inf], size=V),        # signed zeros, -inf
        np.arange(V, dtype=np.float64) * (8.0 / V),         # ascending ramp
        np.arange(V, 0, -1, dtype=np.float64) * (8.0 / V),  # descending ramp
        np.round(g.standard_normal(V) * 2) / 2,             # many ties
        g.standard_normal(V),
    ]
    rows.append(g.standard_normal(V) - 20.0)                 # all negative (log-probability-like)
    rows.append(-np.abs(g.standard_normal(V)))               # non-positive, top keys near -0
    rows.append(np.where(g.random(V) < 0.002, 1.0, -1.0) * g.random(V))  # few positives
    r = g.standard_normal(V)
    r[g.integers(0, V, 40)] = np.nan
    rows.append(r)
    rows.append(g.choice([np.inf, -np.inf, np.nan, 0.0], size=V))
    r = np.full(V, np.nan)
    r[g.integers(0, V, 3)] = -5.0
    rows.append(r)                                          # almost all NaN
    a = np.array(rows)
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(a.astype(np.float32))
    return a.astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V,K", [(5003, 1), (5003, 7), (40000, 16), (40000, 64), (151936, 16), (70, 64), (200000, 32), (262144, 64)])
def test_topk_ties_and_special_values(dtype, V, K):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case topk special {dtype} V={V} K={K}", flush=True)
    rows = _special_rows(V, dtype, seed=V + K)
    R = rows.shape[0]
    dims = dc.Dims(R, 1, K, V, 32, 32, 32, 32, 32, 32, dtype)
    ids, vals = dc.topk(dims, to_dev(rows, dtype))
    torch.cuda.synchronize()
    ref_ids, ref_vals = O.top_k(O.to_f64(rows, dtype), K)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    got = vals.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref_vals))
    np.testing.assert_array_equal(got[~np.isnan(got)], ref_vals[~np.isnan(ref_vals)])
    # the values are the logits themselves: a -0 stays -0 (equal keys, so the
    # id decides the order, but the value written must keep its sign)
    np.testing.assert_array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref_vals[~np.isnan(ref_vals)]))


@pytest.mark.parametrize("R", [1, 3, 16, 32, 100])
def test_topk_rows_cut_into_segments(R):
    """Few rows (at most 32) are cut into column segments and merged; more
    rows stay whole.  The K best must not depend on where the cuts fall.  Rows of a tied top value spread over the
    whole row (lower ids win across segments), the K best packed into one
    narrow band, and the K best one per segment at the cut points' sides."""
    import draft_block_contextual_amd as dc
    import torch
    V, K = 151936, 16
    print(f"case topk segments R={R}", flush=True)
    g = np.random.default_rng(1000 + R)
    rows = np.round(g.standard_normal((R, V)) * 4) / 4
    for i in range(R):
        kind = i % 3
        if kind == 0:       # 40 equal maxima spread evenly: the 16 lowest ids win
            rows[i, np.linspace(0, V - 1, 40).astype(np.int64)] = 30.0
        elif kind == 1:     # the K best in one band of 64 columns
            c = int(g.integers(0, V - 64))
            rows[i, c:c + 64:4] = 20.0 + np.arange(16) * 0.5
        else:               # equal maxima just below and above every multiple of 512
            cols = np.arange(512, V, 512)
            rows[i, cols[g.integers(0, cols.size, 12)] - 1] = 25.0
            rows[i, cols[g.integers(0, cols.size, 12)]] = 25.0
    bits = synth.f32_to_bf16_bits(rows.astype(np.float32))
    dims = dc.Dims(R, 1, K, V, 32, 32, 32, 32, 32, 32, "bf16")
    ids, vals = dc.topk(dims, to_dev(bits, "bf16"))
    torch.cuda.synchronize()
    ref_ids, ref_vals = O.top_k(O.to_f64(bits, "bf16"), K)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_array_equal(vals.cpu().numpy().astype(np.float64), ref_vals)


# ------------------------------------------------------------------- walk

def _select(S, vals, ids):
    import draft_block_contextual_amd as dc
    import torch
    N, B, K = vals.shape
    dims = dc.Dims(N, B, K, max(K, 1), 32, 32, 32, 32, 32, 32, "f32")
    Sd = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).cuda() if B > 1 else None
    if Sd is None:
        Sd = torch.zeros(1, dtype=torch.float32, device="cuda")
    si, st = dc.select(dims, Sd, torch.from_numpy(vals.astype(np.float32)).cuda(),
                       torch.from_numpy(ids.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    return si.cpu().numpy(), st.cpu().numpy()


def test_select_matches_oracle_walk():
    g = np.random.default_rng(3)
    for N, B, K in [(5, 16, 16), (3, 7, 64), (4, 16, 3), (2, 1, 5), (6, 40, 32)]:
        print(f"case select N={N} B={B} K={K}", flush=True)
        S = (np.round(g.standard_normal((N, max(B - 1, 0), K, K)) * 4) / 4).astype(np.float32)
        S[S > 1.7] = np.nan
        vals = np.sort(g.standard_normal((N, B, K)))[..., ::-1].astype(np.float32)
        ids = g.integers(0, 100000, (N, B, K)).astype(np.int32)
        si, st = _select(S, vals, ids)
        ri, rt, _ = O.greedy_walk(S.astype(np.float64), vals.astype(np.float64), ids)
        np.testing.assert_array_equal(si, ri)
        np.testing.assert_array_equal(st, rt)


def test_select_worked_example():
    with open(os.path.join(GOLD, "worked_example.json")) as f:
        W = json.load(f)
    B, K = W["B"], W["K"]
    for name, rd in W["readings"].items():
        for case in rd["cases"]:
            ell = np.array(rd["logits"], np.float32)
            S = np.zeros((1, B - 1, K, K), np.float32)
            for p in range(B - 1):
                S[0, p] = ell[p + 1][None, :]
            for p, a, b, v in case.get("plants", []):
                S[0, p, a, b] += np.float32(v)
            ids = np.arange(B * K, dtype=np.int32).reshape(1, B, K)
            si, st = _select(S, ell[None], ids)
            assert list(si[0]) == case["path"], (name, case)


# ---------------------------------------------------- whole-path rules

def _select_path(S, vals, ids, rule, lam):
    import draft_block_contextual_amd as dc
    import torch
    N, B, K = vals.shape
    dims = dc.Dims(N, B, K, max(K, 1), 32, 32, 32, 32, 32, 32, "f32")
    if B > 1:
        Sd = torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)).cuda()
    else:
        Sd = torch.zeros(1, dtype=torch.float32, device="cuda")
    si, st = dc.select_path(dims, Sd, torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).cuda(),
                            torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda(), rule, lam)
    torch.cuda.synchronize()
    return si.cpu().numpy(), st.cpu().numpy()


def _path_score(S, vals, path, lam):
    """J of one path in float64 with the oracle's weights (NaN terms -inf)."""
    B = len(path)
    terms = [vals[0, path[0]]] + [S[p, path[p], path[p + 1]] for p in range(B - 1)]
    terms = np.array([-np.inf if np.isnan(t) else t for t in terms], np.float64)
    w = lam ** np.arange(B, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        J = float((w * terms).sum())
    return (-np.inf if np.isnan(J) else J), float(np.abs(terms[np.isfinite(terms)]).sum())


@pytest.mark.parametrize("lam", [1.0, 0.5])
def test_select_path_exact_on_integer_grids(lam):
    # integer scores: with lam = 1 every fp32 total is exact at any length,
    # with lam = 0.5 up to 16 slots, so exact ties are ties on both sides and
    # the lexicographic tie rule must give the same path bit for bit
    g = np.random.default_rng(41)
    cases = [(5, 16, 16), (3, 7, 64), (4, 16, 3), (2, 1, 5), (6, 12, 32), (3, 16, 1), (4, 9, 17)]
    if lam == 1.0:
        cases += [(2, 300, 8), (1, 4096, 4), (1, 256, 64)]     # long blocks up to both limits
    for N, B, K in cases:
        print(f"case select_path lam={lam} N={N} B={B} K={K}", flush=True)
        S = g.integers(-3, 4, size=(N, max(B - 1, 0), K, K)).astype(np.float32)
        vals = g.integers(-3, 4, size=(N, B, K)).astype(np.float32)
        if B > 2:
            S[0, 1, :, 0] = np.nan               # NaN terms never win
            S[-1, 0, 0, :] = -np.inf
        ids = g.integers(0, 100000, (N, B, K)).astype(np.int32)
        rule = "global_sum" if lam == 1.0 else "discount"
        si, st = _select_path(S, vals, ids, rule, lam)
        ri, rt, _ = O.best_path(S.astype(np.float64), vals.astype(np.float64), ids, lam)
        np.testing.assert_array_equal(si, ri)
        np.testing.assert_array_equal(st, rt)


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "mid_bf16", "k32_small", "k64_small"])
@pytest.mark.parametrize("lam", [1.0, 0.75])
def test_select_path_on_oracle_scores(name, lam):
    # the oracle's own S (rounded to fp32, the type the entry point takes):
    # the GPU path must be the oracle's, unless the two are within the fp32
    # summation error of each other (then the GPU path's J, in float64, must
    # be within that bound of the optimum)
    print(f"case select_path {name} lam={lam}", flush=True)
    ref = _oracle(name)
    S = ref["S"].astype(np.float32)
    vals = ref["cand_vals"].astype(np.float32)
    ids = ref["cand_ids"].astype(np.int32)
    rule = "global_sum" if lam == 1.0 else "discount"
    si, st = _select_path(S, vals, ids, rule, lam)
    ri, rt, Jb = O.best_path(S.astype(np.float64), vals.astype(np.float64), ids, lam)
    same = 0
    for n in range(vals.shape[0]):
        if np.array_equal(si[n], ri[n]):
            same += 1
            assert np.array_equal(st[n], rt[n])
            continue
        J, mag = _path_score(S[n].astype(np.float64), vals[n].astype(np.float64), si[n], lam)
        assert J >= Jb[n] - 1e-4 * (1.0 + mag), (n, J, Jb[n])
        assert np.array_equal(st[n], ids[n, np.arange(vals.shape[1]), si[n]])
    assert same >= 0.9 * vals.shape[0]


def test_select_path_rules_against_greedy():
    g = np.random.default_rng(42)
    N, B, K = 8, 16, 16
    S = g.standard_normal((N, B - 1, K, K)).astype(np.float32) * 3
    vals = np.sort(g.standard_normal((N, B, K)))[..., ::-1].astype(np.float32)
    ids = g.integers(0, 100000, (N, B, K)).astype(np.int32)
    gi, gt = _select(S, vals, ids)
    # the greedy rule is dcoco_select itself
    si, st = _select_path(S, vals, ids, "greedy", 0.0)
    np.testing.assert_array_equal(si, gi)
    np.testing.assert_array_equal(st, gt)
    # a vanishing discount orders paths by (l_1, S_1, S_2, ...) lexicographically:
    # the greedy walk, on scores with no near-ties
    si, st = _select_path(S, vals, ids, "discount", 1e-6)
    np.testing.assert_array_equal(si, gi)
    # the hand-worked case where the total departs from the greedy walk
    vals2 = np.array([[[1.0, 0.0], [0.0, 0.0]]], np.float32)
    S2 = np.array([[[[0.0, 0.0], [5.0, 4.0]]]], np.float32)
    ids2 = np.array([[[10, 11], [20, 21]]], np.int32)
    for rule, lam, want in (("global_sum", 1.0, [1, 0]), ("discount", 0.75, [1, 0]), ("discount", 0.1, [0, 0])):
        si, st = _select_path(S2, vals2, ids2, rule, lam)
        assert si[0].tolist() == want, (rule, lam)
        assert st[0].tolist() == [ids2[0, 0, want[0]], ids2[0, 1, want[1]]]


# ------------------------------------------------------ representation

def _z_interval(inp, ref):
    """Where the GPU's bf16 z may lie, element by element.  z = bf16(W_f [b; g])
    with b and g the bf16-rounded LayerNorm outputs.  The kernels take the same
    steps in fp32, so two things can move the value that gets rounded away
    from the oracle's fp64 one: a b or g entry that sits within the fp32
    evaluation error of a rounding midpoint may round one bf16 step the other
    way (_flip_size), moving z_o by |W_f[o, j]| times that step; and the fp32
    sum of the 2r products W_f[o, j] x_j is off by at most 2r 2^-24 sum_j
    |W_f[o, j] x_j| (the bound of a recursive sum, in any order).  With delta
    the sum of both, the kernel's z lies between bf16(pre - delta) and
    bf16(pre + delta), pre being the oracle's z before its rounding (rounding
    is monotone)."""
    D = inp["dims"]
    ids = ref["cand_ids"]
    P_e, P_h, W_f = (O.to_f64(inp[k], "bf16") for k in ("P_e", "P_h", "W_f"))
    r = D.r
    Wb, Wg = np.abs(W_f[:, :r]), np.abs(W_f[:, r:])
    fb = _flip_size(_ln64(O.to_f64(inp["E"][ids], "bf16") @ P_e.T, D.ln_eps))     # [N, B, K, r]
    fg = _flip_size(_ln64(O.to_f64(inp["h"], "bf16") @ P_h.T, D.ln_eps))          # [N, B, r]
    b, g = ref["b"], ref["g"]
    pre = b @ W_f[:, :r].T + (g @ W_f[:, r:].T)[:, :, None, :]
    mag = np.abs(b) @ Wb.T + (np.abs(g) @ Wg.T)[:, :, None, :]
    delta = fb @ Wb.T + (fg @ Wg.T)[:, :, None, :] + 2 * r * 2.0 ** -24 * mag
    return O.round_bf16(pre - delta), O.round_bf16(pre + delta)


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_f32", "mid_bf16", "k32_small", "widez_bf16",
                                  "tall_bf16"])
def test_represent_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case represent {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    dims, w, logits, h, E = device_inputs(inp)
    ids = torch.from_numpy(ref["cand_ids"].astype(np.int32)).cuda()
    z, s = dc.represent(dims, w, h, E, ids)
    torch.cuda.synchronize()
    z = _np(z).astype(np.float64)
    s = _np(s).astype(np.float64)
    if D.dtype == "bf16":
        lo, hi = _z_interval(inp, ref)
        zr = ref["z"]
        dz = np.abs(z - zr)
        print(f"  z: max |dz| = {dz.max():.3g}, exact fraction {np.mean(dz == 0):.4f}, "
              f"outside the interval {int(np.sum((z < lo) | (z > hi)))}", flush=True)
        assert np.all((lo <= z) & (z <= hi))
        assert np.mean(dz == 0) > 0.98
        np.testing.assert_allclose(s, ref["s"], rtol=0, atol=2e-2)
    else:
        np.testing.assert_allclose(z, ref["z"], rtol=1e-4, atol=1e-4)
        np.testing.assert_allclose(s, ref["s"], rtol=1e-4, atol=1e-3)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_represent_clamps_ids_of_a_one_row_table(dtype):
    # V = 1: every id is clamped to the table's only row, so ids past either
    # end give exactly the result of id 0 (forward, and the backward's
    # recomputed forward and gathered rows)
    import draft_block_contextual_amd as dc
    import torch
    print(f"case represent V=1 {dtype}", flush=True)
    N, B, K, d, r = 2, 3, 1, 64, 32
    dims = dc.Dims(N, B, K, 1, d, d, r, r, r, 32, dtype)
    g = np.random.default_rng(80)

    def mat(*shape, scale=0.1):
        x = (g.standard_normal(shape) * scale).astype(np.float32)
        return to_dev(synth.f32_to_bf16_bits(x) if dtype == "bf16" else x, dtype)

    w = dc.Weights(P_e=mat(r, d), P_h=mat(r, d), W_f=mat(r, 2 * r), W_pair=mat(r, 2 * d), W1=None, b1=None,
                   w2=None, b2=0.0)
    h = mat(N, B, d, scale=30.0)
    E = mat(1, d, scale=0.02)
    zero = torch.zeros((N, B, K), dtype=torch.int32, device="cuda")
    bad = torch.tensor([[[5], [-3], [1]], [[1 << 20], [-(1 << 30)], [0]]], dtype=torch.int32, device="cuda")
    z0, s0 = dc.represent(dims, w, h, E, zero)
    z1, s1 = dc.represent(dims, w, h, E, bad)
    torch.cuda.synchronize()
    assert torch.equal(z0.view(torch.int16 if dtype == "bf16" else torch.int32),
                       z1.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(s0, s1)
    if dtype == "bf16":
        dz = torch.randn((N, B, K, r), device="cuda")
        ds = torch.randn((N, B - 1, r), device="cuda")
        a = dc.represent_backward(dims, w, h, E, zero, dz, ds)
        b = dc.represent_backward(dims, w, h, E, bad, dz, ds)
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["tiny_bias", "small_bf16", "small_f32", "mid_bf16", "k64_small"])
def test_score_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case score {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    dims, w, logits, h, E = device_inputs(inp)
    zst = ref["z"].astype(np.float32)
    if D.dtype == "bf16":
        zst = synth.f32_to_bf16_bits(zst)      # the oracle's z is bf16-valued: exact
    z = to_dev(zst, D.dtype)
    s = torch.from_numpy(ref["s"].astype(np.float32)).cuda()
    cl = torch.from_numpy(ref["cand_vals"].astype(np.float32)).cuda()
    S = dc.score(dims, w, z, s, cl)
    torch.cuda.synchronize()
    # reference S from the same fp32-stored s
    Sref = O.transition_scores(ref["z"], ref["s"].astype(np.float32).astype(np.float64), ref["cand_vals"],
                               O.to_f64(inp["W1"], D.dtype), O.to_f64(inp["b1"], D.dtype),
                               O.to_f64(inp["w2"], D.dtype), inp["b2"])
    ok, worst, nbad = s_tolerance_ok(_np(S), Sref, D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"


# ---------------------------------------------------------- whole path

@pytest.mark.parametrize("name", SMALL)
def test_correct_block_matches_oracle(name):
    print(f"case correct_block {name}", flush=True)
    inp, out = _run_block(name)
    D = inp["dims"]
    ref = _oracle(name)
    np.testing.assert_array_equal(out["cand_ids"], ref["cand_ids"])
    np.testing.assert_array_equal(out["cand_logits"].astype(np.float64), ref["cand_vals"])
    ok, worst, nbad = s_tolerance_ok(out["S"], ref["S"], D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"
    ok, cmp, tot, fail = lockstep_path_check(out["S"], ref["S"], ref["cand_vals"], out["sel_idx"], ref["sel_idx"])
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"
    # tokens are the selected candidates' ids
    N, B, K = ref["cand_ids"].shape
    np.testing.assert_array_equal(out["sel_tok"], out["cand_ids"][np.arange(N)[:, None], np.arange(B)[None], out["sel_idx"]])
    # the walk on the GPU's own scores is exact
    ri, rt, _ = O.greedy_walk(out["S"].astype(np.float64), out["cand_logits"].astype(np.float64), out["cand_ids"])
    np.testing.assert_array_equal(out["sel_idx"], ri)


@pytest.mark.parametrize("name", ["tiny_zero", "small_bf16", "mid_bf16", "k64_small"])
def test_zero_output_layer_reproduces_drafter(name):
    import dataclasses
    import draft_block_contextual_amd as dc
    import torch
    print(f"case zero output layer {name}", flush=True)
    inp = dict(_inputs(name))
    D = inp["dims"]
    inp["w2"] = np.zeros_like(inp["w2"])
    inp["b2"] = 0.0
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    S = out["S"].cpu().numpy()
    cl = out["cand_logits"].cpu().numpy()
    for p in range(D.B - 1):
        for a in range(D.K):
            np.testing.assert_array_equal(S[:, p, a, :], cl[:, p + 1, :])   # bit-exact
    np.testing.assert_array_equal(out["sel_idx"].cpu().numpy(), 0)
    lg = O.to_f64(inp["logits"], D.dtype)
    np.testing.assert_array_equal(out["sel_tok"].cpu().numpy(), np.argmax(lg, axis=-1))


def test_deterministic_bitwise():
    import draft_block_contextual_amd as dc
    import torch
    print("case determinism mid_bf16", flush=True)
    inp = _inputs("mid_bf16")
    dims, w, logits, h, E = device_inputs(inp)
    a = dc.correct_block(dims, w, logits, h, E, want_all=True)
    a = {k: v.clone() for k, v in a.items()}
    b = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k


def test_worked_example_end_to_end():
    import draft_block_contextual_amd as dc
    import torch
    with open(os.path.join(GOLD, "worked_example.json")) as f:
        W = json.load(f)
    B, K = W["B"], W["K"]
    V, d, r, H = 12, 32, 32, 32
    g = np.random.default_rng(16)
    for name in ["W-lit", "W-rank"]:
        rd = W["readings"][name]
        lg = np.full((B, V), -10.0, np.float32)
        for p in range(B):
            for j in range(K):
                lg[p, 3 * p + j] = rd["logits"][p][j]
        dims = dc.Dims(1, B, K, V, d, d, r, r, r, H, "f32")
        f = lambda *s: torch.from_numpy((g.standard_normal(s) * 0.1).astype(np.float32)).cuda()
        w = dc.Weights(P_e=f(r, d), P_h=f(r, d), W_f=f(r, 2 * r), W_pair=f(r, 2 * d), W1=f(H, 3 * r),
                       b1=None, w2=torch.zeros(H, device="cuda"), b2=0.0)
        out = dc.correct_block(dims, w, torch.from_numpy(lg).cuda(), f(1, B, d) * 300, f(V, d) * 0.2)
        torch.cuda.synchronize()
        toks = out["sel_tok"].cpu().numpy()[0]
        words = [W["tokens"][p][int(t) - 3 * p] for p, t in enumerate(toks)]
        case = [c for c in rd["cases"] if c["delta"] == "zero"][0]
        assert " ".join(words) == case["text"]


# ------------------------------------------------- full-size workloads

def _full_size(name, blocks):
    print(f"case full size {name} blocks={blocks}", flush=True)
    inp, out = _run_block(name)
    D = inp["dims"]
    ref = O.correct_block(inp, blocks=list(blocks))
    sl = list(blocks)
    np.testing.assert_array_equal(out["cand_ids"][sl], ref["cand_ids"])
    ok, worst, nbad = s_tolerance_ok(out["S"][sl], ref["S"], D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"
    ok, cmp, tot, fail = lockstep_path_check(out["S"][sl], ref["S"], ref["cand_vals"], out["sel_idx"][sl],
                                             ref["sel_idx"])
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"
    print(f"  worst |dS| = {worst:.3g}; path steps compared {cmp}/{tot}", flush=True)
    # the planted peaks are each row's known top-K
    cfg = inp["cfg"]
    for n in sl:
        pid, _ = synth.planted_peaks(cfg, n)
        np.testing.assert_array_equal(out["cand_ids"][n], pid[:, :D.K])
    return inp, out


def test_full_q8b_1():
    _full_size("q8b_1", (0,))


def test_full_q8b_32_sampled():
    _full_size("q8b_32", (0, 13, 31))


def test_full_kstress_sampled():
    _full_size("kstress", (5,))


def test_full_large_sampled():
    _full_size("large", (0, 63))


def test_full_rows_max_sampled():
    # 4095 blocks of 16 slots: 65520 rows, near the 65535 the boundary accepts
    _full_size("rows_max", (0, 2047, 4094))


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "widez_bf16", "k64_small", "small_f32", "mid_f32"])
def test_correct_block_walk_ties(name):
    # w2 = 0 and logits on a coarse grid: every row of S_p is l_{p+1}(b) + b2,
    # with many equal values, so each step's argmax is decided by the lowest
    # index among ties.  The walk inside dcoco_correct_block must equal the
    # oracle's walk on the returned S, and dcoco_select's walk on the same S.
    import draft_block_contextual_amd as dc
    import torch
    print(f"case correct_block walk ties {name}", flush=True)
    inp = dict(_inputs(name))
    D = inp["dims"]
    zero = np.zeros_like(np.asarray(inp["w2"]))
    inp["w2"] = zero
    lg = O.to_f64(inp["logits"], D.dtype)
    coarse = np.round(lg)                       # few distinct values per row
    inp["logits"] = synth.f32_to_bf16_bits(coarse.astype(np.float32)) if D.dtype == "bf16" else coarse.astype(np.float32)
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    out = {k: _np(v) for k, v in out.items()}
    N, B, K = out["cand_ids"].shape
    ri, rt, _ = O.greedy_walk(out["S"].astype(np.float64), out["cand_logits"].astype(np.float64), out["cand_ids"])
    np.testing.assert_array_equal(out["sel_idx"], ri)
    np.testing.assert_array_equal(out["sel_tok"], rt)
    S = torch.from_numpy(out["S"]).cuda()
    cl = torch.from_numpy(out["cand_logits"]).cuda()
    ids = torch.from_numpy(out["cand_ids"]).cuda()
    si, st = dc.select(dims, S, cl, ids)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(si), out["sel_idx"])
    # candidates are sorted, so index 0 is always among a row's maxima and the
    # lowest index among equal maxima is 0 at every step
    assert np.all(out["sel_idx"] == 0)


@pytest.mark.parametrize("B,K", [(2100, 2), (300, 32)])
def test_correct_block_walk_fallback_shapes(B, K):
    # blocks too large for the walk over the grid's argmax table (more than
    # 2048 slots, or more than 8192 table entries) take the walk over S; the
    # result must still be the oracle's walk on the returned scores
    import draft_block_contextual_amd as dc
    import torch
    print(f"case correct_block walk fallback B={B} K={K}", flush=True)
    cfg = synth.Config(f"fallback_{B}_{K}", synth._d(1, B, K, 3001, 64, 64, 32, 32, 32, 64, "bf16"),
                       30.0, "peaks", K, 2100 + K, "random")
    inp = synth.make_inputs(cfg)
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    out = {k: _np(v) for k, v in out.items()}
    ri, rt, _ = O.greedy_walk(out["S"].astype(np.float64), out["cand_logits"].astype(np.float64), out["cand_ids"])
    np.testing.assert_array_equal(out["sel_idx"], ri)
    np.testing.assert_array_equal(out["sel_tok"], rt)


@pytest.mark.parametrize("name", ["mid_bf16", "h512_bf16", "k32_small", "k1_bf16", "odd_k_slab", "b30_k7_slab",
                                  "chunks_bf16", "chunks_ragged", "chunks_five", "chunks_long"])
def test_correct_block_equals_separate_calls(name):
    # On these shapes the whole-path call scores with the on-chip slab kernels
    # and one workgroup per block finishes the sums and walks the block (K^2 a
    # multiple of 4 or not); dcoco_score finishes pair by pair and dcoco_select
    # walks separately.  The sums are added in the same order, so S is
    # bit-identical and so is the walk.
    import draft_block_contextual_amd as dc
    import torch
    print(f"case correct_block vs separate calls {name}", flush=True)
    extra = {
        "odd_k_slab": synth.Config("odd_k_slab", synth._d(3, 9, 7, 3001, 128, 128, 64, 64, 64, 96, "bf16"),
                                   30.0, "peaks", 7, 2201, "random"),
        "b30_k7_slab": synth.Config("b30_k7_slab", synth._d(2, 30, 7, 2003, 128, 96, 64, 128, 64, 160, "bf16"),
                                    30.0, "peaks", 7, 2202, "random"),
    }
    inp = synth.make_inputs(extra[name]) if name in extra else _inputs(name)
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    ids, cl = out["cand_ids"], out["cand_logits"]
    z, s = dc.represent(dims, w, h, E, ids)
    S = dc.score(dims, w, z, s, cl)
    si, st = dc.select(dims, S, cl, ids)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(out["S"]), _np(S))
    np.testing.assert_array_equal(_np(out["sel_idx"]), _np(si))
    np.testing.assert_array_equal(_np(out["sel_tok"]), _np(st))
    o = {k: _np(v) for k, v in out.items()}
    ri, rt, _ = O.greedy_walk(o["S"].astype(np.float64), o["cand_logits"].astype(np.float64), o["cand_ids"])
    np.testing.assert_array_equal(o["sel_idx"], ri)
    np.testing.assert_array_equal(o["sel_tok"], rt)


def test_degenerate_shapes_select_the_drafter():
    # B = 1: no transitions, every slot keeps the drafter's top-1; K = 1: the
    # only candidate is chosen whatever the scores
    for name in ("b1_bf16", "k1_bf16"):
        print(f"case degenerate {name}", flush=True)
        inp, out = _run_block(name)
        assert np.all(out["sel_idx"] == 0), name
        np.testing.assert_array_equal(out["sel_tok"], out["cand_ids"][:, :, 0])
        np.testing.assert_array_equal(out["cand_ids"], _oracle(name)["cand_ids"])


def test_score_backward_single_slot_is_zero():
    import draft_block_contextual_amd as dc
    import torch
    name = "b1_bf16"
    print(f"case score_backward {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    dims, w, _, _, _ = device_inputs(inp)
    z = _oracle(name)["z"]
    out = dc.score_backward(dims, w, _bf16_dev(z), None, None)
    torch.cuda.synchronize()
    for key in ("dz", "dW1", "db1", "dw2", "db2", "d_cand_logits"):
        assert np.all(_np(out[key]) == 0), key


# --------------------------------- table of normalised candidate projections

def _bf16_ulp(x):
    return np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))).astype(int) - 7)


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "tall_bf16", "q8b_1", "r512_bf16", "wide_max"])
def test_btable_rows_match_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case btable rows {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    dims, w, logits, h, E = device_inputs(inp)
    tab = dc.build_btable(dims, w, E)
    torch.cuda.synchronize()
    g = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, D.V - 1], g.integers(0, D.V, 2000)]))
    got = tab[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    E_rows = O.to_f64(np.asarray(inp["E"])[rows], D.dtype)
    ref = O.candidate_embedding(E_rows, np.arange(len(rows)), O.to_f64(inp["P_e"], D.dtype), D.ln_eps, True)
    d = np.abs(got - ref)
    print(f"  max |db| = {d.max():.3g}, exact fraction {np.mean(d == 0):.4f}", flush=True)
    # fp32 against fp64 before the bf16 rounding: at most one bf16 step apart,
    # plus the fp32 accumulation error of P_e E_v scaled by 1/sigma, which only
    # shows on values near zero (whose bf16 step is tiny)
    assert np.all(d <= _bf16_ulp(ref) + 1e-4)
    assert np.mean(d == 0) > 0.98


def _check_block(inp, out, ref, sl=None):
    D = inp["dims"]
    sl = slice(None) if sl is None else list(sl)
    np.testing.assert_array_equal(out["cand_ids"][sl], ref["cand_ids"])
    ok, worst, nbad = s_tolerance_ok(out["S"][sl], ref["S"], D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"
    ok, cmp, tot, fail = lockstep_path_check(out["S"][sl], ref["S"], ref["cand_vals"], out["sel_idx"][sl],
                                             ref["sel_idx"])
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"
    return worst


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "k64_small", "k32_small", "widez_bf16", "tall_bf16",
                                  "r512_bf16", "wide_max"])
def test_correct_block_btable_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case correct_block btable {name}", flush=True)
    inp = _inputs(name)
    dims, w, logits, h, E = device_inputs(inp)
    tab = dc.build_btable(dims, w, E)
    out = dc.correct_block(dims, w, logits, h, None, want_all=True, btable=tab)
    torch.cuda.synchronize()
    out = {k: _np(v) for k, v in out.items()}
    _check_block(inp, out, _oracle(name))
    ri, rt, _ = O.greedy_walk(out["S"].astype(np.float64), out["cand_logits"].astype(np.float64), out["cand_ids"])
    np.testing.assert_array_equal(out["sel_idx"], ri)


def test_full_q8b_32_btable_sampled():
    import draft_block_contextual_amd as dc
    import torch
    print("case full size q8b_32 btable blocks=(0, 13, 31)", flush=True)
    inp = _inputs("q8b_32")
    dims, w, logits, h, E = device_inputs(inp)
    tab = dc.build_btable(dims, w, E)
    out_t = dc.correct_block(dims, w, logits, h, None, want_all=True, btable=tab)
    out_p = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    out_t = {k: _np(v) for k, v in out_t.items()}
    out_p = {k: _np(v) for k, v in out_p.items()}
    blocks = (0, 13, 31)
    worst = _check_block(inp, out_t, O.correct_block(inp, blocks=list(blocks)), blocks)
    print(f"  worst |dS| vs the oracle = {worst:.3g}", flush=True)
    # the two device paths differ only in the fp32 summation order of P_e E_v
    np.testing.assert_array_equal(out_t["cand_ids"], out_p["cand_ids"])
    assert np.max(np.abs(out_t["S"] - out_p["S"])) < 3e-2


# ------------------------------------------------------------- training

def _targets(ids, V, seed, absent=0.2):
    """A target token per slot: one of the slot's candidates, or (with
    probability `absent`) a token no candidate list holds."""
    g = np.random.default_rng(seed)
    N, B, K = ids.shape
    pick = ids[np.arange(N)[:, None], np.arange(B)[None, :], g.integers(0, K, (N, B))]
    return np.where(g.random((N, B)) < absent, V + 7, pick).astype(np.int32)


def _dev_f32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _bf16_dev(x):
    # values already representable in bf16: their top 16 bits
    import torch
    bits = (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_f32", "mid_bf16", "k64_small"])
def test_loss_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case loss {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    S = ref["S"].astype(np.float32)
    ids = ref["cand_ids"].astype(np.int32)
    tgt = _targets(ids, D.V, 61)
    dims = dc.Dims.from_synth(D)
    L, pair, dS = dc.loss(dims, _dev_f32(S), _dev_i32(ids), _dev_i32(tgt), rho=4.0)
    torch.cuda.synchronize()
    R = O.corrector_loss(S.astype(np.float64), ids, tgt, 4.0)
    assert R["mask"].any()
    if R["mask"].size >= 20:
        assert not R["mask"].all()      # some pairs are dropped
    # fp32 softmax: each term is within a few ulps of its own size
    assert abs(float(L.cpu()[0]) - R["loss"]) <= 1e-5 * max(1.0, abs(R["loss"]))
    np.testing.assert_allclose(_np(pair), R["pair_loss"], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(_np(dS), R["dS"], rtol=1e-4, atol=1e-7)
    assert np.all(_np(dS)[~R["mask"]] == 0)


def test_loss_degenerate_cases():
    import draft_block_contextual_amd as dc
    import torch
    g = np.random.default_rng(62)
    # every target absent: zero loss and zero gradient
    N, B, K = 3, 5, 4
    S = g.standard_normal((N, B - 1, K, K)).astype(np.float32)
    ids = g.integers(0, 1000, (N, B, K)).astype(np.int32)
    dims = dc.Dims(N, B, K, 2000, 32, 32, 32, 32, 32, 32, "f32")
    L, pair, dS = dc.loss(dims, _dev_f32(S), _dev_i32(ids), _dev_i32(np.full((N, B), 5000)), 4.0)
    torch.cuda.synchronize()
    assert float(L.cpu()[0]) == 0.0 and np.all(_np(dS) == 0) and np.all(_np(pair) == 0)
    # one candidate per slot: the softmax is certain
    ids1 = np.arange(N * B).reshape(N, B, 1).astype(np.int32)
    dims1 = dc.Dims(N, B, 1, 2000, 32, 32, 32, 32, 32, 32, "f32")
    S1 = g.standard_normal((N, B - 1, 1, 1)).astype(np.float32)
    L, pair, dS = dc.loss(dims1, _dev_f32(S1), _dev_i32(ids1), _dev_i32(ids1[:, :, 0]), 4.0)
    torch.cuda.synchronize()
    assert float(L.cpu()[0]) == 0.0 and np.all(_np(dS) == 0)
    # equal scores: log K^2 per active pair, weighted
    ids2 = np.arange(N * B * K).reshape(N, B, K).astype(np.int32)
    L, pair, dS = dc.loss(dims, _dev_f32(np.full((N, B - 1, K, K), 0.25)), _dev_i32(ids2),
                          _dev_i32(ids2[:, :, 2]), 4.0)
    torch.cuda.synchronize()
    want = np.log(K * K) * np.exp(-np.arange(B - 1) / 4.0).sum()
    assert abs(float(L.cpu()[0]) - want) <= 1e-5 * want
    # one slot: no pairs, zero loss
    dimsb = dc.Dims(N, 1, K, 2000, 32, 32, 32, 32, 32, 32, "f32")
    L, _, _ = dc.loss(dimsb, None, _dev_i32(ids[:, :1]), _dev_i32(ids[:, :1, 0]), 4.0)
    torch.cuda.synchronize()
    assert float(L.cpu()[0]) == 0.0


def _grad_check(got, R, name, rel=2e-4):
    """fp32 against float64: each gradient within rel of its largest entry
    (the sums run over thousands of terms of both signs), and no element off by
    more than 1e-3 of its own size beyond that floor."""
    g = got.astype(np.float64)
    r = np.asarray(R, np.float64)
    scale = max(np.abs(r).max(), 1e-30)
    err = np.abs(g - r)
    assert err.max() <= rel * scale, (name, err.max(), scale)
    assert np.all(err <= 1e-3 * np.abs(r) + rel * scale), name


@pytest.mark.parametrize("name", ["tiny", "tiny_bias", "small_bf16", "small_f32", "mid_bf16", "k32_small",
                                  "k64_small", "widez_bf16", "wide_max"])
def test_score_backward_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case score_backward {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    dims, w, _, _, _ = device_inputs(inp)
    g = np.random.default_rng(63)
    G = g.standard_normal(ref["S"].shape) / D.n_blocks        # a dense upstream gradient
    z = ref["z"]
    s32 = ref["s"].astype(np.float32)
    zd = _bf16_dev(z) if D.dtype == "bf16" else _dev_f32(z)
    out = dc.score_backward(dims, w, zd, _dev_f32(s32), _dev_f32(G.astype(np.float32)))
    torch.cuda.synchronize()
    wt = {k: O.to_f64(inp[k], D.dtype) for k in ("W1", "b1", "w2")}
    R = O.score_backward(z, s32.astype(np.float64), wt["W1"], wt["b1"], wt["w2"],
                         G.astype(np.float32).astype(np.float64))
    for key in ("dz", "ds", "dW1", "db1", "dw2", "d_cand_vals"):
        got = _np(out["d_cand_logits" if key == "d_cand_vals" else key])
        _grad_check(got, R[key], f"{name}:{key}")
    assert abs(float(_np(out["db2"])[0]) - R["db2"]) <= 1e-5 * max(1.0, np.abs(G).sum())


def test_score_backward_large_preactivations():
    # W1 scaled by 2^6 (exact in bf16): many pre-activations leave the range
    # where the kernel factors e^-u per side, so both of its paths run
    import draft_block_contextual_amd as dc
    import torch
    name = "small_bf16"
    print(f"case score_backward {name} W1*64", flush=True)
    inp = _inputs(name)
    ref = _oracle(name)
    dims, w, _, _, _ = device_inputs(inp)
    wt = {k: O.to_f64(inp[k], "bf16") for k in ("W1", "b1", "w2")}
    W1 = wt["W1"] * 64.0
    w.W1 = _bf16_dev(W1)
    z = ref["z"]
    s32 = ref["s"].astype(np.float32)
    A = np.abs(z @ W1[:, :z.shape[-1]].T)
    assert (A > 80).mean() > 0.05 and (A <= 80).mean() > 0.05      # both paths taken
    G = np.random.default_rng(64).standard_normal(ref["S"].shape) / inp["dims"].n_blocks
    out = dc.score_backward(dims, w, _bf16_dev(z), _dev_f32(s32), _dev_f32(G.astype(np.float32)))
    torch.cuda.synchronize()
    R = O.score_backward(z, s32.astype(np.float64), W1, wt["b1"], wt["w2"], G.astype(np.float32).astype(np.float64))
    for key in ("dz", "ds", "dW1", "db1", "dw2", "d_cand_vals"):
        got = _np(out["d_cand_logits" if key == "d_cand_vals" else key])
        _grad_check(got, R[key], f"big:{key}")


def test_training_step_end_to_end():
    # loss then backward on one config, as a training step would chain them
    import draft_block_contextual_amd as dc
    import torch
    name = "small_bf16"
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    dims, w, _, _, _ = device_inputs(inp)
    ids = ref["cand_ids"].astype(np.int32)
    tgt = _targets(ids, D.V, 64, absent=0.1)
    S32 = ref["S"].astype(np.float32)
    L, _, dS = dc.loss(dims, _dev_f32(S32), _dev_i32(ids), _dev_i32(tgt), 4.0)
    out = dc.score_backward(dims, w, _bf16_dev(ref["z"]), _dev_f32(ref["s"].astype(np.float32)), dS)
    torch.cuda.synchronize()
    RL = O.corrector_loss(S32.astype(np.float64), ids, tgt, 4.0)
    wt = {k: O.to_f64(inp[k], D.dtype) for k in ("W1", "b1", "w2")}
    R = O.score_backward(ref["z"], ref["s"].astype(np.float32).astype(np.float64), wt["W1"], wt["b1"], wt["w2"],
                         RL["dS"])
    for key in ("dz", "dW1", "dw2", "db1"):
        _grad_check(_np(out[key]), R[key], f"e2e:{key}", rel=5e-4)


def test_score_backward_full_q8b_32_sampled():
    # the full 32-block launch (two-part bf16 MFMA products, split sums) with
    # the upstream gradient nonzero in two blocks only: the oracle computes
    # those two blocks, every other block's dz must be exactly zero
    import draft_block_contextual_amd as dc
    import torch
    D = synth.get_config("q8b_32").dims
    N, B, K, rz, rs, H = D.n_blocks, D.B, D.K, D.r_z, D.r_s, D.H
    print(f"case score_backward q8b_32 N={N} B={B} K={K}", flush=True)
    g = np.random.default_rng(65)

    def bf(x):
        return (np.asarray(x, np.float32).view(np.uint32) + 0x8000 >> 16 << 16).view(np.float32).astype(np.float64)

    z = bf(g.standard_normal((N, B, K, rz)))
    s = (g.standard_normal((N, B - 1, rs)) * 30).astype(np.float32)
    W1 = bf(g.standard_normal((H, 2 * rz + rs)) * np.sqrt(2.0 / (H + 2 * rz + rs)))
    b1 = bf(g.standard_normal(H) * 0.1)
    w2 = bf(g.standard_normal(H) * np.sqrt(2.0 / (H + 1)))
    G = np.zeros((N, B - 1, K, K), np.float32)
    blocks = [0, 17]
    G[blocks] = g.standard_normal((len(blocks), B - 1, K, K)).astype(np.float32) / N
    dims = dc.Dims.from_synth(D)
    w = dc.Weights(P_e=None, P_h=None, W_f=None, W_pair=None, W1=_bf16_dev(W1), b1=_bf16_dev(b1), w2=_bf16_dev(w2),
                   b2=0.0)
    out = dc.score_backward(dims, w, _bf16_dev(z), _dev_f32(s), _dev_f32(G))
    torch.cuda.synchronize()
    R = O.score_backward(z[blocks], s[blocks].astype(np.float64), W1, b1, w2, G[blocks].astype(np.float64))
    dz = _np(out["dz"])
    others = np.setdiff1d(np.arange(N), blocks)
    assert np.all(dz[others] == 0)
    _grad_check(dz[blocks], R["dz"], "full:dz")
    _grad_check(_np(out["ds"])[blocks], R["ds"], "full:ds")
    for key in ("dW1", "db1", "dw2"):
        _grad_check(_np(out[key]), R[key], f"full:{key}")
    _grad_check(_np(out["d_cand_logits"])[blocks], R["d_cand_vals"], "full:dcl")


# ------------------------------------------------- representation backward

def _ln64(x, eps):
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)


def _flip_size(y):
    """How far the bf16 rounding of an LN output may move between the fp64
    oracle and the kernel's fp32 evaluation: the rounding decision is taken
    on values that agree to about 1e-7 of max(1, |y|), so an entry within
    2^-17 of that scale of a rounding midpoint may round either way (by one
    bf16 step); every other entry rounds alike (size 0)."""
    w = 2.0 ** -17 * np.maximum(1.0, np.abs(y))
    return np.abs(O.round_bf16(y + w) - O.round_bf16(y - w))


def _rep_bwd_check(out, h, Er, f64, dz, ds, eps, blocks=None, tag=""):
    R = O.represent_backward(h, Er, f64["P_e"], f64["P_h"], f64["W_f"], f64["W_pair"], dz, ds, eps, True)
    for key in ("dP_e", "dP_h", "dW_pair"):
        _grad_check(_np(out[key]), R[key], f"{tag}:{key}")
    if "dh" in out:
        dh = _np(out["dh"])
        if blocks is not None:
            others = np.setdiff1d(np.arange(dh.shape[0]), blocks)
            assert np.all(dh[others] == 0), tag
            dh = dh[blocks]
        _grad_check(dh, R["dh"], f"{tag}:dh")
    # dW_f multiplies the bf16-rounded b and g: besides the fp32 floor, each
    # entry may move by the upstream gradient times a rounding step wherever
    # the rounding decision is a near-tie
    r = f64["P_e"].shape[0]
    fb = _flip_size(_ln64(Er @ f64["P_e"].T, eps))              # [N, B, K, r]
    fg = _flip_size(_ln64(h @ f64["P_h"].T, eps))               # [N, B, r]
    slack = np.concatenate([np.einsum("nbkz,nbkr->zr", np.abs(dz), fb),
                            np.einsum("nbz,nbr->zr", np.abs(dz.sum(axis=2)), fg)], axis=1)
    got = _np(out["dW_f"]).astype(np.float64)
    ref = R["dW_f"]
    scale = np.abs(ref).max()
    err = np.abs(got - ref)
    assert np.all(err <= 2e-4 * scale + slack), (tag, "dW_f", (err - slack).max(), scale)
    assert got.shape == (f64["W_f"].shape[0], 2 * r)


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16", "k64_small", "k32_small", "widez_bf16", "tall_bf16",
                                  "wide_max"])
def test_represent_backward_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case represent_backward {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = _oracle(name)
    dims, w, _, h, E = device_inputs(inp)
    ids = ref["cand_ids"].astype(np.int32)
    g = np.random.default_rng(67)
    dz = (g.standard_normal((D.n_blocks, D.B, D.K, D.r_z)) / D.n_blocks).astype(np.float32)
    ds = (g.standard_normal((D.n_blocks, D.B - 1, D.r_s)) / D.n_blocks).astype(np.float32)
    out = dc.represent_backward(dims, w, h, E, _dev_i32(ids), _dev_f32(dz), _dev_f32(ds))
    torch.cuda.synchronize()
    f64 = {k: O.to_f64(inp[k], "bf16") for k in ("P_e", "P_h", "W_f", "W_pair")}
    h64 = O.to_f64(inp["h"], "bf16")
    Er = O.to_f64(inp["E"], "bf16")[ids]
    _rep_bwd_check(out, h64, Er, f64, dz.astype(np.float64), ds.astype(np.float64), D.ln_eps, tag=name)


def test_represent_backward_single_slot_and_no_dh():
    # B = 1: no pairs, so dW_pair is zero and dh is the LN path alone; a
    # second call without dh leaves the weight gradients unchanged
    import draft_block_contextual_amd as dc
    import dataclasses
    import torch
    name = "small_bf16"
    print(f"case represent_backward {name} B=1", flush=True)
    inp = _inputs(name)
    D1 = dataclasses.replace(inp["dims"], B=1)
    ids = _oracle(name)["cand_ids"][:, :1].astype(np.int32)
    dims, w, _, _, E = device_inputs(inp)
    dims = dc.Dims.from_synth(D1)
    h1 = np.ascontiguousarray(inp["h"][:, :1])
    hd = to_dev(h1, "bf16", "cuda")
    g = np.random.default_rng(68)
    dz = g.standard_normal((D1.n_blocks, 1, D1.K, D1.r_z)).astype(np.float32)
    out = dc.represent_backward(dims, w, hd, E, _dev_i32(ids), _dev_f32(dz), None)
    out2 = dc.represent_backward(dims, w, hd, E, _dev_i32(ids), _dev_f32(dz), None, want_dh=False)
    torch.cuda.synchronize()
    assert np.all(_np(out["dW_pair"]) == 0)
    for key in ("dP_e", "dP_h", "dW_f"):
        assert np.array_equal(_np(out[key]), _np(out2[key])), key
    f64 = {k: O.to_f64(inp[k], "bf16") for k in ("P_e", "P_h", "W_f", "W_pair")}
    Er = O.to_f64(inp["E"], "bf16")[ids]
    _rep_bwd_check(out, O.to_f64(h1, "bf16"), Er, f64, dz.astype(np.float64),
                   np.zeros((D1.n_blocks, 0, D1.r_s)), D1.ln_eps, tag="B1")


def test_represent_backward_full_q8b_32_sampled():
    # the full 32-block launch with the upstream gradients nonzero in two
    # blocks only: the weight gradients are then those two blocks' sums (the
    # oracle computes them), and dh of every other block is exactly zero
    import draft_block_contextual_amd as dc
    import torch
    D = synth.get_config("q8b_32").dims
    N, B, K, d, e, r, rz, rs = D.n_blocks, D.B, D.K, D.d, D.e, D.r, D.r_z, D.r_s
    print(f"case represent_backward q8b_32 N={N} B={B} K={K}", flush=True)
    g = np.random.default_rng(69)

    def bf(x):
        return (np.asarray(x, np.float32).view(np.uint32) + 0x8000 >> 16 << 16).view(np.float32).astype(np.float64)

    pool = np.sort(g.choice(D.V, 8192, replace=False))
    rows = bf(g.standard_normal((len(pool), e)))
    ids = pool[g.integers(0, len(pool), (N, B, K))].astype(np.int32)
    h = bf(g.standard_normal((N, B, d)) * 30)
    W = {"P_e": bf(g.standard_normal((r, e)) / np.sqrt(e)), "P_h": bf(g.standard_normal((r, d)) / np.sqrt(d)),
         "W_f": bf(g.standard_normal((rz, 2 * r)) / np.sqrt(2 * r)),
         "W_pair": bf(g.standard_normal((rs, 2 * d)) / np.sqrt(2 * d))}
    blocks = [0, 17]
    dz = np.zeros((N, B, K, rz), np.float32)
    ds = np.zeros((N, B - 1, rs), np.float32)
    dz[blocks] = g.standard_normal((2, B, K, rz)).astype(np.float32) / N
    ds[blocks] = g.standard_normal((2, B - 1, rs)).astype(np.float32) / N
    E = torch.zeros((D.V, e), dtype=torch.bfloat16, device="cuda")
    E[torch.from_numpy(pool).cuda()] = _bf16_dev(rows)
    dims = dc.Dims.from_synth(D)
    w = dc.Weights(P_e=_bf16_dev(W["P_e"]), P_h=_bf16_dev(W["P_h"]), W_f=_bf16_dev(W["W_f"]),
                   W_pair=_bf16_dev(W["W_pair"]), W1=None, b1=None, w2=None, b2=0.0)
    out = dc.represent_backward(dims, w, _bf16_dev(h), E, _dev_i32(ids), _dev_f32(dz), _dev_f32(ds))
    torch.cuda.synchronize()
    lookup = np.searchsorted(pool, ids[blocks])
    _rep_bwd_check(out, h[blocks], rows[lookup], W, dz[blocks].astype(np.float64), ds[blocks].astype(np.float64),
                   D.ln_eps, blocks=blocks, tag="full")


# ---------------------------------------------------------- drafter LM head

def _lm_check(ids, vals, logits, K):
    """GPU (ids, vals) per row against the oracle's bf16 logits of that row.
    The GPU rounds an fp32 sum and the oracle an fp64 one, so a logit may sit
    one bf16 step away; within that, the selection must be a valid top-K in
    the pages' order, and it must equal the oracle's exactly in most rows."""
    R, V = logits.shape
    ref_ids, ref_vals = O.top_k(logits, K)
    exact = 0
    for i in range(R):
        g, gv, lg = ids[i].astype(np.int64), vals[i].astype(np.float64), logits[i]
        assert len(set(g.tolist())) == K and g.min() >= 0 and g.max() < V, i
        ulp = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(lg[g]), 2.0 ** -126))).astype(int) - 7)
        assert np.all(np.abs(gv - lg[g]) <= ulp), (i, gv, lg[g])
        # sorted by value, equal values by id
        assert np.all((gv[:-1] > gv[1:]) | ((gv[:-1] == gv[1:]) & (g[:-1] < g[1:]))), i
        # nothing left out beats anything taken by more than one step
        rest = np.delete(lg, g)
        kth = lg[g].min()
        assert rest.max() <= kth + 2 * ulp.max(), (i, rest.max(), kth)
        if np.array_equal(g, ref_ids[i]) and np.array_equal(gv, ref_vals[i]):
            exact += 1
    return exact / R


@pytest.mark.parametrize("name", ["lmh_small", "lmh_rows", "lmh_flat", "lmh_k1", "lmh_k32", "lmh_k64"])
def test_lm_head_topk_matches_oracle(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case lm_head_topk {name}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    L = synth.make_lm_head_inputs(name, inp["E"])
    dims = dc.Dims.from_synth(D)
    ids, vals = dc.lm_head_topk(dims, to_dev(L["hd"], "bf16"), to_dev(L["W_lm"], "bf16"))
    torch.cuda.synchronize()
    logits = O.lm_head_logits(L["hd"], L["W_lm"], "bf16")
    frac = _lm_check(_np(ids), _np(vals), logits, D.K)
    assert frac >= 0.95, frac


def test_lm_head_topk_matches_dcoco_topk_on_stored_logits():
    # the fused path selects what the two-step path selects from the same
    # logits once they are stored (rows where no rounding straddles)
    import draft_block_contextual_amd as dc
    import torch
    name = "lmh_rows"
    inp = _inputs(name)
    D = inp["dims"]
    L = synth.make_lm_head_inputs(name, inp["E"])
    dims = dc.Dims.from_synth(D)
    ids, vals = dc.lm_head_topk(dims, to_dev(L["hd"], "bf16"), to_dev(L["W_lm"], "bf16"))
    stored = synth.f32_to_bf16_bits(O.lm_head_logits(L["hd"], L["W_lm"], "bf16").astype(np.float32))
    ids2, vals2 = dc.topk(dims, to_dev(stored, "bf16"))
    torch.cuda.synchronize()
    same = np.mean([np.array_equal(a, b) for a, b in zip(_np(ids), _np(ids2))])
    assert same >= 0.95, same


def test_full_q8b_32_lm_head_sampled():
    # the full 512 x 151936 x 4096 launch; the oracle computes sampled rows
    import draft_block_contextual_amd as dc
    import torch
    name = "q8b_32"
    print("case lm_head_topk q8b_32", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    L = synth.make_lm_head_inputs(name, inp["E"])
    dims = dc.Dims.from_synth(D)
    ids, vals = dc.lm_head_topk(dims, to_dev(L["hd"], "bf16"), to_dev(L["W_lm"], "bf16"))
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 255, 300, 384, 511]
    logits = O.lm_head_logits(L["hd"], L["W_lm"], "bf16", rows=rows)
    frac = _lm_check(_np(ids)[rows], _np(vals)[rows], logits, D.K)
    assert frac >= 0.75, frac
    # every row: the planted peaks are the top 16 (they stand 12+ above the background)
    np.testing.assert_array_equal(np.sort(_np(ids), axis=1), np.sort(L["planted"], axis=1))


# ------------------------------------------------------ top-K stress rows

@pytest.mark.parametrize("kind,K", [("ramp_up", 16), ("ramp_down", 16), ("constant", 16), ("ramp_up_noisy", 16),
                                    ("normal", 16), ("normal", 64), ("normal", 1)])
def test_topk_stress_rows(kind, K):
    # rows that defeat a sampled threshold: every later element above it
    # (rising), all elements tied (constant); plain N(0, 2^2) rows, whose K-th
    # largest bf16 value is usually tied with others; the result must stay exact
    import draft_block_contextual_amd as dc
    import torch
    print(f"case topk stress {kind} K={K}", flush=True)
    R, V = 24, 151936
    x = np.linspace(-12, 12, V)
    if kind == "ramp_down":
        x = x[::-1]
    if kind == "constant":
        x = np.full(V, 1.5)
    rows = np.tile(x, (R, 1))
    if kind == "ramp_up_noisy":
        rows = rows + np.random.default_rng(70).standard_normal((R, V)) * 0.5
    if kind == "normal":
        rows = np.random.default_rng(71 + K).standard_normal((R, V)) * 2.0
    bits = synth.f32_to_bf16_bits(rows.astype(np.float32))
    dims = dc.Dims(1, R, K, V, 32, 32, 32, 32, 32, 32, "bf16")
    ids, vals = dc.topk(dims, to_dev(bits, "bf16"))
    torch.cuda.synchronize()
    ref_ids, ref_vals = O.top_k(O.to_f64(bits, "bf16"), K)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_array_equal(vals.cpu().numpy().astype(np.float64), ref_vals)
