"""Special cases of the pages checked on the HIP path (through the C ABI).

* Large pre-activations: the scoring grid evaluates w2 SiLU(u) through
  per-candidate factors 2^A', 2^B' while every |A'| of a group of hidden
  units stays within 64, and through 2^(A'+B') per element otherwise (a group
  is one wave's 16 units where A and B are formed on chip, a slab of
  4096 / KR units where they go through memory).  Scores with W1 rows scaled
  by 2^6 (exact in bf16 and fp32) must still match the oracle, with both
  forms taken in the same launch.
* The walk reads one row per pair (review of arXiv 2610.12570, "Contextual
  Correction of Parallel Drafts for Speculative Decoding", part 2 of "New
  approach: DCOCO", paper Sec. 3.3: O(BK) on top of the scoring): poisoning
  every row the walk does not visit leaves its path unchanged.
* Without the candidate state (the fusion W_f = 0, so z = 0: the "-cand state"
  ablation of section "Path selection and ablation", paper Tab. 5/6) the
  correction no longer depends on the candidates and the walk keeps the
  drafter's own choice in every slot.
* With W1's predecessor block zero, S_p(a, b) does not depend on a: every row
  of a pair's grid is the same, bit for bit.
"""
import functools

import numpy as np
import pytest

import synth
from helpers import (device_inputs, ensure_built, lockstep_path_check, s_tolerance_ok, s_tolerance_cancelling,
                     score_magnitude, to_dev, PATH_MARGIN)
from oracle import dcoco_oracle as O

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()


def _np(t):
    import torch
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.cpu().numpy()


@functools.lru_cache(maxsize=8)
def _inputs(name):
    return synth.make_inputs(name)


def _store(x, dtype):
    """float64 values exactly representable in the storage type -> stored array."""
    x = np.asarray(x, np.float64)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x.astype(np.float32))
        assert np.array_equal(O.to_f64(bits, "bf16"), x), "value not exact in bf16"
        return bits
    assert np.array_equal(x.astype(np.float32).astype(np.float64), x)
    return x.astype(np.float32)


def _slab(K):
    """Hidden units per slab in the scoring grid: 4096 / KR, with the candidate
    count padded to KR = 8, 16, 32 or 64."""
    KR = 8 if K <= 8 else 16 if K <= 16 else 32 if K <= 32 else 64
    return 4096 // KR


def _on_chip(D):
    """The library forms A and B on chip for bf16 with K <= 32, r_z of 64, 128
    or 256 and H a multiple of 16: for K <= 16 while blocks x slabs of 64
    units stay within 768, for K > 16 up to 40M grid elements N (B-1) K^2 H;
    otherwise they go through memory to the grid kernel."""
    if not (D.dtype == "bf16" and D.K <= 32 and D.r_z in (64, 128, 256) and D.H % 16 == 0):
        return False
    if D.K <= 16:
        return D.n_blocks * ((D.H + 63) // 64) <= 768
    return D.n_blocks * (D.B - 1) * D.K * D.K * D.H <= 40e6


def _group(D):
    """Hidden units that take one form together: one wave's 16 where A and B
    are formed on chip, else the grid's slab of 4096 / KR units."""
    return 16 if _on_chip(D) else _slab(D.K)


def _slab_counts(z, W1, D):
    """(groups certainly above, groups certainly below) the |A'| = 64 switch,
    where A' = -log2(e) W1a z_{p,a} over a pair's K predecessor rows and one
    group of hidden units (values within 0.1% of 64 count as neither)."""
    N, B, _, rz = z.shape
    H = D.H
    A = np.abs(z[:, :-1] @ W1[:, :rz].T) * LOG2E          # [N, B-1, K, H]
    hs = _group(D)
    hi = lo = 0
    for h0 in range(0, H, hs):
        m = A[..., h0:h0 + hs].max(axis=(-1, -2))         # [N, B-1]
        hi += int((m > 64 * 1.001).sum())
        lo += int((m < 64 * 0.999).sum())
    return hi, lo


def _scaled_w1(inp, units):
    """W1 with the rows of hidden units [0, units) multiplied by 2^6."""
    D = inp["dims"]
    W1 = O.to_f64(inp["W1"], D.dtype).copy()
    W1[:units] *= 64.0
    return W1


# ------------------------------------------------ large pre-activations

def _check_scores(got, Sref, D, z, s, cand_vals, W1, inp):
    """bf16: 3e-2 absolute everywhere.  fp32: 1e-4 max(1, |S|), except that
    pre-activations in the hundreds make a pair's terms cancel to scores far
    below their size M; no fp32 evaluation keeps 1e-4 of |S| there, so every
    score must be within the first-order rounding bound n 2^-24 M of the two
    sums (n = 2 r_z + r_s + H) and 99% of them within 1e-4 max(1, |S|)."""
    if D.dtype == "bf16":
        ok, worst, nbad = s_tolerance_ok(got, Sref, D.dtype)
        print(f"  max |S| = {np.abs(Sref).max():.4g}, worst |dS| = {worst:.3g}", flush=True)
        assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"
        return
    M = score_magnitude(z, s, cand_vals, W1, O.to_f64(inp["b1"], D.dtype), O.to_f64(inp["w2"], D.dtype),
                        inp["b2"])
    ok, worst, n_rel, n_all = s_tolerance_cancelling(got, Sref, M, 2 * D.r_z + D.r_s + D.H)
    print(f"  max |S| = {np.abs(Sref).max():.4g}, max M = {M.max():.4g}, worst |dS| = {worst:.3g}; "
          f"outside 1e-4 max(1, |S|): {n_rel} of {got.size}, outside both: {n_all}", flush=True)
    assert ok, (worst, n_rel, n_all)


@pytest.mark.parametrize("name,mode,tile", [("k32_small", "units", 1), ("k64_small", "units", 1),
                                            ("h512_bf16", "units", 1), ("mid_bf16", "slots", 1),
                                            ("h512_bf16", "units", 33), ("mid_bf16", "slots", 49),
                                            ("k32_f32", "units", 1), ("mid_f32", "slots", 1),
                                            ("small_f32", "slots", 1)])
def test_score_large_preactivations(name, mode, tile):
    # "units": the W1 rows of the first slab of hidden units scaled by 2^6, so
    # that slab of every pair takes the per-element form and the later slabs
    # the factored one.  "slots": z of every even slot scaled by 2^6, so pairs
    # whose predecessor slot is even take the per-element form and the others
    # the factored one (with large B' values on their successor side).
    # tile > 1 repeats the blocks that many times, past the size where the
    # library scores through the A, B buffer and the grid kernel.
    import dataclasses
    import draft_block_contextual_amd as dc
    import torch
    print(f"case score large pre-activations {name} {mode} x{tile}", flush=True)
    inp = _inputs(name)
    D = inp["dims"]
    ref = O.correct_block(inp)
    dims, w, _, _, _ = device_inputs(inp)
    W1 = O.to_f64(inp["W1"], D.dtype)
    # the oracle's z as the entry point receives it (bf16 z is bf16-valued
    # already; fp32 z is rounded to fp32)
    z = ref["z"].astype(np.float32).astype(np.float64)
    if mode == "units":
        W1 = _scaled_w1(inp, _slab(D.K))
        w.W1 = to_dev(_store(W1, D.dtype), D.dtype)
    else:
        z[:, 0::2] *= 64.0
    s32 = ref["s"].astype(np.float32)
    Sref = O.transition_scores(z, s32.astype(np.float64), ref["cand_vals"], W1, O.to_f64(inp["b1"], D.dtype),
                               O.to_f64(inp["w2"], D.dtype), inp["b2"])
    vals, ids = ref["cand_vals"], ref["cand_ids"]
    if tile > 1:
        z, s32, vals, ids, Sref = (np.concatenate([x] * tile) for x in (z, s32, vals, ids, Sref))
        D = dataclasses.replace(D, n_blocks=D.n_blocks * tile)
        dims = dc.Dims.from_synth(D)
    hi, lo = _slab_counts(z, W1, D)
    print(f"  {'on chip' if _on_chip(D) else 'through memory'}; groups above the switch: {hi}, below: {lo}",
          flush=True)
    assert hi > 0 and lo > 0
    assert _on_chip(D) == (tile == 1 and D.dtype == "bf16" and D.K <= 32)
    cl = vals.astype(np.float32)
    S = dc.score(dims, w, to_dev(_store(z, D.dtype), D.dtype), torch.from_numpy(s32).cuda(),
                 torch.from_numpy(cl).cuda())
    torch.cuda.synchronize()
    got = _np(S)
    _check_scores(got, Sref, D, z, s32.astype(np.float64), vals, W1, inp)
    # and the walk over those scores is the oracle's wherever the margin decides
    ri, _, _ = O.greedy_walk(Sref, vals, ids)
    si, _ = dc.select(dims, S, torch.from_numpy(cl).cuda(), torch.from_numpy(ids.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    ok, cmp, tot, fail = lockstep_path_check(got, Sref, vals, _np(si), ri)
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"


@pytest.mark.parametrize("name", ["k32_small", "k64_small", "h512_bf16", "k32_f32"])
def test_correct_block_large_preactivations(name):
    import draft_block_contextual_amd as dc
    import torch
    print(f"case correct_block large pre-activations {name}", flush=True)
    inp = dict(_inputs(name))
    D = inp["dims"]
    W1 = _scaled_w1(inp, _slab(D.K))
    inp["W1"] = _store(W1, D.dtype)
    ref = O.correct_block(inp)
    hi, lo = _slab_counts(ref["z"], W1, D)
    print(f"  groups above the switch: {hi}, below: {lo}", flush=True)
    assert hi > 0 and lo > 0
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    out = {k: _np(v) for k, v in out.items()}
    np.testing.assert_array_equal(out["cand_ids"], ref["cand_ids"])
    _check_scores(out["S"], ref["S"], D, ref["z"], ref["s"], ref["cand_vals"], W1, inp)
    ok, cmp, tot, fail = lockstep_path_check(out["S"], ref["S"], ref["cand_vals"], out["sel_idx"], ref["sel_idx"])
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"
    ri, rt, _ = O.greedy_walk(out["S"].astype(np.float64), out["cand_logits"].astype(np.float64), out["cand_ids"])
    np.testing.assert_array_equal(out["sel_idx"], ri)
    np.testing.assert_array_equal(out["sel_tok"], rt)


# ----------------------------------------------------- walk reads O(BK)

def _select(dims, S, vals, ids):
    import draft_block_contextual_amd as dc
    import torch
    si, st = dc.select(dims, torch.from_numpy(np.ascontiguousarray(S, np.float32)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(vals, np.float32)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda())
    torch.cuda.synchronize()
    return si.cpu().numpy(), st.cpu().numpy()


@pytest.mark.parametrize("poison", [np.nan, -np.inf])
@pytest.mark.parametrize("source", ["oracle_mid_bf16", "oracle_k64_small", "random"])
def test_select_ignores_rows_off_the_path(source, poison):
    import draft_block_contextual_amd as dc
    print(f"case select poisoning {source} {poison}", flush=True)
    if source == "random":
        g = np.random.default_rng(91)
        N, B, K = 6, 16, 16
        S = (np.round(g.standard_normal((N, B - 1, K, K)) * 4) / 4).astype(np.float32)   # many ties
        vals = np.sort(g.standard_normal((N, B, K)))[..., ::-1].astype(np.float32)
        ids = g.integers(0, 100000, (N, B, K)).astype(np.int32)
    else:
        ref = O.correct_block(_inputs(source[len("oracle_"):]))
        S = ref["S"].astype(np.float32)
        vals = ref["cand_vals"].astype(np.float32)
        ids = ref["cand_ids"].astype(np.int32)
    N, B, K = vals.shape
    dims = dc.Dims(N, B, K, 100000, 32, 32, 32, 32, 32, 32, "f32")
    si, st = _select(dims, S, vals, ids)
    ri, rt, _ = O.greedy_walk(S.astype(np.float64), vals.astype(np.float64), ids)
    np.testing.assert_array_equal(si, ri)
    # every row of S_p except the visited row k_p replaced by the poison
    P = np.full_like(S, poison)
    n_idx = np.arange(N)[:, None]
    p_idx = np.arange(B - 1)[None, :]
    P[n_idx, p_idx, si[:, :-1]] = S[n_idx, p_idx, si[:, :-1]]
    assert np.mean(np.isnan(P) | np.isinf(P)) > 0.5
    pi, pt = _select(dims, P, vals, ids)
    np.testing.assert_array_equal(pi, si)
    np.testing.assert_array_equal(pt, st)


# ------------------------------------------------ candidate-blind cases

def _run(inp):
    import draft_block_contextual_amd as dc
    import torch
    dims, w, logits, h, E = device_inputs(inp)
    out = dc.correct_block(dims, w, logits, h, E, want_all=True)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in out.items()}


@pytest.mark.parametrize("name", ["tiny", "small_bf16", "small_f32", "mid_bf16", "k64_small", "k32_f32"])
def test_zero_fusion_keeps_the_drafter_choice(name):
    # W_f = 0: z = 0 for every candidate, so the correction of pair p is one
    # number for all (a, b), S_p(a, b) = l_{p+1}(b) + c_p, and the walk takes
    # index 0 (the drafter's top-1) in every slot
    print(f"case zero fusion {name}", flush=True)
    inp = dict(_inputs(name))
    D = inp["dims"]
    inp["W_f"] = np.zeros_like(inp["W_f"])
    out = _run(inp)
    np.testing.assert_array_equal(out["sel_idx"], 0)
    np.testing.assert_array_equal(out["sel_tok"], out["cand_ids"][:, :, 0])
    S = out["S"]
    if D.B > 1:
        np.testing.assert_array_equal(S.view(np.uint32), np.broadcast_to(S[:, :, :1].view(np.uint32), S.shape))
    ref = O.correct_block(inp)
    np.testing.assert_array_equal(ref["sel_idx"], 0)
    ok, worst, nbad = s_tolerance_ok(S, ref["S"], D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"


@pytest.mark.parametrize("name", ["tiny_bias", "small_bf16", "small_f32", "mid_bf16", "k64_small", "k32_f32"])
def test_zero_predecessor_block_gives_equal_rows(name):
    # W1a = 0: the MLP no longer sees z_{p,a}, so S_p(a, b) is the same for
    # every a, bit for bit (the same fp32 operations run for every a)
    print(f"case zero W1a {name}", flush=True)
    inp = dict(_inputs(name))
    D = inp["dims"]
    W1 = np.array(inp["W1"], copy=True)
    W1[:, :D.r_z] = 0
    inp["W1"] = W1
    out = _run(inp)
    S = out["S"]
    np.testing.assert_array_equal(S.view(np.uint32), np.broadcast_to(S[:, :, :1].view(np.uint32), S.shape))
    ref = O.correct_block(inp)
    ok, worst, nbad = s_tolerance_ok(S, ref["S"], D.dtype)
    assert ok, f"{nbad} scores out of tolerance, worst |dS| = {worst}"
    ok, cmp, tot, fail = lockstep_path_check(S, ref["S"], ref["cand_vals"], out["sel_idx"], ref["sel_idx"])
    assert ok, f"path differs at a step with margin > {PATH_MARGIN}: {fail}"
