"""Seeded synthetic inputs for the DCOCO corrector hot path.

This module only draws random numbers and stores them; it holds none of the
method's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP library's
tests and benchmark read their inputs from here, so the two sides always see
identical bytes.

Shapes follow the workloads the pages describe: draft blocks of B = 16 slots
(review of arXiv 2610.12570, "Contextual Correction of Parallel Drafts for
Speculative Decoding", experimental setup: block size 16), top-16 candidates
(same page, the top-k coverage analysis, paper Fig. 1 / Tab. 7), a drafter of
hidden width d = 4096 (same page, strengths: the Qwen3-8B corrector) and 4-32
concurrent streams (same page, TL;DR and concurrency results, paper Tab. 8).
The pages evaluate on public suites with trained weights; none of those are
available, so these seeded tensors with the same shapes stand in for them.

Recipe (all draws from ``numpy.random.Generator(PCG64)`` seeded through
``SeedSequence``; a tensor's seed depends only on (base seed, tensor role,
stream index), so stream n's data does not depend on how many streams a call
holds):

* weights: Xavier-normal, std = sqrt(2 / (fan_in + fan_out)); b1 = 0, w2
  Xavier-normal (fan_in = H, fan_out = 1), b2 = 0 unless a config asks for the
  random-bias variant (b1, b2 ~ N(0, 0.1^2)) or the zeroed output layer
  (w2 = 0, b2 = 0);
* embedding table E ~ N(0, 0.02^2);
* hidden states h ~ N(0, 1) * h_scale (30, or 40 for the d = 8192 shape);
* logit rows: tiny config: N(0, 1) with +3 added at one random id per slot;
  other configs: N(0, 2^2) clipped to [-12, 12], plus P planted peaks with
  values 20 + 0.5 j (j = 0..P-1, exact in bf16 and distinct) at P distinct
  random ids in random order, so the top-P of every row is tie-free and known.

bf16 storage: values are drawn in float32 and rounded to the nearest bf16
(ties to even); arrays are returned as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = ["Dims", "CONFIGS", "get_config", "make_inputs", "make_lm_head_inputs", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "ROLE"]


@dataclasses.dataclass(frozen=True)
class Dims:
    """Problem shape of one call (notation of the pages where they have one).

    n_blocks  N   draft blocks (decoding streams) per call
    B             slots per draft block
    K             candidates kept per slot
    V             vocabulary size
    d             drafter hidden width (h_i in R^d)
    e             token-embedding width (rows of E)
    r             width of the projected, normalised b_{i,k} and g_i
    r_z           width of the fused candidate representation z_{i,k}
    r_s           width of the pair state s_p
    H             hidden width of the transition MLP Delta_theta
    dtype         "bf16" (bf16 storage, fp32 accumulate) or "f32"
    """
    n_blocks: int
    B: int
    K: int
    V: int
    d: int
    e: int
    r: int
    r_z: int
    r_s: int
    H: int
    dtype: str
    ln_eps: float = 1e-5


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dims: Dims
    h_scale: float
    logit_mode: str          # "tiny" or "peaks"
    n_peaks: int
    seed: int
    mlp_out: str = "random"  # "random", "zero" or "random_bias"
    desc: str = ""


def _d(N, B, K, V, d, e, r, rz, rs, H, dtype):
    return Dims(N, B, K, V, d, e, r, rz, rs, H, dtype)


# Base seed = 1000 + config index for the five named workloads; test-only
# shapes use their own seeds.
CONFIGS = {
    # tiny fp32 workload: 1 stream, B=4, K=3, d=64, V=1000
    "tiny": Config("tiny", _d(1, 4, 3, 1000, 64, 64, 32, 32, 32, 64, "f32"),
                   30.0, "tiny", 1, 1000, "random",
                   "1 stream, B=4, K=3, d=64, V=1000, e=64, r=32, H=64, fp32"),
    "tiny_zero": Config("tiny_zero", _d(1, 4, 3, 1000, 64, 64, 32, 32, 32, 64, "f32"),
                        30.0, "tiny", 1, 1000, "zero",
                        "tiny workload with the MLP output layer zeroed"),
    "tiny_bias": Config("tiny_bias", _d(1, 4, 3, 1000, 64, 64, 32, 32, 32, 64, "f32"),
                        30.0, "tiny", 1, 1000, "random_bias",
                        "tiny workload with random b1, b2 ~ N(0, 0.1^2)"),
    # Qwen3-8B-shaped block, one stream
    "q8b_1": Config("q8b_1", _d(1, 16, 16, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                    30.0, "peaks", 16, 1001, "random",
                    "1 stream, B=16, K=16, d=4096, V=151936, e=4096, r=256, H=512, bf16"),
    # the measured workload: same shapes, 32 streams
    "q8b_32": Config("q8b_32", _d(32, 16, 16, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                     30.0, "peaks", 16, 1002, "random",
                     "32 streams, B=16, K=16, d=4096, V=151936, e=4096, r=256, H=512, bf16"),
    "q8b_4": Config("q8b_4", _d(4, 16, 16, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                    30.0, "peaks", 16, 1002, "random", "stream sweep: 4 streams"),
    "q8b_8": Config("q8b_8", _d(8, 16, 16, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                    30.0, "peaks", 16, 1002, "random", "stream sweep: 8 streams"),
    "q8b_16": Config("q8b_16", _d(16, 16, 16, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                     30.0, "peaks", 16, 1002, "random", "stream sweep: 16 streams"),
    # K-stress: 64 candidates per slot, 16 streams
    "kstress": Config("kstress", _d(16, 16, 64, 151936, 4096, 4096, 256, 256, 256, 512, "bf16"),
                      30.0, "peaks", 64, 1003, "random",
                      "16 streams, B=16, K=64, d=4096, V=151936, r=256, H=512, bf16"),
    # large-target shape
    "large": Config("large", _d(64, 16, 32, 262144, 8192, 8192, 512, 512, 512, 1024, "bf16"),
                    40.0, "peaks", 32, 1004, "random",
                    "64 streams, B=16, K=32, d=8192, V=262144, e=8192, r=512, H=1024, bf16"),
    # test-only shapes: several tiles plus ragged tails everywhere
    "small_bf16": Config("small_bf16", _d(3, 5, 7, 5003, 256, 128, 64, 96, 32, 160, "bf16"),
                         30.0, "peaks", 9, 2001, "random",
                         "ragged bf16 test shape (V not a multiple of 8, K=7)"),
    "small_f32": Config("small_f32", _d(2, 6, 5, 3001, 128, 96, 64, 32, 64, 96, "f32"),
                        30.0, "peaks", 5, 2002, "random_bias",
                        "ragged fp32 test shape"),
    "mid_bf16": Config("mid_bf16", _d(4, 16, 16, 20000, 1024, 512, 128, 128, 128, 256, "bf16"),
                       30.0, "peaks", 16, 2003, "random",
                       "mid-size bf16 shape that spans many tiles"),
    "mid_f32": Config("mid_f32", _d(2, 16, 16, 20000, 512, 256, 128, 128, 128, 256, "f32"),
                      30.0, "peaks", 16, 2004, "random",
                      "mid-size fp32 shape"),
    "k64_small": Config("k64_small", _d(2, 4, 64, 9000, 256, 256, 64, 64, 64, 192, "bf16"),
                        30.0, "peaks", 64, 2005, "random", "K = 64 on a small shape"),
    "k32_small": Config("k32_small", _d(2, 5, 32, 9000, 512, 256, 128, 128, 128, 320, "bf16"),
                        30.0, "peaks", 32, 2006, "random", "K = 32 on a small shape"),
    "widez_bf16": Config("widez_bf16", _d(2, 6, 8, 7001, 256, 192, 160, 320, 96, 128, "bf16"),
                         30.0, "peaks", 8, 2007, "random",
                         "r = 160 (20 k chunks) and d_z = 320 (two column chunks, the second partial)"),
    "tall_bf16": Config("tall_bf16", _d(3, 15, 50, 6007, 256, 512, 256, 256, 64, 256, "bf16"),
                        30.0, "peaks", 50, 2008, "random",
                        "2250 candidate rows (ragged over 128-row tiles) with 256-wide projections"),
    # degenerate and limit shapes: one slot (no transitions), one candidate,
    # the widest projections the boundary accepts, the most rows it accepts
    "b1_bf16": Config("b1_bf16", _d(3, 1, 8, 5003, 128, 128, 64, 64, 64, 64, "bf16"),
                      30.0, "peaks", 8, 2009, "random", "B = 1: no pairs, the drafter's top-1 per slot"),
    "k1_bf16": Config("k1_bf16", _d(3, 6, 1, 5003, 128, 128, 64, 64, 64, 64, "bf16"),
                      30.0, "peaks", 1, 2010, "random", "K = 1: one candidate per slot"),
    "wide_max": Config("wide_max", _d(2, 4, 4, 3001, 256, 256, 2048, 2048, 2048, 256, "bf16"),
                       30.0, "peaks", 4, 2011, "random", "d_proj = d_z = d_pair = 2048 (the widest accepted)"),
    "rows_max": Config("rows_max", _d(4095, 16, 4, 1024, 64, 64, 32, 32, 32, 64, "bf16"),
                       30.0, "peaks", 4, 2012, "random", "65520 slot rows (the most accepted is 65535)"),
    # several hidden-unit slabs per pair in the scoring grid: K = 32 in fp32,
    # and K = 16 with H = 512 as in the Qwen3-8B-shaped workload
    "k32_f32": Config("k32_f32", _d(2, 5, 32, 9000, 256, 256, 128, 128, 128, 320, "f32"),
                      30.0, "peaks", 32, 2013, "random", "K = 32, H = 320 in fp32"),
    "h512_bf16": Config("h512_bf16", _d(3, 6, 16, 7001, 256, 256, 128, 128, 128, 512, "bf16"),
                        30.0, "peaks", 16, 2014, "random", "K = 16 with H = 512 on a small shape"),
    # d_proj = 512, as in the d = 8192 workload: the table path's GEMM gathers the rows
    "r512_bf16": Config("r512_bf16", _d(2, 6, 16, 6007, 512, 512, 512, 256, 128, 256, "bf16"),
                        30.0, "peaks", 16, 2015, "random", "d_proj = 512 on a small shape"),
    # many blocks, so that on-chip scoring gives each workgroup a run of
    # three pairs (a whole and a ragged slab count)
    "chunks_bf16": Config("chunks_bf16", _d(128, 16, 16, 3001, 64, 64, 64, 64, 64, 64, "bf16"),
                          30.0, "peaks", 16, 2016, "random", "128 blocks of B = 16, K = 16, H = 64"),
    "chunks_ragged": Config("chunks_ragged", _d(64, 16, 12, 3001, 64, 64, 64, 128, 64, 96, "bf16"),
                            30.0, "peaks", 12, 2017, "random", "64 blocks of B = 16, K = 12, H = 96"),
    # on-chip scoring with the pair term formed in the scoring launch at its
    # limit (five pairs, fifteen operand rows per workgroup), and with runs
    # of six pairs, where the pair term comes from its own product
    "chunks_five": Config("chunks_five", _d(256, 16, 4, 3001, 64, 64, 64, 64, 64, 64, "bf16"),
                          30.0, "peaks", 4, 2018, "random", "256 blocks of B = 16, K = 4, H = 64"),
    "chunks_long": Config("chunks_long", _d(8, 64, 8, 3001, 64, 64, 64, 64, 64, 512, "bf16"),
                          30.0, "peaks", 8, 2019, "random", "8 blocks of B = 64, K = 8, H = 512"),
    # LM-head shapes (head tied to E, so d == e): ragged vocabulary tiles,
    # ragged row tiles, rows without planted peaks (bf16 ties at the K-th)
    "lmh_small": Config("lmh_small", _d(2, 8, 16, 5003, 256, 256, 64, 64, 64, 64, "bf16"),
                        30.0, "peaks", 16, 2101, "random", "LM head: 16 rows, V = 5003, d = 256"),
    "lmh_rows": Config("lmh_rows", _d(25, 8, 16, 9001, 320, 320, 64, 64, 64, 64, "bf16"),
                       30.0, "peaks", 16, 2102, "random", "LM head: 200 rows (two row tiles), d = 320"),
    "lmh_flat": Config("lmh_flat", _d(3, 16, 12, 20011, 512, 512, 64, 64, 64, 64, "bf16"),
                       30.0, "peaks", 0, 2103, "random", "LM head: background only, K = 12, V = 20011"),
    "lmh_k1": Config("lmh_k1", _d(2, 4, 1, 3001, 128, 128, 64, 64, 64, 64, "bf16"),
                     30.0, "peaks", 1, 2104, "random", "LM head: K = 1"),
    "lmh_k32": Config("lmh_k32", _d(3, 8, 32, 12007, 256, 256, 64, 64, 64, 64, "bf16"),
                      30.0, "peaks", 0, 2105, "random", "LM head: K = 32, background only (ties at the K-th)"),
    "lmh_k64": Config("lmh_k64", _d(5, 8, 64, 9001, 320, 320, 64, 64, 64, 64, "bf16"),
                      30.0, "peaks", 64, 2106, "random", "LM head: K = 64, 40 rows"),
}

# tensor roles, in the fixed order their seeds are spawned
ROLE = {"E": 0, "P_e": 1, "P_h": 2, "W_f": 3, "W_pair": 4, "W1": 5, "b1": 6,
        "w2": 7, "b2": 8, "stream": 9}
STREAM_ROLE = {"h": 0, "logit_bg": 1, "peak_pos": 2, "peak_perm": 3}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _xavier(seed, role, shape, chunk_rows=None):
    fan_out, fan_in = shape
    std = np.sqrt(2.0 / (fan_in + fan_out))
    g = _rng(seed, ROLE[role])
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def _embedding(seed: int, V: int, e: int, dtype: str) -> np.ndarray:
    """E ~ N(0, 0.02^2), drawn in row chunks to bound peak host memory."""
    g = _rng(seed, ROLE["E"])
    out = np.empty((V, e), dtype=np.uint16 if dtype == "bf16" else np.float32)
    step = max(1, (1 << 24) // e)
    for r0 in range(0, V, step):
        r1 = min(V, r0 + step)
        blk = g.standard_normal((r1 - r0, e), dtype=np.float32) * np.float32(0.02)
        out[r0:r1] = _store(blk, dtype)
    return out


def _logit_row_block(cfg: Config, stream: int, seed: int) -> np.ndarray:
    D = cfg.dims
    if cfg.logit_mode == "tiny":
        g = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["logit_bg"])
        x = g.standard_normal((D.B, D.V), dtype=np.float32)
        gp = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["peak_pos"])
        pos = gp.integers(0, D.V, size=D.B)
        x[np.arange(D.B), pos] += np.float32(3.0)
        return x
    g = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["logit_bg"])
    x = np.clip(g.standard_normal((D.B, D.V), dtype=np.float32) * np.float32(2.0),
                -12.0, 12.0).astype(np.float32)
    gp = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["peak_pos"])
    gq = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["peak_perm"])
    P = cfg.n_peaks
    vals = (20.0 + 0.5 * np.arange(P)).astype(np.float32)
    for i in range(D.B):
        pos = gp.choice(D.V, size=P, replace=False)
        x[i, pos] = vals[gq.permutation(P)]
    return x


def planted_peaks(cfg: Config, stream: int, seed: int | None = None):
    """Return (ids, values) of the planted peaks of each slot of one stream,
    ids sorted by planted value descending: the known top-P of every row.

    Only defined for the "peaks" logit mode.
    """
    assert cfg.logit_mode == "peaks"
    D = cfg.dims
    seed = cfg.seed if seed is None else seed
    gp = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["peak_pos"])
    gq = _rng(seed, ROLE["stream"], stream, STREAM_ROLE["peak_perm"])
    P = cfg.n_peaks
    vals = (20.0 + 0.5 * np.arange(P)).astype(np.float32)
    ids = np.empty((D.B, P), np.int64)
    pv = np.empty((D.B, P), np.float32)
    for i in range(D.B):
        pos = gp.choice(D.V, size=P, replace=False)
        v = vals[gq.permutation(P)]
        order = np.argsort(-v, kind="stable")
        ids[i] = pos[order]
        pv[i] = v[order]
    return ids, pv


def make_inputs(cfg: Config | str, seed: int | None = None, n_blocks: int | None = None,
                with_E: bool = True) -> dict:
    """Draw every input of one call.

    Returns a dict of numpy arrays: logits [N,B,V], h [N,B,d], E [V,e],
    P_e [r,e], P_h [r,d], W_f [r_z,2r], W_pair [r_s,2d], W1 [H,2r_z+r_s],
    b1 [H], w2 [H] (uint16 bf16 bits or float32, per the config's dtype) and
    b2 (python float), plus "dims" (a Dims with n_blocks overridden when
    asked) and "cfg".
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    D = cfg.dims if n_blocks is None else dataclasses.replace(cfg.dims, n_blocks=n_blocks)
    dt = D.dtype
    out = {"dims": D, "cfg": cfg, "seed": seed}
    out["E"] = _embedding(seed, D.V, D.e, dt) if with_E else None
    out["P_e"] = _store(_xavier(seed, "P_e", (D.r, D.e)), dt)
    out["P_h"] = _store(_xavier(seed, "P_h", (D.r, D.d)), dt)
    out["W_f"] = _store(_xavier(seed, "W_f", (D.r_z, 2 * D.r)), dt)
    out["W_pair"] = _store(_xavier(seed, "W_pair", (D.r_s, 2 * D.d)), dt)
    out["W1"] = _store(_xavier(seed, "W1", (D.H, 2 * D.r_z + D.r_s)), dt)
    if cfg.mlp_out == "zero":
        w2 = np.zeros(D.H, np.float32)
        b1 = np.zeros(D.H, np.float32)
        b2 = 0.0
    else:
        w2 = _xavier(seed, "w2", (1, D.H))[0]
        if cfg.mlp_out == "random_bias":
            b1 = _rng(seed, ROLE["b1"]).standard_normal(D.H, dtype=np.float32) * np.float32(0.1)
            b2 = float(_rng(seed, ROLE["b2"]).standard_normal(dtype=np.float32) * np.float32(0.1))
        else:
            b1 = np.zeros(D.H, np.float32)
            b2 = 0.0
    out["b1"] = _store(b1, dt)
    out["w2"] = _store(w2, dt)
    # b2 is a scalar passed by value in fp32; round it through bf16 in the
    # bf16 configs so that every parameter is a bf16 value there.
    if dt == "bf16":
        b2 = float(bf16_bits_to_f32(f32_to_bf16_bits(np.array([b2], np.float32)))[0])
    out["b2"] = float(np.float32(b2))
    h = np.empty((D.n_blocks, D.B, D.d), np.uint16 if dt == "bf16" else np.float32)
    logits = np.empty((D.n_blocks, D.B, D.V), np.uint16 if dt == "bf16" else np.float32)
    for n in range(D.n_blocks):
        gh = _rng(seed, ROLE["stream"], n, STREAM_ROLE["h"])
        h[n] = _store(gh.standard_normal((D.B, D.d), dtype=np.float32) * np.float32(cfg.h_scale), dt)
        logits[n] = _store(_logit_row_block(cfg, n, seed), dt)
    out["h"] = h
    out["logits"] = logits
    return out


def make_stream_inputs(cfg: Config | str, seed: int, n_blocks: int | None = None) -> dict:
    """Only the per-stream tensors (logits [N,B,V] and h [N,B,d]) of an input
    set drawn with ``seed``; weights and E are shared across rotating sets."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    D = cfg.dims if n_blocks is None else dataclasses.replace(cfg.dims, n_blocks=n_blocks)
    dt = D.dtype
    h = np.empty((D.n_blocks, D.B, D.d), np.uint16 if dt == "bf16" else np.float32)
    logits = np.empty((D.n_blocks, D.B, D.V), np.uint16 if dt == "bf16" else np.float32)
    for n in range(D.n_blocks):
        gh = _rng(seed, ROLE["stream"], n, STREAM_ROLE["h"])
        h[n] = _store(gh.standard_normal((D.B, D.d), dtype=np.float32) * np.float32(cfg.h_scale), dt)
        logits[n] = _store(_logit_row_block(cfg, n, seed), dt)
    return {"h": h, "logits": logits, "dims": D, "seed": seed}


def make_lm_head_inputs(cfg: Config | str, E: np.ndarray, seed: int | None = None,
                        n_blocks: int | None = None) -> dict:
    """Inputs of the drafter's LM head for one call, with the head tied to the
    token-embedding table (W_lm = E, rows = vocabulary; needs d == e).

    hd [N*B, d]: the final hidden state of each slot, N(0, s^2) with
    s = 100 / sqrt(d) (so the background logits hd . E[v] have a standard
    deviation near 2, as the logit rows above), plus, per row, P planted
    directions that lift P distinct random ids to 20 + 0.5 j: the row gains
    the combination of those P rows of E that brings their dot products to
    the targets (a P x P solve), so after rounding to bf16 the planted logits
    land close to their targets.  At d = 4096 they stand clear of the
    background; at small widths the added direction also lifts other ids,
    which is just another logit row to select from.
    Returns {"hd": bits or float32, "W_lm": E, "planted": [N*B, P] ids,
    "dims": Dims}.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    D = cfg.dims if n_blocks is None else dataclasses.replace(cfg.dims, n_blocks=n_blocks)
    assert D.d == D.e, "a tied head needs d == e"
    dt = D.dtype
    P = cfg.n_peaks
    R = D.n_blocks * D.B
    hd = np.empty((R, D.d), np.uint16 if dt == "bf16" else np.float32)
    planted = np.empty((R, P), np.int64)
    s = np.float32(100.0 / np.sqrt(D.d))
    targets = (20.0 + 0.5 * np.arange(P)).astype(np.float64)
    for n in range(D.n_blocks):
        g = _rng(seed, ROLE["stream"], n, STREAM_ROLE["h"] + 16)
        gp = _rng(seed, ROLE["stream"], n, STREAM_ROLE["peak_pos"] + 16)
        for i in range(D.B):
            x = g.standard_normal(D.d, dtype=np.float32).astype(np.float64) * s
            ids = gp.choice(D.V, size=P, replace=False)
            if P:
                t = targets[gp.permutation(P)]
                rows = to_float(E[ids], dt).astype(np.float64)
                x = x + np.linalg.solve(rows @ rows.T, t - rows @ x) @ rows
            hd[n * D.B + i] = _store(x.astype(np.float32)[None, :], dt)[0]
            planted[n * D.B + i] = ids
    return {"hd": hd, "W_lm": E, "planted": planted, "dims": D}


def to_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """View stored values as float32 (bf16 bits are widened exactly)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a, np.float32)


def make_inputs_device(cfg: Config | str, seed: int | None = None, sets: int = 1, device="cuda:0") -> dict:
    """The same recipe as ``make_inputs``, drawn on the GPU with torch's
    seeded generator (Philox), for throughput runs at shapes whose host-side
    draw would take minutes (the 4.3 GB embedding table of the d = 8192
    workload).  The values follow the same distributions but are not the
    numpy draws, so nothing is compared against the oracle with them.

    Returns torch tensors on ``device`` (bf16 or fp32 per the config): E,
    P_e, P_h, W_f, W_pair, W1, b1, w2, b2 (float), and ``sets`` independent
    (logits [N*B, V], h [N, B, d]) pairs under "sets".
    """
    import torch
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    D = cfg.dims
    dt = torch.bfloat16 if D.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device).manual_seed(seed)

    def normal(shape, std):
        return (torch.randn(shape, generator=gen, device=device) * std).to(dt)

    def xavier(shape):
        return normal(shape, float(np.sqrt(2.0 / (shape[0] + shape[1]))))

    out = {"dims": D, "cfg": cfg}
    E = torch.empty((D.V, D.e), dtype=dt, device=device)
    step = max(1, (1 << 26) // D.e)
    for r0 in range(0, D.V, step):
        r1 = min(D.V, r0 + step)
        E[r0:r1] = normal((r1 - r0, D.e), 0.02)
    out["E"] = E
    out["P_e"] = xavier((D.r, D.e))
    out["P_h"] = xavier((D.r, D.d))
    out["W_f"] = xavier((D.r_z, 2 * D.r))
    out["W_pair"] = xavier((D.r_s, 2 * D.d))
    out["W1"] = xavier((D.H, 2 * D.r_z + D.r_s))
    out["b1"] = torch.zeros(D.H, dtype=dt, device=device)
    out["w2"] = xavier((1, D.H))[0].contiguous()
    out["b2"] = 0.0
    R = D.n_blocks * D.B
    P = cfg.n_peaks
    peak_vals = 20.0 + 0.5 * torch.arange(P, device=device, dtype=torch.float32)
    out["sets"] = []
    for _ in range(sets):
        h = normal((D.n_blocks, D.B, D.d), cfg.h_scale)
        lg = torch.empty((R, D.V), dtype=dt, device=device)
        for r0 in range(0, R, 64):
            r1 = min(R, r0 + 64)
            x = (torch.randn((r1 - r0, D.V), generator=gen, device=device) * 2.0).clamp_(-12.0, 12.0)
            if P:
                # P distinct random ids per row, given the planted values in a random order
                pos = torch.rand((r1 - r0, D.V), generator=gen, device=device).topk(P, dim=1).indices
                order = torch.rand((r1 - r0, P), generator=gen, device=device).argsort(dim=1)
                x.scatter_(1, pos, peak_vals[order])
            lg[r0:r1] = x.to(dt)
        out["sets"].append((lg, h))
    # the draws ran on torch's current stream; finish them so that a caller
    # reading these tensors on another stream sees the values
    torch.cuda.synchronize(device)
    return out
