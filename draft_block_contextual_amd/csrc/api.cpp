// C ABI of libdcoco: argument checks, workspace layout and the launch sequence
// of each entry point on the caller's stream.  The operations themselves are
// specified in include/dcoco.h.
#include "../../include/dcoco.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "kernels.h"

using namespace dcoco;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == DCOCO_BF16 ? 2 : 4; }

int check_width(int32_t w, int32_t maxw) {
  if (w <= 0) return DCOCO_ERR_INVALID_ARG;
  if (w % 32 != 0 || w > maxw) return DCOCO_ERR_UNSUPPORTED;
  return DCOCO_OK;
}

int check_dims(const dcoco_dims* d, bool need_widths) {
  if (!d) return DCOCO_ERR_INVALID_ARG;
  if (d->dtype != DCOCO_F32 && d->dtype != DCOCO_BF16) return DCOCO_ERR_INVALID_ARG;
  if (d->n_blocks < 1 || d->B < 1 || d->K < 1 || d->V < 1 || d->K > d->V) return DCOCO_ERR_INVALID_ARG;
  if (!(d->ln_eps > 0.0f) || !std::isfinite(d->ln_eps)) return DCOCO_ERR_INVALID_ARG;
  if (d->K > 64 || d->V > (1 << 30)) return DCOCO_ERR_UNSUPPORTED;
  const long long rows = static_cast<long long>(d->n_blocks) * d->B;
  if (rows * d->K > (1ll << 30) || rows > 65535) return DCOCO_ERR_UNSUPPORTED;
  if (need_widths) {
    int rc;
    if ((rc = check_width(d->d_hidden, 1 << 16)) != DCOCO_OK) return rc;
    if ((rc = check_width(d->d_embed, 1 << 16)) != DCOCO_OK) return rc;
    if ((rc = check_width(d->d_proj, 2048)) != DCOCO_OK) return rc;
    if ((rc = check_width(d->d_z, 2048)) != DCOCO_OK) return rc;
    if ((rc = check_width(d->d_pair, 2048)) != DCOCO_OK) return rc;
    if ((rc = check_width(d->d_mlp, 1 << 16)) != DCOCO_OK) return rc;
  }
  return DCOCO_OK;
}

int check_weights(const dcoco_weights* w, bool rep, bool score) {
  if (!w) return DCOCO_ERR_INVALID_ARG;
  if (rep) {
    if (!w->P_e || !w->P_h || !w->W_f || !w->W_pair) return DCOCO_ERR_INVALID_ARG;
    if (!aligned16(w->P_e) || !aligned16(w->P_h) || !aligned16(w->W_f) || !aligned16(w->W_pair))
      return DCOCO_ERR_INVALID_ARG;
  }
  if (score) {
    if (!w->W1 || !w->w2) return DCOCO_ERR_INVALID_ARG;
    if (!aligned16(w->W1) || !aligned16(w->w2) || (w->b1 && !aligned16(w->b1))) return DCOCO_ERR_INVALID_ARG;
    if (!std::isfinite(w->b2)) return DCOCO_ERR_INVALID_ARG;
  }
  return DCOCO_OK;
}

bool ptr_ok(const void* p) { return p && aligned16(p); }
bool opt_ok(const void* p) { return !p || aligned16(p); }

// Sequential carve-up of a caller workspace.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct RepLayout {
  int split_slot, split_cand;
  float* Y;       // [split_slot][R][r + 2 rs]
  float* U;       // [split_cand][R K][r]
  void* g;        // [R][r]
  float* gf;      // [R][rz]
  void* b;        // [R K][r]
};

// cand = false: no buffers for the gathered projection (table path)
RepLayout carve_rep(Carve& c, const dcoco_dims* d, bool cand = true) {
  RepLayout L;
  const int R = d->n_blocks * d->B;
  const int RK = R * d->K;
  const int ns = d->d_proj + 2 * d->d_pair;
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  L.split_slot = gemm_pick_split(R, ns, d->d_hidden, dt, dt);
  L.split_cand = gemm_pick_split(RK, d->d_proj, d->d_embed, dt, dt);
  L.Y = static_cast<float*>(c.take(sizeof(float) * L.split_slot * static_cast<size_t>(R) * ns));
  L.U = cand ? static_cast<float*>(c.take(sizeof(float) * L.split_cand * static_cast<size_t>(RK) * d->d_proj))
             : nullptr;
  L.g = c.take(esize(d->dtype) * static_cast<size_t>(R) * d->d_proj);
  L.gf = static_cast<float*>(c.take(sizeof(float) * static_cast<size_t>(R) * d->d_z));
  L.b = cand ? c.take(esize(d->dtype) * static_cast<size_t>(RK) * d->d_proj) : nullptr;
  return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DCOCO_OK : DCOCO_ERR_HIP; }

// ---- representation stage, in parts that can run on two streams

// slot side: [P_h; W_L; W_R] h (split-K partials), s_p (+ its bf16 split when
// s3 is given), gf = W_fg LN(P_h h)
// slot side, first half: [P_h; W_pair halves] h as fp32 partials (split k ranges)
GemmProblem slot_gemm_problem(const dcoco_dims* d, const dcoco_weights* w, const void* h, const RepLayout& L,
                              int split) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int R = d->n_blocks * d->B;
  const int r = d->d_proj, rs = d->d_pair, dh = d->d_hidden;
  const int ns = r + 2 * rs;
  GemmProblem q{};
  q.M = R; q.N = ns; q.Kd = dh;
  q.A = h; q.lda = dh; q.a_rows = nullptr; q.a_dtype = dt;
  q.w[0] = w->P_h; q.ldw[0] = dh; q.col0[0] = 0; q.seg_end[0] = r;
  q.w[1] = w->W_pair; q.ldw[1] = 2ll * dh; q.col0[1] = 0; q.seg_end[1] = r + rs;
  q.w[2] = w->W_pair; q.ldw[2] = 2ll * dh; q.col0[2] = dh; q.seg_end[2] = ns;
  q.w_dtype = dt;
  q.split = split; q.out_f32 = L.Y; q.ldo = ns; q.out = nullptr;
  return q;
}

// slot side, second half: gf = W_fg LN(P_h h) and the pair states (and their
// bf16 split into s3 when given) from `split` partials; without pairs the
// pair states are left to the z launch (bf16 path)
hipError_t slot_finish(const dcoco_dims* d, const dcoco_weights* w, float* s, void* s3, const RepLayout& L,
                       int split, hipStream_t st, bool pairs = true) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int R = d->n_blocks * d->B;
  const int r = d->d_proj, rs = d->d_pair, rz = d->d_z;
  const int ns = r + 2 * rs;
  hipError_t e;
  if (!pairs) {
    if (dt != kDtypeBf16) return hipErrorInvalidValue;
    return launch_ln_gemm_gf(L.Y, split, R, ns, r, d->ln_eps, w->W_f, 2ll * r, r, rz, L.gf, st);
  }
  if (dt == kDtypeBf16 && ln_gemm_pair_supported(r, rs))
    return launch_ln_gemm_pair(L.Y, split, R, ns, r, d->ln_eps, w->W_f, 2ll * r, r, rz, L.gf, d->B, r,
                               r + rs, rs, s, s3, st);
  if ((e = launch_pair_state(L.Y, split, d->n_blocks, d->B, ns, r, r + rs, rs, s, s3, st)) != hipSuccess)
    return e;
  if (dt == kDtypeBf16)
    return launch_ln_gemm(L.Y, split, R, ns, 0, r, d->ln_eps, w->W_f, 2ll * r, r, rz, L.gf, nullptr,
                          nullptr, 1, st);
  if ((e = launch_ln_rows(L.Y, split, R, ns, 0, r, d->ln_eps, L.g, dt, st)) != hipSuccess) return e;
  GemmProblem q{};
  q.M = R; q.N = rz; q.Kd = r;
  q.A = L.g; q.lda = r; q.a_dtype = dt;
  q.w[0] = w->W_f; q.ldw[0] = 2ll * r; q.col0[0] = r; q.seg_end[0] = rz;
  q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = rz;
  q.w_dtype = dt;
  q.split = 1; q.out_f32 = L.gf; q.ldo = rz; q.out = nullptr;
  return launch_gemm(q, st);
}

hipError_t slot_part(const dcoco_dims* d, const dcoco_weights* w, const void* h, float* s, void* s3,
                     const RepLayout& L, hipStream_t st) {
  hipError_t e;
  if ((e = launch_gemm(slot_gemm_problem(d, w, h, L, L.split_slot), st)) != hipSuccess) return e;
  return slot_finish(d, w, s, s3, L, L.split_slot, st);
}

constexpr int kTopkGemmSlots = 3 * 256;   // resident workgroups of the joint launch: three per CU

// top-K of the logits and the slot side.  Where the rows and the slot GEMM
// can share one launch (bf16, aligned rows, K <= 16), the GEMM's k split is
// cut until its tiles and the rows fit the resident workgroup slots once;
// otherwise the slot side and top-K run one after the other.  With pairs
// false the pair states are left to the z launch; *split gets the k split
// of the slot partial sums.
hipError_t topk_and_slot(const dcoco_dims* d, const dcoco_weights* w, const void* logits, const void* h, float* s,
                         void* s3, const RepLayout& L, void* topk_ws, int32_t* ids, float* cl, hipStream_t st,
                         bool pairs = true, int* split = nullptr) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int R = d->n_blocks * d->B;
  if (dt == kDtypeBf16) {
    GemmProblem q = slot_gemm_problem(d, w, h, L, L.split_slot);
    const int row_wgs = topk_gemm_row_workgroups(R, d->V);
    while (q.split > 1 && topk_gemm_workgroups(q) + row_wgs > kTopkGemmSlots) q.split /= 2;
    if (topk_gemm_supported(d->V, d->K, logits, q)) {
      hipError_t e = launch_topk_gemm(logits, R, d->V, d->K, ids, cl, q, topk_ws, st);
      if (e != hipSuccess) return e;
      if (split) *split = q.split;
      return slot_finish(d, w, s, s3, L, q.split, st, pairs);
    }
  }
  if (split) *split = L.split_slot;
  hipError_t e = launch_gemm(slot_gemm_problem(d, w, h, L, L.split_slot), st);
  if (e == hipSuccess) e = slot_finish(d, w, s, s3, L, L.split_slot, st, pairs);
  if (e != hipSuccess) return e;
  return launch_topk(dt, logits, R, d->V, d->K, topk_ws, ids, cl, st);
}

// The pair states can ride on the z launch (bf16, r <= 256): the arguments
// for it, from the slot partial sums of k split `split`.
bool z_pairs(const dcoco_dims* d, const RepLayout& L, int split, float* s, void* s3, PairStateArgs* ps) {
  const long long RK = static_cast<long long>(d->n_blocks) * d->B * d->K;
  const int P = d->n_blocks * (d->B - 1);
  const int r = d->d_proj, rs = d->d_pair;
  if (d->dtype != DCOCO_BF16 || r > 256 || P <= 0 || RK > (1ll << 30) || split > 4 ||
      !ln_gemm_pair_supported(r, rs) || !ln_gemm_pairs_fit(static_cast<int>(RK), P, rs))
    return false;
  if (ps == nullptr) return true;
  ps->Y = L.Y; ps->split = split; ps->ldy = r + 2 * rs; ps->B = d->B; ps->cl = r; ps->cr = r + rs; ps->rs = rs;
  ps->P = P; ps->s = s; ps->s3 = s3;
  return true;
}

// candidate side, first half: P_e E[c] over gathered rows (split-K partials)
hipError_t cand_gemm(const dcoco_dims* d, const dcoco_weights* w, const void* E, const int32_t* ids,
                     const RepLayout& L, hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int RK = d->n_blocks * d->B * d->K;
  const int r = d->d_proj;
  GemmProblem q{};
  q.M = RK; q.N = r; q.Kd = d->d_embed;
  q.A = E; q.lda = d->d_embed; q.a_rows = ids; q.a_rows_max = d->V - 1; q.a_dtype = dt;
  q.w[0] = w->P_e; q.ldw[0] = d->d_embed; q.col0[0] = 0; q.seg_end[0] = r;
  q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = r;
  q.w_dtype = dt;
  q.split = L.split_cand; q.out_f32 = L.U; q.ldo = r; q.out = nullptr;
  return launch_gemm(q, st);
}

// candidate side, second half (needs gf): z = W_fb LN(P_e E[c]) + gf[slot]
// (bf16: with ps, the pair states in the same launch)
hipError_t cand_finish(const dcoco_dims* d, const dcoco_weights* w, void* z, const RepLayout& L,
                       hipStream_t st, const PairStateArgs* ps = nullptr) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int RK = d->n_blocks * d->B * d->K;
  const int r = d->d_proj, rz = d->d_z;
  if (dt == kDtypeBf16)
    return launch_ln_gemm(L.U, L.split_cand, RK, r, 0, r, d->ln_eps, w->W_f, 2ll * r, 0, rz, nullptr, z, L.gf,
                          d->K, st, ps);
  if (ps) return hipErrorInvalidValue;
  hipError_t e;
  if ((e = launch_ln_rows(L.U, L.split_cand, RK, r, 0, r, d->ln_eps, L.b, dt, st)) != hipSuccess) return e;
  GemmProblem q{};
  q.M = RK; q.N = rz; q.Kd = r;
  q.A = L.b; q.lda = r; q.a_dtype = dt;
  q.w[0] = w->W_f; q.ldw[0] = 2ll * r; q.col0[0] = 0; q.seg_end[0] = rz;
  q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = rz;
  q.w_dtype = dt;
  q.split = 1; q.out = z; q.out_dtype = dt; q.ldo = rz;
  q.row_bias = L.gf; q.row_bias_div = d->K; q.col_bias = nullptr;
  return launch_gemm(q, st);
}

// representation stage on one stream (see dcoco_represent)
hipError_t run_represent(const dcoco_dims* d, const dcoco_weights* w, const void* h, const void* E,
                         const int32_t* ids, void* z, float* s, const RepLayout& L, hipStream_t st) {
  hipError_t e;
  if ((e = slot_part(d, w, h, s, nullptr, L, st)) != hipSuccess) return e;
  if ((e = cand_gemm(d, w, E, ids, L, st)) != hipSuccess) return e;
  return cand_finish(d, w, z, L, st);
}

// the scores come from the on-chip slab kernels (no A, B buffer)
bool use_slab(const dcoco_dims* d) {
  return score_slab_preferred(d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32, d->n_blocks, d->B, d->K, d->d_z,
                              d->d_mlp);
}

// scoring stage buffers
struct ScoreLayout {
  void* s3;       // bf16 [3, P, rs] (bf16 path only)
  float* C;       // fp32 [nq, P, H]; null when the slab launch forms the pair term
  float* AB;      // fp32 [N*B*K, 2H] (A, B through memory), else null
  float* part;    // fp32 [nslab, P, K, K] (slab kernels), else null
  bool c_chip;    // the slab launch forms W1s s_p from s3 (no C buffer, no pair-term GEMM)
};

// with_ab: the A, B buffer even where the slab kernels score (training needs it)
ScoreLayout carve_score(Carve& c, const dcoco_dims* d, bool with_ab = false) {
  ScoreLayout L;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  const size_t RK = static_cast<size_t>(d->n_blocks) * d->B * d->K;
  const int nq = d->dtype == DCOCO_BF16 ? 3 : 1;
  const bool slab = use_slab(d);
  L.c_chip = slab && !with_ab && d->dtype == DCOCO_BF16 &&
             score_slab_c_on_chip(d->n_blocks, d->B, d->K, d->d_mlp, d->d_pair);
  L.s3 = c.take(d->dtype == DCOCO_BF16 ? 3 * P * d->d_pair * 2 : 0);
  L.C = L.c_chip ? nullptr : static_cast<float*>(c.take(sizeof(float) * nq * P * d->d_mlp));
  L.AB = (with_ab || !slab) ? static_cast<float*>(c.take(sizeof(float) * RK * 2 * d->d_mlp)) : nullptr;
  L.part = slab ? static_cast<float*>(c.take(score_slab_part_bytes(d->n_blocks, d->B, d->K, d->d_mlp)))
                : nullptr;
  return L;
}

// pair term: C_p parts = W1s s_p (bf16 path: s split into hi/mid/lo rows; the
// split is made here unless s3_ready).  Where the slab launch forms the
// product itself, only the split is made.
hipError_t pair_term(const dcoco_dims* d, const dcoco_weights* w, const float* s, const ScoreLayout& L,
                     bool s3_ready, hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int P = d->n_blocks * (d->B - 1);
  if (P == 0) return hipSuccess;
  const int rz = d->d_z, rs = d->d_pair, H = d->d_mlp;
  const int nq = dt == kDtypeBf16 ? 3 : 1;
  hipError_t e;
  if (dt == kDtypeBf16 && !s3_ready &&
      (e = launch_split3(s, static_cast<long long>(P) * rs, L.s3, st)) != hipSuccess)
    return e;
  if (L.c_chip) return hipSuccess;
  GemmProblem q{};
  q.M = nq * P; q.N = H; q.Kd = rs;
  q.A = dt == kDtypeBf16 ? L.s3 : static_cast<const void*>(s); q.lda = rs; q.a_dtype = dt;
  q.w[0] = w->W1; q.ldw[0] = 2ll * rz + rs; q.col0[0] = 2 * rz; q.seg_end[0] = H;
  q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = H;
  q.w_dtype = dt;
  q.split = 1; q.out_f32 = L.C; q.ldo = H; q.out = nullptr;
  return launch_gemm(q, st);
}

// AB = z [W1a; W1b]^T (fp32)
hipError_t ab_gemm(const dcoco_dims* d, const dcoco_weights* w, const void* z, const ScoreLayout& L,
                   hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int rz = d->d_z, rs = d->d_pair, H = d->d_mlp;
  const int RK = d->n_blocks * d->B * d->K;
  const long long ldw1 = 2ll * rz + rs;
  GemmProblem q{};
  q.M = RK; q.N = 2 * H; q.Kd = rz;
  q.A = z; q.lda = rz; q.a_dtype = dt;
  q.w[0] = w->W1; q.ldw[0] = ldw1; q.col0[0] = 0; q.seg_end[0] = H;
  q.w[1] = w->W1; q.ldw[1] = ldw1; q.col0[1] = rz; q.seg_end[1] = 2 * H;
  q.w[2] = w->W1; q.ldw[2] = ldw1; q.col0[2] = rz; q.seg_end[2] = 2 * H;
  q.w_dtype = dt;
  q.split = 1; q.out_f32 = L.AB; q.ldo = 2 * H; q.out = nullptr;
  return launch_gemm(q, st);
}

// The walk's outputs, when the scoring launches may also walk.
struct WalkOut {
  const int32_t* ids;
  int32_t* sel_idx;
  int32_t* sel_tok;
};

// the scores (need the pair term): the slab kernels, else A, B through memory
// and the grid.  With best, the walk's table.  With wk on the slab path (and a
// block that fits), the finishing launch walks each block itself and
// *walked is set; the caller then launches no walk.
hipError_t score_tail(const dcoco_dims* d, const dcoco_weights* w, const void* z, const float* cl, float* S,
                      const ScoreLayout& L, hipStream_t st, int32_t* best = nullptr, const WalkOut* wk = nullptr,
                      bool* walked = nullptr) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int P = d->n_blocks * (d->B - 1);
  if (walked) *walked = false;
  if (P == 0) return hipSuccess;
  const int H = d->d_mlp;
  hipError_t e;
  if (L.part != nullptr) {
    ScoreSlabProblem q{};
    q.N = d->n_blocks; q.B = d->B; q.K = d->K; q.H = H; q.rz = d->d_z;
    q.z = z; q.W1 = w->W1; q.ldw1 = 2ll * d->d_z + d->d_pair;
    q.C = L.C; q.nq = dt == kDtypeBf16 ? 3 : 1; q.b1 = w->b1; q.w2 = w->w2; q.b2 = w->b2;
    q.s3 = L.c_chip ? L.s3 : nullptr; q.rs = d->d_pair;
    q.cand_logits = cl; q.part = L.part; q.S = S; q.best = best;
    const bool walk = wk != nullptr && block_finish_walk_fits(d->B, d->K, d->d_mlp);
    if (walk) {
      q.cand_ids = wk->ids; q.sel_idx = wk->sel_idx; q.sel_tok = wk->sel_tok;
    }
    e = launch_score_slab(q, st);
    if (e == hipSuccess && walked) *walked = walk;
    return e;
  }
  if ((e = ab_gemm(d, w, z, L, st)) != hipSuccess) return e;
  GridProblem g{};
  g.N = d->n_blocks; g.B = d->B; g.K = d->K; g.H = H; g.dtype = dt;
  g.AB = L.AB; g.C = L.C; g.nq = dt == kDtypeBf16 ? 3 : 1; g.b1 = w->b1; g.w2 = w->w2; g.b2 = w->b2;
  g.cand_logits = cl; g.S = S; g.best = best;
  return launch_grid(g, st);
}

// The greedy walk after the grid: from the grid's argmax table when the block
// fits the table walk, else from S.
hipError_t walk_after_grid(const float* S, const int32_t* best, const float* cl, const int32_t* ids,
                           const dcoco_dims* d, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st) {
  if (best != nullptr)
    return launch_walk_table(best, cl, ids, d->n_blocks, d->B, d->K, sel_idx, sel_tok, st);
  return launch_walk(S, cl, ids, d->n_blocks, d->B, d->K, sel_idx, sel_tok, st);
}

hipError_t run_score(const dcoco_dims* d, const dcoco_weights* w, const void* z, const float* s,
                     const float* cl, float* S, const ScoreLayout& L, hipStream_t st) {
  hipError_t e;
  if ((e = pair_term(d, w, s, L, false, st)) != hipSuccess) return e;
  return score_tail(d, w, z, cl, S, L, st);
}

constexpr int kTableChunk = 8192;   // table rows projected per launch pair

int check_ws(void* ws, size_t* bytes, size_t need) {
  if (!bytes) return DCOCO_ERR_INVALID_ARG;
  need = need < kAlign ? kAlign : need;   // never 0: NULL always means "size query"
  if (!ws) {
    *bytes = need;
    return 1;   // size query answered
  }
  if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0 || *bytes < need) return DCOCO_ERR_WORKSPACE;
  return DCOCO_OK;
}

constexpr int kMaxGradSplit = 16;

// bf16 storage: the two large gradient products run on bf16 MFMA over a
// two-part split of the fp32 gradients (the row-reduction kernel)
bool bwd_on_mfma(const dcoco_dims* d) { return d->dtype == DCOCO_BF16; }

size_t wgrad_part_floats(int M, int N, int Kd);

struct BwdLayout {
  ScoreLayout SL;
  float* dAB;      // [N*B*K, 2H]
  float* dC;       // [P, H]
  float* dw2p;     // [P, H]
  float* part;     // split partial products
  size_t part_floats;
  float* red;      // partial sums of the reductions
};

BwdLayout carve_bwd(Carve& c, const dcoco_dims* d) {
  BwdLayout L;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  const size_t RK = static_cast<size_t>(d->n_blocks) * d->B * d->K;
  const size_t H = d->d_mlp;
  L.SL = carve_score(c, d, true);  // the backward reads A and B
  L.dAB = static_cast<float*>(c.take(sizeof(float) * RK * 2 * H));
  L.dC = static_cast<float*>(c.take(sizeof(float) * P * H));
  L.dw2p = static_cast<float*>(c.take(sizeof(float) * P * H));
  L.part_floats = kMaxGradSplit * std::max(H, P) * std::max(d->d_z, d->d_pair);
  if (bwd_on_mfma(d))
    L.part_floats = std::max({L.part_floats, wgrad_part_floats(static_cast<int>(RK), d->d_z, 2 * d->d_mlp),
                              wgrad_part_floats(2 * d->d_mlp, d->d_z, static_cast<int>(RK))});
  L.part = static_cast<float*>(c.take(sizeof(float) * L.part_floats));
  const size_t red = static_cast<size_t>(mlp_reduce_floats(static_cast<int>(P), static_cast<int>(H), d->n_blocks,
                                                            d->B, d->K));
  L.red = static_cast<float*>(c.take(sizeof(float) * red));
  return L;
}

// C[M, N] = sum over Kd of A(m, k) B(k, n), split over k so the launch has
// about 256 workgroups, the splits added in order into out (row stride ldo)
hipError_t grad_product(GemmF32Args q, int a_dt, int b_dt, float* part, float* out, long long ldo,
                        hipStream_t st) {
  const int tiles = ((q.M + 63) / 64) * ((q.N + 63) / 64);
  int splits = std::max(1, std::min(kMaxGradSplit, 256 / std::max(tiles, 1)));
  splits = std::min(splits, std::max(1, q.K / 64));
  q.k_split = ((q.K + splits - 1) / splits + 15) / 16 * 16;
  splits = (q.K + q.k_split - 1) / q.k_split;
  q.C = part; q.ldc = q.N; q.c_split = static_cast<long long>(q.M) * q.N; q.accumulate = 0;
  hipError_t e = launch_gemm_f32(q, a_dt, b_dt, st);
  if (e != hipSuccess) return e;
  return launch_sum_splits(part, splits, q.M, q.N, out, ldo, st);
}

// ---- gradient products on the row-reduction kernel

// one destination of a product's output rows (consecutive segments)
struct OutSeg {
  float* c;
  long long ld;
  int rows;
};

// split-K choice for a product, never more than the partial buffer holds
int wgrad_split_for(int M, int N, int Kd, size_t part_floats) {
  int split = wgrad_pick_split(M, N, Kd);
  while (split > 1 && static_cast<size_t>(split) * M * N > part_floats) split /= 2;
  return split;
}

size_t wgrad_part_floats(int M, int N, int Kd) {
  const int split = wgrad_pick_split(M, N, Kd);
  return split > 1 ? static_cast<size_t>(split) * M * N : 0;
}

// runs the product p (A, B, M, N, Kd set) with its output rows going to
// segs[0..nseg) in order; with a k split, through fp32 partials summed in order
hipError_t wgrad_run(WgradArgs p, bool rr, const OutSeg* segs, int nseg, float* part, size_t part_floats,
                     hipStream_t st) {
  const int split = wgrad_split_for(p.M, p.N, p.Kd, part_floats);
  if (split == 1) {
    p.c0 = segs[0].c; p.ldc0 = segs[0].ld; p.cend0 = segs[0].rows;
    if (nseg > 1) { p.c1 = segs[1].c; p.ldc1 = segs[1].ld; p.cend1 = segs[0].rows + segs[1].rows; }
    if (nseg > 2) { p.c2 = segs[2].c; p.ldc2 = segs[2].ld; }
    return launch_wgrad(p, rr, 1, st);
  }
  p.c0 = part; p.ldc0 = p.N; p.c_split = static_cast<long long>(p.M) * p.N;
  hipError_t e = launch_wgrad(p, rr, split, st);
  if (e != hipSuccess) return e;
  SegOut o{};
  o.out0 = segs[0].c; o.ld0 = segs[0].ld; o.end0 = segs[0].rows;
  o.out1 = nseg > 1 ? segs[1].c : segs[0].c; o.ld1 = nseg > 1 ? segs[1].ld : segs[0].ld;
  o.end1 = nseg > 1 ? segs[0].rows + segs[1].rows : p.M;
  o.out2 = nseg > 2 ? segs[2].c : o.out1; o.ld2 = nseg > 2 ? segs[2].ld : o.ld1;
  return launch_sum_splits_seg(part, wgrad_grid_splits(p.Kd, split), p.c_split, p.M, p.N, o, st);
}

// ---- representation backward (bf16 storage)

struct RepBwdLayout {
  int split_h, split_e;    // forward recompute: split-K of P_h h and P_e E[c]
  float* Y;                // [split_h][R][r]: P_h h partials
  float* U;                // [split_e][RK][r]: P_e E[c] partials
  float* dBG;              // [RK, 2 r]: dz W_f (db | per-candidate part of dg)
  void* BG;                // bf16 [RK, 2 r]: b | g repeated over the slot's candidates
  float* dxe;              // [RK, r]
  float* Acat;             // [R, C]: dx_h | ds at the left slot | ds at the right slot
  float* part;             // split partial products
  size_t part_floats;
};

RepBwdLayout carve_rep_bwd(Carve& c, const dcoco_dims* d) {
  RepBwdLayout L;
  const int R = d->n_blocks * d->B;
  const int RK = R * d->K;
  const int r = d->d_proj, rz = d->d_z, rs = d->d_pair, dh = d->d_hidden, de = d->d_embed;
  const int C = r + 2 * rs;
  L.split_h = gemm_pick_split(R, r, dh, kDtypeBf16, kDtypeBf16);
  L.split_e = gemm_pick_split(RK, r, de, kDtypeBf16, kDtypeBf16);
  const size_t RKs = RK, Rs = R;
  L.Y = static_cast<float*>(c.take(4 * L.split_h * Rs * r));
  L.U = static_cast<float*>(c.take(4 * L.split_e * RKs * r));
  L.dBG = static_cast<float*>(c.take(4 * RKs * 2 * r));
  L.BG = c.take(2 * RKs * 2 * r);
  L.dxe = static_cast<float*>(c.take(4 * RKs * r));
  L.Acat = static_cast<float*>(c.take(4 * Rs * C));
  L.part_floats = std::max({wgrad_part_floats(RK, 2 * r, rz), wgrad_part_floats(rz, 2 * r, RK),
                            wgrad_part_floats(r, de, RK), wgrad_part_floats(C, dh, R), wgrad_part_floats(R, dh, C)});
  L.part = static_cast<float*>(c.take(4 * std::max<size_t>(L.part_floats, 1)));
  return L;
}

hipError_t run_rep_backward(const dcoco_dims* d, const dcoco_weights* w, const void* h, const void* E,
                            const int32_t* ids, const float* dz, const float* ds, const dcoco_rep_grads* g,
                            float* dh_out, const RepBwdLayout& L, hipStream_t st) {
  const int N = d->n_blocks, B = d->B, K = d->K;
  const int R = N * B, RK = R * K;
  const int r = d->d_proj, rz = d->d_z, rs = d->d_pair, dh = d->d_hidden, de = d->d_embed;
  const int C = r + 2 * rs;
  const uint16_t* Wf = static_cast<const uint16_t*>(w->W_f);
  const uint16_t* Wp = static_cast<const uint16_t*>(w->W_pair);
  uint16_t* BG = static_cast<uint16_t*>(L.BG);
  hipError_t e = hipSuccess;
  // forward recompute: x_h = P_h h, x_e = P_e E[c] (split-K partials)
  {
    GemmProblem q{};
    q.M = R; q.N = r; q.Kd = dh;
    q.A = h; q.lda = dh; q.a_dtype = kDtypeBf16;
    q.w[0] = w->P_h; q.ldw[0] = dh; q.col0[0] = 0;
    q.seg_end[0] = q.seg_end[1] = q.seg_end[2] = r;
    q.w_dtype = kDtypeBf16;
    q.split = L.split_h; q.out_f32 = L.Y; q.ldo = r; q.out = nullptr;
    e = launch_gemm(q, st);
  }
  if (e == hipSuccess) {
    GemmProblem q{};
    q.M = RK; q.N = r; q.Kd = de;
    q.A = E; q.lda = de; q.a_rows = ids; q.a_rows_max = d->V - 1; q.a_dtype = kDtypeBf16;
    q.w[0] = w->P_e; q.ldw[0] = de; q.col0[0] = 0;
    q.seg_end[0] = q.seg_end[1] = q.seg_end[2] = r;
    q.w_dtype = kDtypeBf16;
    q.split = L.split_e; q.out_f32 = L.U; q.ldo = r; q.out = nullptr;
    e = launch_gemm(q, st);
  }
  // dBG = dz [W_fb | W_fg]
  if (e == hipSuccess) {
    WgradArgs p;
    p.M = RK; p.N = 2 * r; p.Kd = rz;
    p.A = dz; p.lda = rz;
    p.b0 = Wf; p.ldb0 = 2ll * r;
    const OutSeg o{L.dBG, 2ll * r, RK};
    e = wgrad_run(p, false, &o, 1, L.part, L.part_floats, st);
  }
  // LayerNorm forward (b, and g once per candidate, into BG) and backward
  // (dx_e; dx_h into Acat); ds placed by slot
  if (e == hipSuccess)
    e = launch_ln_fwd_bwd(L.U, L.split_e, RK, r, 0, r, d->ln_eps, L.dBG, 2ll * r, 0, 1, BG, 2ll * r, 1, L.dxe, r, st);
  if (e == hipSuccess)
    e = launch_ln_fwd_bwd(L.Y, L.split_h, R, r, 0, r, d->ln_eps, L.dBG, 2ll * r, r, K, BG + r, 2ll * r, K, L.Acat, C,
                          st);
  if (e == hipSuccess) e = launch_pack_ds(ds, N, B, rs, r, C, L.Acat, st);
  // dW_f = dz^T [b | g]
  if (e == hipSuccess) {
    WgradArgs p;
    p.M = rz; p.N = 2 * r; p.Kd = RK;
    p.A = dz; p.lda = rz;
    p.b0 = BG; p.ldb0 = 2ll * r;
    const OutSeg o{g->dW_f, 2ll * r, rz};
    e = wgrad_run(p, true, &o, 1, L.part, L.part_floats, st);
  }
  // dP_e = dx_e^T E[c] (E rows gathered by candidate id)
  if (e == hipSuccess) {
    WgradArgs p;
    p.M = r; p.N = de; p.Kd = RK;
    p.A = L.dxe; p.lda = r;
    p.b0 = static_cast<const uint16_t*>(E); p.ldb0 = de;
    p.bmap.mode = 1; p.bmap.ids = ids; p.bmap.idmax = d->V - 1;
    const OutSeg o{g->dP_e, de, r};
    e = wgrad_run(p, true, &o, 1, L.part, L.part_floats, st);
  }
  // [dP_h; dW_L; dW_R] = Acat^T h
  if (e == hipSuccess) {
    WgradArgs p;
    p.M = C; p.N = dh; p.Kd = R;
    p.A = L.Acat; p.lda = C;
    p.b0 = static_cast<const uint16_t*>(h); p.ldb0 = dh;
    const OutSeg o[3] = {{g->dP_h, dh, r}, {g->dW_pair, 2ll * dh, rs}, {g->dW_pair + dh, 2ll * dh, rs}};
    e = wgrad_run(p, true, o, 3, L.part, L.part_floats, st);
  }
  if (!dh_out || e != hipSuccess) return e;
  // dh = Acat [P_h; W_L; W_R]
  WgradArgs p;
  p.M = R; p.N = dh; p.Kd = C;
  p.A = L.Acat; p.lda = C;
  p.b0 = static_cast<const uint16_t*>(w->P_h); p.ldb0 = dh; p.bend0 = r;
  p.b1 = Wp; p.ldb1 = 2ll * dh; p.bend1 = r + rs;
  p.b2 = Wp + dh; p.ldb2 = 2ll * dh;
  const OutSeg o{dh_out, dh, R};
  return wgrad_run(p, false, &o, 1, L.part, L.part_floats, st);
}

// ---- the static scratch buffer of dcoco_correct_block_static

// One buffer per GPU, in the library's code object (each device that loads the
// library holds its own copy until the process ends).  Host code never uses
// this name as an address: the device address comes from hipGetSymbolAddress.
__device__ __align__(256) char scratch[DCOCO_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch`, looked up once per device
int static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DCOCO_ERR_HIP;
  if (dev >= kMaxDevices) return DCOCO_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return DCOCO_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DCOCO_OK;
}

}  // namespace

extern "C" {

int dcoco_abi_version(void) { return 108; }

size_t dcoco_static_scratch_bytes(void) { return DCOCO_STATIC_SCRATCH_BYTES; }

const char* dcoco_status_string(int status) {
  switch (status) {
    case DCOCO_OK: return "ok";
    case DCOCO_ERR_INVALID_ARG: return "invalid argument";
    case DCOCO_ERR_UNSUPPORTED: return "unsupported shape";
    case DCOCO_ERR_WORKSPACE: return "workspace too small or misaligned";
    case DCOCO_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dcoco_topk(const dcoco_dims* d, const void* logits, int32_t* cand_ids, float* cand_logits,
               void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, false);
  if (rc != DCOCO_OK) return rc;
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  if (!topk_supported(dt, d->V, d->K)) return DCOCO_ERR_UNSUPPORTED;
  const int R = d->n_blocks * d->B;
  Carve c(nullptr);
  c.take(topk_workspace_bytes(dt, R, d->V, d->K));
  rc = check_ws(workspace, workspace_bytes, c.off);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if (!ptr_ok(logits) || !ptr_ok(cand_ids) || !ptr_ok(cand_logits)) return DCOCO_ERR_INVALID_ARG;
  return hip_status(launch_topk(dt, logits, R, d->V, d->K, workspace, cand_ids, cand_logits,
                                static_cast<hipStream_t>(stream)));
}

int dcoco_represent(const dcoco_dims* d, const dcoco_weights* w, const void* h, const void* E,
                    const int32_t* cand_ids, void* z, float* s, void* workspace,
                    size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  Carve c(nullptr);
  carve_rep(c, d);
  rc = check_ws(workspace, workspace_bytes, c.off);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if ((rc = check_weights(w, true, false)) != DCOCO_OK) return rc;
  if (!ptr_ok(h) || !ptr_ok(E) || !ptr_ok(cand_ids) || !ptr_ok(z)) return DCOCO_ERR_INVALID_ARG;
  if (d->B > 1 && !ptr_ok(s)) return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  const RepLayout L = carve_rep(cw, d);
  return hip_status(run_represent(d, w, h, E, cand_ids, z, s, L, static_cast<hipStream_t>(stream)));
}

int dcoco_score(const dcoco_dims* d, const dcoco_weights* w, const void* z, const float* s,
                const float* cand_logits, float* S, void* workspace, size_t* workspace_bytes,
                void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  Carve c(nullptr);
  carve_score(c, d);
  rc = check_ws(workspace, workspace_bytes, c.off);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if ((rc = check_weights(w, false, true)) != DCOCO_OK) return rc;
  if (P == 0) return DCOCO_OK;
  if (!ptr_ok(z) || !ptr_ok(s) || !ptr_ok(cand_logits) || !ptr_ok(S)) return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  const ScoreLayout SL = carve_score(cw, d);
  return hip_status(run_score(d, w, z, s, cand_logits, S, SL, static_cast<hipStream_t>(stream)));
}

int dcoco_select(const dcoco_dims* d, const float* S, const float* cand_logits, const int32_t* cand_ids,
                 int32_t* sel_idx, int32_t* sel_tok, void* stream) {
  int rc = check_dims(d, false);
  if (rc != DCOCO_OK) return rc;
  if (!ptr_ok(cand_logits) || !ptr_ok(cand_ids) || !ptr_ok(sel_tok) || !opt_ok(sel_idx))
    return DCOCO_ERR_INVALID_ARG;
  if (d->B > 1 && !ptr_ok(S)) return DCOCO_ERR_INVALID_ARG;
  return hip_status(launch_walk(S, cand_logits, cand_ids, d->n_blocks, d->B, d->K, sel_idx, sel_tok,
                                static_cast<hipStream_t>(stream)));
}

int dcoco_select_path(const dcoco_dims* d, const float* S, const float* cand_logits, const int32_t* cand_ids,
                      int rule, float lambda, int32_t* sel_idx, int32_t* sel_tok, void* stream) {
  if (rule == DCOCO_PATH_GREEDY) return dcoco_select(d, S, cand_logits, cand_ids, sel_idx, sel_tok, stream);
  if (rule != DCOCO_PATH_GLOBAL_SUM && rule != DCOCO_PATH_DISCOUNT) return DCOCO_ERR_INVALID_ARG;
  const float lam = rule == DCOCO_PATH_GLOBAL_SUM ? 1.0f : lambda;
  if (!(lam > 0.0f && lam <= 1.0f)) return DCOCO_ERR_INVALID_ARG;   // also rejects NaN
  int rc = check_dims(d, false);
  if (rc != DCOCO_OK) return rc;
  if (!ptr_ok(cand_logits) || !ptr_ok(cand_ids) || !ptr_ok(sel_tok) || !opt_ok(sel_idx))
    return DCOCO_ERR_INVALID_ARG;
  if (d->B > 1 && !ptr_ok(S)) return DCOCO_ERR_INVALID_ARG;
  if (!path_supported(d->B, d->K)) return DCOCO_ERR_UNSUPPORTED;
  return hip_status(launch_path(S, cand_logits, cand_ids, d->n_blocks, d->B, d->K, lam, sel_idx, sel_tok,
                                static_cast<hipStream_t>(stream)));
}

int dcoco_lm_head_topk(const dcoco_dims* d, const void* hd, const void* W_lm, int32_t* cand_ids,
                       float* cand_logits, void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, false);
  if (rc != DCOCO_OK) return rc;
  const int M = d->n_blocks * d->B;
  if (d->dtype != DCOCO_BF16 || !lm_head_topk_supported(M, d->V, d->d_hidden, d->K)) return DCOCO_ERR_UNSUPPORTED;
  rc = check_ws(workspace, workspace_bytes, lm_head_workspace_bytes(M, d->V, d->K));
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if (!ptr_ok(hd) || !ptr_ok(W_lm) || !ptr_ok(cand_ids) || !ptr_ok(cand_logits)) return DCOCO_ERR_INVALID_ARG;
  return hip_status(launch_lm_head_topk(hd, W_lm, M, d->V, d->d_hidden, d->K, workspace, cand_ids, cand_logits,
                                        static_cast<hipStream_t>(stream)));
}

int dcoco_loss(const dcoco_dims* d, const float* S, const int32_t* cand_ids, const int32_t* target_tok,
               float rho, float* loss, float* pair_loss, float* dS, void* stream) {
  int rc = check_dims(d, false);
  if (rc != DCOCO_OK) return rc;
  if (!(rho > 0.0f) || !std::isfinite(rho)) return DCOCO_ERR_INVALID_ARG;
  if (!ptr_ok(cand_ids) || !ptr_ok(target_tok) || !ptr_ok(loss)) return DCOCO_ERR_INVALID_ARG;
  if (d->B > 1 && (!ptr_ok(S) || !ptr_ok(pair_loss) || !ptr_ok(dS))) return DCOCO_ERR_INVALID_ARG;
  return hip_status(launch_loss(S, cand_ids, target_tok, d->n_blocks, d->B, d->K, rho, pair_loss, loss, dS,
                                static_cast<hipStream_t>(stream)));
}

int dcoco_score_backward(const dcoco_dims* d, const dcoco_weights* w, const void* z, const float* s,
                         const float* dS, float* dz, float* ds, float* d_cand_logits, const dcoco_mlp_grads* g,
                         void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  Carve c(nullptr);
  carve_bwd(c, d);
  rc = check_ws(workspace, workspace_bytes, c.off);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if ((rc = check_weights(w, false, true)) != DCOCO_OK) return rc;
  if (!g || !ptr_ok(g->dW1) || !ptr_ok(g->db1) || !ptr_ok(g->dw2) || !ptr_ok(g->db2) || !ptr_ok(dz) ||
      !opt_ok(ds) || !opt_ok(d_cand_logits))
    return DCOCO_ERR_INVALID_ARG;
  const int P = d->n_blocks * (d->B - 1);
  if (P > 0 && (!ptr_ok(z) || !ptr_ok(s) || !ptr_ok(dS))) return DCOCO_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int rz = d->d_z, rs = d->d_pair, H = d->d_mlp;
  const int RK = d->n_blocks * d->B * d->K;
  const long long ldw1 = 2ll * rz + rs;
  hipError_t e = hipSuccess;
  if (P == 0) {
    // no transitions: every gradient is zero
    if (e == hipSuccess) e = launch_fill(dz, static_cast<long long>(RK) * rz, 0.f, st);
    if (e == hipSuccess) e = launch_fill(g->dW1, H * ldw1, 0.f, st);
    if (e == hipSuccess) e = launch_fill(g->db1, H, 0.f, st);
    if (e == hipSuccess) e = launch_fill(g->dw2, H, 0.f, st);
    if (e == hipSuccess) e = launch_fill(g->db2, 1, 0.f, st);
    if (e == hipSuccess && d_cand_logits) e = launch_fill(d_cand_logits, RK, 0.f, st);
    return hip_status(e);
  }
  Carve cw(workspace);
  const BwdLayout L = carve_bwd(cw, d);
  const char* W1 = static_cast<const char*>(w->W1);
  const size_t es = esize(d->dtype);
  // forward recompute: the pair term and A, B
  if (e == hipSuccess) e = pair_term(d, w, s, L.SL, false, st);
  if (e == hipSuccess) e = ab_gemm(d, w, z, L.SL, st);
  if (e == hipSuccess) {
    GridBwdArgs a{};
    a.B = d->B; a.K = d->K; a.H = H; a.P = P; a.nq = dt == kDtypeBf16 ? 3 : 1;
    a.AB = L.SL.AB; a.C = L.SL.C; a.b1 = w->b1; a.w2 = w->w2; a.dS = dS;
    a.dAB = L.dAB; a.dC = L.dC; a.dw2p = L.dw2p;
    e = launch_grid_bwd(a, dt, st);
  }
  if (e == hipSuccess)
    e = launch_mlp_reduce(L.dw2p, L.dC, P, H, dS, d->n_blocks, d->B, d->K, L.red, g->dw2, g->db1, g->db2,
                          d_cand_logits, st);
  if (bwd_on_mfma(d)) {
    const uint16_t* W1u = static_cast<const uint16_t*>(w->W1);
    // dz = dA W1a + dB W1b: one product over 2H, W1's two column blocks
    // stacked along k
    if (e == hipSuccess) {
      WgradArgs p;
      p.M = RK; p.N = rz; p.Kd = 2 * H;
      p.A = L.dAB; p.lda = 2ll * H;
      p.b0 = W1u; p.ldb0 = ldw1; p.bend0 = H;
      p.b1 = W1u + rz; p.ldb1 = ldw1;
      const OutSeg o{dz, rz, RK};
      e = wgrad_run(p, false, &o, 1, L.part, L.part_floats, st);
    }
    // [dW1a; dW1b] = [dA | dB]^T z, reduced over the N*B*K candidate rows
    if (e == hipSuccess) {
      WgradArgs p;
      p.M = 2 * H; p.N = rz; p.Kd = RK;
      p.A = L.dAB; p.lda = 2ll * H;
      p.b0 = static_cast<const uint16_t*>(z); p.ldb0 = rz;
      const OutSeg o[2] = {{g->dW1, ldw1, H}, {g->dW1 + rz, ldw1, H}};
      e = wgrad_run(p, true, o, 2, L.part, L.part_floats, st);
    }
  } else {
    // fp32 products: dW1a, dW1b, then dz = dA W1a + dB W1b
    for (int part = 0; part < 2 && e == hipSuccess; ++part) {
      GemmF32Args q{};
      q.M = H; q.N = rz; q.K = RK;
      q.A = L.dAB + part * H; q.a_m = 1; q.a_k = 2ll * H;
      q.B = z; q.b_k = rz; q.b_n = 1;
      e = grad_product(q, kDtypeF32, dt, L.part, g->dW1 + part * rz, ldw1, st);
    }
    for (int part = 0; part < 2 && e == hipSuccess; ++part) {
      GemmF32Args q{};
      q.M = RK; q.N = rz; q.K = H; q.k_split = H;
      q.A = L.dAB + part * H; q.a_m = 2ll * H; q.a_k = 1;
      q.B = W1 + es * part * rz; q.b_k = ldw1; q.b_n = 1;
      q.C = dz; q.ldc = rz; q.c_split = 0; q.accumulate = part;
      e = launch_gemm_f32(q, kDtypeF32, dt, st);
    }
  }
  // dW1s = dC^T s (fp32: s stays fp32)
  if (e == hipSuccess) {
    GemmF32Args q{};
    q.M = H; q.N = rs; q.K = P;
    q.A = L.dC; q.a_m = 1; q.a_k = H;
    q.B = s; q.b_k = rs; q.b_n = 1;
    e = grad_product(q, kDtypeF32, kDtypeF32, L.part, g->dW1 + 2 * rz, ldw1, st);
  }
  if (e == hipSuccess && ds) {
    GemmF32Args q{};
    q.M = P; q.N = rs; q.K = H;
    q.A = L.dC; q.a_m = H; q.a_k = 1;
    q.B = W1 + es * 2 * rz; q.b_k = ldw1; q.b_n = 1;
    e = grad_product(q, kDtypeF32, dt, L.part, ds, rs, st);
  }
  return hip_status(e);
}

int dcoco_represent_backward(const dcoco_dims* d, const dcoco_weights* w, const void* h, const void* E,
                             const int32_t* cand_ids, const float* dz, const float* ds, const dcoco_rep_grads* g,
                             float* dh, void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  if (d->dtype != DCOCO_BF16) return DCOCO_ERR_UNSUPPORTED;
  Carve c(nullptr);
  carve_rep_bwd(c, d);
  rc = check_ws(workspace, workspace_bytes, c.off);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if ((rc = check_weights(w, true, false)) != DCOCO_OK) return rc;
  if (!g || !ptr_ok(g->dP_e) || !ptr_ok(g->dP_h) || !ptr_ok(g->dW_f) || !ptr_ok(g->dW_pair) || !opt_ok(dh))
    return DCOCO_ERR_INVALID_ARG;
  if (!ptr_ok(h) || !ptr_ok(E) || !ptr_ok(cand_ids) || !ptr_ok(dz)) return DCOCO_ERR_INVALID_ARG;
  if (d->B > 1 && !ptr_ok(ds)) return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  const RepBwdLayout L = carve_rep_bwd(cw, d);
  return hip_status(run_rep_backward(d, w, h, E, cand_ids, dz, d->B > 1 ? ds : nullptr, g, dh, L,
                                     static_cast<hipStream_t>(stream)));
}

int dcoco_correct_block(const dcoco_dims* d, const dcoco_weights* w, const void* logits, const void* h,
                        const void* E, void* workspace, size_t* workspace_bytes, int32_t* sel_tok,
                        int32_t* sel_idx, float* S_out, int32_t* cand_ids_out, float* cand_logits_out,
                        void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  if (!topk_supported(dt, d->V, d->K)) return DCOCO_ERR_UNSUPPORTED;
  const int R = d->n_blocks * d->B;
  const size_t RK = static_cast<size_t>(R) * d->K;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  auto layout = [&](Carve& c, void** topk_ws, int32_t** ids, float** cl, RepLayout* L, void** z,
                    float** s, float** S, ScoreLayout* SL, int32_t** best) {
    *topk_ws = c.take(topk_workspace_bytes(dt, R, d->V, d->K));
    *ids = static_cast<int32_t*>(c.take(sizeof(int32_t) * RK));
    *cl = static_cast<float*>(c.take(sizeof(float) * RK));
    *L = carve_rep(c, d);
    *z = c.take(esize(d->dtype) * RK * d->d_z);
    *s = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->d_pair));
    *S = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->K * d->K));
    *SL = carve_score(c, d);
    *best = walk_table_supported(d->B, d->K) && P > 0
                ? static_cast<int32_t*>(c.take(sizeof(int32_t) * P * d->K)) : nullptr;
  };
  void* topk_ws; int32_t* ids; float* cl; RepLayout L; void* z; float* s; float* S; ScoreLayout SL;
  int32_t* best;
  {
    Carve c(nullptr);
    layout(c, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL, &best);
    rc = check_ws(workspace, workspace_bytes, c.off);
    if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  }
  if ((rc = check_weights(w, true, true)) != DCOCO_OK) return rc;
  if (!ptr_ok(logits) || !ptr_ok(h) || !ptr_ok(E) || !ptr_ok(sel_tok)) return DCOCO_ERR_INVALID_ARG;
  if (!opt_ok(sel_idx) || !opt_ok(S_out) || !opt_ok(cand_ids_out) || !opt_ok(cand_logits_out))
    return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  layout(cw, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL, &best);
  if (cand_ids_out) ids = cand_ids_out;
  if (cand_logits_out) cl = cand_logits_out;
  if (S_out) S = S_out;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = dt == kDtypeBf16;
  // the launch that makes the pair states also writes the bf16 split of s
  // that the pair term reads: the z launch where it can carry them, else
  // the gf launch
  const bool zp = bf && z_pairs(d, L, L.split_slot, s, SL.s3, nullptr);
  int split = 0;
  hipError_t e = topk_and_slot(d, w, logits, h, s, bf ? SL.s3 : nullptr, L, topk_ws, ids, cl, st, !zp, &split);
  PairStateArgs ps{};
  if (zp && !z_pairs(d, L, split, s, SL.s3, &ps)) e = hipErrorInvalidValue;
  if (e == hipSuccess) e = cand_gemm(d, w, E, ids, L, st);
  if (e == hipSuccess) e = cand_finish(d, w, z, L, st, zp ? &ps : nullptr);
  if (e == hipSuccess) e = pair_term(d, w, s, SL, bf, st);
  const WalkOut wk{ids, sel_idx, sel_tok};
  bool walked = false;
  if (e == hipSuccess) e = score_tail(d, w, z, cl, S, SL, st, best, &wk, &walked);
  if (e == hipSuccess && !walked) e = walk_after_grid(S, best, cl, ids, d, sel_idx, sel_tok, st);
  return hip_status(e);
}

int dcoco_correct_block_static(const dcoco_dims* d, const dcoco_weights* w, const void* logits, const void* h,
                               const void* E, int32_t* sel_tok, int32_t* sel_idx, float* S_out,
                               int32_t* cand_ids_out, float* cand_logits_out, void* stream) {
  // the size this call needs (a pure query: nothing is launched)
  size_t need = 0;
  int rc = dcoco_correct_block(d, w, nullptr, nullptr, nullptr, nullptr, &need, nullptr, nullptr, nullptr,
                               nullptr, nullptr, stream);
  if (rc != DCOCO_OK) return rc;
  if (need > DCOCO_STATIC_SCRATCH_BYTES) return DCOCO_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if ((rc = static_scratch(&ws)) != DCOCO_OK) return rc;
  size_t have = DCOCO_STATIC_SCRATCH_BYTES;
  return dcoco_correct_block(d, w, logits, h, E, ws, &have, sel_tok, sel_idx, S_out, cand_ids_out,
                             cand_logits_out, stream);
}

int dcoco_build_btable(const dcoco_dims* d, const dcoco_weights* w, const void* E, void* table,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  if (d->dtype != DCOCO_BF16) return DCOCO_ERR_UNSUPPORTED;
  const int dt = kDtypeBf16;
  const int r = d->d_proj;
  const int chunk = d->V < kTableChunk ? d->V : kTableChunk;
  // room for the largest split any chunk can pick (4)
  const size_t need = sizeof(float) * 4 * static_cast<size_t>(chunk) * r;
  rc = check_ws(workspace, workspace_bytes, need);
  if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  if (!w || !ptr_ok(w->P_e) || !ptr_ok(E) || !ptr_ok(table)) return DCOCO_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  float* U = static_cast<float*>(workspace);
  hipError_t e = hipSuccess;
  for (int v0 = 0; v0 < d->V && e == hipSuccess; v0 += chunk) {
    const int M = d->V - v0 < chunk ? d->V - v0 : chunk;
    GemmProblem q{};
    q.M = M; q.N = r; q.Kd = d->d_embed;
    q.A = static_cast<const uint16_t*>(E) + static_cast<size_t>(v0) * d->d_embed; q.lda = d->d_embed;
    q.a_rows = nullptr; q.a_dtype = dt;
    q.w[0] = w->P_e; q.ldw[0] = d->d_embed; q.col0[0] = 0; q.seg_end[0] = r;
    q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = r;
    q.w_dtype = dt;
    q.split = gemm_pick_split(M, r, d->d_embed, dt, dt); q.out_f32 = U; q.ldo = r; q.out = nullptr;
    e = launch_gemm(q, st);
    if (e == hipSuccess)
      e = launch_ln_rows(U, q.split, M, r, 0, r, d->ln_eps, static_cast<uint16_t*>(table) + static_cast<size_t>(v0) * r,
                         dt, st);
  }
  return hip_status(e);
}

int dcoco_correct_block_btable(const dcoco_dims* d, const dcoco_weights* w, const void* logits, const void* h,
                               const void* btable, void* workspace, size_t* workspace_bytes, int32_t* sel_tok,
                               int32_t* sel_idx, float* S_out, int32_t* cand_ids_out, float* cand_logits_out,
                               void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  if (d->dtype != DCOCO_BF16) return DCOCO_ERR_UNSUPPORTED;
  const int dt = kDtypeBf16;
  if (!topk_supported(dt, d->V, d->K)) return DCOCO_ERR_UNSUPPORTED;
  const int R = d->n_blocks * d->B;
  const size_t RK = static_cast<size_t>(R) * d->K;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  auto layout = [&](Carve& c, void** topk_ws, int32_t** ids, float** cl, RepLayout* L, void** z,
                    float** s, float** S, ScoreLayout* SL, int32_t** best) {
    *topk_ws = c.take(topk_workspace_bytes(dt, R, d->V, d->K));
    *ids = static_cast<int32_t*>(c.take(sizeof(int32_t) * RK));
    *cl = static_cast<float*>(c.take(sizeof(float) * RK));
    *L = carve_rep(c, d, false);
    *z = c.take(esize(d->dtype) * RK * d->d_z);
    *s = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->d_pair));
    *S = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->K * d->K));
    *SL = carve_score(c, d);
    *best = walk_table_supported(d->B, d->K) && P > 0
                ? static_cast<int32_t*>(c.take(sizeof(int32_t) * P * d->K)) : nullptr;
  };
  void* topk_ws; int32_t* ids; float* cl; RepLayout L; void* z; float* s; float* S; ScoreLayout SL;
  int32_t* best;
  {
    Carve c(nullptr);
    layout(c, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL, &best);
    rc = check_ws(workspace, workspace_bytes, c.off);
    if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  }
  if ((rc = check_weights(w, false, true)) != DCOCO_OK) return rc;
  if (!ptr_ok(w->P_h) || !ptr_ok(w->W_f) || !ptr_ok(w->W_pair)) return DCOCO_ERR_INVALID_ARG;
  if (!ptr_ok(logits) || !ptr_ok(h) || !ptr_ok(btable) || !ptr_ok(sel_tok)) return DCOCO_ERR_INVALID_ARG;
  if (!opt_ok(sel_idx) || !opt_ok(S_out) || !opt_ok(cand_ids_out) || !opt_ok(cand_logits_out))
    return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  layout(cw, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL, &best);
  if (cand_ids_out) ids = cand_ids_out;
  if (cand_logits_out) cl = cand_logits_out;
  if (S_out) S = S_out;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int r = d->d_proj;
  // the pair states ride on the gathered z launch where it can carry them
  const bool zp = gather_gemm_supported(r) && z_pairs(d, L, L.split_slot, s, SL.s3, nullptr);
  int split = 0;
  hipError_t e = topk_and_slot(d, w, logits, h, s, SL.s3, L, topk_ws, ids, cl, st, !zp, &split);
  PairStateArgs ps{};
  if (zp && !z_pairs(d, L, split, s, SL.s3, &ps)) e = hipErrorInvalidValue;
  if (e == hipSuccess) {
    if (gather_gemm_supported(r)) {
      // table rows gathered into the LDS operand tile, W_fb slice resident in LDS
      e = launch_gather_gemm(btable, ids, d->V - 1, static_cast<int>(RK), r, w->W_f, 2ll * r, 0, d->d_z, z, L.gf,
                             d->K, st, zp ? &ps : nullptr);
    } else {
      // wider rows: the GEMM gathers table rows by id, z = W_fb b[c] + gf[slot]
      GemmProblem q{};
      q.M = static_cast<int>(RK); q.N = d->d_z; q.Kd = r;
      q.A = btable; q.lda = r; q.a_rows = ids; q.a_rows_max = d->V - 1; q.a_dtype = dt;
      q.w[0] = w->W_f; q.ldw[0] = 2ll * r; q.col0[0] = 0; q.seg_end[0] = d->d_z;
      q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = d->d_z;
      q.w_dtype = dt;
      q.split = 1; q.out = z; q.out_dtype = dt; q.ldo = d->d_z;
      q.row_bias = L.gf; q.row_bias_div = d->K; q.col_bias = nullptr;
      e = launch_gemm(q, st);
    }
  }
  if (e == hipSuccess) e = pair_term(d, w, s, SL, true, st);
  const WalkOut wk{ids, sel_idx, sel_tok};
  bool walked = false;
  if (e == hipSuccess) e = score_tail(d, w, z, cl, S, SL, st, best, &wk, &walked);
  if (e == hipSuccess && !walked) e = walk_after_grid(S, best, cl, ids, d, sel_idx, sel_tok, st);
  return hip_status(e);
}

}  // extern "C"
