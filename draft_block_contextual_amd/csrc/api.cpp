// C ABI of libdcoco: argument checks, workspace layout and the launch sequence
// of each entry point on the caller's stream.  The operations themselves are
// specified in include/dcoco.h.
#include "../../include/dcoco.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

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
hipError_t slot_part(const dcoco_dims* d, const dcoco_weights* w, const void* h, float* s, void* s3,
                     const RepLayout& L, hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int R = d->n_blocks * d->B;
  const int r = d->d_proj, rs = d->d_pair, rz = d->d_z, dh = d->d_hidden;
  const int ns = r + 2 * rs;
  hipError_t e;
  {
    GemmProblem q{};
    q.M = R; q.N = ns; q.Kd = dh;
    q.A = h; q.lda = dh; q.a_rows = nullptr; q.a_dtype = dt;
    q.w[0] = w->P_h; q.ldw[0] = dh; q.col0[0] = 0; q.seg_end[0] = r;
    q.w[1] = w->W_pair; q.ldw[1] = 2ll * dh; q.col0[1] = 0; q.seg_end[1] = r + rs;
    q.w[2] = w->W_pair; q.ldw[2] = 2ll * dh; q.col0[2] = dh; q.seg_end[2] = ns;
    q.w_dtype = dt;
    q.split = L.split_slot; q.out_f32 = L.Y; q.ldo = ns; q.out = nullptr;
    if ((e = launch_gemm(q, st)) != hipSuccess) return e;
  }
  if (dt == kDtypeBf16 && ln_gemm_pair_supported(r, rs))
    return launch_ln_gemm_pair(L.Y, L.split_slot, R, ns, r, d->ln_eps, w->W_f, 2ll * r, r, rz, L.gf, d->B, r,
                               r + rs, rs, s, s3, st);
  if ((e = launch_pair_state(L.Y, L.split_slot, d->n_blocks, d->B, ns, r, r + rs, rs, s, s3, st)) != hipSuccess)
    return e;
  if (dt == kDtypeBf16)
    return launch_ln_gemm(L.Y, L.split_slot, R, ns, 0, r, d->ln_eps, w->W_f, 2ll * r, r, rz, L.gf, nullptr,
                          nullptr, 1, st);
  if ((e = launch_ln_rows(L.Y, L.split_slot, R, ns, 0, r, d->ln_eps, L.g, dt, st)) != hipSuccess) return e;
  GemmProblem q{};
  q.M = R; q.N = rz; q.Kd = r;
  q.A = L.g; q.lda = r; q.a_dtype = dt;
  q.w[0] = w->W_f; q.ldw[0] = 2ll * r; q.col0[0] = r; q.seg_end[0] = rz;
  q.w[1] = q.w[2] = nullptr; q.seg_end[1] = q.seg_end[2] = rz;
  q.w_dtype = dt;
  q.split = 1; q.out_f32 = L.gf; q.ldo = rz; q.out = nullptr;
  return launch_gemm(q, st);
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
hipError_t cand_finish(const dcoco_dims* d, const dcoco_weights* w, void* z, const RepLayout& L,
                       hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int RK = d->n_blocks * d->B * d->K;
  const int r = d->d_proj, rz = d->d_z;
  if (dt == kDtypeBf16)
    return launch_ln_gemm(L.U, L.split_cand, RK, r, 0, r, d->ln_eps, w->W_f, 2ll * r, 0, rz, nullptr, z, L.gf,
                          d->K, st);
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

// scoring stage buffers
struct ScoreLayout {
  void* s3;       // bf16 [3, P, rs] (bf16 path only)
  float* C;       // fp32 [nq, P, H]
  float* AB;      // fp32 [N*B*K, 2H]
};

ScoreLayout carve_score(Carve& c, const dcoco_dims* d) {
  ScoreLayout L;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  const size_t RK = static_cast<size_t>(d->n_blocks) * d->B * d->K;
  const int nq = d->dtype == DCOCO_BF16 ? 3 : 1;
  L.s3 = c.take(d->dtype == DCOCO_BF16 ? 3 * P * d->d_pair * 2 : 0);
  L.C = static_cast<float*>(c.take(sizeof(float) * nq * P * d->d_mlp));
  L.AB = static_cast<float*>(c.take(sizeof(float) * RK * 2 * d->d_mlp));
  return L;
}

// pair term: C_p parts = W1s s_p (bf16 path: s split into hi/mid/lo rows; the
// split is made here unless s3_ready)
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

// AB, then the grid (needs the pair term)
hipError_t score_tail(const dcoco_dims* d, const dcoco_weights* w, const void* z, const float* cl, float* S,
                      const ScoreLayout& L, hipStream_t st) {
  const int dt = d->dtype == DCOCO_BF16 ? kDtypeBf16 : kDtypeF32;
  const int P = d->n_blocks * (d->B - 1);
  if (P == 0) return hipSuccess;
  const int H = d->d_mlp;
  hipError_t e;
  if ((e = ab_gemm(d, w, z, L, st)) != hipSuccess) return e;
  GridProblem g{};
  g.N = d->n_blocks; g.B = d->B; g.K = d->K; g.H = H; g.dtype = dt;
  g.AB = L.AB; g.C = L.C; g.nq = dt == kDtypeBf16 ? 3 : 1; g.b1 = w->b1; g.w2 = w->w2; g.b2 = w->b2;
  g.cand_logits = cl; g.S = S;
  return launch_grid(g, st);
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

// bf16 storage with N*B*K a multiple of 32: the two large gradient products
// run on bf16 MFMA over a two-part split of the fp32 gradients
bool bwd_on_mfma(const dcoco_dims* d) {
  return d->dtype == DCOCO_BF16 && (static_cast<long long>(d->n_blocks) * d->B * d->K) % 32 == 0;
}

struct BwdLayout {
  ScoreLayout SL;
  float* dAB;      // [N*B*K, 2H]
  float* dC;       // [P, H]
  float* dw2p;     // [P, H]
  float* part;     // [kMaxGradSplit, max(H, P), max(d_z, d_pair)]
  float* red;      // partial sums of the reductions
  void* A1;        // bf16 [N*B*K, 4H]: [dA | dB] hi, then lo
  void* At;        // bf16 [2H, 2 N*B*K]: its transpose, parts side by side
  void* Zt;        // bf16 [d_z, 2 N*B*K]: z transposed, twice
  void* W1t;       // bf16 [d_z, 4H]
};

BwdLayout carve_bwd(Carve& c, const dcoco_dims* d) {
  BwdLayout L;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  const size_t RK = static_cast<size_t>(d->n_blocks) * d->B * d->K;
  const size_t H = d->d_mlp;
  L.SL = carve_score(c, d);
  L.dAB = static_cast<float*>(c.take(sizeof(float) * RK * 2 * H));
  L.dC = static_cast<float*>(c.take(sizeof(float) * P * H));
  L.dw2p = static_cast<float*>(c.take(sizeof(float) * P * H));
  L.part = static_cast<float*>(
      c.take(sizeof(float) * kMaxGradSplit * std::max(H, P) * std::max(d->d_z, d->d_pair)));
  const size_t red = 2 * (static_cast<size_t>(colsum_blocks(static_cast<int>(P))) + 1) * H +
                     P * d->K * d->K / 8192 + 2;
  L.red = static_cast<float*>(c.take(sizeof(float) * red));
  const bool mf = bwd_on_mfma(d);
  L.A1 = c.take(mf ? 2 * RK * 4 * H : 0);
  L.At = c.take(mf ? 2 * 2 * H * 2 * RK : 0);
  L.Zt = c.take(mf ? 2 * static_cast<size_t>(d->d_z) * 2 * RK : 0);
  L.W1t = c.take(mf ? 2 * static_cast<size_t>(d->d_z) * 4 * H : 0);
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

// ---- representation backward (bf16 storage)

int pad64(int x) { return (x + 63) / 64 * 64; }

struct RepBwdLayout {
  int split_h, split_e;    // forward recompute: split-K of P_h h and P_e E[c]
  int s_f, s_e, s_h, s_dh; // splits of the gradient products
  int Rp, RKp;             // row counts padded to 64 (reduction length)
  float* Y;                // [split_h][R][r]: P_h h partials
  float* U;                // [split_e][RK][r]: P_e E[c] partials
  void* A1z;               // bf16 [RK, 2 d_z]: dz hi | lo
  void* dzT;               // bf16 [2 d_z, RKp]: dz^T, hi rows then lo rows
  void* WfT2;              // bf16 [2 r, 2 d_z]: W_f^T, twice along k
  float* dBG;              // [RK, 2 r]: dz W_f (db | per-candidate part of dg)
  void* bq;                // bf16 [RK, r]: b
  void* gq;                // bf16 [R, r]: g
  float* dxe;              // [RK, r]
  void* BGT;               // bf16 [2 r, RKp]: b^T, then g^T repeated over k
  void* dxeT;              // bf16 [2 r, RKp]: dx_e^T hi rows then lo rows
  void* EcT;               // bf16 [d_embed, RKp]: the gathered E rows, transposed
  float* Acat;             // [R, C]: dx_h | ds at the left slot | ds at the right slot
  void* A1cat;             // bf16 [R, 2C]
  void* AcatT;             // bf16 [2C, Rp]
  void* hT;                // bf16 [d_hidden, Rp]
  void* WcatT2;            // bf16 [d_hidden, 2C]: [P_h; W_L; W_R]^T, twice along k
  float* part;             // split partial products
};

RepBwdLayout carve_rep_bwd(Carve& c, const dcoco_dims* d) {
  RepBwdLayout L;
  const int R = d->n_blocks * d->B;
  const int RK = R * d->K;
  const int r = d->d_proj, rz = d->d_z, rs = d->d_pair, dh = d->d_hidden, de = d->d_embed;
  const int C = r + 2 * rs;
  L.Rp = pad64(R);
  L.RKp = pad64(RK);
  L.split_h = gemm_pick_split(R, r, dh, kDtypeBf16, kDtypeBf16);
  L.split_e = gemm_pick_split(RK, r, de, kDtypeBf16, kDtypeBf16);
  L.s_f = gemm_pick_split_max(2 * rz, 2 * r, L.RKp, kMaxGradSplit);
  L.s_e = gemm_pick_split_max(2 * r, de, L.RKp, kMaxGradSplit);
  L.s_h = gemm_pick_split_max(2 * C, dh, L.Rp, kMaxGradSplit);
  L.s_dh = gemm_pick_split_max(R, dh, 2 * C, 4);
  const size_t bf = 2, f4 = 4;
  const size_t RKs = RK, Rs = R, RKps = L.RKp, Rps = L.Rp;
  L.Y = static_cast<float*>(c.take(f4 * L.split_h * Rs * r));
  L.U = static_cast<float*>(c.take(f4 * L.split_e * RKs * r));
  L.A1z = c.take(bf * RKs * 2 * rz);
  L.dzT = c.take(bf * 2 * rz * RKps);
  L.WfT2 = c.take(bf * 2 * r * 2 * rz);
  L.dBG = static_cast<float*>(c.take(f4 * RKs * 2 * r));
  L.bq = c.take(bf * RKs * r);
  L.gq = c.take(bf * Rs * r);
  L.dxe = static_cast<float*>(c.take(f4 * RKs * r));
  L.BGT = c.take(bf * 2 * r * RKps);
  L.dxeT = c.take(bf * 2 * r * RKps);
  L.EcT = c.take(bf * de * RKps);
  L.Acat = static_cast<float*>(c.take(f4 * Rs * C));
  L.A1cat = c.take(bf * Rs * 2 * C);
  L.AcatT = c.take(bf * 2 * C * Rps);
  L.hT = c.take(bf * dh * Rps);
  L.WcatT2 = c.take(bf * dh * 2 * C);
  const size_t part = std::max({static_cast<size_t>(L.s_f) * 2 * rz * 2 * r, static_cast<size_t>(L.s_e) * 2 * r * de,
                                static_cast<size_t>(L.s_h) * 2 * C * dh, static_cast<size_t>(L.s_dh) * Rs * dh});
  L.part = static_cast<float*>(c.take(f4 * part));
  return L;
}

// C [M, N] = A [M, Kd] W^T (W rows [N][Kd], both bf16, Kd % 64 == 0) into
// fp32 split partials part [split][M][N]
hipError_t bf16_product(int M, int N, int Kd, const void* A, long long lda, const void* W, long long ldw, int split,
                        float* part, hipStream_t st) {
  GemmProblem q{};
  q.M = M; q.N = N; q.Kd = Kd;
  q.A = A; q.lda = lda; q.a_dtype = kDtypeBf16;
  q.w[0] = W; q.ldw[0] = ldw; q.col0[0] = 0;
  q.seg_end[0] = q.seg_end[1] = q.seg_end[2] = N;
  q.w_dtype = kDtypeBf16;
  q.split = split; q.out_f32 = part; q.ldo = N; q.out = nullptr;
  return launch_gemm(q, st);
}

hipError_t run_rep_backward(const dcoco_dims* d, const dcoco_weights* w, const void* h, const void* E,
                            const int32_t* ids, const float* dz, const float* ds, const dcoco_rep_grads* g,
                            float* dh_out, const RepBwdLayout& L, hipStream_t st) {
  const int N = d->n_blocks, B = d->B, K = d->K;
  const int R = N * B, RK = R * K;
  const int r = d->d_proj, rz = d->d_z, rs = d->d_pair, dh = d->d_hidden, de = d->d_embed;
  const int C = r + 2 * rs;
  const int Rp = L.Rp, RKp = L.RKp;
  const long long RKpl = RKp, Rpl = Rp;
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
  // dBG = dz [W_fb | W_fg]: dz as two bf16 parts against W_f^T twice
  if (e == hipSuccess)
    e = launch_split_t_ex(dz, true, rz, RK, RKp, rz, RowMap{}, L.A1z, L.dzT, RKpl, 0, static_cast<long long>(rz) * RKpl,
                          st);
  if (e == hipSuccess)
    e = launch_split_t_ex(w->W_f, false, 2ll * r, rz, rz, 2 * r, RowMap{}, nullptr, L.WfT2, 2ll * rz, 0, rz, st);
  if (e == hipSuccess) e = bf16_product(RK, 2 * r, 2 * rz, L.A1z, 2ll * rz, L.WfT2, 2ll * rz, 1, L.dBG, st);
  // LayerNorm forward (b, g) and backward (dx_e; dx_h into Acat), ds placed by slot
  if (e == hipSuccess)
    e = launch_ln_fwd_bwd(L.U, L.split_e, RK, r, 0, r, d->ln_eps, L.dBG, 2ll * r, 0, 1, L.bq, L.dxe, r, st);
  if (e == hipSuccess)
    e = launch_ln_fwd_bwd(L.Y, L.split_h, R, r, 0, r, d->ln_eps, L.dBG, 2ll * r, r, K, L.gq, L.Acat, C, st);
  if (e == hipSuccess) e = launch_pack_ds(ds, N, B, rs, r, C, L.Acat, st);
  // transposed operands of the weight-gradient products (reduction over rows)
  if (e == hipSuccess) e = launch_split_t_ex(L.bq, false, r, RK, RKp, r, RowMap{}, nullptr, L.BGT, RKpl, 0, 0, st);
  if (e == hipSuccess) {
    RowMap rep;
    rep.mode = 2;
    rep.rep = K;
    e = launch_split_t_ex(L.gq, false, r, RK, RKp, r, rep, nullptr, static_cast<char*>(L.BGT) + 2ll * r * RKpl,
                          RKpl, 0, 0, st);
  }
  if (e == hipSuccess)
    e = launch_split_t_ex(L.dxe, true, r, RK, RKp, r, RowMap{}, nullptr, L.dxeT, RKpl, 0, static_cast<long long>(r) * RKpl,
                          st);
  if (e == hipSuccess) {
    RowMap gat;
    gat.mode = 1;
    gat.ids = ids;
    gat.idmax = d->V - 1;
    e = launch_split_t_ex(E, false, de, RK, RKp, de, gat, nullptr, L.EcT, RKpl, 0, 0, st);
  }
  if (e == hipSuccess)
    e = launch_split_t_ex(L.Acat, true, C, R, Rp, C, RowMap{}, L.A1cat, L.AcatT, Rpl, 0, static_cast<long long>(C) * Rpl,
                          st);
  if (e == hipSuccess) e = launch_split_t_ex(h, false, dh, R, Rp, dh, RowMap{}, nullptr, L.hT, Rpl, 0, 0, st);
  // dW_f = dz^T [b | g repeated]: hi and lo parts stacked along M, then added
  if (e == hipSuccess) e = bf16_product(2 * rz, 2 * r, RKp, L.dzT, RKpl, L.BGT, RKpl, L.s_f, L.part, st);
  if (e == hipSuccess)
    e = launch_sum_splits_ex(L.part, 2 * L.s_f, static_cast<long long>(rz) * 2 * r, rz, 2 * r, 2ll * r, g->dW_f, 2ll * r,
                             st);
  // dP_e = dx_e^T E[c]
  if (e == hipSuccess) e = bf16_product(2 * r, de, RKp, L.dxeT, RKpl, L.EcT, RKpl, L.s_e, L.part, st);
  if (e == hipSuccess)
    e = launch_sum_splits_ex(L.part, 2 * L.s_e, static_cast<long long>(r) * de, r, de, de, g->dP_e, de, st);
  // [dP_h; dW_L; dW_R] = Acat^T h
  if (e == hipSuccess) e = bf16_product(2 * C, dh, Rp, L.AcatT, Rpl, L.hT, Rpl, L.s_h, L.part, st);
  const long long slice = static_cast<long long>(C) * dh;
  if (e == hipSuccess) e = launch_sum_splits_ex(L.part, 2 * L.s_h, slice, r, dh, dh, g->dP_h, dh, st);
  if (e == hipSuccess)
    e = launch_sum_splits_ex(L.part + static_cast<long long>(r) * dh, 2 * L.s_h, slice, rs, dh, dh, g->dW_pair, 2ll * dh,
                             st);
  if (e == hipSuccess)
    e = launch_sum_splits_ex(L.part + static_cast<long long>(r + rs) * dh, 2 * L.s_h, slice, rs, dh, dh,
                             g->dW_pair + dh, 2ll * dh, st);
  if (!dh_out || e != hipSuccess) return e;
  // dh = Acat [P_h; W_L; W_R]: Acat as two bf16 parts against the weights twice
  const long long ldc2 = 2ll * C;
  e = launch_split_t_ex(w->P_h, false, dh, r, r, dh, RowMap{}, nullptr, L.WcatT2, ldc2, 0, C, st);
  if (e == hipSuccess)
    e = launch_split_t_ex(w->W_pair, false, 2ll * dh, rs, rs, dh, RowMap{}, nullptr, L.WcatT2, ldc2, r, C, st);
  if (e == hipSuccess)
    e = launch_split_t_ex(static_cast<const char*>(w->W_pair) + 2ll * dh, false, 2ll * dh, rs, rs, dh, RowMap{},
                          nullptr, L.WcatT2, ldc2, r + rs, C, st);
  if (e != hipSuccess) return e;
  if (L.s_dh == 1) return bf16_product(R, dh, 2 * C, L.A1cat, ldc2, L.WcatT2, ldc2, 1, dh_out, st);
  e = bf16_product(R, dh, 2 * C, L.A1cat, ldc2, L.WcatT2, ldc2, L.s_dh, L.part, st);
  if (e == hipSuccess) e = launch_sum_splits(L.part, L.s_dh, R, dh, dh_out, dh, st);
  return e;
}

}  // namespace

extern "C" {

int dcoco_abi_version(void) { return 105; }

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
  float* red2 = L.red + 2 * (colsum_blocks(P) + 1) * static_cast<long long>(H);
  if (e == hipSuccess) e = launch_colsum(L.dw2p, P, H, H, L.red, g->dw2, st);
  if (e == hipSuccess) e = launch_colsum(L.dC, P, H, H, L.red, g->db1, st);
  if (e == hipSuccess) e = launch_sum(dS, static_cast<long long>(P) * d->K * d->K, red2, g->db2, st);
  if (e == hipSuccess && d_cand_logits) e = launch_dlogit(dS, d->n_blocks, d->B, d->K, d_cand_logits, st);
  if (bwd_on_mfma(d)) {
    // [dA | dB] = hi + lo (two bf16 parts); z and W1 are bf16 already
    if (e == hipSuccess) e = launch_split_t(L.dAB, true, RK, 2 * H, L.A1, L.At, st);
    if (e == hipSuccess) e = launch_split_t(z, false, RK, rz, nullptr, L.Zt, st);
    if (e == hipSuccess) e = launch_w1t(w->W1, H, rz, ldw1, L.W1t, st);
    // dz = [dA | dB]_hi [W1a; W1b] + [dA | dB]_lo [W1a; W1b], one product over 4H
    if (e == hipSuccess) {
      GemmProblem q{};
      q.M = RK; q.N = rz; q.Kd = 4 * H;
      q.A = L.A1; q.lda = 4ll * H; q.a_dtype = kDtypeBf16;
      q.w[0] = L.W1t; q.ldw[0] = 4ll * H; q.col0[0] = 0;
      q.seg_end[0] = q.seg_end[1] = q.seg_end[2] = rz;
      q.w_dtype = kDtypeBf16;
      q.split = 1; q.out_f32 = dz; q.ldo = rz; q.out = nullptr;
      e = launch_gemm(q, st);
    }
    // dW1a, dW1b: (dA or dB)^T z over 2 N*B*K (both parts), split over k
    for (int part = 0; part < 2 && e == hipSuccess; ++part) {
      GemmProblem q{};
      q.M = H; q.N = rz; q.Kd = 2 * RK;
      q.A = static_cast<const char*>(L.At) + 2ll * part * H * 2 * RK; q.lda = 2ll * RK; q.a_dtype = kDtypeBf16;
      q.w[0] = L.Zt; q.ldw[0] = 2ll * RK; q.col0[0] = 0;
      q.seg_end[0] = q.seg_end[1] = q.seg_end[2] = rz;
      q.w_dtype = kDtypeBf16;
      int split = 1;
      while (split < kMaxGradSplit && ((H + 63) / 64) * ((rz + 63) / 64) * split < 256 && q.Kd / (2 * split) >= 256)
        split *= 2;
      q.split = split; q.out_f32 = L.part; q.ldo = rz; q.out = nullptr;
      e = launch_gemm(q, st);
      if (e == hipSuccess) e = launch_sum_splits(L.part, split, H, rz, g->dW1 + part * rz, ldw1, st);
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
                    float** s, float** S, ScoreLayout* SL) {
    *topk_ws = c.take(topk_workspace_bytes(dt, R, d->V, d->K));
    *ids = static_cast<int32_t*>(c.take(sizeof(int32_t) * RK));
    *cl = static_cast<float*>(c.take(sizeof(float) * RK));
    *L = carve_rep(c, d);
    *z = c.take(esize(d->dtype) * RK * d->d_z);
    *s = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->d_pair));
    *S = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->K * d->K));
    *SL = carve_score(c, d);
  };
  void* topk_ws; int32_t* ids; float* cl; RepLayout L; void* z; float* s; float* S; ScoreLayout SL;
  {
    Carve c(nullptr);
    layout(c, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL);
    rc = check_ws(workspace, workspace_bytes, c.off);
    if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  }
  if ((rc = check_weights(w, true, true)) != DCOCO_OK) return rc;
  if (!ptr_ok(logits) || !ptr_ok(h) || !ptr_ok(E) || !ptr_ok(sel_tok)) return DCOCO_ERR_INVALID_ARG;
  if (!opt_ok(sel_idx) || !opt_ok(S_out) || !opt_ok(cand_ids_out) || !opt_ok(cand_logits_out))
    return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  layout(cw, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL);
  if (cand_ids_out) ids = cand_ids_out;
  if (cand_logits_out) cl = cand_logits_out;
  if (S_out) S = S_out;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = dt == kDtypeBf16;
  // the pair-state kernel also writes the bf16 split of s that the pair term reads
  hipError_t e = slot_part(d, w, h, s, bf ? SL.s3 : nullptr, L, st);
  if (e == hipSuccess) e = pair_term(d, w, s, SL, bf, st);
  if (e == hipSuccess) e = launch_topk(dt, logits, R, d->V, d->K, topk_ws, ids, cl, st);
  if (e == hipSuccess) e = cand_gemm(d, w, E, ids, L, st);
  if (e == hipSuccess) e = cand_finish(d, w, z, L, st);
  if (e == hipSuccess) e = score_tail(d, w, z, cl, S, SL, st);
  if (e == hipSuccess) e = launch_walk(S, cl, ids, d->n_blocks, d->B, d->K, sel_idx, sel_tok, st);
  return hip_status(e);
}

int dcoco_build_btable(const dcoco_dims* d, const dcoco_weights* w, const void* E, void* table,
                       void* workspace, size_t* workspace_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != DCOCO_OK) return rc;
  if (d->dtype != DCOCO_BF16 || !gather_gemm_supported(d->d_proj)) return DCOCO_ERR_UNSUPPORTED;
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
  if (d->dtype != DCOCO_BF16 || !gather_gemm_supported(d->d_proj)) return DCOCO_ERR_UNSUPPORTED;
  const int dt = kDtypeBf16;
  if (!topk_supported(dt, d->V, d->K)) return DCOCO_ERR_UNSUPPORTED;
  const int R = d->n_blocks * d->B;
  const size_t RK = static_cast<size_t>(R) * d->K;
  const size_t P = static_cast<size_t>(d->n_blocks) * (d->B - 1);
  auto layout = [&](Carve& c, void** topk_ws, int32_t** ids, float** cl, RepLayout* L, void** z,
                    float** s, float** S, ScoreLayout* SL) {
    *topk_ws = c.take(topk_workspace_bytes(dt, R, d->V, d->K));
    *ids = static_cast<int32_t*>(c.take(sizeof(int32_t) * RK));
    *cl = static_cast<float*>(c.take(sizeof(float) * RK));
    *L = carve_rep(c, d, false);
    *z = c.take(esize(d->dtype) * RK * d->d_z);
    *s = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->d_pair));
    *S = static_cast<float*>(c.take(sizeof(float) * (P ? P : 1) * d->K * d->K));
    *SL = carve_score(c, d);
  };
  void* topk_ws; int32_t* ids; float* cl; RepLayout L; void* z; float* s; float* S; ScoreLayout SL;
  {
    Carve c(nullptr);
    layout(c, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL);
    rc = check_ws(workspace, workspace_bytes, c.off);
    if (rc != DCOCO_OK) return rc > 0 ? DCOCO_OK : rc;
  }
  if ((rc = check_weights(w, false, true)) != DCOCO_OK) return rc;
  if (!ptr_ok(w->P_h) || !ptr_ok(w->W_f) || !ptr_ok(w->W_pair)) return DCOCO_ERR_INVALID_ARG;
  if (!ptr_ok(logits) || !ptr_ok(h) || !ptr_ok(btable) || !ptr_ok(sel_tok)) return DCOCO_ERR_INVALID_ARG;
  if (!opt_ok(sel_idx) || !opt_ok(S_out) || !opt_ok(cand_ids_out) || !opt_ok(cand_logits_out))
    return DCOCO_ERR_INVALID_ARG;
  Carve cw(workspace);
  layout(cw, &topk_ws, &ids, &cl, &L, &z, &s, &S, &SL);
  if (cand_ids_out) ids = cand_ids_out;
  if (cand_logits_out) cl = cand_logits_out;
  if (S_out) S = S_out;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int r = d->d_proj;
  hipError_t e = slot_part(d, w, h, s, SL.s3, L, st);
  if (e == hipSuccess) e = pair_term(d, w, s, SL, true, st);
  if (e == hipSuccess) e = launch_topk(dt, logits, R, d->V, d->K, topk_ws, ids, cl, st);
  if (e == hipSuccess)
    e = launch_gather_gemm(btable, ids, d->V - 1, static_cast<int>(RK), r, w->W_f, 2ll * r, 0, d->d_z, z, L.gf,
                           d->K, st);
  if (e == hipSuccess) e = score_tail(d, w, z, cl, S, SL, st);
  if (e == hipSuccess) e = launch_walk(S, cl, ids, d->n_blocks, d->B, d->K, sel_idx, sel_tok, st);
  return hip_status(e);
}

}  // extern "C"
