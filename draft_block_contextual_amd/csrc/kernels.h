// Host-side launchers of the DCOCO kernels (internal to libdcoco).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dcoco {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

// ---------------------------------------------------------------- top-K
size_t topk_workspace_bytes(int dtype, int rows, int V, int K);
bool topk_supported(int dtype, int V, int K);
hipError_t launch_topk(int dtype, const void* logits, int rows, int V, int K, void* partial,
                       int32_t* ids, float* vals, hipStream_t st);

// ----------------------------------------------------------------- GEMM
// out = A (M x Kd) * W^T, W being the row-wise concatenation of up to three
// segments (rows [0,end0) from w[0], [end0,end1) from w[1], [end1,N) from w[2];
// segment s reads W row j as w[s] + (j - start_s) * ldw[s] + col0[s]).
// A row m is A + m * lda, or A + a_rows[m] * lda when a_rows is given.
struct GemmProblem {
  int M, N, Kd;
  const void* A;
  long long lda;
  const int32_t* a_rows;
  int a_rows_max;              // gathered ids are clamped into [0, a_rows_max]
  int a_dtype;                 // kDtypeBf16 / kDtypeF32
  const void* w[3];
  long long ldw[3];
  int col0[3];
  int seg_end[3];              // seg_end[2] == N
  int w_dtype;
  // epilogue
  int split;                   // > 1: fp32 partial sums out_f32[split][M][ldo]
  float* out_f32;
  int ldo;
  void* out;                   // split == 1 and out != nullptr: converted store
  int out_dtype;
  const float* row_bias;       // optional fp32 bias [M / row_bias_div][N]
  int row_bias_div;
  const void* col_bias;        // optional bias [N] of type w_dtype
};
hipError_t launch_gemm(const GemmProblem& p, hipStream_t st);
// number of K-splits and partial-buffer bytes chosen for a problem size
int gemm_pick_split(int M, int N, int Kd, int a_dtype, int w_dtype);

// bf16 top-K of `rows` rows (aligned rows, K <= 16) and a bf16 GEMM q with
// fp32 partials (no gather) in one launch: the GEMM's 64 x 64 tiles (times
// q.split) and the rows share the CUs, three workgroups per CU.
bool topk_gemm_supported(int V, int K, const void* logits, const GemmProblem& q);
// With few rows each row is cut into segments (topk_gemm_row_workgroups
// counts the row workgroups) whose composites go to `partial`
// (topk_workspace_bytes of the rows) and a merge launch follows.
int topk_gemm_workgroups(const GemmProblem& q);
int topk_gemm_row_workgroups(int rows, int V);
hipError_t launch_topk_gemm(const void* logits, int rows, int V, int K, int32_t* ids, float* vals,
                            const GemmProblem& q, void* partial, hipStream_t st);
// bf16 products with a long reduction (weight gradients): splits (a power of
// two up to max_split) for about 256 workgroups, each split >= 128 deep
int gemm_pick_split_max(int M, int N, int Kd, int max_split);

// ------------------------------------------------------ row LayerNorm
// y[m, :] = LN(sum_s x[s][m][col0 : col0 + r]) (non-affine), stored as out_dtype.
hipError_t launch_ln_rows(const float* x, int split, int M, int ldx, int col0, int r, float eps,
                          void* y, int out_dtype, hipStream_t st);

// Pair states made by a z launch beside its rows: pair p = n (B - 1) + i
// gets s_p = sum_s Y[s][n B + i][cl : cl + rs] + sum_s Y[s][n B + i + 1][cr : cr + rs]
// (splits added in order) and, with s3, its three bf16 parts (s3[q P rs + p rs + j]).
struct PairStateArgs {
  const float* Y;
  int split, ldy, B, cl, cr, rs, P;
  float* s;
  void* s3;
};
// the z launch over M rows can carry the P pair states of width rs
bool ln_gemm_pairs_fit(int M, int P, int rs);

// bf16 only: out[m, :] = W[:, wcol0 : wcol0 + r] LN(sum_s x[s][m][col0 : col0 + r]) with the
// LN output rounded to bf16; fp32 out (out_bf == nullptr) or bf16 out with
// + row_bias[m / row_div][n] (out_bf != nullptr; then, with ps, the pair
// states too: r <= 256 and ln_gemm_pairs_fit).
hipError_t launch_ln_gemm(const float* x, int split, int M, int ldx, int col0, int r, float eps,
                          const void* W, long long ldw, int wcol0, int N, float* out_f32, void* out_bf,
                          const float* row_bias, int row_div, hipStream_t st, const PairStateArgs* ps = nullptr);

// s[n, p, :] = sum_s Y[s][n*B+p][cl : cl+rs] + sum_s Y[s][n*B+p+1][cr : cr+rs]
// s3 (optional): the same values as three bf16 rows hi, mid, lo (s3[q * n + i])
// gf = W_fg LN(Y[:, 0:r]) plus, in the same launch, the pair states s and
// their bf16 split (bf16 path; needs ln_gemm_pair_supported)
bool ln_gemm_pair_supported(int r, int rs);
hipError_t launch_ln_gemm_pair(const float* Y, int split, int M, int ldy, int r, float eps, const void* W,
                               long long ldw, int wcol0, int N, float* gf, int B, int cl, int cr, int rs, float* s,
                               void* s3, hipStream_t st);
// the same gf launch without the pair states (r <= 256)
hipError_t launch_ln_gemm_gf(const float* Y, int split, int M, int ldy, int r, float eps, const void* W,
                             long long ldw, int wcol0, int N, float* gf, hipStream_t st);
// z rows from a table of normalised projections (bf16): out = W[:, wcol0 .. +r]
// tab[ids[m]] + row_bias[m / row_div], bf16 out [M][N]
bool gather_gemm_supported(int r);
hipError_t launch_gather_gemm(const void* tab, const int32_t* ids, int idmax, int M, int r, const void* W,
                              long long ldw, int wcol0, int N, void* out_bf, const float* row_bias, int row_div,
                              hipStream_t st, const PairStateArgs* ps = nullptr);
hipError_t launch_pair_state(const float* Y, int split, int N, int B, int ldy, int cl, int cr,
                             int rs, float* s, void* s3, hipStream_t st);

// ----------------------------------------------------- scoring and walk
struct GridProblem {
  int N, B, K, H;
  int dtype;                   // storage type of b1 and w2
  const float* AB;             // [N*B*K, 2H] fp32: W1a z | W1b z
  const float* C;              // [nq, N*(B-1), H] fp32: parts of W1s s_p (summed)
  int nq;
  const void* b1;              // [H] (dtype) or null
  const void* w2;              // [H] (dtype)
  float b2;
  const float* cand_logits;    // [N, B, K]
  float* S;                    // [N, B-1, K, K]
  int32_t* best;               // [N, B-1, K] or null: argmax_b S_p(a, b) per row a
};
hipError_t launch_grid(const GridProblem& p, hipStream_t st);

// The same scores with A = W1a z and B = W1b z formed on chip (bf16 only):
// one workgroup per (block, 64-unit slab, chunk of pairs) stores each slab's
// sum per pair in part [nslab, N*(B-1), K, K]; a second launch adds the slabs,
// l_{p+1}(b) and b2 into S and fills best.
struct ScoreSlabProblem {
  int N, B, K, H, rz;
  const void* z;               // [N*B*K, rz] bf16
  const void* W1;              // [H, ldw1] bf16: columns [z_a | z_b | s]
  long long ldw1;
  const float* C;              // [nq, N*(B-1), H] fp32: parts of W1s s_p (summed), when s3 is null
  int nq;
  // with s3 (bf16 [3, N*(B-1), rs]: the parts of s_p), the launch forms
  // W1s s_p itself and C is not read; needs score_slab_c_on_chip
  const void* s3;
  int rs;
  const void* b1;              // [H] bf16 or null
  const void* w2;              // [H] bf16
  float b2;
  const float* cand_logits;    // [N, B, K]
  float* part;                 // [nslab, N*(B-1), K, K] fp32 scratch
  float* S;                    // [N, B-1, K, K]
  int32_t* best;               // [N, B-1, K] or null
  // with sel_tok (and block_finish_walk_fits), one launch per block finishes
  // the scores and walks: sel_idx (may be null) and sel_tok from cand_ids;
  // best is then not written
  const int32_t* cand_ids;
  int32_t* sel_idx;
  int32_t* sel_tok;
};
bool score_slab_supported(int dtype, int K, int rz, int H);
bool block_finish_walk_fits(int B, int K, int H);
bool score_slab_c_on_chip(int N, int B, int K, int H, int rs);
int score_slab_count(int H);
bool score_slab_preferred(int dtype, int N, int B, int K, int rz, int H);
size_t score_slab_part_bytes(int N, int B, int K, int H);
int score_slab_pairs_per_chunk(int N, int B, int K, int H);
hipError_t launch_score_slab(const ScoreSlabProblem& p, hipStream_t st);

// s3 = three bf16 rows per value of s (hi, mid, lo), s3[q * n + i]
hipError_t launch_split3(const float* s, long long n, void* s3, hipStream_t st);

hipError_t launch_walk(const float* S, const float* cand_logits, const int32_t* cand_ids, int N,
                       int B, int K, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st);
// The same walk from the grid's per-row argmax table best [N, B-1, K]; false
// from walk_table_supported means the block does not fit (use launch_walk).
bool walk_table_supported(int B, int K);
hipError_t launch_walk_table(const int32_t* best, const float* cand_logits, const int32_t* cand_ids, int N,
                             int B, int K, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st);

// Whole-path rules: maximise sum_j lam^j sigma_j over all K^B paths (slot j
// 0-based; sigma_0 = l_0(k_0), sigma_j = S_{j-1}(k_{j-1}, k_j)).
bool path_supported(int B, int K);
hipError_t launch_path(const float* S, const float* cand_logits, const int32_t* cand_ids, int N, int B, int K,
                       float lam, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st);

// ----------------------------------------------- LM head fused with top-K
// top-K of bf16(hd W_lm^T) per row without storing the logits (gemm.hip)
bool lm_head_topk_supported(int M, int V, int d, int K);
size_t lm_head_workspace_bytes(int M, int V, int K);
hipError_t launch_lm_head_topk(const void* hd, const void* W_lm, int M, int V, int d, int K, void* workspace,
                               int32_t* ids, float* vals, hipStream_t st);

// ------------------------------------------------------------ training side
// loss per pair, its sum into loss[0], and dL/dS (see train.hip)
hipError_t launch_loss(const float* S, const int32_t* cand_ids, const int32_t* target_tok, int N, int B, int K,
                       float rho, float* pair_loss, float* loss, float* dS, hipStream_t st);

struct GridBwdArgs {
  int B, K, H, P, nq;
  const float* AB;     // [N*B*K, 2H]: W1a z | W1b z
  const float* C;      // [nq, P, H]: parts of W1s s_p
  const void* b1;      // [H] (dtype) or null
  const void* w2;      // [H] (dtype)
  const float* dS;     // [P, K, K]
  float* dAB;          // out [N*B*K, 2H]: dA | dB
  float* dC;           // out [P, H]
  float* dw2p;         // out [P, H]: per-pair parts of dw2
};
hipError_t launch_grid_bwd(const GridBwdArgs& g, int dtype, hipStream_t st);

// C[m, n] (+)= sum_k A(m, k) B(k, n), A(m, k) = A[m a_m + k a_k],
// B(k, n) = B[k b_k + n b_n]; split z writes C + z c_split
struct GemmF32Args {
  int M, N, K, k_split;
  const void* A;
  long long a_m, a_k;
  const void* B;
  long long b_k, b_n;
  float* C;
  long long ldc, c_split;
  int accumulate;
};
hipError_t launch_gemm_f32(const GemmF32Args& g, int a_dtype, int b_dtype, hipStream_t st);
hipError_t launch_sum_splits(const float* part, int splits, int rows, int cols, float* out, long long ld_out,
                             hipStream_t st);
// which source row an operand row m reads: m itself or a clamped id
// (gathered rows)
struct RowMap {
  int mode = 0;                // 0 identity, 1 ids
  const int32_t* ids = nullptr;
  int idmax = 0;
  __device__ __forceinline__ long long row(int m) const {
    if (mode == 1) {
      const int id = ids[m];
      return id < 0 ? 0 : (id > idmax ? idmax : id);
    }
    return m;
  }
};
// Gradient products on bf16 MFMA (wgrad.hip): C[m, n] = sum_k A(m, k) B(k, n),
// A fp32 split into two bf16 parts on chip, B bf16 stored [k][n].
//   row reduction: A(m, k) = A[k * lda + m], else A[m * lda + k]
//   B row k: k < bend0: b0 + bmap.row(k) * ldb0; k < bend1: b1 + (k - bend0) * ldb1;
//            else b2 + (k - bend1) * ldb2 (b1, b2 may be null when unused)
//   C row m: m < cend0: c0 + m * ldc0; m < cend1: c1 + (m - cend0) * ldc1;
//            else c2 + (m - cend1) * ldc2; split z of k adds z * c_split
// Needs N % 8 == 0, lda % 4 == 0, ldb % 8 == 0, 16-byte aligned A and B, and
// M % 4 == 0 (row reduction) or Kd % 8 == 0.
struct WgradArgs {
  int M = 0, N = 0, Kd = 0, ksplit = 0;
  const float* A = nullptr;
  long long lda = 0;
  const uint16_t* b0 = nullptr;
  const uint16_t* b1 = nullptr;
  const uint16_t* b2 = nullptr;
  long long ldb0 = 0, ldb1 = 0, ldb2 = 0;
  int bend0 = 0x7fffffff, bend1 = 0x7fffffff;
  RowMap bmap;
  float* c0 = nullptr;
  float* c1 = nullptr;
  float* c2 = nullptr;
  long long ldc0 = 0, ldc1 = 0, ldc2 = 0;
  int cend0 = 0x7fffffff, cend1 = 0x7fffffff;
  long long c_split = 0;
};
// splits of k for about 256 workgroups (a power of two up to 16, each >= 128 deep)
int wgrad_pick_split(int M, int N, int Kd);
// number of k splits the launch actually runs (partials written) for `splits`
int wgrad_grid_splits(int Kd, int splits);
hipError_t launch_wgrad(WgradArgs p, bool row_reduction, int splits, hipStream_t st);
// row r of part [rows, cols] summed over its splits (split_stride apart) into
// out0 (r < end0), out1 (r < end1) or out2, each with its own row stride
struct SegOut {
  float* out0; long long ld0; int end0;
  float* out1; long long ld1; int end1;
  float* out2; long long ld2;
};
hipError_t launch_sum_splits_seg(const float* part, int splits, long long split_stride, int rows, int cols,
                                 const SegOut& o, hipStream_t st);
// out[r][c] (row stride ld_out) = sum over s of part[s * split_stride + r * ld_part + c]
hipError_t launch_sum_splits_ex(const float* part, int splits, long long split_stride, int rows, int cols,
                                long long ld_part, float* out, long long ld_out, hipStream_t st);
// LayerNorm forward and backward of the rows of x = sum_s x[s][M][ldx]
// (columns col0 .. col0 + r - 1): y = LN(x) stored as bf16 into rows
// m y_rep .. m y_rep + y_rep - 1 of y_bf (row stride ld_y); with the upstream
// gradient dy(m) = sum over q < rep of dY[(m rep + q) * ld_dy + c] (columns
// dy_col0 ..), dx = (dy - mean(dy) - y mean(dy y)) / sigma into dX [M, ld_dx] fp32
hipError_t launch_ln_fwd_bwd(const float* x, int split, int M, int ldx, int col0, int r, float eps, const float* dY,
                             long long ld_dy, int dy_col0, int rep, void* y_bf, long long ld_y, int y_rep, float* dX,
                             long long ld_dx, hipStream_t st);
// Acat [N B, C] fp32 columns r .. r + 2 rs: the pair-state gradients ds [N, B-1, rs]
// placed at their left slot (columns r ..) and right slot (columns r + rs ..),
// zeros where a slot has no such pair
hipError_t launch_pack_ds(const float* ds, int N, int B, int rs, int r, int C, float* Acat, hipStream_t st);
// the scoring backward's reductions in two launches: dw2 and db1 (column sums
// of dw2p and dC [P, H]), d l (into dcl_out, or tmp when null) and db2 = sum
// of d l; tmp holds mlp_reduce_floats(...) floats
int mlp_reduce_floats(int P, int H, int N, int B, int K);
hipError_t launch_mlp_reduce(const float* dw2p, const float* dC, int P, int H, const float* dS, int N, int B, int K,
                             float* tmp, float* dw2, float* db1, float* db2, float* dcl_out, hipStream_t st);
hipError_t launch_fill(float* x, long long n, float v, hipStream_t st);

}  // namespace dcoco
