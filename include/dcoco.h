/*
 * dcoco.h - C ABI of the DCOCO contextual-corrector hot path for AMD MI355X
 * (gfx950).
 *
 * DCOCO re-selects the tokens of a parallel draft block.  For every block of
 * B slots it keeps each slot's top-K draft candidates, builds a representation
 * of every candidate and of every pair of neighbouring slots, scores all
 * (B-1)K^2 transitions between neighbouring candidates with one shared
 * two-layer MLP added to the later candidate's draft logit, and walks the
 * scored grid left to right, each slot taking the best successor of the token
 * actually chosen before it.
 *
 * Sources, cited by page title and section:
 *   [P1] Two Delta, "Two Delta makes NVIDIA Nemotron 3.5 Super even faster
 *        with DCOCO" (twodelta.com/blog/dcoco), section "How DCOCO works".
 *   [P2] review of arXiv 2610.12570, "Contextual Correction of Parallel Drafts
 *        for Speculative Decoding" (jaehun.me/posts/paper-2610-12570), section
 *        "New approach: DCOCO", parts 1 (paper Sec. 3.2) and 2 (paper
 *        Sec. 3.3), part 3 (training, paper Sec. 3.2 and App. A), and
 *        section "Path selection and ablation" (paper Sec. 4.3).
 *
 * Conventions for every entry point
 *   - All array arguments are DEVICE pointers on the current HIP device,
 *     16-byte aligned, row-major, owned by the caller.  The library never
 *     allocates or frees device memory and keeps no pointer after returning.
 *   - Matrices use the [out, in] layout of a linear layer: y = W x reads row o
 *     of W for output o.
 *   - dims->dtype selects the storage type of logits, h, E, the weight
 *     matrices, b1, w2 and of the representation z: DCOCO_BF16 (bf16 values,
 *     fp32 accumulation) or DCOCO_F32.  Candidate logits, pair states s and
 *     scores S are always fp32; ids and indices int32.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting.  Buffers must stay valid until the
 *     stream has finished the work.  Calls on different streams with separate
 *     workspaces may run concurrently.
 *   - Entry points that take `workspace`: with workspace == NULL the call
 *     stores the number of bytes it needs in *workspace_bytes and returns
 *     DCOCO_OK without launching anything.  Otherwise *workspace_bytes must
 *     hold the size of the caller's buffer (256-byte aligned), which must be
 *     at least that number (never less than 256).  The workspace holds no
 *     state between calls.
 *   - Arguments are checked before anything is launched; a failed check
 *     returns a negative dcoco_status and enqueues nothing.  No C++ exception
 *     crosses this interface.  A launch failure returns DCOCO_ERR_HIP.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     run after run.
 *
 * Supported shapes: n_blocks >= 1, B >= 1, 1 <= K <= min(V, 64); d_hidden,
 * d_embed, d_proj, d_z, d_pair and d_mlp positive multiples of 32, with
 * d_proj, d_z, d_pair <= 2048; ln_eps > 0.  Valid shapes outside
 * this set return DCOCO_ERR_UNSUPPORTED.
 */
#ifndef DCOCO_H
#define DCOCO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DCOCO_OK = 0,
  DCOCO_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size, bad eps */
  DCOCO_ERR_UNSUPPORTED = -2,   /* valid but outside the supported shape set */
  DCOCO_ERR_WORKSPACE = -3,     /* workspace too small or misaligned */
  DCOCO_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} dcoco_status;

typedef enum { DCOCO_F32 = 0, DCOCO_BF16 = 1 } dcoco_dtype;

/* Problem shape.  Notation: B slots per draft block, K candidates per slot,
 * V vocabulary size, d_hidden = d (h_i in R^d), d_embed = e (rows of E),
 * d_proj = r (width of b_{i,k} and g_i), d_z = width of z_{i,k},
 * d_pair = width of s_p, d_mlp = H (hidden width of Delta_theta). */
typedef struct {
  int32_t n_blocks;   /* N: independent draft blocks (decoding streams) per call */
  int32_t B, K, V;
  int32_t d_hidden, d_embed, d_proj, d_z, d_pair, d_mlp;
  int32_t dtype;      /* dcoco_dtype */
  float ln_eps;       /* LayerNorm epsilon (> 0) */
} dcoco_dims;

/* Corrector parameters, shared by every slot and transition ([P2] part 1,
 * paper Sec. 3.2).  Storage type = dims.dtype; b2 is passed by value.  The
 * MLP's activation is SiLU, the only one supported: the pages do not name
 * the activation and SiLU is the reading taken, so no field selects it.
 * Layout:
 *   P_e    [d_proj, d_embed]        candidate embedding projection
 *   P_h    [d_proj, d_hidden]       slot hidden-state projection
 *   W_f    [d_z, 2*d_proj]          fusion f; columns [b | g]
 *   W_pair [d_pair, 2*d_hidden]     pair state; columns [h_p | h_{p+1}]
 *   W1     [d_mlp, 2*d_z + d_pair]  MLP layer 1; columns [z_a | z_b | s]
 *   b1     [d_mlp]                  MLP layer-1 bias (NULL means zeros)
 *   w2     [d_mlp]                  MLP output layer (scalar output)
 *   b2                              MLP output bias */
typedef struct {
  const void *P_e, *P_h, *W_f, *W_pair, *W1, *b1, *w2;
  float b2;
} dcoco_weights;

/* Top-K candidate extraction ([P1] "Keep the leading candidates"; [P2]
 * part 1, paper Sec. 3.2).
 *   logits      [n_blocks*B, V] dtype    the drafter's raw logits
 *   cand_ids    [n_blocks*B, K] int32    out: c_{i,k}
 *   cand_logits [n_blocks*B, K] fp32     out: l_i(k), the logit value widened
 * Each row's K largest logits, sorted by value descending; equal values go to
 * the lower id; -0 equals +0; NaN ranks below every number.
 * Workspace: none, except for bf16 calls of at most 32 rows, whose rows are
 * cut into column segments: it then holds each segment's K results
 * (rows * segments * K * 8 bytes, at most 128 KB) until a merge ranks them. */
int dcoco_topk(const dcoco_dims* dims, const void* logits, int32_t* cand_ids,
               float* cand_logits, void* workspace, size_t* workspace_bytes,
               void* stream);

/* Candidate and slot representations and pair states ([P1] "Score
 * neighboring candidates in parallel"; [P2] part 1, paper Sec. 3.2).
 *   h        [n_blocks, B, d_hidden] dtype   drafter hidden states h_i
 *   E        [V, d_embed] dtype              frozen token-embedding table
 *   cand_ids [n_blocks, B, K] int32          candidates (ids must be < V)
 *   z        [n_blocks, B, K, d_z] dtype     out: z_{i,k} = W_f [b_{i,k}; g_i]
 *   s        [n_blocks, B-1, d_pair] fp32    out: s_p = W_pair [h_p; h_{p+1}]
 * with g_i = LN(P_h h_i), b_{i,k} = LN(P_e E[c_{i,k}]), LN non-affine.  In
 * bf16 mode g, b and z are rounded to bf16 (nearest-even); s is not. */
int dcoco_represent(const dcoco_dims* dims, const dcoco_weights* w, const void* h,
                    const void* E, const int32_t* cand_ids, void* z, float* s,
                    void* workspace, size_t* workspace_bytes, void* stream);

/* Transition scores ([P1] "Score neighboring candidates in parallel"; [P2]
 * part 1, paper Sec. 3.2):
 *   S[n,p,a,b] = l_{p+1}(b) + w2 . SiLU(W1 [z_{p,a}; z_{p+1,b}; s_p] + b1) + b2
 *   z           [n_blocks, B, K, d_z] dtype
 *   s           [n_blocks, B-1, d_pair] fp32
 *   cand_logits [n_blocks, B, K] fp32
 *   S           [n_blocks, B-1, K, K] fp32   out (unnormalised) */
int dcoco_score(const dcoco_dims* dims, const dcoco_weights* w, const void* z,
                const float* s, const float* cand_logits, float* S,
                void* workspace, size_t* workspace_bytes, void* stream);

/* Prefix-first greedy walk ([P1] "Select using the realized token
 * identities"; [P2] part 2, paper Sec. 3.3): k_1 = argmax_k l_1(k);
 * k_{p+1} = argmax_b S_p(k_p, b); y_p = c_{p, k_p}.  argmax takes the lowest
 * index among equal maxima and never picks NaN (index 0 if a row is all NaN).
 *   S        [n_blocks, B-1, K, K] fp32
 *   cand_logits [n_blocks, B, K] fp32
 *   cand_ids [n_blocks, B, K] int32
 *   sel_idx  [n_blocks, B] int32   out: k_p (may be NULL)
 *   sel_tok  [n_blocks, B] int32   out: y_p */
int dcoco_select(const dcoco_dims* dims, const float* S, const float* cand_logits,
                 const int32_t* cand_ids, int32_t* sel_idx, int32_t* sel_tok,
                 void* stream);

/* Path-selection rules compared with the greedy walk on the same score grid
 * ([P2] section "Path selection and ablation", paper Sec. 4.3 and Tab. 3).
 *   DCOCO_PATH_GREEDY      the prefix-first walk of dcoco_select (lambda unused)
 *   DCOCO_PATH_GLOBAL_SUM  maximise the total path score
 *   DCOCO_PATH_DISCOUNT    maximise the geometrically discounted score
 * The page gives no formula; the reading used: over all K^B paths k_1..k_B,
 *   J(k) = sum_{j=1..B} lambda^(j-1) sigma_j,
 *   sigma_1 = l_1(k_1), sigma_j = S_{j-1}(k_{j-1}, k_j) (j >= 2),
 * with lambda = 1 for Global-Sum and 0 < lambda <= 1 for the discount (the
 * page evaluates 0.75).  The first slot is free; a NaN term counts as -inf;
 * among paths of equal J (in fp32 arithmetic) the lexicographically smallest
 * index sequence wins.  Arguments as dcoco_select.  Errors: an unknown rule
 * or, for DCOCO_PATH_DISCOUNT, lambda outside (0, 1] -> DCOCO_ERR_INVALID_ARG;
 * for the two whole-path rules, B > 4096 or B*K > 16384 ->
 * DCOCO_ERR_UNSUPPORTED.  One workgroup per block; O(B K^2) work. */
typedef enum {
  DCOCO_PATH_GREEDY = 0,
  DCOCO_PATH_GLOBAL_SUM = 1,
  DCOCO_PATH_DISCOUNT = 2
} dcoco_path_rule;
int dcoco_select_path(const dcoco_dims* dims, const float* S, const float* cand_logits,
                      const int32_t* cand_ids, int rule, float lambda, int32_t* sel_idx,
                      int32_t* sel_tok, void* stream);

/* The drafter's LM head fused with top-K ([P1] "Keep the leading
 * candidates": the candidates are the drafter's own top-K; [P1] "Score
 * neighboring candidates in parallel": the corrector reuses what the drafter
 * pass already computed).  For every row i (one slot of one block),
 *   l_i(v) = bf16( sum_k hd[i,k] W_lm[v,k] )   (fp32 accumulation, rounded
 *            to nearest-even bf16: the logit the drafter would store),
 * and the K largest are selected exactly as dcoco_topk does (value
 * descending, equal values to the lower id), without writing the
 * [n_blocks*B, V] logits anywhere.
 *   hd          [n_blocks*B, d_hidden] bf16   the drafter's final hidden states
 *   W_lm        [V, d_hidden] bf16            LM head (rows = vocabulary)
 *   cand_ids    [n_blocks*B, K] int32         out
 *   cand_logits [n_blocks*B, K] fp32          out: the bf16 logits, widened
 * bf16 storage only; K <= 64 and d_hidden a multiple of 64, else
 * DCOCO_ERR_UNSUPPORTED.  Workspace: query with workspace == NULL (a few MB:
 * per-workgroup candidate lists).  Deterministic. */
int dcoco_lm_head_topk(const dcoco_dims* dims, const void* hd, const void* W_lm,
                       int32_t* cand_ids, float* cand_logits, void* workspace,
                       size_t* workspace_bytes, void* stream);

/* Training loss of the corrector ([P1] "How we train the corrector"; [P2]
 * part 3, paper Sec. 3.2 and App. A).  The label of pair p is the pair of
 * target tokens of slots p and p+1 (the target model's choices under the
 * training context): a*_p and b*_p are their positions among the candidates
 * of the two slots, and the pair counts (m_p = 1) only when both are
 * present.  The pages lose the formula; the reading implemented:
 *   L = (1/N) sum_n sum_{p=1..B-1} m_p exp(-(p-1)/rho) CE_p,
 *   CE_p = log sum_{a,b} exp(S_p(a,b)) - S_p(a*_p, b*_p)  (joint softmax),
 *   dL/dS_p(a,b) = (1/N) m_p exp(-(p-1)/rho) (softmax(S_p)(a,b) - [a=a*,b=b*]).
 *   S          [n_blocks, B-1, K, K] fp32   scores (finite)
 *   cand_ids   [n_blocks, B, K] int32       candidates
 *   target_tok [n_blocks, B] int32          target token per slot
 *   rho        > 0 (the pages train with 4)
 *   loss       [1] fp32                     out: L
 *   pair_loss  [n_blocks, B-1] fp32         out: each pair's term of L
 *   dS         [n_blocks, B-1, K, K] fp32   out: dL/dS
 * S, pair_loss and dS may be NULL when B == 1 (then L = 0).  Errors:
 * rho <= 0 or not finite -> DCOCO_ERR_INVALID_ARG.  Deterministic. */
int dcoco_loss(const dcoco_dims* dims, const float* S, const int32_t* cand_ids,
               const int32_t* target_tok, float rho, float* loss, float* pair_loss,
               float* dS, void* stream);

/* Gradients of the shared scoring MLP, fp32, overwritten (not accumulated). */
typedef struct {
  float* dW1;   /* [d_mlp, 2 d_z + d_pair], columns as W1: [z_a | z_b | s] */
  float* db1;   /* [d_mlp] (also when b1 is NULL) */
  float* dw2;   /* [d_mlp] */
  float* db2;   /* [1] */
} dcoco_mlp_grads;

/* Backward of the transition scores ([P2] part 1, paper Sec. 3.2): given
 * G = dL/dS (e.g. from dcoco_loss), with x = [z_{p,a}; z_{p+1,b}; s_p] and
 * u = W1 x + b1,
 *   dw2 = sum G SiLU(u), db2 = sum G, du = G w2 SiLU'(u),
 *   dW1 = sum du x^T, db1 = sum du, dx = W1^T du -> dz_{p,a}, dz_{p+1,b}, ds_p,
 *   d l_{p+1}(b) = sum_a G(a, b)  (the draft logit term).
 * Sums run over every pair and candidate pair; the forward's bf16 rounding of
 * z counts as the identity.  A, B and the pair term are recomputed here.
 *   z             [n_blocks, B, K, d_z] dtype   the forward's z
 *   s             [n_blocks, B-1, d_pair] fp32  the forward's s
 *   dS            [n_blocks, B-1, K, K] fp32    G
 *   dz            [n_blocks, B, K, d_z] fp32    out
 *   ds            [n_blocks, B-1, d_pair] fp32  out (may be NULL)
 *   d_cand_logits [n_blocks, B, K] fp32         out (may be NULL; slot 1 gets 0)
 *   grads                                       out (every pointer required)
 * Workspace as for dcoco_score (query with workspace == NULL).  Deterministic:
 * split sums are added in a fixed order. */
int dcoco_score_backward(const dcoco_dims* dims, const dcoco_weights* w, const void* z,
                         const float* s, const float* dS, float* dz, float* ds,
                         float* d_cand_logits, const dcoco_mlp_grads* grads,
                         void* workspace, size_t* workspace_bytes, void* stream);

/* Gradients of the representation weights, fp32, overwritten. */
typedef struct {
  float* dP_e;     /* [d_proj, d_embed] */
  float* dP_h;     /* [d_proj, d_hidden] */
  float* dW_f;     /* [d_z, 2 d_proj], columns as W_f: [b | g] */
  float* dW_pair;  /* [d_pair, 2 d_hidden], columns as W_pair: [h_p | h_{p+1}] */
} dcoco_rep_grads;

/* Backward of the representations ([P2] part 1, paper Sec. 3.2, with the
 * forward of dcoco_represent): given dz = dL/dz and ds = dL/ds (e.g. from
 * dcoco_score_backward), with x_e = P_e E[c], x_h = P_h h, b = LN(x_e),
 * g = LN(x_h), sigma = sqrt(var + eps) per row:
 *   dW_f = sum_{i,k} dz_{i,k} [b_{i,k}; g_i]^T,
 *   db = W_fb^T dz,  dg_i = W_fg^T sum_k dz_{i,k},
 *   dx = (dy - mean(dy) - y mean(dy y)) / sigma  (LN backward, y = LN(x)),
 *   dP_e = sum dx_e E[c]^T,  dP_h = sum dx_h h^T,
 *   dW_pair = sum_p ds_p [h_p; h_{p+1}]^T,
 *   dh_i = P_h^T dx_{h,i} + W_L^T ds_i + W_R^T ds_{i-1}  (pairs that exist).
 * E is frozen (no gradient).  x_e and x_h are recomputed; the bf16 roundings
 * of b and g count as the identity, and dW_f takes the rounded b and g.
 * bf16 storage only (fp32 storage: DCOCO_ERR_UNSUPPORTED).
 *   h, E, cand_ids  as dcoco_represent
 *   dz   [n_blocks, B, K, d_z] fp32
 *   ds   [n_blocks, B-1, d_pair] fp32   (may be NULL when B == 1)
 *   grads                               out (every pointer required)
 *   dh   [n_blocks, B, d_hidden] fp32   out, may be NULL (not computed)
 * The gradient products run on bf16 MFMA over a two-part bf16 split of the
 * fp32 gradients (relative remainder <= 2^-17) with fp32 accumulation.
 * Workspace queried as for the other entry points.  Deterministic. */
int dcoco_represent_backward(const dcoco_dims* dims, const dcoco_weights* w, const void* h,
                             const void* E, const int32_t* cand_ids, const float* dz,
                             const float* ds, const dcoco_rep_grads* grads, float* dh,
                             void* workspace, size_t* workspace_bytes, void* stream);

/* The whole corrector for n_blocks draft blocks, on one stream: top-K
 * ([P1] "Keep the leading candidates"), representations and pair states
 * ([P1] "Score neighboring candidates in parallel"; [P2] part 1, paper
 * Sec. 3.2), transition scores (same passages) and the prefix-first greedy
 * walk ([P1] "Select using the realized token identities"; [P2] part 2,
 * paper Sec. 3.3).  It reads only what one drafter pass leaves behind (its
 * logits and hidden states) plus the frozen embedding table and the
 * corrector's own parameters, and returns the corrected block y_1..y_B
 * ([P2] part 1: no extra drafter pass).  Each step is exactly the entry
 * point of the same name above; the intermediates live in the workspace.
 *   logits [n_blocks*B, V], h [n_blocks, B, d_hidden], E [V, d_embed]: dtype
 *   sel_tok         [n_blocks, B] int32           out: the corrected block
 *   sel_idx         [n_blocks, B] int32           out, may be NULL
 *   S_out           [n_blocks, B-1, K, K] fp32    out, may be NULL
 *   cand_ids_out    [n_blocks, B, K] int32        out, may be NULL
 *   cand_logits_out [n_blocks, B, K] fp32         out, may be NULL */
int dcoco_correct_block(const dcoco_dims* dims, const dcoco_weights* w,
                        const void* logits, const void* h, const void* E,
                        void* workspace, size_t* workspace_bytes,
                        int32_t* sel_tok, int32_t* sel_idx, float* S_out,
                        int32_t* cand_ids_out, float* cand_logits_out,
                        void* stream);

/* dcoco_correct_block with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The intermediates live in a static
 * buffer of DCOCO_STATIC_SCRATCH_BYTES (96 MiB) inside the library, one per
 * GPU, held from the library's load until the process ends; the call
 * allocates nothing.  Arguments, outputs, ordering and results are those of
 * dcoco_correct_block (the same kernels run).  A problem whose workspace
 * (dcoco_correct_block's size query) exceeds the buffer returns
 * DCOCO_ERR_UNSUPPORTED before anything is launched; the 32-stream
 * B = 16, K = 16, d = 4096, V = 151936 workload fits.  Every call on one GPU
 * uses that GPU's single buffer: calls that overlap in time on one GPU (two
 * streams, two threads) race and corrupt each other's results; serialise
 * them.  No part of the buffer needs to start at any value, so what an
 * earlier call left there does not matter.  dcoco_static_scratch_bytes()
 * returns the buffer's size. */
#define DCOCO_STATIC_SCRATCH_BYTES (96u << 20)
int dcoco_correct_block_static(const dcoco_dims* dims, const dcoco_weights* w,
                               const void* logits, const void* h, const void* E,
                               int32_t* sel_tok, int32_t* sel_idx, float* S_out,
                               int32_t* cand_ids_out, float* cand_logits_out,
                               void* stream);
size_t dcoco_static_scratch_bytes(void);

/* Table of normalised candidate projections, a re-association of step a2
 * beyond the per-call path: E is frozen and P_e fixed at inference ([P1]
 * "Score neighboring candidates in parallel"; [P2] part 1), so
 * b_v = LN(P_e E_v) can be formed once for every token v and gathered per
 * call instead of gathering E rows and projecting them.  bf16 only (fp32
 * storage returns DCOCO_ERR_UNSUPPORTED); any d_proj the other entry points
 * accept.
 *   E     [V, d_embed] bf16
 *   table [V, d_proj] bf16   out: b_v rounded to bf16 (the per-call rounding
 *                            point of b); uses only w->P_e.
 * Workspace as for the other entry points (the fp32 partial sums of one
 * chunk of 8192 rows).  Run once per weight set; the table is the caller's. */
int dcoco_build_btable(const dcoco_dims* dims, const dcoco_weights* w, const void* E,
                       void* table, void* workspace, size_t* workspace_bytes, void* stream);

/* dcoco_correct_block with b_{i,k} read from a table made by
 * dcoco_build_btable (table [V, d_proj] bf16) instead of projecting gathered
 * E rows; w->P_e is not used.  Same outputs, ordering and errors; the result
 * equals the per-call path up to the fp32 summation order of P_e E_v.  bf16
 * only. */
int dcoco_correct_block_btable(const dcoco_dims* dims, const dcoco_weights* w,
                               const void* logits, const void* h, const void* btable,
                               void* workspace, size_t* workspace_bytes,
                               int32_t* sel_tok, int32_t* sel_idx, float* S_out,
                               int32_t* cand_ids_out, float* cand_logits_out,
                               void* stream);

/* Static description of a status code. */
const char* dcoco_status_string(int status);

/* ABI version of this header (major * 100 + minor): 101 adds the table
 * entry points, 102 dcoco_select_path, 103 dcoco_loss and
 * dcoco_score_backward, 104 dcoco_lm_head_topk, 105
 * dcoco_represent_backward, 106 dcoco_correct_block_static, 107 the table
 * entry points for any d_proj, 108 dcoco_lm_head_topk for K up to 64. */
int dcoco_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DCOCO_H */
