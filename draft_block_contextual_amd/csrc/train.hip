// Training side of the corrector on the same score grid: the masked,
// decay-weighted joint-softmax loss and its gradient dL/dS, and the backward
// of the shared scoring MLP (gradients of W1, b1, w2, b2, of z and s, and of
// the draft logits).  Sources: Two Delta, "Two Delta makes NVIDIA Nemotron
// 3.5 Super even faster with DCOCO", section "How we train the corrector";
// review of arXiv 2610.12570, section "New approach: DCOCO", parts 1 and 3
// (paper Sec. 3.2, App. A).
#include "common.h"
#include "kernels.h"

namespace dcoco {
namespace {

constexpr int kThreads = 256;

// fixed-order sum over the 256 threads of a workgroup (tree over LDS); every
// thread gets the result
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
#pragma unroll
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
#pragma unroll
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// One workgroup per pair (n, p).  The label (a*, b*) is the position of the
// target token of slot p among c_p and of slot p+1 among c_{p+1}; a pair
// whose targets are not both present gets zero loss and zero gradient.
// Otherwise, with the joint softmax over the pair's K^2 scores and the
// weight w_p = exp(-p / rho) (p 0-based here):
//   pair_loss = w_p / N * (logsumexp(S_p) - S_p(a*, b*)),
//   dS_p      = w_p / N * (softmax(S_p) - onehot(a*, b*)).
__global__ void __launch_bounds__(kThreads)
loss_kernel(const float* __restrict__ S, const int32_t* __restrict__ ids, const int32_t* __restrict__ tgt,
            int B, int K, float rho, float inv_n, float* __restrict__ pair_loss, float* __restrict__ dS) {
  __shared__ float red[kThreads];
  __shared__ int s_pos[2];
  const int np = blockIdx.x;
  const int Bm1 = B - 1;
  const int n = np / Bm1;
  const int p = np - n * Bm1;
  const int tid = threadIdx.x;
  const int l = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int per = K * K;
  const float* Sp = S + static_cast<long long>(np) * per;
  float* dSp = dS + static_cast<long long>(np) * per;
  if (wv < 2) {
    // wave 0 looks for slot p's target, wave 1 for slot p+1's
    const long long slot = static_cast<long long>(n) * B + p + wv;
    const int t = tgt[slot];
    const bool hit = l < K && ids[slot * K + min(l, K - 1)] == t;
    const uint64_t m = ballot(hit);
    if (l == 0) s_pos[wv] = m ? __builtin_ctzll(m) : -1;
  }
  __syncthreads();
  const int a = s_pos[0];
  const int b = s_pos[1];
  if (a < 0 || b < 0) {
    for (int i = tid; i < per; i += kThreads) dSp[i] = 0.f;
    if (tid == 0) pair_loss[np] = 0.f;
    return;
  }
  float mx = -INFINITY;
  for (int i = tid; i < per; i += kThreads) mx = fmaxf(mx, Sp[i]);
  mx = block_max(mx, red);
  float se = 0.f;
  for (int i = tid; i < per; i += kThreads) se += expf(Sp[i] - mx);
  se = block_sum(se, red);
  const float coef = expf(-static_cast<float>(p) / rho) * inv_n;
  const float inv_se = 1.0f / se;
  const int label = a * K + b;
  for (int i = tid; i < per; i += kThreads) {
    const float sm = expf(Sp[i] - mx) * inv_se;
    dSp[i] = coef * (i == label ? sm - 1.0f : sm);
  }
  if (tid == 0) pair_loss[np] = coef * ((mx + logf(se)) - Sp[label]);
}

// out[blockIdx.x] = sum of x[blockIdx.x * chunk, ...+chunk) in a fixed order;
// eight independent loads per thread and round (indices clamped, masked)
__global__ void __launch_bounds__(kThreads) sum_kernel(const float* __restrict__ x, long long n, long long chunk,
                                                       float* __restrict__ out) {
  __shared__ float red[kThreads];
  const long long b0 = static_cast<long long>(blockIdx.x) * chunk;
  const long long b1 = min(n, b0 + chunk);
  float v = 0.f;
  for (long long i0 = b0 + threadIdx.x; i0 < b1; i0 += 8 * kThreads) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = x[min(i0 + j * kThreads, n - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += i0 + j * kThreads < b1 ? t[j] : 0.f;
  }
  v = block_sum(v, red);
  if (threadIdx.x == 0) out[blockIdx.x] = v;
}

// Column sums in a fixed order work on blocks of 64 columns x kColRows rows:
// four row groups of eight rows, loads all in flight, combined through LDS.
constexpr int kColRows = 32;

// The reductions after the grid backward in two launches.  First: the
// 32-row partial column sums of dw2p and dC (colsum_block, one block per
// (64 columns, 32 rows) of each) and d l (one thread per entry, the sum over a
// in order), side by side.
// Second: the partial rows added in order into dw2 and db1, and db2 as the
// sum of d l (every dS element enters d l exactly once, slot 0 holds zeros).
__device__ __forceinline__ void colsum_block(const float* __restrict__ x, int rows, int cols, long long ld, int bx,
                                             int by, float* red, float* __restrict__ out) {
  const int c = bx * 64 + (threadIdx.x & 63);
  const int g = threadIdx.x >> 6;
  const int cc = min(c, cols - 1);
  const int r0 = by * kColRows + g * (kColRows / 4);
  float t[kColRows / 4];
#pragma unroll
  for (int j = 0; j < kColRows / 4; ++j) t[j] = x[static_cast<long long>(min(r0 + j, rows - 1)) * ld + cc];
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < kColRows / 4; ++j) v += r0 + j < rows ? t[j] : 0.f;
  red[threadIdx.x] = v;
  __syncthreads();
  if (g == 0 && c < cols)
    out[static_cast<long long>(by) * cols + c] =
        (red[threadIdx.x] + red[threadIdx.x + 64]) + (red[threadIdx.x + 128] + red[threadIdx.x + 192]);
}

__global__ void __launch_bounds__(kThreads) mlp_reduce1_kernel(const float* __restrict__ dw2p,
                                                               const float* __restrict__ dC, int P, int H,
                                                               const float* __restrict__ dS, int N, int B, int K,
                                                               float* __restrict__ part_w, float* __restrict__ part_c,
                                                               float* __restrict__ dcl) {
  __shared__ float red[kThreads];
  const int cb = (H + 63) / 64;
  const int rb = (P + kColRows - 1) / kColRows;
  const int nb = cb * rb;
  const int blk = blockIdx.x;
  if (blk < nb) {
    colsum_block(dw2p, P, H, H, blk % cb, blk / cb, red, part_w);
  } else if (blk < 2 * nb) {
    colsum_block(dC, P, H, H, (blk - nb) % cb, (blk - nb) / cb, red, part_c);
  } else {
    const long long idx = static_cast<long long>(blk - 2 * nb) * kThreads + threadIdx.x;
    if (idx >= static_cast<long long>(N) * B * K) return;
    const int b = static_cast<int>(idx % K);
    const long long ni = idx / K;
    const int i = static_cast<int>(ni % B);
    const long long n = ni / B;
    float v = 0.f;
    if (i > 0) {
      const float* g = dS + ((n * (B - 1) + i - 1) * K) * K + b;
      for (int a = 0; a < K; ++a) v += g[static_cast<long long>(a) * K];
    }
    dcl[idx] = v;
  }
}

__global__ void __launch_bounds__(kThreads) mlp_reduce2_kernel(const float* __restrict__ part_w,
                                                               const float* __restrict__ part_c, int P, int H,
                                                               const float* __restrict__ dcl, long long ncl,
                                                               float* __restrict__ dw2, float* __restrict__ db1,
                                                               float* __restrict__ db2) {
  __shared__ float red[kThreads];
  const int cb = (H + 63) / 64;
  const int rb = (P + kColRows - 1) / kColRows;
  const int blk = blockIdx.x;
  if (blk < 2 * cb) {
    const float* part = blk < cb ? part_w : part_c;
    float* out = blk < cb ? dw2 : db1;
    const int bx = blk % cb;
    if (rb <= kColRows) {
      colsum_block(part, rb, H, H, bx, 0, red, out);
    } else {
      // many row blocks: one thread per column adds them in order
      const int c = bx * 64 + static_cast<int>(threadIdx.x);
      if (threadIdx.x < 64 && c < H) {
        float v = 0.f;
        for (int r = 0; r < rb; ++r) v += part[static_cast<long long>(r) * H + c];
        out[c] = v;
      }
    }
    return;
  }
  // db2: fixed-order sum of d l over one workgroup
  float v = 0.f;
  for (long long i = threadIdx.x; i < ncl; i += kThreads) v += dcl[i];
  red[threadIdx.x] = v;
  __syncthreads();
#pragma unroll
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (static_cast<int>(threadIdx.x) < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) db2[0] = red[0];
}

__global__ void __launch_bounds__(kThreads) fill_kernel(float* __restrict__ x, long long n, float v) {
  const long long i = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) x[i] = v;
}

// Backward of the scoring grid.  One thread per (pair, hidden unit h): with
// A' = A_{p,a,h} + C_{p,h} (C already holds b1) and B_b = B_{p+1,b,h},
//   u = A' + B_b, sig = 1 / (1 + e^-u), SiLU = u sig,
//   SiLU' = sig (1 + u (1 - sig)), du = dS(a, b) w2_h SiLU',
//   dA(a, h) = sum_b du, dB(b, h) = sum_a du, dC(h) = sum du,
//   dw2 part(h) = sum dS(a, b) SiLU.
// e^-u is formed as e^-A' e^-B when both exponents are within +-40 (no
// overflow of the product), else per element.  No cross-thread reductions:
// every sum above runs inside one thread.  The pair that ends at the last
// slot also zeroes that slot's dA rows, and the pair that starts at slot 0
// zeroes slot 0's dB rows, so dAB holds a full [N*B*K, 2H] gradient.
template <int KR, typename T>
__global__ void __launch_bounds__(kThreads) grid_bwd_kernel(GridBwdArgs g) {
  __shared__ float sG[KR * KR];
  const int np = blockIdx.x;
  const int Bm1 = g.B - 1;
  const int n = np / Bm1;
  const int p = np - n * Bm1;
  const int K = g.K;
  const int H = g.H;
  const int tid = threadIdx.x;
  const int h = blockIdx.y * kThreads + tid;
  const int hh = min(h, H - 1);
  const long long ld = 2ll * H;
  for (int i = tid; i < K * K; i += kThreads) sG[i] = g.dS[static_cast<long long>(np) * K * K + i];

  float c = 0.f;
  for (int q = 0; q < g.nq; ++q) c += g.C[(static_cast<long long>(q) * g.P + np) * H + hh];
  if (g.b1) c += Elem<T>::to_f32(static_cast<const T*>(g.b1)[hh]);
  const float w2h = Elem<T>::to_f32(static_cast<const T*>(g.w2)[hh]);
  const float* Arow = g.AB + (static_cast<long long>(n) * g.B + p) * K * ld + hh;
  const float* Brow = g.AB + (static_cast<long long>(n) * g.B + p + 1) * K * ld + H + hh;

  // every row of B (and, for KR <= 32, of A) is loaded before the first use:
  // unconditional loads with the row clamped, so none waits for another
  constexpr int KA = KR <= 32 ? KR : 1;
  float bv[KR], eb[KR], db[KR], av[KA];
#pragma unroll
  for (int b = 0; b < KR; ++b) bv[b] = Brow[static_cast<long long>(min(b, K - 1)) * ld];
  if constexpr (KR <= 32) {
#pragma unroll
    for (int a = 0; a < KR; ++a) av[a] = Arow[static_cast<long long>(min(a, K - 1)) * ld];
  }
  // the pair term joins the B side: u = A(a) + (B(b) + c).  sigma(u) =
  // 1 / (1 + e^-A e^-(B+c)) is exact in the factored form whenever e^-A is a
  // normal number (|A| <= 80): a B-side factor of 0 or inf then still gives
  // sigma = 1 or 0
#pragma unroll
  for (int b = 0; b < KR; ++b) {
    bv[b] += c;
    eb[b] = expf(-bv[b]);
    db[b] = 0.f;
  }
  __syncthreads();
  float dw2 = 0.f, dc = 0.f;
  float* dArow = g.dAB + (static_cast<long long>(n) * g.B + p) * K * ld + h;
  for (int a = 0; a < K; ++a) {
    float ar;
    if constexpr (KR <= 32) {
      ar = av[0];
#pragma unroll
      for (int t = 1; t < KR; ++t) ar = a == t ? av[t] : ar;
    } else {
      ar = Arow[static_cast<long long>(a) * ld];
    }
    const float ap = ar;
    const float* ga = sG + a * K;
    float da = 0.f;
    if (fabsf(ap) <= 80.f) {
      const float ea = expf(-ap);
#pragma unroll
      for (int b = 0; b < KR; ++b) {
        if (b < K) {
          const float u = ap + bv[b];
          const float sg = __builtin_amdgcn_rcpf(fmaf(ea, eb[b], 1.0f));
          const float gab = ga[b];
          const float du = gab * w2h * (sg * fmaf(u, 1.0f - sg, 1.0f));
          dw2 = fmaf(gab, u * sg, dw2);
          da += du;
          db[b] += du;
        }
      }
    } else {
#pragma unroll
      for (int b = 0; b < KR; ++b) {
        if (b < K) {
          const float u = ap + bv[b];
          const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * u));
          const float gab = ga[b];
          const float du = gab * w2h * (sg * fmaf(u, 1.0f - sg, 1.0f));
          dw2 = fmaf(gab, u * sg, dw2);
          da += du;
          db[b] += du;
        }
      }
    }
    dc += da;
    if (h < H) dArow[static_cast<long long>(a) * ld] = da;
  }
  if (h >= H) return;
  float* dBrow = g.dAB + (static_cast<long long>(n) * g.B + p + 1) * K * ld + H + h;
#pragma unroll
  for (int b = 0; b < KR; ++b)
    if (b < K) dBrow[static_cast<long long>(b) * ld] = db[b];
  g.dC[static_cast<long long>(np) * H + h] = dc;
  g.dw2p[static_cast<long long>(np) * H + h] = dw2;
  if (p == Bm1 - 1) {
    float* z = g.dAB + (static_cast<long long>(n) * g.B + Bm1) * K * ld + h;
    for (int a = 0; a < K; ++a) z[static_cast<long long>(a) * ld] = 0.f;
  }
  if (p == 0) {
    float* z = g.dAB + static_cast<long long>(n) * g.B * K * ld + H + h;
    for (int b = 0; b < K; ++b) z[static_cast<long long>(b) * ld] = 0.f;
  }
}

// Plain fp32 tiled product C[m, n] (+)= sum_k A(m, k) B(k, n) with element
// strides, for the gradient products (operands read as stored, bf16 or fp32,
// and widened).  64 x 64 tile, 256 threads of 4 x 4 outputs, 16-deep k
// stages through LDS; the load order follows whichever index of an operand is
// contiguous.  Loads are unconditional (indices clamped) and masked to zero.
// blockIdx.z takes one k range of a split; its partial goes to C + z * c_split.
template <typename TA, typename TB>
__global__ void __launch_bounds__(kThreads) gemm_f32_kernel(GemmF32Args g) {
  __shared__ __align__(16) float sA[16][68];
  __shared__ __align__(16) float sB[16][68];
  const int tid = threadIdx.x;
  const int tx = tid & 15;
  const int ty = tid >> 4;
  const int m0 = blockIdx.y * 64;
  const int n0 = blockIdx.x * 64;
  const int kb = blockIdx.z * g.k_split;
  const int ke = min(g.K, kb + g.k_split);
  const TA* A = static_cast<const TA*>(g.A);
  const TB* Bm = static_cast<const TB*>(g.B);
  const bool a_mc = g.a_m == 1;   // A contiguous along m
  const bool b_nc = g.b_n == 1;   // B contiguous along n
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 16) {
    float av[4], bw[4];
    int am[4], ak[4], bk[4], bn[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      am[r] = a_mc ? (tid & 63) : (tid >> 4) + 16 * r;
      ak[r] = a_mc ? (tid >> 6) + 4 * r : (tid & 15);
      bn[r] = b_nc ? (tid & 63) : (tid >> 4) + 16 * r;
      bk[r] = b_nc ? (tid >> 6) + 4 * r : (tid & 15);
      const int mm = min(m0 + am[r], g.M - 1);
      const int ka = min(k0 + ak[r], ke - 1);
      const int nn = min(n0 + bn[r], g.N - 1);
      const int kk = min(k0 + bk[r], ke - 1);
      av[r] = Elem<TA>::to_f32(A[mm * g.a_m + ka * g.a_k]);
      bw[r] = Elem<TB>::to_f32(Bm[kk * g.b_k + nn * g.b_n]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sA[ak[r]][am[r]] = (m0 + am[r] < g.M && k0 + ak[r] < ke) ? av[r] : 0.f;
      sB[bk[r]][bn[r]] = (n0 + bn[r] < g.N && k0 + bk[r] < ke) ? bw[r] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4*>(&sA[kk][ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&sB[kk][tx * 4]);
      const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
      const float br[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* C = g.C + static_cast<long long>(blockIdx.z) * g.c_split;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nn = n0 + tx * 4 + j;
      if (nn >= g.N) continue;
      float* o = C + static_cast<long long>(m) * g.ldc + nn;
      *o = g.accumulate ? *o + acc[i][j] : acc[i][j];
    }
  }
}

// out[r * ld_out + c] = sum over the splits s (in order) of
// part[s * split_stride + r * ld_part + c]
__global__ void __launch_bounds__(kThreads) sum_splits_kernel(const float* __restrict__ part, int splits,
                                                              long long split_stride, int rows, int cols,
                                                              long long ld_part, float* __restrict__ out,
                                                              long long ld_out) {
  const long long idx = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<long long>(rows) * cols) return;
  const long long r = idx / cols;
  const long long c = idx % cols;
  const float* src = part + r * ld_part + c;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += src[s * split_stride];
  out[r * ld_out + c] = v;
}

// LayerNorm forward and backward per row, one wave per row (4 rows per
// workgroup), VPL values per lane (column l + 64 i).  Forward as in the
// representation stage: the split partials added in order, two-pass mean and
// variance in fp32, y = (x - mean) / sqrt(var + eps).  Backward:
// dx = (dy - mean(dy) - y mean(dy y)) / sqrt(var + eps), dy being the sum
// (in order) of rep upstream rows.  The bf16 y of row m is stored into rows
// m y_rep .. m y_rep + y_rep - 1 of y_bf (row stride ld_y).
template <int VPL>
__global__ void __launch_bounds__(kThreads)
ln_fwd_bwd_kernel(const float* __restrict__ x, int split, int M, int ldx, int col0, int r, float eps,
                  const float* __restrict__ dY, long long ld_dy, int dy_col0, int rep, uint16_t* __restrict__ y_bf,
                  long long ld_y, int y_rep, float* __restrict__ dX, long long ld_dx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= M) return;
  const float inv_r = 1.0f / static_cast<float>(r);
  float v[VPL], g[VPL];
  int cc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    cc[i] = min(l + i * 64, r - 1);       // lanes past r re-read a valid column
    v[i] = 0.f;
    g[i] = 0.f;
  }
  // loads unconditional and several rows deep, sums in a fixed order
  for (int s = 0; s < split; ++s) {
    const float* xs = x + (static_cast<long long>(s) * M + row) * ldx + col0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] += xs[cc[i]];
  }
#pragma unroll 4
  for (int q = 0; q < rep; ++q) {
    const float* dq = dY + (static_cast<long long>(row) * rep + q) * ld_dy + dy_col0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) g[i] += dq[cc[i]];
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    if (l + i * 64 >= r) v[i] = g[i] = 0.f;
    sum += v[i];
  }
  const float mean = wave_sum(sum) * inv_r;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] = (l + i * 64) < r ? v[i] - mean : 0.f;
    sq += v[i] * v[i];
  }
  const float inv = 1.0f / sqrtf(wave_sum(sq) * inv_r + eps);
  float sg = 0.f, sgy = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    v[i] *= inv;                       // y
    sg += g[i];
    sgy += g[i] * v[i];
  }
  const float mg = wave_sum(sg) * inv_r;
  const float mgy = wave_sum(sgy) * inv_r;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * 64;
    if (c < r) {
      const uint16_t yb = f32_to_bf16(v[i]);
      for (int q = 0; q < y_rep; ++q) y_bf[(static_cast<long long>(row) * y_rep + q) * ld_y + c] = yb;
      dX[static_cast<long long>(row) * ld_dx + c] = (g[i] - mg - v[i] * mgy) * inv;
    }
  }
}

// The same per row with one workgroup per row (thread t takes columns t,
// t + 256, ...): for few rows with many upstream rows each, where one wave
// per row leaves most of the chip idle.  Sums over the workgroup: each wave's
// DPP sum, then the four added in wave order.
template <int VPT>
__global__ void __launch_bounds__(kThreads)
ln_fwd_bwd_wg_kernel(const float* __restrict__ x, int split, int M, int ldx, int col0, int r, float eps,
                     const float* __restrict__ dY, long long ld_dy, int dy_col0, int rep,
                     uint16_t* __restrict__ y_bf, long long ld_y, int y_rep, float* __restrict__ dX,
                     long long ld_dx) {
  __shared__ float red[4][4];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const float inv_r = 1.0f / static_cast<float>(r);
  float v[VPT], g[VPT];
  int cc[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    cc[i] = min(tid + i * kThreads, r - 1);
    v[i] = 0.f;
    g[i] = 0.f;
  }
  for (int s = 0; s < split; ++s) {
    const float* xs = x + (static_cast<long long>(s) * M + row) * ldx + col0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) v[i] += xs[cc[i]];
  }
#pragma unroll 8
  for (int q = 0; q < rep; ++q) {
    const float* dq = dY + (static_cast<long long>(row) * rep + q) * ld_dy + dy_col0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) g[i] += dq[cc[i]];
  }
  // workgroup sum of up to two values, fixed order
  auto wg_sum2 = [&](float a, float b, int slot, float& ra, float& rb) {
    a = wave_sum(a);
    b = wave_sum(b);
    if ((tid & 63) == 0) {
      red[slot][wv] = a;
      red[slot + 1][wv] = b;
    }
    __syncthreads();
    ra = (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
    rb = (red[slot + 1][0] + red[slot + 1][1]) + (red[slot + 1][2] + red[slot + 1][3]);
  };
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    if (tid + i * kThreads >= r) v[i] = g[i] = 0.f;
    sum += v[i];
  }
  float tot, unused;
  wg_sum2(sum, 0.f, 0, tot, unused);
  const float mean = tot * inv_r;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    v[i] = (tid + i * kThreads) < r ? v[i] - mean : 0.f;
    sq += v[i] * v[i];
  }
  float sqt;
  wg_sum2(sq, 0.f, 2, sqt, unused);
  const float inv = 1.0f / sqrtf(sqt * inv_r + eps);
  float sg = 0.f, sgy = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    v[i] *= inv;
    sg += g[i];
    sgy += g[i] * v[i];
  }
  __syncthreads();                         // red[0..1] is reused
  float tg, tgy;
  wg_sum2(sg, sgy, 0, tg, tgy);
  const float mg = tg * inv_r;
  const float mgy = tgy * inv_r;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int c = tid + i * kThreads;
    if (c < r) {
      const uint16_t yb = f32_to_bf16(v[i]);
      for (int q = 0; q < y_rep; ++q) y_bf[(static_cast<long long>(row) * y_rep + q) * ld_y + c] = yb;
      dX[static_cast<long long>(row) * ld_dx + c] = (g[i] - mg - v[i] * mgy) * inv;
    }
  }
}

// Acat[i][r + c] = ds of the pair whose left slot is i, Acat[i][r + rs + c] =
// ds of the pair whose right slot is i (zeros at the block ends)
__global__ void __launch_bounds__(kThreads) pack_ds_kernel(const float* __restrict__ ds, int N, int B, int rs, int r,
                                                           int C, float* __restrict__ Acat) {
  const long long idx = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<long long>(N) * B * 2 * rs) return;
  const long long i = idx / (2 * rs);
  const int c2 = static_cast<int>(idx % (2 * rs));
  const int side = c2 / rs;              // 0: i is the left slot, 1: the right slot
  const int c = c2 % rs;
  const long long n = i / B;
  const int j = static_cast<int>(i % B) - side;   // pair index within the block
  float v = 0.f;
  if (j >= 0 && j < B - 1) v = ds[(n * (B - 1) + j) * rs + c];
  Acat[i * C + r + c2] = v;
}

inline unsigned blocks_for(long long n) { return static_cast<unsigned>((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_loss(const float* S, const int32_t* cand_ids, const int32_t* target_tok, int N, int B, int K,
                       float rho, float* pair_loss, float* loss, float* dS, hipStream_t st) {
  const int P = N * (B - 1);
  if (P > 0)
    hipLaunchKernelGGL(loss_kernel, dim3(P), dim3(kThreads), 0, st, S, cand_ids, target_tok, B, K, rho,
                       1.0f / static_cast<float>(N), pair_loss, dS);
  hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(kThreads), 0, st, pair_loss, static_cast<long long>(P),
                     static_cast<long long>(P), loss);
  return hipGetLastError();
}

hipError_t launch_ln_fwd_bwd(const float* x, int split, int M, int ldx, int col0, int r, float eps, const float* dY,
                             long long ld_dy, int dy_col0, int rep, void* y_bf, long long ld_y, int y_rep, float* dX,
                             long long ld_dx, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  uint16_t* yb = static_cast<uint16_t*>(y_bf);
  if (M < 4096 && r <= 2048) {
    // few rows: a workgroup per row
    const int vpt = (r + kThreads - 1) / kThreads;
#define DCOCO_LNW(V)                                                                                              \
  hipLaunchKernelGGL((ln_fwd_bwd_wg_kernel<V>), dim3(M), dim3(kThreads), 0, st, x, split, M, ldx, col0, r, eps, dY, \
                     ld_dy, dy_col0, rep, yb, ld_y, y_rep, dX, ld_dx)
    if (vpt <= 1) DCOCO_LNW(1);
    else if (vpt <= 2) DCOCO_LNW(2);
    else if (vpt <= 4) DCOCO_LNW(4);
    else DCOCO_LNW(8);
#undef DCOCO_LNW
    return hipGetLastError();
  }
  const int vpl = (r + 63) / 64;
  const dim3 grid((M + 3) / 4);
#define DCOCO_LNB(V)                                                                                              \
  hipLaunchKernelGGL((ln_fwd_bwd_kernel<V>), grid, dim3(kThreads), 0, st, x, split, M, ldx, col0, r, eps, dY, ld_dy, \
                     dy_col0, rep, yb, ld_y, y_rep, dX, ld_dx)
  if (vpl <= 4) DCOCO_LNB(4);
  else if (vpl <= 8) DCOCO_LNB(8);
  else if (vpl <= 16) DCOCO_LNB(16);
  else if (vpl <= 32) DCOCO_LNB(32);
  else return hipErrorInvalidValue;
#undef DCOCO_LNB
  return hipGetLastError();
}

hipError_t launch_pack_ds(const float* ds, int N, int B, int rs, int r, int C, float* Acat, hipStream_t st) {
  const long long n = static_cast<long long>(N) * B * 2 * rs;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_ds_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, st, ds, N, B, rs, r, C, Acat);
  return hipGetLastError();
}

hipError_t launch_fill(float* x, long long n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, st, x, n, v);
  return hipGetLastError();
}

hipError_t launch_grid_bwd(const GridBwdArgs& g, int dtype, hipStream_t st) {
  const dim3 grid(g.P, (g.H + kThreads - 1) / kThreads);
#define DCOCO_BWD(KRV)                                                                           \
  do {                                                                                           \
    if (dtype == kDtypeBf16)                                                                     \
      hipLaunchKernelGGL((grid_bwd_kernel<KRV, bf16>), grid, dim3(kThreads), 0, st, g);          \
    else                                                                                         \
      hipLaunchKernelGGL((grid_bwd_kernel<KRV, float>), grid, dim3(kThreads), 0, st, g);         \
  } while (0)
  if (g.K <= 8) DCOCO_BWD(8);
  else if (g.K <= 16) DCOCO_BWD(16);
  else if (g.K <= 32) DCOCO_BWD(32);
  else DCOCO_BWD(64);
#undef DCOCO_BWD
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmF32Args& g, int a_dtype, int b_dtype, hipStream_t st) {
  const dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, (g.K + g.k_split - 1) / g.k_split);
  if (a_dtype == kDtypeBf16 && b_dtype == kDtypeBf16)
    hipLaunchKernelGGL((gemm_f32_kernel<bf16, bf16>), grid, dim3(kThreads), 0, st, g);
  else if (a_dtype == kDtypeBf16)
    hipLaunchKernelGGL((gemm_f32_kernel<bf16, float>), grid, dim3(kThreads), 0, st, g);
  else if (b_dtype == kDtypeBf16)
    hipLaunchKernelGGL((gemm_f32_kernel<float, bf16>), grid, dim3(kThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<float, float>), grid, dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int splits, int rows, int cols, float* out, long long ld_out,
                             hipStream_t st) {
  return launch_sum_splits_ex(part, splits, static_cast<long long>(rows) * cols, rows, cols, cols, out, ld_out, st);
}

// rows of part [M, cols] (splits split_stride apart) into up to three
// destinations: rows [0, end0) to out0, [end0, end1) to out1, the rest to out2
__global__ void __launch_bounds__(kThreads) sum_splits_seg_kernel(const float* __restrict__ part, int splits,
                                                                  long long split_stride, int rows, int cols,
                                                                  SegOut o) {
  const long long idx = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  if (idx >= static_cast<long long>(rows) * cols) return;
  const int r = static_cast<int>(idx / cols);
  const int c = static_cast<int>(idx % cols);
  const float* src = part + idx;
  float v = 0.f;
  for (int s = 0; s < splits; ++s) v += src[s * split_stride];
  float* dst;
  if (r < o.end0) dst = o.out0 + static_cast<long long>(r) * o.ld0;
  else if (r < o.end1) dst = o.out1 + static_cast<long long>(r - o.end0) * o.ld1;
  else dst = o.out2 + static_cast<long long>(r - o.end1) * o.ld2;
  dst[c] = v;
}

hipError_t launch_sum_splits_seg(const float* part, int splits, long long split_stride, int rows, int cols,
                                 const SegOut& o, hipStream_t st) {
  const long long n = static_cast<long long>(rows) * cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_splits_seg_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, st, part, splits, split_stride,
                     rows, cols, o);
  return hipGetLastError();
}

hipError_t launch_sum_splits_ex(const float* part, int splits, long long split_stride, int rows, int cols,
                                long long ld_part, float* out, long long ld_out, hipStream_t st) {
  const long long n = static_cast<long long>(rows) * cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_splits_kernel, dim3(blocks_for(n)), dim3(kThreads), 0, st, part, splits, split_stride,
                     rows, cols, ld_part, out, ld_out);
  return hipGetLastError();
}

int mlp_reduce_floats(int P, int H, int N, int B, int K) {
  const int rb = (P + kColRows - 1) / kColRows;
  return 2 * rb * H + N * B * K;
}

hipError_t launch_mlp_reduce(const float* dw2p, const float* dC, int P, int H, const float* dS, int N, int B, int K,
                             float* tmp, float* dw2, float* db1, float* db2, float* dcl_out, hipStream_t st) {
  const int cb = (H + 63) / 64;
  const int rb = (P + kColRows - 1) / kColRows;
  float* part_w = tmp;
  float* part_c = tmp + static_cast<long long>(rb) * H;
  float* dcl = dcl_out ? dcl_out : tmp + 2ll * rb * H;
  const long long ncl = static_cast<long long>(N) * B * K;
  const unsigned nb1 = static_cast<unsigned>(2 * cb * rb) + blocks_for(ncl);
  hipLaunchKernelGGL(mlp_reduce1_kernel, dim3(nb1), dim3(kThreads), 0, st, dw2p, dC, P, H, dS, N, B, K, part_w,
                     part_c, dcl);
  hipLaunchKernelGGL(mlp_reduce2_kernel, dim3(2 * cb + 1), dim3(kThreads), 0, st, part_w, part_c, P, H, dcl, ncl,
                     dw2, db1, db2);
  return hipGetLastError();
}

}  // namespace dcoco
