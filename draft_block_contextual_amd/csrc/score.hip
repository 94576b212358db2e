// Transition scoring and the prefix-first greedy walk.
//
// Scoring ([P1] "Score neighboring candidates in parallel"; [P2] part 1, paper
// Sec. 3.2): for every pair of neighbouring slots (p, p+1) and every candidate
// pair (a, b)
//   S_p(a,b) = l_{p+1}(b) + w2 . SiLU(W1a z_{p,a} + W1b z_{p+1,b} + W1s s_p + b1) + b2,
// i.e. the shared MLP applied to [z_{p,a}; z_{p+1,b}; s_p] with W1 split by
// its column blocks.  The per-candidate products W1a z and W1b z are formed
// once per slot on MFMA (not once per pair), the pair part C_p = W1s s_p + b1
// once per pair (by the GEMM before this kernel), and only the broadcast sum,
// SiLU and the w2 dot product run over the K x K x H grid, on the vector ALU
// in fp32.  With t = -log2(e) u:  SiLU(u) w2 = (-ln 2 w2) * t / (1 + 2^t), so
// each grid element costs one add, exp2, add, rcp, mul and fma.
//
// Walk ([P1] "Select using the realized token identities"; [P2] part 2, paper
// Sec. 3.3): k_1 = argmax l_1, k_{p+1} = argmax_b S_p(k_p, b); the lowest
// index wins ties and NaN never wins.  One wave walks one block; the whole
// block's scores are first staged in LDS so the sequential steps read LDS,
// not memory.
//
// P1 = Two Delta, "Two Delta makes NVIDIA Nemotron 3.5 Super even faster with
// DCOCO"; P2 = review of arXiv 2610.12570, "Contextual Correction of Parallel
// Drafts for Speculative Decoding".
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dcoco {

namespace {

constexpr int kHC = 128;                 // MLP hidden units per LDS chunk
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

struct GridDev {
  int N, B, K, rz, H;
  const void* z;
  const void* W1;
  long long ldw1;
  const float* C;
  const void* w2;
  float b2;
  const float* cand_logits;
  float* S;
};

__device__ __forceinline__ void load8_f32(const bf16* p, float (&f)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8_f32(const float* p, float (&f)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// MFMA operand fragment: 8 consecutive k values of one row.
template <typename T> struct FragT;
template <> struct FragT<bf16> {
  bf16x8_t v;
  __device__ void load(const bf16* p, bool ok) {
    const uint4 u = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
    v = __builtin_bit_cast(bf16x8_t, u);
  }
};
template <> struct FragT<float> {
  float v[8];
  __device__ void load(const float* p, bool ok) {
    if (ok) {
      load8_f32(p, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
  }
};

__device__ __forceinline__ f32x4_t mma(const FragT<bf16>& a, const FragT<bf16>& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma(const FragT<float>& a, const FragT<float>& b, f32x4_t c) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[t], b.v[t], c, 0, 0, 0);
  return c;
}

// One workgroup per (block n, pair p).  TA = ceil(K/16): the K candidate rows
// are padded to 16*TA, and thread t scores the (a, b) = (t/16 + 16i,
// t%16 + 16j) entries, i, j < TA.
template <typename T, int TA>
__global__ void __launch_bounds__(256) grid_kernel(GridDev g) {
  constexpr int KR = 16 * TA;
  constexpr int kStr = kHC + 4;
  __shared__ __align__(16) float sA[KR * kStr];
  __shared__ __align__(16) float sB[KR * kStr];
  __shared__ __align__(16) float sW2[kHC];

  const int np = blockIdx.x;
  const int Bm1 = g.B - 1;
  const int n = np / Bm1;
  const int p = np % Bm1;
  const int K = g.K;
  const int rz = g.rz;
  const T* za = static_cast<const T*>(g.z) + (static_cast<long long>(n) * g.B + p) * K * rz;
  const T* zb = za + static_cast<long long>(K) * rz;
  const T* W1 = static_cast<const T*>(g.W1);
  const T* w2 = static_cast<const T*>(g.w2);
  const float* Cp = g.C + static_cast<long long>(np) * g.H;

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int ta = tid >> 4;
  const int tb = tid & 15;
  const int frow = l & 15;
  const int fk = (l >> 4) * 8;

  float acc[TA][TA];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) acc[i][j] = 0.f;

  for (int hc0 = 0; hc0 < g.H; hc0 += kHC) {
    const int hlen = min(kHC, g.H - hc0);
    // ---- per-candidate products on MFMA: wave wv owns 32 hidden units
    if (wv * 32 < hlen) {
      f32x4_t accA[TA][2], accB[TA][2];
#pragma unroll
      for (int i = 0; i < TA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          accA[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          accB[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      for (int k = 0; k < rz; k += 32) {
        FragT<T> fa[TA], fb[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          const int row = i * 16 + frow;
          fa[i].load(za + static_cast<long long>(row) * rz + k + fk, row < K);
          fb[i].load(zb + static_cast<long long>(row) * rz + k + fk, row < K);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int h = hc0 + wv * 32 + j * 16 + frow;
          const T* wrow = W1 + static_cast<long long>(h) * g.ldw1 + k + fk;
          FragT<T> wa, wb;
          wa.load(wrow, true);
          wb.load(wrow + rz, true);
#pragma unroll
          for (int i = 0; i < TA; ++i) {
            accA[i][j] = mma(fa[i], wa, accA[i][j]);
            accB[i][j] = mma(fb[i], wb, accB[i][j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wv * 32 + j * 16 + (l & 15);
        const float c = Cp[hc0 + col];
#pragma unroll
        for (int i = 0; i < TA; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = i * 16 + (l >> 4) * 4 + v;
            sA[row * kStr + col] = kNegLog2e * accA[i][j][v];
            sB[row * kStr + col] = kNegLog2e * (accB[i][j][v] + c);
          }
      }
    }
    if (tid < hlen) sW2[tid] = kNegLn2 * Elem<T>::to_f32(w2[hc0 + tid]);
    __syncthreads();
    // ---- the K x K x hlen grid on the vector ALU
    for (int h = 0; h < hlen; h += 4) {
      float4 av[TA], bv[TA];
#pragma unroll
      for (int i = 0; i < TA; ++i) {
        av[i] = *reinterpret_cast<const float4*>(&sA[(ta + 16 * i) * kStr + h]);
        bv[i] = *reinterpret_cast<const float4*>(&sB[(tb + 16 * i) * kStr + h]);
      }
      const float4 wq = *reinterpret_cast<const float4*>(&sW2[h]);
      const float w4[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          const float a4[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
          for (int j = 0; j < TA; ++j) {
            const float b4[4] = {bv[j].x, bv[j].y, bv[j].z, bv[j].w};
            const float t = a4[c] + b4[c];
            const float e = __builtin_amdgcn_exp2f(t);
            const float r = __builtin_amdgcn_rcpf(1.0f + e);
            acc[i][j] = fmaf(w4[c], t * r, acc[i][j]);
          }
        }
      }
    }
    __syncthreads();
  }
  const float* lnext = g.cand_logits + (static_cast<long long>(n) * g.B + p + 1) * K;
  float* Sp = g.S + static_cast<long long>(np) * K * K;
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) {
      const int a = ta + 16 * i;
      const int b = tb + 16 * j;
      if (a < K && b < K) Sp[a * K + b] = lnext[b] + (acc[i][j] + g.b2);
    }
}

constexpr int kWalkLds = 8192;   // floats of scores staged per batch

__device__ __forceinline__ uint64_t arg_comp(float v, int idx) {
  return (static_cast<uint64_t>(order_key(v)) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(idx));
}

__global__ void __launch_bounds__(256)
walk_kernel(const float* __restrict__ S, const float* __restrict__ cl, const int32_t* __restrict__ ids,
            int B, int K, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_tok) {
  __shared__ __align__(16) float sS[kWalkLds];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int per = K * K;
  const int batch = max(1, kWalkLds / per);
  const int Bm1 = B - 1;
  const float* Sn = S + static_cast<long long>(n) * Bm1 * per;
  const float* cln = cl + static_cast<long long>(n) * B * K;
  const int32_t* idn = ids + static_cast<long long>(n) * B * K;
  int k = 0;
  if (tid < kWave) {
    const uint64_t c = l < K ? arg_comp(cln[l], l) : 0ull;
    const uint64_t best = wave_max_u64(c);
    k = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
    if (l == 0) {
      if (sel_idx) sel_idx[static_cast<long long>(n) * B] = k;
      sel_tok[static_cast<long long>(n) * B] = idn[k];
    }
  }
  for (int p0 = 0; p0 < Bm1; p0 += batch) {
    const int cnt = min(batch, Bm1 - p0);
    const int nval = cnt * per;
    __syncthreads();
    for (int i = tid; i < nval; i += 256) sS[i] = Sn[static_cast<long long>(p0) * per + i];
    __syncthreads();
    if (tid < kWave) {
      for (int q = 0; q < cnt; ++q) {
        const int p = p0 + q;
        const uint64_t c = l < K ? arg_comp(sS[q * per + k * K + l], l) : 0ull;
        const uint64_t best = wave_max_u64(c);
        k = static_cast<int>(0xffffffffu - static_cast<uint32_t>(best));
        if (l == 0) {
          if (sel_idx) sel_idx[static_cast<long long>(n) * B + p + 1] = k;
          sel_tok[static_cast<long long>(n) * B + p + 1] = idn[(p + 1) * K + k];
        }
      }
    }
  }
}

template <typename T>
hipError_t launch_grid_t(const GridProblem& q, hipStream_t st) {
  GridDev g;
  g.N = q.N; g.B = q.B; g.K = q.K; g.rz = q.rz; g.H = q.H;
  g.z = q.z; g.W1 = q.W1; g.ldw1 = q.ldw1; g.C = q.C; g.w2 = q.w2; g.b2 = q.b2;
  g.cand_logits = q.cand_logits; g.S = q.S;
  const int blocks = q.N * (q.B - 1);
  if (blocks <= 0) return hipSuccess;
  const int ta = (q.K + 15) / 16;
#define DCOCO_GRID(TAV) hipLaunchKernelGGL((grid_kernel<T, TAV>), dim3(blocks), dim3(256), 0, st, g)
  if (ta <= 1) DCOCO_GRID(1);
  else if (ta == 2) DCOCO_GRID(2);
  else if (ta == 3) DCOCO_GRID(3);
  else DCOCO_GRID(4);
#undef DCOCO_GRID
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grid(const GridProblem& q, hipStream_t st) {
  if (q.dtype == kDtypeBf16) return launch_grid_t<bf16>(q, st);
  return launch_grid_t<float>(q, st);
}

hipError_t launch_walk(const float* S, const float* cand_logits, const int32_t* cand_ids, int N,
                       int B, int K, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st) {
  hipLaunchKernelGGL(walk_kernel, dim3(N), dim3(256), 0, st, S, cand_logits, cand_ids, B, K, sel_idx,
                     sel_tok);
  return hipGetLastError();
}

}  // namespace dcoco
