// Transition scoring and the prefix-first greedy walk.
//
// Scoring ([P1] "Score neighboring candidates in parallel"; [P2] part 1, paper
// Sec. 3.2): for every pair of neighbouring slots (p, p+1) and every candidate
// pair (a, b)
//   S_p(a,b) = l_{p+1}(b) + w2 . SiLU(W1a z_{p,a} + W1b z_{p+1,b} + W1s s_p + b1) + b2,
// i.e. the shared MLP applied to [z_{p,a}; z_{p+1,b}; s_p] with W1 split by
// its column blocks.  The per-candidate products W1a z and W1b z are formed
// once per slot and pair on MFMA, the pair part C_p = W1s s_p + b1 once per
// pair, and only the broadcast sum, SiLU and the w2 dot product run over the
// K x K x H grid, on the vector ALU in fp32.  s_p stays fp32: in the bf16 path
// it is split exactly into three bf16 parts (hi + mid + lo; 3 x 8 significand
// bits cover fp32's 24) that form three rows of an MFMA operand, and the three
// product rows are added in fp32.  With t = -log2(e) u:  SiLU(u) w2 = (-ln 2 w2) * t / (1 + 2^t), so
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

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

struct GridDev {
  int N, B, K, rz, rs, H;
  const void* z;
  const float* s;        // [N, B-1, rs] pair states (fp32)
  const void* W1;        // [H, 2 rz + rs]
  long long ldw1;
  const void* b1;        // [H] or null
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

// One workgroup (4 waves) per (block n, pair p).  The hidden units are cut
// into chunks of 32; wave w takes chunks w, w+4, ...  For a chunk, the wave
// forms A = -log2(e) W1a z_{p,a} and B = -log2(e) (W1b z_{p+1,b} + C_p) for
// its 32 units on MFMA into its own LDS tile, then runs the K x K x 32 grid
// from LDS.  Lane (la, lb) of the 8 x 8 lane grid owns the TA x TA outputs
// a = TA la + i, b = TA lb + j (K <= 8 TA).  The four waves' partial sums are
// added in a fixed order at the end.
constexpr int kChunkH = 32;
constexpr int kChunkStr = kChunkH + 4;     // LDS row stride (floats)
constexpr int kMaxPair = 2048;             // largest supported pair width

template <int TA>
struct GridSmem {
  static constexpr int KR = 8 * TA;
  static constexpr int KRM = ((KR + 15) / 16) * 16;
  static constexpr int kTile = KRM * kChunkStr;
  static constexpr int kRed = KR * KR;
  static constexpr int kWork = 2 * kTile + 2 * kChunkH;   // A, B tiles, w2', C
  static constexpr int kPerWave = kWork > kRed ? kWork : kRed;
};

template <typename T, int TA>
__global__ void __launch_bounds__(256) grid_kernel(GridDev g) {
  using SM = GridSmem<TA>;
  constexpr int KR = SM::KR;
  constexpr int MT = SM::KRM / 16;
  __shared__ __align__(16) float smem[4 * SM::kPerWave];

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

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int frow = l & 15;
  const int fk = (l >> 4) * 8;
  const int la = l >> 3;
  const int lb = l & 7;
  float* sA = smem + wv * SM::kPerWave;
  float* sB = sA + SM::kTile;
  float* sW = sB + SM::kTile;
  float* sC = sW + kChunkH;
  // s_p as MFMA operand rows: bf16 path hi/mid/lo parts in rows 0..2, fp32
  // path s_p itself in row 0
  constexpr int kSRows = std::is_same<T, bf16>::value ? 3 : 1;
  __shared__ __align__(16) T sS[kSRows * kMaxPair];
  const int rs = g.rs;
  const float* sp = g.s + static_cast<long long>(np) * rs;
  for (int k = tid; k < rs; k += 256) {
    const float x = sp[k];
    if constexpr (std::is_same<T, bf16>::value) {
      const uint16_t hi = f32_to_bf16(x);
      const float r1 = x - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
      sS[k] = bf16{hi};
      sS[kMaxPair + k] = bf16{mid};
      sS[2 * kMaxPair + k] = bf16{lo};
    } else {
      sS[k] = x;
    }
  }
  __syncthreads();

  float acc[TA][TA];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) acc[i][j] = 0.f;

  const int nchunks = g.H / kChunkH;
  for (int c = wv; c < nchunks; c += 4) {
    const int h0 = c * kChunkH;
    // ---- per-candidate products for 32 hidden units on MFMA
    f32x4_t accA[MT][2], accB[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        accA[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        accB[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    for (int k = 0; k < rz; k += 32) {
      FragT<T> fa[MT], fb[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int row = m * 16 + frow;
        fa[m].load(za + static_cast<long long>(row) * rz + k + fk, row < K);
        fb[m].load(zb + static_cast<long long>(row) * rz + k + fk, row < K);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const T* wrow = W1 + static_cast<long long>(h0 + t * 16 + frow) * g.ldw1 + k + fk;
        FragT<T> wa, wb;
        wa.load(wrow, true);
        wb.load(wrow + rz, true);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          accA[m][t] = mma(fa[m], wa, accA[m][t]);
          accB[m][t] = mma(fb[m], wb, accB[m][t]);
        }
      }
    }
    // ---- C_p = W1s s_p + b1 for the chunk's 32 units
    {
      f32x4_t accC[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
      for (int k = 0; k < rs; k += 32) {
        FragT<T> fs;
        fs.load(&sS[(frow < kSRows ? frow : 0) * kMaxPair + k + fk], frow < kSRows);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          FragT<T> ws;
          ws.load(W1 + static_cast<long long>(h0 + t * 16 + frow) * g.ldw1 + 2 * rz + k + fk, true);
          accC[t] = mma(fs, ws, accC[t]);
        }
      }
      // rows 0..kSRows-1 of the product live in lanes 0..15
      if (l < 16) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float cv = accC[t][0];
          if constexpr (kSRows == 3) cv = (cv + accC[t][1]) + accC[t][2];
          if (g.b1) cv += Elem<T>::to_f32(static_cast<const T*>(g.b1)[h0 + t * 16 + l]);
          sC[t * 16 + l] = cv;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = t * 16 + (l & 15);
      const float cb = sC[col];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = m * 16 + (l >> 4) * 4 + v;
          sA[row * kChunkStr + col] = kNegLog2e * accA[m][t][v];
          sB[row * kChunkStr + col] = kNegLog2e * (accB[m][t][v] + cb);
        }
    }
    if (l < kChunkH) sW[l] = kNegLn2 * Elem<T>::to_f32(w2[h0 + l]);
    // LDS operations of one wave complete in order: the reads below see the
    // writes above without a barrier
    __builtin_amdgcn_wave_barrier();
    // ---- the K x K x 32 grid
#pragma unroll 2
    for (int h = 0; h < kChunkH; h += 4) {
      float4 av[TA], bv[TA];
#pragma unroll
      for (int i = 0; i < TA; ++i) {
        av[i] = *reinterpret_cast<const float4*>(&sA[(la * TA + i) * kChunkStr + h]);
        bv[i] = *reinterpret_cast<const float4*>(&sB[(lb * TA + i) * kChunkStr + h]);
      }
      const float4 wq = *reinterpret_cast<const float4*>(&sW[h]);
      const float w4[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          const float a4[4] = {av[i].x, av[i].y, av[i].z, av[i].w};
#pragma unroll
          for (int j = 0; j < TA; ++j) {
            const float b4[4] = {bv[j].x, bv[j].y, bv[j].z, bv[j].w};
            const float t = a4[cc] + b4[cc];
            const float e = __builtin_amdgcn_exp2f(t);
            const float r = __builtin_amdgcn_rcpf(1.0f + e);
            acc[i][j] = fmaf(w4[cc], t * r, acc[i][j]);
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // ---- add the four waves' partial sums in a fixed order
  __syncthreads();
  float* red = smem + wv * SM::kPerWave;
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) red[(la * TA + i) * KR + lb * TA + j] = acc[i][j];
  __syncthreads();
  const float* lnext = g.cand_logits + (static_cast<long long>(n) * g.B + p + 1) * K;
  float* Sp = g.S + static_cast<long long>(np) * K * K;
  for (int idx = tid; idx < K * K; idx += 256) {
    const int a = idx / K;
    const int b = idx - a * K;
    const int o = a * KR + b;
    const float sum = ((smem[o] + smem[SM::kPerWave + o]) + smem[2 * SM::kPerWave + o]) +
                      smem[3 * SM::kPerWave + o];
    Sp[idx] = lnext[b] + (sum + g.b2);
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
  g.N = q.N; g.B = q.B; g.K = q.K; g.rz = q.rz; g.rs = q.rs; g.H = q.H;
  g.z = q.z; g.s = q.s; g.W1 = q.W1; g.ldw1 = q.ldw1; g.b1 = q.b1; g.w2 = q.w2; g.b2 = q.b2;
  g.cand_logits = q.cand_logits; g.S = q.S;
  const int blocks = q.N * (q.B - 1);
  if (blocks <= 0) return hipSuccess;
#define DCOCO_GRID(TAV) hipLaunchKernelGGL((grid_kernel<T, TAV>), dim3(blocks), dim3(256), 0, st, g)
  if (q.K <= 8) DCOCO_GRID(1);
  else if (q.K <= 16) DCOCO_GRID(2);
  else if (q.K <= 32) DCOCO_GRID(4);
  else DCOCO_GRID(8);
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
