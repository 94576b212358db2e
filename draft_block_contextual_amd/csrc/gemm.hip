// MFMA GEMMs of the representation stage: out = A * W^T for the slot
// projections (P_h, W_pair), the gathered candidate-embedding projection P_e,
// the two halves of the fusion W_f, and the pair-state part of the MLP's first
// layer (review of arXiv 2610.12570, "Contextual Correction of Parallel
// Drafts for Speculative Decoding", part 1 of "New approach: DCOCO", paper
// Sec. 3.2).
//
// Tiling for gfx950: 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a
// (BM/2) x (BN/2) block of 16 x 16 MFMA tiles.  bf16 x bf16 uses
// v_mfma_f32_16x16x32_bf16 with a 64-deep k stage; anything with an fp32
// operand runs v_mfma_f32_16x16x4_f32 (fp32 products and sums) with a 32-deep
// stage.  A and W tiles are staged in LDS (rows padded by 16 bytes against
// bank conflicts) and the next stage's global loads are issued before the
// current stage's MFMAs.  A lane holds 8 consecutive k values of one row in
// both operands, so any k order the instruction uses pairs them correctly.
// Large reductions are split over grid.z into fp32 partial sums that the
// consumer adds in a fixed order (deterministic, no atomics).
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace dcoco {

namespace {

constexpr int kGemmThreads = 256;

struct GemmDev {
  int M, N, Kd, ksplit;
  const char* A;
  long long lda;
  const int32_t* a_rows;
  int a_rows_max;              // clamp for gathered row ids
  const char* w0;
  const char* w1;
  const char* w2;
  long long ldw0, ldw1, ldw2;
  int col00, col01, col02;
  int end0, end1;
  float* out_f32;
  int ldo;
  void* out;
  const float* row_bias;
  int row_bias_div;
  const void* col_bias;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ void unpack_bf16x8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T>
__device__ __forceinline__ void lds_frag_f32(const char* p, float (&f)[8]) {
  if constexpr (std::is_same<T, bf16>::value) {
    unpack_bf16x8(*reinterpret_cast<const uint4*>(p), f);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 16);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

__device__ __forceinline__ f32x4_t mma_f32x8(const float (&a)[8], const float (&b)[8], f32x4_t c) {
#pragma unroll
  for (int t = 0; t < 8; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], c, 0, 0, 0);
  return c;
}

template <typename TA, typename TW, typename TO, int BM, int BN, int MODE>
__global__ void __launch_bounds__(kGemmThreads) gemm_kernel(GemmDev p) {
  constexpr bool kBF = std::is_same<TA, bf16>::value && std::is_same<TW, bf16>::value;
  constexpr int BK = kBF ? 64 : 32;
  constexpr int kRowA = BK * static_cast<int>(sizeof(TA));
  constexpr int kRowW = BK * static_cast<int>(sizeof(TW));
  constexpr int kStrA = kRowA + 16;
  constexpr int kStrW = kRowW + 16;
  constexpr int kCpA = kRowA / 16;
  constexpr int kCpW = kRowW / 16;
  constexpr int kLdA = (BM * kCpA + kGemmThreads - 1) / kGemmThreads;
  constexpr int kLdW = (BN * kCpW + kGemmThreads - 1) / kGemmThreads;
  constexpr int TM = BM / 32;
  constexpr int TN = BN / 32;
  constexpr int kElA = 16 / static_cast<int>(sizeof(TA));
  constexpr int kElW = 16 / static_cast<int>(sizeof(TW));

  __shared__ __align__(16) char sA[BM * kStrA];
  __shared__ __align__(16) char sW[BN * kStrW];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1;
  const int wn = wv & 1;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * BM;
  const int zs = blockIdx.z;
  const int kbeg = zs * p.ksplit;
  const int kend = min(p.Kd, kbeg + p.ksplit);

  // fixed per-thread sources of the 16-byte chunks this thread stages
  const char* srcA[kLdA];
  int dstA[kLdA];
  int kA[kLdA];
  bool okA[kLdA];
#pragma unroll
  for (int i = 0; i < kLdA; ++i) {
    const int c = tid + i * kGemmThreads;
    const int r = c / kCpA;
    const int cc = c % kCpA;
    okA[i] = c < BM * kCpA && (m0 + r) < p.M;
    long long row = m0 + r;
    if (okA[i] && p.a_rows) {
      int id = p.a_rows[m0 + r];
      id = id < 0 ? 0 : (id > p.a_rows_max ? p.a_rows_max : id);
      row = id;
    }
    srcA[i] = p.A + (row * p.lda) * static_cast<long long>(sizeof(TA)) + cc * 16;
    dstA[i] = r * kStrA + cc * 16;
    kA[i] = cc * kElA;
  }
  const char* srcW[kLdW];
  int dstW[kLdW];
  int kW[kLdW];
  bool okW[kLdW];
#pragma unroll
  for (int i = 0; i < kLdW; ++i) {
    const int c = tid + i * kGemmThreads;
    const int r = c / kCpW;
    const int cc = c % kCpW;
    const int j = n0 + r;
    okW[i] = c < BN * kCpW && j < p.N;
    const char* base;
    long long ld;
    int col0, j0;
    if (j < p.end0) { base = p.w0; ld = p.ldw0; col0 = p.col00; j0 = 0; }
    else if (j < p.end1) { base = p.w1; ld = p.ldw1; col0 = p.col01; j0 = p.end0; }
    else { base = p.w2; ld = p.ldw2; col0 = p.col02; j0 = p.end1; }
    srcW[i] = base + (static_cast<long long>(j - j0) * ld + col0) * static_cast<long long>(sizeof(TW)) + cc * 16;
    dstW[i] = r * kStrW + cc * 16;
    kW[i] = cc * kElW;
  }

  uint4 ra[kLdA], rw[kLdW];
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kLdA; ++i)
      ra[i] = (okA[i] && k0 + kA[i] < kend)
                  ? *reinterpret_cast<const uint4*>(srcA[i] + static_cast<long long>(k0) * sizeof(TA))
                  : zero4;
#pragma unroll
    for (int i = 0; i < kLdW; ++i)
      rw[i] = (okW[i] && k0 + kW[i] < kend)
                  ? *reinterpret_cast<const uint4*>(srcW[i] + static_cast<long long>(k0) * sizeof(TW))
                  : zero4;
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int frow = l & 15;
  const int fk = (l >> 4) * 8;

  if (kbeg < kend) gload(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
#pragma unroll
    for (int i = 0; i < kLdA; ++i)
      if (tid + i * kGemmThreads < BM * kCpA) *reinterpret_cast<uint4*>(sA + dstA[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < kLdW; ++i)
      if (tid + i * kGemmThreads < BN * kCpW) *reinterpret_cast<uint4*>(sW + dstW[i]) = rw[i];
    __syncthreads();
    if (k0 + BK < kend) gload(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      if constexpr (kBF) {
        bf16x8_t fa[TM], fw[TN];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          fa[a] = as_bf16x8(*reinterpret_cast<const uint4*>(
              sA + (wm * (BM / 2) + a * 16 + frow) * kStrA + (ks + fk) * 2));
#pragma unroll
        for (int b = 0; b < TN; ++b)
          fw[b] = as_bf16x8(*reinterpret_cast<const uint4*>(
              sW + (wn * (BN / 2) + b * 16 + frow) * kStrW + (ks + fk) * 2));
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fw[b], acc[a][b], 0, 0, 0);
      } else {
        float fa[TM][8], fw[TN][8];
#pragma unroll
        for (int a = 0; a < TM; ++a)
          lds_frag_f32<TA>(sA + (wm * (BM / 2) + a * 16 + frow) * kStrA +
                               (ks + fk) * static_cast<int>(sizeof(TA)), fa[a]);
#pragma unroll
        for (int b = 0; b < TN; ++b)
          lds_frag_f32<TW>(sW + (wn * (BN / 2) + b * 16 + frow) * kStrW +
                               (ks + fk) * static_cast<int>(sizeof(TW)), fw[b]);
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b) acc[a][b] = mma_f32x8(fa[a], fw[b], acc[a][b]);
      }
    }
    __syncthreads();
  }

  // epilogue: lane l holds column (l & 15), rows 4 (l >> 4) + v of each tile
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * (BM / 2) + a * 16 + (l >> 4) * 4 + v;
        const int n = n0 + wn * (BN / 2) + b * 16 + (l & 15);
        if (m < p.M && n < p.N) {
          if constexpr (MODE == 0) {
            p.out_f32[(static_cast<long long>(zs) * p.M + m) * p.ldo + n] = acc[a][b][v];
          } else {
            float x = acc[a][b][v];
            if (p.row_bias) x += p.row_bias[static_cast<long long>(m / p.row_bias_div) * p.N + n];
            if (p.col_bias) x += Elem<TW>::to_f32(static_cast<const TW*>(p.col_bias)[n]);
            static_cast<TO*>(p.out)[static_cast<long long>(m) * p.ldo + n] = Elem<TO>::from_f32(x);
          }
        }
      }
}

// bf16 x bf16 with a multi-stage ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: each wave instruction writes 64 lanes x 16 bytes
// = 1 KB of LDS, so staging costs no VGPRs and several k stages stay in
// flight per workgroup).  A stage holds 64 k values: 128-byte tile rows.  Row
// r's 16-byte chunk c is stored at position c ^ ((r >> 1) & 7), so the 16
// rows a fragment read touches hit 16 distinct 4-bank groups.
constexpr int kDmaRow = 128;

__device__ __forceinline__ int dma_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// WM x WN waves, each owning a (BM / WM) x (BN / WN) block of the tile.
template <int BM, int BN, int WM, int WN, int STAGES, int MODE>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_bf16_dma_kernel(GemmDev p, int tiles_m, int tiles_n, int remap) {
  constexpr int NW = WM * WN;
  constexpr int kABytes = BM * kDmaRow;
  constexpr int kWBytes = BN * kDmaRow;
  constexpr int kStage = kABytes + kWBytes;
  constexpr int AJ = kABytes / 1024 / NW;  // A load instructions per wave per stage
  constexpr int WJ = kWBytes / 1024 / NW;
  constexpr int IPS = AJ + WJ;
  constexpr int MW = BM / WM;              // wave block
  constexpr int NWB = BN / WN;
  constexpr int TM = MW / 16;
  constexpr int TN = NWB / 16;
  static_assert(AJ >= 1 && WJ >= 1 && AJ * NW * 1024 == kABytes && WJ * NW * 1024 == kWBytes,
                "tile does not split into whole 1 KB copies per wave");
  static_assert(TM >= 1 && TN >= 1 && TM * 16 * WM == BM && TN * 16 * WN == BN, "wave grid");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  // one LDS object per ring slot: the compiler tracks direct-to-LDS loads per
  // object, so reads of one slot need not wait for loads into the others
  __shared__ __align__(1024) char sm0[kStage];
  __shared__ __align__(1024) char sm1[kStage];
  __shared__ __align__(1024) char sm2[STAGES >= 3 ? kStage : 16];
  __shared__ __align__(1024) char sm3[STAGES == 4 ? kStage : 16];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / WN;
  const int wn = wv % WN;
  int bid = blockIdx.x;
  if (remap) bid = (bid % 8) * (static_cast<int>(gridDim.x) / 8) + bid / 8;
  const int tn = bid % tiles_n;
  bid /= tiles_n;
  const int tm = bid % tiles_m;
  const int zs = bid / tiles_m;
  const int n0 = tn * BN;
  const int m0 = tm * BM;
  const int kbeg = zs * p.ksplit;
  const int kend = min(p.Kd, kbeg + p.ksplit);
  const int nk = kend > kbeg ? (kend - kbeg) / 64 : 0;

  // every lane always issues its loads (rows past the edge re-read a valid
  // row and are never stored), so vmcnt counts are exact
  const char* srcA[AJ];
#pragma unroll
  for (int j = 0; j < AJ; ++j) {
    const int r = 8 * (wv + NW * j) + (l >> 3);
    const int c = dma_swz(r, l & 7);
    const int m = min(m0 + r, p.M - 1);
    long long row = m;
    if (p.a_rows) {
      int id = p.a_rows[m];
      id = id < 0 ? 0 : (id > p.a_rows_max ? p.a_rows_max : id);
      row = id;
    }
    srcA[j] = p.A + row * p.lda * 2 + c * 16;
  }
  const char* srcW[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int r = 8 * (wv + NW * j) + (l >> 3);
    const int c = dma_swz(r, l & 7);
    const int jn = min(n0 + r, p.N - 1);
    const char* base;
    long long ld;
    int col0, j0;
    if (jn < p.end0) { base = p.w0; ld = p.ldw0; col0 = p.col00; j0 = 0; }
    else if (jn < p.end1) { base = p.w1; ld = p.ldw1; col0 = p.col01; j0 = p.end0; }
    else { base = p.w2; ld = p.ldw2; col0 = p.col02; j0 = p.end1; }
    srcW[j] = base + (static_cast<long long>(jn - j0) * ld + col0) * 2 + c * 16;
  }
  auto issue = [&](char* base, int k0) {
    const uint32_t b0 = __builtin_amdgcn_readfirstlane(lds_offset(base) + wv * 1024);
#pragma unroll
    for (int j = 0; j < AJ; ++j) dma16(srcA[j] + static_cast<long long>(k0) * 2, b0 + j * NW * 1024);
#pragma unroll
    for (int j = 0; j < WJ; ++j)
      dma16(srcW[j] + static_cast<long long>(k0) * 2, b0 + kABytes + j * NW * 1024);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto slot = [&](auto S) -> char* {
    constexpr int kS = decltype(S)::value;
    if constexpr (kS == 0) return sm0;
    else if constexpr (kS == 1) return sm1;
    else if constexpr (kS == 2) return sm2;
    else return sm3;
  };
  const int frow = l & 15;
  auto compute = [&](const char* sa) {
    const char* sw = sa + kABytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + (l >> 4);
      bf16x8_t fa[TM], fw[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int row = wm * MW + a * 16 + frow;
        fa[a] = as_bf16x8(*reinterpret_cast<const uint4*>(sa + row * kDmaRow + dma_swz(row, c) * 16));
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int row = wn * NWB + b * 16 + frow;
        fw[b] = as_bf16x8(*reinterpret_cast<const uint4*>(sw + row * kDmaRow + dma_swz(row, c) * 16));
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fw[b], acc[a][b], 0, 0, 0);
    }
  };
  // one pipeline step on ring slot S: wait for its loads, barrier, refill the
  // slot consumed in the previous step, then compute on slot S
  auto step = [&](auto S, int it) {
    constexpr int kS = decltype(S)::value;
    if (it + STAGES - 2 < nk) wait_vmcnt_barrier<(STAGES - 2) * IPS>();
    else wait_vmcnt_barrier<0>();
    if (it + STAGES - 1 < nk)
      issue(slot(std::integral_constant<int, (kS + STAGES - 1) % STAGES>{}),
            kbeg + (it + STAGES - 1) * 64);
    compute(slot(S));
  };
  if (0 < nk) issue(sm0, kbeg);
  if constexpr (STAGES >= 3) {
    if (1 < nk) issue(sm1, kbeg + 64);
  }
  if constexpr (STAGES == 4) {
    if (2 < nk) issue(sm2, kbeg + 128);
  }
  for (int it = 0; it < nk; it += STAGES) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < nk) step(std::integral_constant<int, 1>{}, it + 1);
    if constexpr (STAGES >= 3) {
      if (it + 2 < nk) step(std::integral_constant<int, 2>{}, it + 2);
    }
    if constexpr (STAGES == 4) {
      if (it + 3 < nk) step(std::integral_constant<int, 3>{}, it + 3);
    }
  }

  // epilogue; with a bias, all bias values are fetched (clamped, branch-free)
  // before any store so the loads overlap
  if constexpr (MODE == 1) {
    float bias[TM][TN][4];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = min(m0 + wm * MW + a * 16 + (l >> 4) * 4 + v, p.M - 1);
          const int n = min(n0 + wn * NWB + b * 16 + (l & 15), p.N - 1);
          float x = 0.f;
          if (p.row_bias) x += p.row_bias[static_cast<long long>(m / p.row_bias_div) * p.N + n];
          if (p.col_bias) x += bf16_to_f32(static_cast<const bf16*>(p.col_bias)[n].bits);
          bias[a][b][v] = x;
        }
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm * MW + a * 16 + (l >> 4) * 4 + v;
          const int n = n0 + wn * NWB + b * 16 + (l & 15);
          if (m < p.M && n < p.N)
            static_cast<bf16*>(p.out)[static_cast<long long>(m) * p.ldo + n] =
                bf16{f32_to_bf16(acc[a][b][v] + bias[a][b][v])};
        }
  } else {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm * MW + a * 16 + (l >> 4) * 4 + v;
          const int n = n0 + wn * NWB + b * 16 + (l & 15);
          if (m < p.M && n < p.N)
            p.out_f32[(static_cast<long long>(zs) * p.M + m) * p.ldo + n] = acc[a][b][v];
        }
  }
}

struct Tile {
  int bm, bn;
};

// bf16 x bf16 with Kd % 64 == 0 runs on the DMA kernel, which also has a
// 128 x 256 tile (8 waves): tall products with N >= 256 read each A row once
// per 256 columns
Tile pick_tile(int M, int N, bool dma) {
  const long long t128 = static_cast<long long>((M + 127) / 128) * ((N + 127) / 128);
  if (dma && M >= 2048 && N >= 256 && N % 256 == 0) return {128, 256};
  if (M >= 1024 && N >= 128 && t128 >= 64) return {128, 128};
  return {64, 64};
}

int pick_split(int M, int N, int Kd, int bk, bool dma) {
  const Tile t = pick_tile(M, N, dma);
  const long long tiles = static_cast<long long>((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  int split = 1;
  while (tiles * split < 256 && split < 4 && Kd / (split * 2) >= 4 * bk) split *= 2;
  return split;
}

template <typename TA, typename TW, typename TO>
hipError_t launch_gemm_t(const GemmProblem& q, hipStream_t st) {
  constexpr bool kBF = std::is_same<TA, bf16>::value && std::is_same<TW, bf16>::value;
  constexpr int BK = kBF ? 64 : 32;
  GemmDev p;
  p.M = q.M; p.N = q.N; p.Kd = q.Kd;
  const int split = q.split;
  int ks = (q.Kd + split - 1) / split;
  ks = (ks + BK - 1) / BK * BK;
  p.ksplit = ks;
  p.A = static_cast<const char*>(q.A);
  p.lda = q.lda;
  p.a_rows = q.a_rows;
  p.a_rows_max = q.a_rows_max > 0 ? q.a_rows_max : 0x7fffffff;
  p.w0 = static_cast<const char*>(q.w[0]);
  p.w1 = static_cast<const char*>(q.w[1] ? q.w[1] : q.w[0]);
  p.w2 = static_cast<const char*>(q.w[2] ? q.w[2] : q.w[0]);
  p.ldw0 = q.ldw[0]; p.ldw1 = q.ldw[1]; p.ldw2 = q.ldw[2];
  p.col00 = q.col0[0]; p.col01 = q.col0[1]; p.col02 = q.col0[2];
  p.end0 = q.seg_end[0]; p.end1 = q.seg_end[1];
  p.out_f32 = q.out_f32; p.ldo = q.ldo; p.out = q.out;
  p.row_bias = q.row_bias; p.row_bias_div = q.row_bias_div > 0 ? q.row_bias_div : 1;
  p.col_bias = q.col_bias;
  const bool dma = kBF && q.Kd % 64 == 0;
  const Tile t = pick_tile(q.M, q.N, dma);
  const bool partial = q.out == nullptr;
  if constexpr (kBF) {
    if (dma) {
      const int tiles_m = (q.M + t.bm - 1) / t.bm;
      const int tiles_n = (q.N + t.bn - 1) / t.bn;
      const int total = tiles_m * tiles_n * split;
      const int remap = (total % 8 == 0) ? 1 : 0;
#define DCOCO_DMA(BMV, BNV, WMV, WNV, ST, MODEV)                                                  \
  hipLaunchKernelGGL((gemm_bf16_dma_kernel<BMV, BNV, WMV, WNV, ST, MODEV>), dim3(total),              \
                     dim3(64 * WMV * WNV), 0, st, p, tiles_m, tiles_n, remap)
      if (t.bn == 256) {
        if (partial) DCOCO_DMA(128, 256, 2, 4, 3, 0); else DCOCO_DMA(128, 256, 2, 4, 3, 1);
      } else if (t.bm == 128) {
        if (partial) DCOCO_DMA(128, 128, 2, 2, 4, 0); else DCOCO_DMA(128, 128, 2, 2, 4, 1);
      } else {
        if (partial) DCOCO_DMA(64, 64, 2, 2, 4, 0); else DCOCO_DMA(64, 64, 2, 2, 4, 1);
      }
#undef DCOCO_DMA
      return hipGetLastError();
    }
  }
  dim3 grid((q.N + t.bn - 1) / t.bn, (q.M + t.bm - 1) / t.bm, split);
#define DCOCO_GEMM(BMV, BNV, MODEV)                                                       \
  hipLaunchKernelGGL((gemm_kernel<TA, TW, TO, BMV, BNV, MODEV>), grid, dim3(kGemmThreads), 0, st, p)
  if (t.bm == 128) {
    if (partial) DCOCO_GEMM(128, 128, 0); else DCOCO_GEMM(128, 128, 1);
  } else {
    if (partial) DCOCO_GEMM(64, 64, 0); else DCOCO_GEMM(64, 64, 1);
  }
#undef DCOCO_GEMM
  return hipGetLastError();
}

}  // namespace

int gemm_pick_split(int M, int N, int Kd, int a_dtype, int w_dtype) {
  const int bk = (a_dtype == kDtypeBf16 && w_dtype == kDtypeBf16) ? 64 : 32;
  const bool dma = a_dtype == kDtypeBf16 && w_dtype == kDtypeBf16 && Kd % 64 == 0;
  return pick_split(M, N, Kd, bk, dma);
}

hipError_t launch_gemm(const GemmProblem& q, hipStream_t st) {
  if (q.a_dtype == kDtypeBf16 && q.w_dtype == kDtypeBf16) return launch_gemm_t<bf16, bf16, bf16>(q, st);
  if (q.a_dtype == kDtypeF32 && q.w_dtype == kDtypeF32) return launch_gemm_t<float, float, float>(q, st);
  if (q.a_dtype == kDtypeF32 && q.w_dtype == kDtypeBf16) return launch_gemm_t<float, bf16, float>(q, st);
  return hipErrorInvalidValue;
}

}  // namespace dcoco
