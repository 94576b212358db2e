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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "gemm_tile.h"
#include "kernels.h"
#include "select.h"
#include "wave.h"

namespace dcoco {

namespace {

constexpr int kGemmThreads = 256;



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

// One output tile (or one k split of it) per workgroup.
template <int BM, int BN, int WM, int WN, int STAGES, int MODE>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_bf16_dma_kernel(GemmDev p, int tiles_m, int tiles_n, int remap) {
  using G = DmaTile<BM, BN, WM, WN, STAGES>;
  constexpr int MW = G::MW, NWB = G::NWB, TM = G::TM, TN = G::TN, kStage = G::kStage;
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

  f32x4_t acc[TM][TN];
  dma_tile_mainloop<BM, BN, WM, WN, STAGES>(p, m0, n0, kbeg, kend, sm0, sm1, sm2, sm3, acc);

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
  const GemmDev p = gemm_dev(q, BK);
  const int split = q.split;
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

// ---------------------------------------------------------------------------
// Drafter LM head fused with top-K: logits l_i(v) = W_lm[v] . hd_i are formed
// tile by tile on MFMA, rounded to bf16 (the drafter's stored logit), and
// each workgroup keeps, per row, the top K of every vocabulary tile it has
// seen; the logits never reach memory.  Workgroup (tm, g) takes rows
// [BM tm, +BM) and vocabulary tiles g, g + groups, ...  Per tile, after the
// k loop, the BM x 256 keys are staged in the (now idle) LDS ring.  With K <= 16
// each row is then merged by one lane (all of the workgroup's rows at once, one
// per lane of the first BM / 64 waves): the lane marks its row's keys above the
// list's K-th best (or, while the list is not full, at or above a bound that K
// of the tile's keys reach: the K-th largest of the 64 per-lane maxima of the
// row, found by one wave beforehand), then pushes each marked composite through
// a fixed insertion network over its 16 list entries (a composite below the
// K-th best leaves the list as it is).  With K <= 64 one wave merges each row:
// the tile's composites above the row's K-th best go into its sorted list (a
// few: inserted one by one; many: an exact selection over list + tile).  The
// lists of all groups are merged by lm_head_merge_kernel.
constexpr int kLmBN = 256;
constexpr int kLmMaxK = 64;
// row tile: 256 rows (16 waves) where the lists are short (K <= 16), else
// 128 (8 waves); each wave owns 64 x 64 outputs; two ring slots
constexpr int lm_rows(int K) { return K <= 16 ? 256 : 128; }
template <int BM>
using LmTile = DmaTile<BM, kLmBN, BM / 64, 4, 2>;

__device__ __forceinline__ uint32_t key16_of(float x) { return order_key(bf16{f32_to_bf16(x)}); }

// The order keys of the bf16 roundings (to nearest, ties to even) of x0 and
// x1 in the low and high half: the packed conversion instruction rounds both,
// then per half a negative h maps to 0x8000 - (h & 0x7fff) (its two's
// complement) and a non-negative one to h + 0x8000; NaN maps to 0.  The same
// keys as key16_of.
__device__ __forceinline__ uint32_t key16x2(float x0, float x1) {
  const uint32_t h = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x0))) |
                     (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x1))) << 16);
  const uint32_t sgn = ((h >> 15) & 0x00010001u) * 0xffffu;       // 0xffff in each negative half
  const uint32_t neg = (~h & 0x7fff7fffu) + 0x00010001u;          // per half 0x8000 - (h & 0x7fff)
  const uint32_t pos = h | 0x80008000u;
  uint32_t k = (neg & sgn) | (pos & ~sgn);
  if (x0 != x0) k &= 0xffff0000u;
  if (x1 != x1) k &= 0x0000ffffu;
  return k;
}

// lane l gets lane l - 1's v (lane 0 gets 0): a DPP wave shift, no LDS permute
__device__ __forceinline__ uint64_t shift_up_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), 0x138, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), 0x138, 0xf, 0xf,
                                             false);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

// v from a wave-uniform lane, through the scalar unit (no LDS permute)
__device__ __forceinline__ uint64_t read_lane_u64(uint64_t v, int lane) {
  const uint32_t lo = read_lane_u32(static_cast<uint32_t>(v), lane);
  const uint32_t hi = read_lane_u32(static_cast<uint32_t>(v >> 32), lane);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// KMAX (16 or 64) bounds K: the rows' lists take BM KMAX composites of LDS
// beside the two ring slots: 128 + 16 KB for 256-row tiles at KMAX = 16,
// 96 + 64 KB for 128-row tiles at KMAX = 64.
template <int KMAX, int BM>
__global__ void __launch_bounds__(BM * 4) lm_head_topk_kernel(GemmDev p, int K, int tiles_m, int tiles_n, int groups,
                                                             int xcd_map, uint64_t* __restrict__ part) {
  using LT = LmTile<BM>;
  constexpr int kSlots = 2;
  constexpr int NWV = LT::NW;          // waves
  constexpr int NT = NWV * 64;         // threads
  constexpr int kLmBM = BM;
  constexpr int TM = LT::TM, TN = LT::TN, MW = LT::MW, NWB = LT::NWB;
  // K <= 16: a list entry is (key << 16) | (0xffff - the column's index within
  // the group: 256 x the group's tiles before it + column), 0 = empty; the
  // group holds at most 256 tiles.  K <= 64: the 64-bit composite.
  using TopT = std::conditional_t<KMAX == 16, uint32_t, uint64_t>;
  static_assert(kSlots * LT::kStage + kLmBM * KMAX * sizeof(TopT) <= 160 * 1024, "LDS");
  __shared__ __align__(1024) char sm0[LT::kStage];
  __shared__ __align__(1024) char sm1[LT::kStage];
  __shared__ TopT s_top[kLmBM][KMAX];   // per row, sorted; entry K - 1 is 0 until K are held
  // entry j of row r sits at j ^ (r & 15) for KMAX = 16, so the lanes that each
  // read their own row's entry j fall on different banks
  constexpr int kRowBytes = kLmBN * 2;                   // staged keys of one row
  constexpr int kRowsSlot = LT::kStage / kRowBytes;      // rows of keys one ring slot holds
  static_assert(kLmBM <= kSlots * kRowsSlot, "keys fit the ring");

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / 4;
  const int wn = wv % 4;
  const int b = blockIdx.x;
  int tm, g;
  if (xcd_map) {
    // the row tiles of one vocabulary group share an XCD (and its L2)
    const int idx = b / 8;
    tm = idx % tiles_m;
    g = (idx / tiles_m) * 8 + b % 8;
  } else {
    tm = b % tiles_m;
    g = b / tiles_m;
  }
  const int m0 = tm * kLmBM;
  auto keyrow = [&](int r) -> uint16_t* {
    return reinterpret_cast<uint16_t*>(r < kRowsSlot ? sm0 + r * kRowBytes : sm1 + (r - kRowsSlot) * kRowBytes);
  };
  auto tp = [](int r, int j) { return KMAX == 16 ? (j ^ (r & 15)) : j; };
  for (int i = tid; i < kLmBM * KMAX; i += NT) (&s_top[0][0])[i] = 0;

  int ord = 0;   // the group's tiles before this one
  for (int tn = g; tn < tiles_n; tn += groups, ++ord) {
    const int n0 = tn * kLmBN;
    f32x4_t acc[TM][TN];
    dma_tile_mainloop<kLmBM, kLmBN, kLmBM / 64, 4, 2>(p, m0, n0, 0, p.Kd, sm0, sm1, sm0, sm0, acc);
    __syncthreads();                         // every wave is done with the ring
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int bb = 0; bb < TN; ++bb) {
        const int c = wn * NWB + bb * 16 + (l & 15);
        const bool live = n0 + c < p.N;
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const int r = wm * MW + a * 16 + (l >> 4) * 4 + v;
          const uint32_t k2 = live ? key16x2(acc[a][bb][v], acc[a][bb][v + 1]) : 0u;
          keyrow(r)[c] = static_cast<uint16_t>(k2);
          keyrow(r + 1)[c] = static_cast<uint16_t>(k2 >> 16);
        }
      }
    __syncthreads();
    for (int i = 0; i < kLmBM / NWV; ++i) {
      const int r = wv + NWV * i;
      const uint16_t* kr = keyrow(r);
      if constexpr (KMAX == 16) {
        // a list not full yet: the K-th largest of the lanes' maxima over keys
        // 4 l .. 4 l + 3 (K of the tile's keys reach it), left in the list's
        // empty entry K - 1 as (1 << 16) | bound (no entry has key 1) for the
        // row's lane
        if (s_top[r][tp(r, K - 1)] == 0u) {
          const uint64_t v = *reinterpret_cast<const uint64_t*>(kr + 4 * l);
          const uint32_t m0 = max(static_cast<uint32_t>(v) & 0xffffu, static_cast<uint32_t>(v >> 16) & 0xffffu);
          const uint32_t m1 = max(static_cast<uint32_t>(v >> 32) & 0xffffu, static_cast<uint32_t>(v >> 48));
          const uint32_t mx = max(m0, m1);
          uint32_t tb = 0;
          for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = tb | (1u << bit);
            if (__popcll(ballot(mx >= cand)) >= K) tb = cand;
          }
          if (l == 0) s_top[r][tp(r, K - 1)] = (1u << 16) | tb;
        }
      } else {
      const uint64_t thr = s_top[r][K - 1];   // the row's K-th best so far (0 while not full)
      uint64_t c[5];
      c[0] = l < K ? s_top[r][l] : 0ull;     // the current list, sorted
      int n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = q * 64 + l;
        const uint32_t key = kr[col];
        const uint64_t cc = key ? make_comp(key, static_cast<uint32_t>(n0 + col)) : 0ull;
        c[q + 1] = cc > thr ? cc : 0ull;
        n += __popcll(ballot(c[q + 1] != 0ull));
      }
      if (n == 0) continue;
      if (n > 32) {
        // many newcomers (as on a row's first tile): only keys at or above
        // the K-th largest of the lanes' largest keys can make the list
        // (at least K newcomers reach it)
        uint32_t mk = 0;
#pragma unroll
        for (int q = 1; q < 5; ++q) mk = max(mk, comp_key(c[q]));
        uint32_t tk = 0;
        for (int bit = 15; bit >= 0; --bit) {
          const uint32_t cand = tk | (1u << bit);
          if (__popcll(ballot(mk >= cand)) >= K) tk = cand;
        }
        n = 0;
#pragma unroll
        for (int q = 1; q < 5; ++q) {
          c[q] = comp_key(c[q]) >= tk ? c[q] : 0ull;
          n += __popcll(ballot(c[q] != 0ull));
        }
      }
      uint64_t cur = c[0];
      if (n <= 32) {
        // insert each newcomer into the sorted list (lanes 0..K-1)
#pragma unroll
        for (int q = 1; q < 5; ++q) {
          uint64_t m = ballot(c[q] != 0ull);
          while (m) {
            const int src = __builtin_ctzll(m);
            m &= m - 1;
            const uint64_t x = read_lane_u64(c[q], src);
            const int pos = __popcll(ballot(l < K && cur > x));
            const uint64_t up = shift_up_u64(cur);
            cur = l < pos ? cur : (l == pos ? x : up);
          }
        }
      } else {
        bool sel[5];
        select_topk<5, 16>(c, K, sel);
        // compact the selection into lanes 0..K-1, then sort it
        uint64_t* scratch = &s_top[r][0];
        int base = 0;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
          const uint64_t m = ballot(sel[q]);
          __builtin_amdgcn_wave_barrier();
          if (sel[q]) scratch[base + lanes_below(m)] = c[q];
          base += __popcll(m);
        }
        __builtin_amdgcn_wave_barrier();
        const uint64_t mine = l < base ? scratch[l] : 0ull;
        int rank = 0;
        for (int j = 0; j < base; ++j) rank += read_lane_u64(mine, j) > mine ? 1 : 0;
        cur = 0ull;
        for (int j = 0; j < base; ++j) {
          const uint64_t xj = read_lane_u64(mine, j);
          const int rj = static_cast<int>(read_lane_u32(static_cast<uint32_t>(rank), j));
          cur = l == rj ? xj : cur;
        }
      }
      if (l < K) s_top[r][l] = cur;
      }
    }
    if constexpr (KMAX == 16) {
      __syncthreads();                       // the bounds of the rows not full yet
      if (tid < kLmBM) {
        // one lane per row: bit w of mw marks the row's 8-byte word (w + r) mod
        // 64 (the lanes start at different words, so their reads fall on
        // different banks) when one of its four keys beats the K-th best (full
        // list) or reaches the bound (list not full)
        const int r = tid;
        const uint32_t T = s_top[r][tp(r, K - 1)];
        const bool bound = (T >> 16) == 1u;
        const int tk = bound ? static_cast<int>(T & 0xffffu) - 1 : static_cast<int>(T >> 16);
        const uint16_t* kr = keyrow(r);
        auto word = [&](int w) { return *reinterpret_cast<const uint64_t*>(kr + 4 * ((w + r) & 63)); };
        auto key_of = [](uint64_t v, int j) { return static_cast<int>(static_cast<uint32_t>(v >> (16 * j)) & 0xffffu); };
        uint64_t mw = 0ull;
#pragma unroll 1
        for (int w8 = 0; w8 < 64; w8 += 8) {
          uint32_t m8 = 0u;
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const uint64_t v = word(w8 + w);
            const int mx = max(max(key_of(v, 0), key_of(v, 1)), max(key_of(v, 2), key_of(v, 3)));
            m8 |= (mx > tk ? 1u : 0u) << w;
          }
          mw |= static_cast<uint64_t>(m8) << w8;
        }
        uint32_t L[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t e = s_top[r][j ^ (r & 15)];
          L[j] = (bound && j == K - 1) ? 0u : e;   // the bound's entry was empty
        }
        // one marked key per lane and round, until no lane has any left (a
        // marked word holds at least one)
        uint64_t cur = 0ull;   // the current word's keys
        uint32_t ks = 0u;      // its marked keys not yet taken
        int wc = 0;            // its word index
        const bool any = mw != 0ull;
        while (ballot(mw != 0ull || ks != 0u) != 0ull) {
          if (ks == 0u && mw != 0ull) {
            wc = __builtin_ctzll(mw);
            mw &= mw - 1;
            cur = word(wc);
#pragma unroll
            for (int j = 0; j < 4; ++j) ks |= (key_of(cur, j) > tk ? 1u : 0u) << j;
          }
          uint32_t x = 0u;
          if (ks != 0u) {
            const int j = __builtin_ctz(ks);
            ks &= ks - 1;
            const int col = (((wc + r) & 63) << 2) | j;
            const uint32_t key = static_cast<uint32_t>(key_of(cur, j));   // 0: a pad column or NaN
            x = key ? (key << 16) | (0xffffu - static_cast<uint32_t>(ord * kLmBN + col)) : 0u;
          }
          // sorted insertion of x into L[0..15], the smallest falling out; the
          // first K entries depend only on the first K and x
#pragma unroll
          for (int j = 15; j >= 1; --j) L[j] = max(L[j], min(L[j - 1], x));
          L[0] = max(L[0], x);
        }
        if (any || bound) {
#pragma unroll
          for (int j = 0; j < 16; ++j) s_top[r][j ^ (r & 15)] = L[j];
        }
      }
    }
    __syncthreads();                         // the next tile's loads reuse the ring
  }
  for (int i = tid; i < kLmBM * K; i += NT) {
    const int r = i / K;
    const int j = i - r * K;
    uint64_t c;
    if constexpr (KMAX == 16) {
      // back to the global composite: column index 256 o + col of the group
      // is vocabulary id 256 (g + o groups) + col
      const uint32_t e = s_top[r][tp(r, j)];
      const uint32_t li = 0xffffu - (e & 0xffffu);
      c = e ? make_comp(e >> 16, static_cast<uint32_t>((g + static_cast<int>(li >> 8) * groups) * kLmBN +
                                                       static_cast<int>(li & 255u)))
            : 0ull;
    } else {
      c = s_top[r][j];
    }
    if (m0 + r < p.M) part[(static_cast<long long>(g) * p.M + m0 + r) * K + j] = c;
  }
}

// bf16 pattern of an order key (keys of -0 and +0 coincide: +0 comes back)
__device__ __forceinline__ float value_of_key16(uint32_t k) {
  const uint32_t bits = k >= 0x8000u ? k - 0x8000u : ((0x8000u - k) | 0x8000u);
  return bf16_to_f32(static_cast<uint16_t>(bits));
}

// One wave per row: the top K of the groups' lists, sorted (value desc, id
// asc), ids and bf16 values out.  Each list is sorted, so the K-th largest key
// among the groups' first entries bounds the answer from below (K entries
// reach it); the entries at or above it (a few more than K for the drafter's
// logits) are ranked directly.  Beyond 64 of them an exact selection over all
// entries runs instead.
template <int Q>
__global__ void __launch_bounds__(64) lm_head_merge_kernel(const uint64_t* __restrict__ part, int groups, int M,
                                                           int K, int32_t* __restrict__ ids, float* __restrict__ vals) {
  __shared__ uint64_t s_fin[64];
  const int row = blockIdx.x;
  const int l = threadIdx.x;
  uint64_t c[Q];
  bool sel[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = q * kWave + l;
    const int gq = i / K;
    c[q] = gq < groups ? part[(static_cast<long long>(gq) * M + row) * K + (i - gq * K)] : 0ull;
  }
  // the groups' first entries, one group per lane and round (groups <= 64 Q)
  uint32_t kf[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int gq = q * kWave + l;
    kf[q] = (q * kWave < groups && gq < groups)
                ? comp_key(part[(static_cast<long long>(gq) * M + row) * K]) : 0u;
  }
  uint32_t kb = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t cand = kb | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (q * kWave < groups) cnt += __popcll(ballot(kf[q] >= cand));
    if (cnt >= K) kb = cand;
  }
  int n = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) n += __popcll(ballot(c[q] != 0ull && comp_key(c[q]) >= kb));
  int base = 0;
  if (n <= kWave) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const bool in = c[q] != 0ull && comp_key(c[q]) >= kb;
      const uint64_t m = ballot(in);
      if (in) s_fin[base + lanes_below(m)] = c[q];
      base += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    const uint64_t mine = l < base ? s_fin[l] : 0ull;
    int rank = 0;
    for (int j = 0; j < base; ++j) rank += s_fin[j] > mine ? 1 : 0;
    if (l < base && rank < K) {
      ids[static_cast<long long>(row) * K + rank] = static_cast<int32_t>(0xffffffffu - comp_inv(mine));
      vals[static_cast<long long>(row) * K + rank] = value_of_key16(comp_key(mine));
    }
    return;
  }
  select_topk<Q, 16>(c, K, sel);
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t m = ballot(sel[q]);
    if (sel[q]) s_fin[base + lanes_below(m)] = c[q];
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  if (l < K) {
    const uint64_t mine = l < base ? s_fin[l] : 0ull;
    int rank = 0;
    for (int j = 0; j < base; ++j) rank += s_fin[j] > mine ? 1 : 0;
    if (l < base) {
      ids[static_cast<long long>(row) * K + rank] = static_cast<int32_t>(0xffffffffu - comp_inv(mine));
      vals[static_cast<long long>(row) * K + rank] = value_of_key16(comp_key(mine));
    }
  }
}

}  // namespace

GemmDev gemm_dev(const GemmProblem& q, int bk) {
  GemmDev p;
  p.M = q.M; p.N = q.N; p.Kd = q.Kd;
  int ks = (q.Kd + q.split - 1) / q.split;
  ks = (ks + bk - 1) / bk * bk;
  p.ksplit = ks;
  p.A = static_cast<const char*>(q.A);
  p.lda = q.lda;
  p.a_rows = q.a_rows;
  // gathered rows are always clamped into [0, a_rows_max] (0 is a valid
  // maximum: a one-row table); without a gather the clamp is never read
  p.a_rows_max = q.a_rows ? (q.a_rows_max > 0 ? q.a_rows_max : 0) : 0x7fffffff;
  p.w0 = static_cast<const char*>(q.w[0]);
  p.w1 = static_cast<const char*>(q.w[1] ? q.w[1] : q.w[0]);
  p.w2 = static_cast<const char*>(q.w[2] ? q.w[2] : q.w[0]);
  p.ldw0 = q.ldw[0]; p.ldw1 = q.ldw[1]; p.ldw2 = q.ldw[2];
  p.col00 = q.col0[0]; p.col01 = q.col0[1]; p.col02 = q.col0[2];
  p.end0 = q.seg_end[0]; p.end1 = q.seg_end[1];
  p.out_f32 = q.out_f32; p.ldo = q.ldo; p.out = q.out;
  p.row_bias = q.row_bias; p.row_bias_div = q.row_bias_div > 0 ? q.row_bias_div : 1;
  p.col_bias = q.col_bias;
  return p;
}

bool lm_head_topk_supported(int M, int V, int d, int K) {
  return M >= 1 && V >= K && K >= 1 && K <= kLmMaxK && d >= 64 && d % 64 == 0;
}

namespace {

// vocabulary groups for row tiles of `rows` rows
int lm_groups_for(int M, int V, int K, int rows) {
  const int tiles_m = (M + rows - 1) / rows;
  const int tiles_n = (V + kLmBN - 1) / kLmBN;
  int groups = std::max(1, 256 / tiles_m);
  groups = std::min(groups, 2048 / K);         // the merge holds 2048 composites per row
  groups = std::min(groups, tiles_n);
  if (groups >= 8) groups -= groups % 8;
  return groups;
}

// K <= 16 takes the 256-row kernel with 32-bit list entries while no group
// holds more than 256 vocabulary tiles; otherwise the 128-row kernel
bool lm_short_lists(int M, int V, int K) {
  if (K > 16) return false;
  const int tiles_n = (V + kLmBN - 1) / kLmBN;
  const int groups = lm_groups_for(M, V, K, lm_rows(16));
  return (tiles_n + groups - 1) / groups <= 256;
}

int lm_rows_for(int M, int V, int K) { return lm_short_lists(M, V, K) ? lm_rows(16) : lm_rows(64); }

}  // namespace

int lm_head_groups(int M, int V, int K) { return lm_groups_for(M, V, K, lm_rows_for(M, V, K)); }

size_t lm_head_workspace_bytes(int M, int V, int K) {
  return sizeof(uint64_t) * static_cast<size_t>(lm_head_groups(M, V, K)) * M * K;
}

hipError_t launch_lm_head_topk(const void* hd, const void* W_lm, int M, int V, int d, int K, void* workspace,
                               int32_t* ids, float* vals, hipStream_t st) {
  if (!lm_head_topk_supported(M, V, d, K)) return hipErrorInvalidValue;
  GemmDev p{};
  p.M = M; p.N = V; p.Kd = d; p.ksplit = d;
  p.A = static_cast<const char*>(hd); p.lda = d;
  p.w0 = p.w1 = p.w2 = static_cast<const char*>(W_lm);
  p.ldw0 = p.ldw1 = p.ldw2 = d;
  p.end0 = p.end1 = V;
  p.row_bias_div = 1;
  const int rows = lm_rows_for(M, V, K);
  const int tiles_m = (M + rows - 1) / rows;
  const int tiles_n = (V + kLmBN - 1) / kLmBN;
  const int groups = lm_head_groups(M, V, K);
  const int xcd_map = groups % 8 == 0 ? 1 : 0;
  uint64_t* part = static_cast<uint64_t*>(workspace);
  if (lm_short_lists(M, V, K))
    hipLaunchKernelGGL((lm_head_topk_kernel<16, lm_rows(16)>), dim3(tiles_m * groups), dim3(lm_rows(16) * 4), 0,
                       st, p, K, tiles_m, tiles_n, groups, xcd_map, part);
  else
    hipLaunchKernelGGL((lm_head_topk_kernel<64, lm_rows(64)>), dim3(tiles_m * groups), dim3(lm_rows(64) * 4), 0,
                       st, p, K, tiles_m, tiles_n, groups, xcd_map, part);
  const int count = groups * K;
#define DCOCO_LMM(QV) \
  hipLaunchKernelGGL((lm_head_merge_kernel<QV>), dim3(M), dim3(64), 0, st, part, groups, M, K, ids, vals)
  if (count <= 64) DCOCO_LMM(1);
  else if (count <= 256) DCOCO_LMM(4);
  else if (count <= 512) DCOCO_LMM(8);
  else if (count <= 1024) DCOCO_LMM(16);
  else DCOCO_LMM(32);
#undef DCOCO_LMM
  return hipGetLastError();
}

int gemm_pick_split(int M, int N, int Kd, int a_dtype, int w_dtype) {
  const int bk = (a_dtype == kDtypeBf16 && w_dtype == kDtypeBf16) ? 64 : 32;
  const bool dma = a_dtype == kDtypeBf16 && w_dtype == kDtypeBf16 && Kd % 64 == 0;
  return pick_split(M, N, Kd, bk, dma);
}

int gemm_pick_split_max(int M, int N, int Kd, int max_split) {
  const Tile t = pick_tile(M, N, Kd % 64 == 0);
  const long long tiles = static_cast<long long>((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
  int split = 1;
  while (tiles * split < 256 && split < max_split && Kd / (split * 2) >= 256) split *= 2;
  return split;
}

hipError_t launch_gemm(const GemmProblem& q, hipStream_t st) {
  if (q.a_dtype == kDtypeBf16 && q.w_dtype == kDtypeBf16) return launch_gemm_t<bf16, bf16, bf16>(q, st);
  if (q.a_dtype == kDtypeF32 && q.w_dtype == kDtypeF32) return launch_gemm_t<float, float, float>(q, st);
  if (q.a_dtype == kDtypeF32 && q.w_dtype == kDtypeBf16) return launch_gemm_t<float, bf16, float>(q, st);
  return hipErrorInvalidValue;
}

}  // namespace dcoco
