// The tile machinery shared by the GEMM kernels and by the launch that runs
// the slot-side GEMM tiles beside the top-K rows: the device-side problem
// description and the bf16 k loop that stages both operands through an LDS
// ring with direct global->LDS loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace dcoco {

// A GemmProblem as the kernels read it.
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

// bf16 x bf16 with a multi-stage ring filled by direct global->LDS loads
// (global_load_lds_dwordx4: each wave instruction writes 64 lanes x 16 bytes
// = 1 KB of LDS, so staging costs no VGPRs and several k stages stay in
// flight per workgroup).  A stage holds 64 k values: 128-byte tile rows.  Row
// r's 16-byte chunk c is stored at position c ^ ((r >> 1) & 7), so the 16
// rows a fragment read touches hit 16 distinct 4-bank groups.
constexpr int kDmaRow = 128;

__device__ __forceinline__ int dma_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// Geometry of a BM x BN tile computed by WM x WN waves, each owning a
// (BM / WM) x (BN / WN) block of 16 x 16 MFMA tiles, with a ring of STAGES
// 64-deep k stages.
template <int BM, int BN, int WM, int WN, int STAGES>
struct DmaTile {
  static constexpr int NW = WM * WN;
  static constexpr int kABytes = BM * kDmaRow;
  static constexpr int kWBytes = BN * kDmaRow;
  static constexpr int kStage = kABytes + kWBytes;
  static constexpr int AJ = kABytes / 1024 / NW;  // A load instructions per wave per stage
  static constexpr int WJ = kWBytes / 1024 / NW;
  static constexpr int IPS = AJ + WJ;
  static constexpr int MW = BM / WM;              // wave block
  static constexpr int NWB = BN / WN;
  static constexpr int TM = MW / 16;
  static constexpr int TN = NWB / 16;
  static_assert(AJ >= 1 && WJ >= 1 && AJ * NW * 1024 == kABytes && WJ * NW * 1024 == kWBytes,
                "tile does not split into whole 1 KB copies per wave");
  static_assert(TM >= 1 && TN >= 1 && TM * 16 * WM == BM && TN * 16 * WN == BN, "wave grid");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
};

// The k loop of one tile: acc = A[m0 : m0 + BM, kbeg : kend] W[n0 : n0 + BN,
// kbeg : kend]^T (kend - kbeg a multiple of 64) through the LDS ring sm0..sm3
// (one LDS object per slot: the compiler tracks direct-to-LDS loads per
// object, so reads of one slot need not wait for loads into the others).
// Every lane always issues its loads (rows past the edge re-read a valid row
// and are never stored), so vmcnt counts are exact.  Leaves every load
// complete; the caller synchronises before it reuses the ring.
template <int BM, int BN, int WM, int WN, int STAGES>
__device__ __forceinline__ void dma_tile_mainloop(
    const GemmDev& p, int m0, int n0, int kbeg, int kend, char* sm0, char* sm1, char* sm2, char* sm3,
    f32x4_t (&acc)[DmaTile<BM, BN, WM, WN, STAGES>::TM][DmaTile<BM, BN, WM, WN, STAGES>::TN]) {
  using G = DmaTile<BM, BN, WM, WN, STAGES>;
  constexpr int NW = G::NW, AJ = G::AJ, WJ = G::WJ, IPS = G::IPS, MW = G::MW, NWB = G::NWB;
  constexpr int TM = G::TM, TN = G::TN, kABytes = G::kABytes;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv / WN;
  const int wn = wv % WN;
  const int nk = kend > kbeg ? (kend - kbeg) / 64 : 0;

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
  // fragments of both 32-deep halves of a stage are read first (so the MFMAs
  // issue back to back behind the reads) unless the wave tile is large or
  // the workgroup has more than 8 waves (fewer registers per wave), where
  // each half is read in turn
  constexpr int KH = (NW <= 8 && (TM + TN) * 2 <= 16) ? 2 : 1;
  auto compute = [&](const char* sa) {
    const char* sw = sa + kABytes;
#pragma unroll
    for (int k0 = 0; k0 < 2; k0 += KH) {
      bf16x8_t fa[KH][TM], fw[KH][TN];
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        const int c = (k0 + kh) * 4 + (l >> 4);
#pragma unroll
        for (int a = 0; a < TM; ++a) {
          const int row = wm * MW + a * 16 + frow;
          fa[kh][a] = as_bf16x8(*reinterpret_cast<const uint4*>(sa + row * kDmaRow + dma_swz(row, c) * 16));
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int row = wn * NWB + b * 16 + frow;
          fw[kh][b] = as_bf16x8(*reinterpret_cast<const uint4*>(sw + row * kDmaRow + dma_swz(row, c) * 16));
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kh][a], fw[kh][b], acc[a][b], 0, 0, 0);
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
}

// The device-side description of q (k split into q.split ranges, each a
// multiple of bk).
GemmDev gemm_dev(const GemmProblem& q, int bk);

}  // namespace dcoco
