// Gradient products of the training side on bf16 MFMA:
//   C[m, n] = sum_k A(m, k) B(k, n)
// with A fp32 and B bf16, both read in the layout the backward produces them
// in.  Weight gradients reduce over the rows of both operands (A(m, k) =
// A[k][m], "row reduction"); input gradients reduce over the columns of A
// (A(m, k) = A[m][k]) against a weight stored [k][n].  B is always stored
// [k][n] (n contiguous), its rows optionally gathered by id, repeated, or
// taken from up to three stacked matrices.  Sources of the operations: review
// of arXiv 2610.12570, section "New approach: DCOCO", parts 1 and 3 (paper
// Sec. 3.2, App. A); Two Delta, "Two Delta makes NVIDIA Nemotron 3.5 Super even
// faster with DCOCO", section "How we train the corrector".
//
// Each operand tile is transposed while it is staged from registers into LDS,
// so no transposed copy of an operand ever reaches memory, and the fp32
// operand is split there into two bf16 parts, hi = bf16(a) and lo = bf16(a -
// hi) (|a - hi - lo| <= 2^-17 |a|); both parts meet the same B fragment, so
// the product is the fp32 one up to that remainder and fp32 accumulation.
#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace dcoco {
namespace {

constexpr int kWgThreads = 256;
constexpr int kWgBM = 128;
constexpr int kWgBN = 128;
constexpr int kWgBK = 64;
constexpr int kWgRow = kWgBK * 2;    // LDS bytes per tile row (8 chunks of 8 bf16)

// chunk position of 16-byte chunk c in LDS row r: rows r and r + 1 start 32
// banks apart, and the XOR spreads 16 consecutive rows over all 64 banks
__device__ __forceinline__ int wg_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ bf16x8_t wg_x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// two floats rounded to bf16 (nearest-even, the hardware conversion), packed
// with the first in the low half
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// hi and lo bf16 parts of two floats: hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt2(a, b);
  lo = cvt2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// hi and lo parts of 8 floats, packed in k order
__device__ __forceinline__ void split8(const float (&x)[8], uint4& hi, uint4& lo) {
  split2(x[0], x[1], hi.x, lo.x);
  split2(x[2], x[3], hi.y, lo.y);
  split2(x[4], x[5], hi.z, lo.z);
  split2(x[6], x[7], hi.w, lo.w);
}

__device__ __forceinline__ uint32_t dw(uint4 v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// 16-bit element n of row u (low) and of row v (high) in one word (byte permute)
__device__ __forceinline__ uint32_t pick16(uint4 u, uint4 v, int n) {
  return __builtin_amdgcn_perm(dw(v, n >> 1), dw(u, n >> 1), (n & 1) ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ const uint16_t* b_row(const WgradArgs& p, int k) {
  if (k < p.bend0) return p.b0 + p.bmap.row(k) * p.ldb0;
  if (k < p.bend1) return p.b1 + static_cast<long long>(k - p.bend0) * p.ldb1;
  return p.b2 + static_cast<long long>(k - p.bend1) * p.ldb2;
}

// Per-thread staging of one 64-deep k tile: a task is 8 consecutive k of one
// 16-byte chunk (kg) of 4 A columns (row reduction), of one A row (two float4),
// or of 8 B columns (threads 0..127).
struct WgTask {
  int kg, mg, ng;
  bool b_task;
};

// one k tile's operands into registers; gathered B rows use the ids fetched
// one load ahead (idn), and fetch the ids `ahead` rows further on
template <bool RR>
__device__ __forceinline__ void wg_load(const WgradArgs& p, const WgTask& t, int m0, int n0, int k0, int kend,
                                        int ahead, float4 (&ra)[8], uint4 (&rb)[8], int (&idn)[8]) {
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint4 zu = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (RR) {
    const int m = m0 + 4 * t.mg;
    const bool mok = m < p.M;
    const int mc = mok ? m : 0;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = k0 + t.kg * 8 + kk;
      const int kc = min(k, kend - 1);
      const float4 v = *reinterpret_cast<const float4*>(p.A + static_cast<long long>(kc) * p.lda + mc);
      ra[kk] = (mok && k < kend) ? v : z4;
    }
  } else {
    const int kc = min(k0 + t.kg * 8, kend - 8);
    const bool kok = k0 + t.kg * 8 < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + t.mg + 32 * i;
      const int mc = min(m, p.M - 1);
      const float* src = p.A + static_cast<long long>(mc) * p.lda + kc;
      const float4 v0 = *reinterpret_cast<const float4*>(src);
      const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
      const bool ok = kok && m < p.M;
      ra[2 * i] = ok ? v0 : z4;
      ra[2 * i + 1] = ok ? v1 : z4;
    }
  }
  if (t.b_task) {
    const int n = n0 + 8 * t.ng;
    const bool nok = n < p.N;
    const int nc = nok ? n : 0;
    if (p.bmap.mode == 1) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k = k0 + t.kg * 8 + kk;
        const int row = min(max(idn[kk], 0), p.bmap.idmax);
        const uint4 v = *reinterpret_cast<const uint4*>(p.b0 + static_cast<long long>(row) * p.ldb0 + nc);
        rb[kk] = (nok && k < kend) ? v : zu;
      }
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) idn[kk] = p.bmap.ids[min(k0 + ahead + t.kg * 8 + kk, kend - 1)];
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int k = k0 + t.kg * 8 + kk;
        const int kc = min(k, kend - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(b_row(p, kc) + nc);
        rb[kk] = (nok && k < kend) ? v : zu;
      }
    }
  }
}

// registers -> LDS: A split into its hi and lo parts, B transposed, both in
// the [row][k] layout the MFMA fragments read
template <bool RR>
__device__ __forceinline__ void wg_stage(const WgTask& t, const float4 (&ra)[8], const uint4 (&rb)[8], char* sAh,
                                         char* sAl, char* sB) {
  if constexpr (RR) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) x[kk] = j == 0 ? ra[kk].x : j == 1 ? ra[kk].y : j == 2 ? ra[kk].z : ra[kk].w;
      uint4 hi, lo;
      split8(x, hi, lo);
      const int r = 4 * t.mg + j;
      const int off = r * kWgRow + wg_swz(r, t.kg) * 16;
      *reinterpret_cast<uint4*>(sAh + off) = hi;
      *reinterpret_cast<uint4*>(sAl + off) = lo;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x[8] = {ra[2 * i].x, ra[2 * i].y, ra[2 * i].z, ra[2 * i].w,
                          ra[2 * i + 1].x, ra[2 * i + 1].y, ra[2 * i + 1].z, ra[2 * i + 1].w};
      uint4 hi, lo;
      split8(x, hi, lo);
      const int r = t.mg + 32 * i;
      const int off = r * kWgRow + wg_swz(r, t.kg) * 16;
      *reinterpret_cast<uint4*>(sAh + off) = hi;
      *reinterpret_cast<uint4*>(sAl + off) = lo;
    }
  }
  if (t.b_task) {
    // 8 x 8 transpose of 16-bit values: tile row n takes element n of each
    // of the 8 k rows
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const uint4 v = make_uint4(pick16(rb[0], rb[1], n), pick16(rb[2], rb[3], n), pick16(rb[4], rb[5], n),
                                 pick16(rb[6], rb[7], n));
      const int r = 8 * t.ng + n;
      *reinterpret_cast<uint4*>(sB + r * kWgRow + wg_swz(r, t.kg) * 16) = v;
    }
  }
}

// the MFMA work of one staged k tile: wave (wm, wn) owns a 64 x 64 block
__device__ __forceinline__ void wg_compute(const char* sAh, const char* sAl, const char* sB, int wm, int wn, int l,
                                           f32x4_t (&acc)[4][4]) {
  const int frow = l & 15;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = ks * 4 + (l >> 4);
    uint4 fb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = wn * 64 + b * 16 + frow;
      fb[b] = *reinterpret_cast<const uint4*>(sB + r * kWgRow + wg_swz(r, c) * 16);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = wm * 64 + a * 16 + frow;
      const int off = r * kWgRow + wg_swz(r, c) * 16;
      const uint4 fh = *reinterpret_cast<const uint4*>(sAh + off);
      const uint4 fl = *reinterpret_cast<const uint4*>(sAl + off);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg_x8(fh), wg_x8(fb[b]), acc[a][b], 0, 0, 0);
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wg_x8(fl), wg_x8(fb[b]), acc[a][b], 0, 0, 0);
      }
    }
  }
}

// One 128 x 128 output tile (of one k split) per workgroup; 4 waves as 2 x 2,
// each 64 x 64 = 4 x 4 MFMA tiles of 16 x 16.  With SETS = 2, two register
// sets alternate over the 64-deep k tiles, so the loads of tile t + 2 are in
// flight while tile t is staged and multiplied (vector loads complete in issue
// order, and each staging waits only for its own set); this takes the whole
// register file (one wave per SIMD).  With SETS = 1, one set: the next tile
// loads while this one is multiplied, at two waves per SIMD.
// RR: A(m, k) = A[k * lda + m] (row reduction), else A[m * lda + k].
template <bool RR, int SETS>
__global__ void __launch_bounds__(kWgThreads, SETS == 2 ? 1 : 2) wgrad_kernel(WgradArgs p) {
  __shared__ __align__(16) char sAh[kWgBM * kWgRow];
  __shared__ __align__(16) char sAl[kWgBM * kWgRow];
  __shared__ __align__(16) char sB[kWgBN * kWgRow];
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1;
  const int wn = wv & 1;
  const int n0 = blockIdx.x * kWgBN;
  const int m0 = blockIdx.y * kWgBM;
  const int z = blockIdx.z;
  const int kbeg = z * p.ksplit;
  const int kend = min(p.Kd, kbeg + p.ksplit);
  WgTask t;
  t.kg = tid & 7;
  t.mg = tid >> 3;
  t.ng = tid >> 3;
  t.b_task = tid < 128;

  float4 ra0[8], ra1[8];
  uint4 rb0[8], rb1[8];
  int id0[8], id1[8];                      // ids of each set's next gathered B tile
  if (p.bmap.mode == 1 && t.b_task) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      id0[kk] = p.bmap.ids[min(kbeg + t.kg * 8 + kk, kend - 1)];
      if constexpr (SETS == 2) id1[kk] = p.bmap.ids[min(kbeg + kWgBK + t.kg * 8 + kk, kend - 1)];
    }
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int kAhead = SETS * kWgBK;
  if constexpr (SETS == 1) {
    if (kbeg < kend) wg_load<RR>(p, t, m0, n0, kbeg, kend, kAhead, ra0, rb0, id0);
    for (int k0 = kbeg; k0 < kend; k0 += kWgBK) {
      wg_stage<RR>(t, ra0, rb0, sAh, sAl, sB);
      __syncthreads();
      if (k0 + kWgBK < kend) wg_load<RR>(p, t, m0, n0, k0 + kWgBK, kend, kAhead, ra0, rb0, id0);
      wg_compute(sAh, sAl, sB, wm, wn, l, acc);
      __syncthreads();
    }
  } else {
  if (kbeg < kend) wg_load<RR>(p, t, m0, n0, kbeg, kend, kAhead, ra0, rb0, id0);
  if (kbeg + kWgBK < kend) wg_load<RR>(p, t, m0, n0, kbeg + kWgBK, kend, kAhead, ra1, rb1, id1);
  for (int k0 = kbeg; k0 < kend; k0 += 2 * kWgBK) {
    wg_stage<RR>(t, ra0, rb0, sAh, sAl, sB);
    __syncthreads();
    if (k0 + 2 * kWgBK < kend) wg_load<RR>(p, t, m0, n0, k0 + 2 * kWgBK, kend, kAhead, ra0, rb0, id0);
    wg_compute(sAh, sAl, sB, wm, wn, l, acc);
    __syncthreads();
    if (k0 + kWgBK >= kend) break;
    wg_stage<RR>(t, ra1, rb1, sAh, sAl, sB);
    __syncthreads();
    if (k0 + 3 * kWgBK < kend) wg_load<RR>(p, t, m0, n0, k0 + 3 * kWgBK, kend, kAhead, ra1, rb1, id1);
    wg_compute(sAh, sAl, sB, wm, wn, l, acc);
    __syncthreads();
  }
  }

  // epilogue: output row m goes to the segment that holds it
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * 64 + a * 16 + (l >> 4) * 4 + v;
      if (m >= p.M) continue;
      float* row;
      if (m < p.cend0) row = p.c0 + static_cast<long long>(m) * p.ldc0;
      else if (m < p.cend1) row = p.c1 + static_cast<long long>(m - p.cend0) * p.ldc1;
      else row = p.c2 + static_cast<long long>(m - p.cend1) * p.ldc2;
      row += z * p.c_split;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int n = n0 + wn * 64 + b * 16 + (l & 15);
        if (n < p.N) row[n] = acc[a][b][v];
      }
    }
}

// ---------------------------------------------------------------------------
// The same products with the operands' raw tiles streamed into LDS by direct
// global->LDS loads (global_load_lds_dwordx4: one wave instruction moves 64
// lanes x 16 bytes), two tiles ahead, in a 2-slot ring; a transform pass then
// reads each raw tile, splits / transposes it with the staging code above
// into the MFMA layout, and the waves multiply.  No staging registers and no
// compiler-counted loads in the loop: the waits are fixed vmcnt counts.
// Raw layouts, one 1 KB instruction after another:
//   row reduction A: 64 k-rows x 512 B (128 fp32 of m), chunk c of row r at
//     position c ^ ((r >> 3) & 7), so the transform's column reads of 8 rows
//     fall on different banks;
//   column reduction A: 128 m-rows x 256 B (64 fp32 of k), natural order;
//   B: 64 k-rows x 256 B (128 bf16 of n), chunk c of row r at c ^ ((r >> 3) & 7).
// Gathered B rows take their ids from LDS (staged once per workgroup).
constexpr int kRawA = kWgBK * kWgBM * 4;     // 32 KB
constexpr int kRawB = kWgBK * kWgBN * 2;     // 16 KB
constexpr int kRawBytes = kRawA + kRawB;
constexpr int kDmaA = kRawA / 1024 / 4;      // A instructions per wave per tile (8)
constexpr int kDmaB = kRawB / 1024 / 4;      // B instructions per wave per tile (4)
constexpr int kIdsCap = 2048;                // gathered ids staged per workgroup

__device__ __forceinline__ int raw_swz(int r) { return (r >> 3) & 7; }

template <bool RR>
__device__ __forceinline__ void wg_issue(const WgradArgs& p, const int32_t* s_ids, int kbeg, int m0, int n0, int k0,
                                         int kend, uint32_t raw, int wv, int l) {
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int j = wv * kDmaA + i;
    const float* src;
    if constexpr (RR) {
      const int r = 2 * j + (l >> 5);
      const int c = (l & 31) ^ raw_swz(r);
      const int k = min(k0 + r, kend - 1);
      const int m = min(m0 + c * 4, p.M - 4);
      src = p.A + static_cast<long long>(k) * p.lda + m;
    } else {
      const int r = 4 * j + (l >> 4);
      const int m = min(m0 + r, p.M - 1);
      const int k = min(k0 + (l & 15) * 4, kend - 4);
      src = p.A + static_cast<long long>(m) * p.lda + k;
    }
    dma16(src, __builtin_amdgcn_readfirstlane(raw + j * 1024));
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int j = wv * kDmaB + i;
    const int r = 4 * j + (l >> 4);
    const int c = (l & 15) ^ raw_swz(r);
    const int k = min(k0 + r, kend - 1);
    const int n = min(n0 + c * 8, p.N - 8);
    const uint16_t* row = p.bmap.mode == 1 ? p.b0 + static_cast<long long>(s_ids[k - kbeg]) * p.ldb0 : b_row(p, k);
    dma16(row + n, __builtin_amdgcn_readfirstlane(raw + kRawA + j * 1024));
  }
}

// one raw tile (LDS) into the staging registers, masked like wg_load
template <bool RR>
__device__ __forceinline__ void wg_from_raw(const WgradArgs& p, const char* raw, const WgTask& t, int m0, int n0,
                                            int k0, int kend, float4 (&ra)[8], uint4 (&rb)[8]) {
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint4 zu = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (RR) {
    const bool mok = m0 + 4 * t.mg < p.M;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r = t.kg * 8 + kk;
      const float4 v = *reinterpret_cast<const float4*>(raw + r * 512 + ((t.mg ^ raw_swz(r)) * 16));
      ra[kk] = (mok && k0 + r < kend) ? v : z4;
    }
  } else {
    const bool kok = k0 + t.kg * 8 < kend;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = t.mg + 32 * i;
      const char* q = raw + m * 256 + t.kg * 32;
      const float4 v0 = *reinterpret_cast<const float4*>(q);
      const float4 v1 = *reinterpret_cast<const float4*>(q + 16);
      const bool ok = kok && m0 + m < p.M;
      ra[2 * i] = ok ? v0 : z4;
      ra[2 * i + 1] = ok ? v1 : z4;
    }
  }
  if (t.b_task) {
    const bool nok = n0 + 8 * t.ng < p.N;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int r = t.kg * 8 + kk;
      const uint4 v = *reinterpret_cast<const uint4*>(raw + kRawA + r * 256 + ((t.ng ^ raw_swz(r)) * 16));
      rb[kk] = (nok && k0 + r < kend) ? v : zu;
    }
  }
}

__device__ __forceinline__ void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

template <bool RR>
__global__ void __launch_bounds__(kWgThreads, 1) wgrad_dma_kernel(WgradArgs p) {
  __shared__ __align__(1024) char raw0[kRawBytes];
  __shared__ __align__(1024) char raw1[kRawBytes];
  __shared__ __align__(16) char sAh[kWgBM * kWgRow];
  __shared__ __align__(16) char sAl[kWgBM * kWgRow];
  __shared__ __align__(16) char sB[kWgBN * kWgRow];
  __shared__ int32_t s_ids[kIdsCap];
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1;
  const int wn = wv & 1;
  const int n0 = blockIdx.x * kWgBN;
  const int m0 = blockIdx.y * kWgBM;
  const int z = blockIdx.z;
  const int kbeg = z * p.ksplit;
  const int kend = min(p.Kd, kbeg + p.ksplit);
  WgTask t;
  t.kg = tid & 7;
  t.mg = tid >> 3;
  t.ng = tid >> 3;
  t.b_task = tid < 128;
  if (p.bmap.mode == 1) {
    for (int i = tid; i < kend - kbeg; i += kWgThreads) {
      const int id = p.bmap.ids[kbeg + i];
      s_ids[i] = id < 0 ? 0 : (id > p.bmap.idmax ? p.bmap.idmax : id);
    }
  }
  lds_only_barrier();
  const uint32_t r0 = __builtin_amdgcn_readfirstlane(lds_offset(raw0));
  const uint32_t r1 = __builtin_amdgcn_readfirstlane(lds_offset(raw1));

  f32x4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kbeg < kend) wg_issue<RR>(p, s_ids, kbeg, m0, n0, kbeg, kend, r0, wv, l);
  if (kbeg + kWgBK < kend) wg_issue<RR>(p, s_ids, kbeg, m0, n0, kbeg + kWgBK, kend, r1, wv, l);
  int par = 0;
  for (int k0 = kbeg; k0 < kend; k0 += kWgBK, par ^= 1) {
    // this tile's raw data has landed when at most the next tile's loads are
    // still in flight; the barrier also ends every wave's reads of the
    // previous MFMA tile
    if (k0 + kWgBK < kend) wait_vmcnt_barrier<kDmaA + kDmaB>();
    else wait_vmcnt_barrier<0>();
    {
      float4 ra[8];
      uint4 rb[8];
      wg_from_raw<RR>(p, par ? raw1 : raw0, t, m0, n0, k0, kend, ra, rb);
      wg_stage<RR>(t, ra, rb, sAh, sAl, sB);
    }
    lds_only_barrier();                      // MFMA tile complete, this raw slot free
    if (k0 + 2 * kWgBK < kend) wg_issue<RR>(p, s_ids, kbeg, m0, n0, k0 + 2 * kWgBK, kend, par ? r1 : r0, wv, l);
    wg_compute(sAh, sAl, sB, wm, wn, l, acc);
  }

#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * 64 + a * 16 + (l >> 4) * 4 + v;
      if (m >= p.M) continue;
      float* row;
      if (m < p.cend0) row = p.c0 + static_cast<long long>(m) * p.ldc0;
      else if (m < p.cend1) row = p.c1 + static_cast<long long>(m - p.cend0) * p.ldc1;
      else row = p.c2 + static_cast<long long>(m - p.cend1) * p.ldc2;
      row += z * p.c_split;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int n = n0 + wn * 64 + b * 16 + (l & 15);
        if (n < p.N) row[n] = acc[a][b][v];
      }
    }
}

}  // namespace

// weight gradients with bf16 operands take the direct global->LDS kernel
constexpr bool kWgradUseDma = true;

int wgrad_pick_split(int M, int N, int Kd) {
  const long long tiles = static_cast<long long>((M + kWgBM - 1) / kWgBM) * ((N + kWgBN - 1) / kWgBN);
  int split = 1;
  while (tiles * split < 512 && split < 32 && Kd / (split * 2) >= 256) split *= 2;
  return split;
}

hipError_t launch_wgrad(WgradArgs p, bool row_reduction, int splits, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  if (p.N % 8 != 0 || p.lda % 4 != 0 || !al16(p.A) || splits < 1) return hipErrorInvalidValue;
  if (row_reduction ? (p.M % 4 != 0) : (p.Kd % 8 != 0)) return hipErrorInvalidValue;
  if (!p.b1) { p.b1 = p.b0; p.ldb1 = p.ldb0; }
  if (!p.b2) { p.b2 = p.b1; p.ldb2 = p.ldb1; }
  const uint16_t* bs[3] = {p.b0, p.b1, p.b2};
  const long long lds[3] = {p.ldb0, p.ldb1, p.ldb2};
  for (int s = 0; s < 3; ++s)
    if (!bs[s] || !al16(bs[s]) || lds[s] % 8 != 0) return hipErrorInvalidValue;
  if (!p.c1) { p.c1 = p.c0; p.ldc1 = p.ldc0; }
  if (!p.c2) { p.c2 = p.c1; p.ldc2 = p.ldc1; }
  int ks = (p.Kd + splits - 1) / splits;
  ks = (ks + kWgBK - 1) / kWgBK * kWgBK;
  p.ksplit = ks;
  const int gz = p.Kd > 0 ? (p.Kd + ks - 1) / ks : 1;
  const dim3 grid((p.N + kWgBN - 1) / kWgBN, (p.M + kWgBM - 1) / kWgBM, gz);
  // the DMA ring takes a whole CU per workgroup (its LDS), so it pays when the
  // grid fits one workgroup per CU; larger grids run two register-staged
  // workgroups per CU, whose transforms and MFMAs then overlap
  const long long wgs = static_cast<long long>(grid.x) * grid.y * grid.z;
  const bool dma = kWgradUseDma && wgs <= 256 && (p.bmap.mode != 1 || ks <= kIdsCap);
  if (dma) {
    if (row_reduction)
      hipLaunchKernelGGL((wgrad_dma_kernel<true>), grid, dim3(kWgThreads), 0, st, p);
    else
      hipLaunchKernelGGL((wgrad_dma_kernel<false>), grid, dim3(kWgThreads), 0, st, p);
    return hipGetLastError();
  }
  // register staging: row reductions at two waves per SIMD; column reductions
  // (short k per workgroup, A rows read whole) gain more from two sets
  if (row_reduction)
    hipLaunchKernelGGL((wgrad_kernel<true, 1>), grid, dim3(kWgThreads), 0, st, p);
  else
    hipLaunchKernelGGL((wgrad_kernel<false, 2>), grid, dim3(kWgThreads), 0, st, p);
  return hipGetLastError();
}

int wgrad_grid_splits(int Kd, int splits) {
  int ks = (Kd + splits - 1) / splits;
  ks = (ks + kWgBK - 1) / kWgBK * kWgBK;
  return Kd > 0 ? (Kd + ks - 1) / ks : 1;
}

}  // namespace dcoco
