// Row LayerNorm and pair-state assembly of the representation stage (review
// of arXiv 2610.12570, "Contextual Correction of Parallel Drafts for
// Speculative Decoding", part 1 of "New approach: DCOCO", paper Sec. 3.2):
//   g_i     = LN(P_h h_i),  b_{i,k} = LN(P_e E[c_{i,k}])   (non-affine LN)
//   s_p     = W_pair [h_p; h_{p+1}] = W_L h_p + W_R h_{p+1}
// The projections arrive as fp32 split-K partial sums, added here in a fixed
// order.  LN statistics are two-pass in fp32 (mean, then mean of squared
// deviations), one wave64 per row.
#include "common.h"
#include "dma.h"
#include "kernels.h"
#include "wave.h"
#include "ln_tile.h"

namespace dcoco {

namespace {

template <typename TO, int VPL>
__global__ void __launch_bounds__(256)
ln_rows_kernel(const float* __restrict__ x, int split, int M, int ldx, int col0, int r, float eps,
               TO* __restrict__ y) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane_id();
  if (row >= M) return;
  float v[VPL];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    float a = 0.f;
    if (c < r) {
      for (int s = 0; s < split; ++s)
        a += x[(static_cast<long long>(s) * M + row) * ldx + col0 + c];
    }
    v[i] = a;
    sum += a;
  }
  const float mean = wave_sum(sum) / static_cast<float>(r);
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    v[i] = c < r ? v[i] - mean : 0.f;
    sq += v[i] * v[i];
  }
  const float var = wave_sum(sq) / static_cast<float>(r);
  const float inv = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int c = l + i * kWave;
    if (c < r) y[static_cast<long long>(row) * r + c] = Elem<TO>::from_f32(v[i] * inv);
  }
}

__global__ void __launch_bounds__(256)
pair_state_kernel(const float* __restrict__ Y, int split, int N, int B, int ldy, int cl, int cr,
                  int rs, float* __restrict__ s, uint16_t* __restrict__ s3) {
  const long long total = static_cast<long long>(N) * (B - 1) * rs;
  const long long M = static_cast<long long>(N) * B;
  for (long long t = blockIdx.x * 256ll + threadIdx.x; t < total; t += 256ll * gridDim.x) {
    const int j = static_cast<int>(t % rs);
    const long long np = t / rs;
    const long long n = np / (B - 1);
    const long long p = np % (B - 1);
    const long long rl = n * B + p;
    float left = 0.f, right = 0.f;
    for (int q = 0; q < split; ++q) {
      left += Y[(q * M + rl) * ldy + cl + j];
      right += Y[(q * M + rl + 1) * ldy + cr + j];
    }
    const float x = left + right;
    s[t] = x;
    if (s3) {
      // x = hi + mid + lo exactly (three bf16 parts of 8 significand bits)
      const uint16_t hi = f32_to_bf16(x);
      const float r1 = x - bf16_to_f32(hi);
      const uint16_t mid = f32_to_bf16(r1);
      s3[t] = hi;
      s3[total + t] = mid;
      s3[2 * total + t] = f32_to_bf16(r1 - bf16_to_f32(mid));
    }
  }
}

// bf16 path: LayerNorm of BM rows straight into an LDS operand tile, then
// y = W x for those rows on MFMA (W rows streamed from L2 as 16-byte
// fragments, one k step prefetched).  Used for gf = W_fg g (fp32 out) and
// z = W_fb b + gf[slot] (bf16 out), so the normalised g and b never leave the
// chip.  The LN phase keeps several rows' loads (all SPLIT partial sums of
// each) in flight at once: a wave normalises RP rows per pass.
template <int BM, int RMAX, int SPLIT, int MODE>
__global__ void __launch_bounds__(256)
ln_gemm_kernel(const float* __restrict__ x, int M, int ldx, int col0, int r, float eps,
               const bf16* __restrict__ W, long long ldw, int wcol0, int N, float* __restrict__ out_f32,
               bf16* __restrict__ out_bf, const float* __restrict__ row_bias, int row_div) {
  constexpr int kStr = RMAX * 2 + 16;              // LDS bytes per tile row
  constexpr int VPL = RMAX / kWave;
  constexpr int RP0 = 64 / (VPL * SPLIT);
  constexpr int RP = RP0 < 1 ? 1 : (RP0 > BM / 4 ? BM / 4 : RP0);
  constexpr int WM = BM >= 32 ? 2 : 1;             // wave grid: WM x (4 / WM)
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / (16 * WM);
  constexpr int TN = 8;                            // 128 columns per wave pass
  __shared__ __align__(16) char tile[BM * kStr];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int m0 = blockIdx.x * BM;

  // ---- LayerNorm: wave wv owns rows wv*RP + 4*RP*j + q, q < RP
  for (int rb = wv * RP; rb < BM; rb += 4 * RP) {
    float v[RP][VPL];
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      const int m = min(m0 + rb + q, M - 1);
      float part[SPLIT][VPL];
#pragma unroll
      for (int s2 = 0; s2 < SPLIT; ++s2)
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int c = l + i * kWave;
          part[s2][i] = c < r ? x[(static_cast<long long>(s2) * M + m) * ldx + col0 + c] : 0.f;
        }
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        float a = part[0][i];
#pragma unroll
        for (int s2 = 1; s2 < SPLIT; ++s2) a += part[s2][i];
        v[q][i] = a;
      }
    }
#pragma unroll
    for (int q = 0; q < RP; ++q) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i) sum += v[q][i];
      const float mean = wave_sum(sum) / static_cast<float>(r);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int c = l + i * kWave;
        v[q][i] = c < r ? v[q][i] - mean : 0.f;
        sq += v[q][i] * v[q][i];
      }
      const float inv = 1.0f / sqrtf(wave_sum(sq) / static_cast<float>(r) + eps);
      const bool live = m0 + rb + q < M;
      uint16_t* trow = reinterpret_cast<uint16_t*>(tile + (rb + q) * kStr);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int c = l + i * kWave;
        if (c < r) trow[c] = live ? f32_to_bf16(v[q][i] * inv) : 0;
      }
    }
  }
  __syncthreads();

  // ---- y = W x on MFMA
  const int wm = wv / WN;
  const int wn = wv % WN;
  const int frow = l & 15;
  const int fk = (l >> 4) * 8;
  for (int n0 = wn * 128; n0 < N; n0 += WN * 128) {
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bf16* wrow[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b)
      wrow[b] = W + static_cast<long long>(min(n0 + b * 16 + frow, N - 1)) * ldw + wcol0 + fk;
    auto kstep = [&](int k, const uint4 (&wf)[TN]) {
      bf16x8_t fa[TM];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        fa[a] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    tile + (wm * (BM / WM) + a * 16 + frow) * kStr + (k + fk) * 2));
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const bf16x8_t fw = __builtin_bit_cast(bf16x8_t, wf[b]);
#pragma unroll
        for (int a = 0; a < TM; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fw, acc[a][b], 0, 0, 0);
      }
    };
    // two fragment buffers, one k step in flight ahead of the MFMAs
    uint4 w0[TN], w1[TN];
#pragma unroll
    for (int b = 0; b < TN; ++b) w0[b] = *reinterpret_cast<const uint4*>(wrow[b]);
    for (int k = 0; k < r; k += 64) {
      const bool two = k + 32 < r;
      if (two) {
#pragma unroll
        for (int b = 0; b < TN; ++b) w1[b] = *reinterpret_cast<const uint4*>(wrow[b] + k + 32);
      }
      kstep(k, w0);
      if (k + 64 < r) {
#pragma unroll
        for (int b = 0; b < TN; ++b) w0[b] = *reinterpret_cast<const uint4*>(wrow[b] + k + 64);
      }
      if (two) kstep(k + 32, w1);
    }
    // epilogue: every bias value is fetched (clamped, branch-free) before
    // any store, so the loads overlap
    int mrow[TM][4];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) mrow[a][v] = m0 + wm * (BM / WM) + a * 16 + (l >> 4) * 4 + v;
    if constexpr (MODE == 1) {
      float bias[TM][4][TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float* rb = row_bias + static_cast<long long>(min(mrow[a][v], M - 1) / row_div) * N;
#pragma unroll
          for (int b = 0; b < TN; ++b) bias[a][v][b] = rb[min(n0 + b * 16 + (l & 15), N - 1)];
        }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int n = n0 + b * 16 + (l & 15);
            if (mrow[a][v] < M && n < N)
              out_bf[static_cast<long long>(mrow[a][v]) * N + n] = bf16{f32_to_bf16(acc[a][b][v] + bias[a][v][b])};
          }
    } else {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int n = n0 + b * 16 + (l & 15);
            if (mrow[a][v] < M && n < N) out_f32[static_cast<long long>(mrow[a][v]) * N + n] = acc[a][b][v];
          }
    }
  }
}

// bf16 path for r <= 256, with the weight slice resident in LDS: a chunk of
// 256 output columns of W (256 rows x r k values) is copied into LDS with
// direct global->LDS loads issued before the LayerNorm phase, so the copy
// overlaps the LN loads and arithmetic and the MFMA phase then reads both
// operands from LDS only.  W rows are 512 bytes apart; row n's 16-byte k chunk
// c sits in slot c ^ (n & 15), so the 16 rows one fragment read touches fall
// on distinct banks.  LN: each wave normalises BM / 4 rows, one float4 of
// every split partial per lane and row, all loads in flight together.
constexpr int kLgCols = 256;                 // W rows (output columns) per LDS chunk
constexpr int kLgRowBytes = 512;             // LDS bytes per W row (k <= 256)

// Pair states assembled by the same launch: s_p = Y_L[m] + Y_R[m + 1] for
// slot row m = n B + i of pair p = n (B - 1) + i (split partials added in
// order) and its exact three-way bf16 split.  By rows (gf mode): the pairs
// of the workgroup's slot rows, from the operand x.  By workgroup (z mode):
// workgroup x takes pairs x ppw .. x ppw + ppw - 1, one float4 item of 4
// columns per thread, from y.
struct PairArgs {
  int B, cl, cr, rs;
  float* s;
  uint16_t* s3;
  long long total;      // N (B - 1) rs
  const float* y;       // z mode: slot partial sums [split][N B][ldy]
  int split, ldy, ppw, P;
};

// s_p's four columns at t = p rs + j and their bf16 split
__device__ __forceinline__ void store_pair_state(const PairArgs& pa, long long t, float4 sum) {
  *reinterpret_cast<float4*>(pa.s + t) = sum;
  if (pa.s3 == nullptr) return;
  const float v4[4] = {sum.x, sum.y, sum.z, sum.w};
  uint16_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    hi[c] = f32_to_bf16(v4[c]);
    const float r1 = v4[c] - bf16_to_f32(hi[c]);
    mid[c] = f32_to_bf16(r1);
    lo[c] = f32_to_bf16(r1 - bf16_to_f32(mid[c]));
  }
  auto pack4 = [](const uint16_t (&h)[4]) {
    return make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16), h[2] | (static_cast<uint32_t>(h[3]) << 16));
  };
  *reinterpret_cast<uint2*>(pa.s3 + t) = pack4(hi);
  *reinterpret_cast<uint2*>(pa.s3 + pa.total + t) = pack4(mid);
  *reinterpret_cast<uint2*>(pa.s3 + 2 * pa.total + t) = pack4(lo);
}

constexpr int kPairMaxSplit = 4;

// Rows taken from a bf16 table instead of normalised here (GATHER mode): row
// m of the operand is table row ids[m] (clamped into [0, idmax]), r values.
struct GatherArgs {
  const uint16_t* tab;
  const int32_t* ids;
  int idmax;
};

// NCOL W rows (output columns) per LDS chunk, NCOL / 4 per wave.  Workgroup
// (x, y) takes rows [x BM, +BM) and output columns [y ncols_wg, +ncols_wg) in
// chunks of NCOL; a launch with one column group per workgroup row has
// gridDim.y == 1 and ncols_wg == N.  With several column groups each one
// normalises the same rows (cheap next to the loads), and in gf mode
// assembles its share of the pair-state columns.
// PAIR: 0 no pair states, 1 by rows (gf mode), 2 by workgroup (z mode).
template <int BM, int SPLIT, int MODE, int PAIR, bool GATHER = false, int NCOL = kLgCols>
__global__ void __launch_bounds__(256)
ln_gemm_w_kernel(const float* __restrict__ x, int M, int ldx, int col0, int r, float eps,
                 const bf16* __restrict__ W, long long ldw, int wcol0, int N, float* __restrict__ out_f32,
                 bf16* __restrict__ out_bf, const float* __restrict__ row_bias, int row_div, PairArgs pa,
                 GatherArgs ga, int ncols_wg) {
  constexpr int kStr = 256 * 2 + 16;         // LDS bytes per normalised row
  constexpr int RPW = BM / 4;                // LN rows per wave
  constexpr int TM = BM / 16;
  constexpr int TN = NCOL / 64;              // NCOL / 4 columns per wave
  constexpr int CW = NCOL / 4;
  static_assert(NCOL % 64 == 0 && NCOL <= kLgCols, "column chunk");
  __shared__ __align__(1024) char wl[NCOL * kLgRowBytes];
  __shared__ __align__(16) char tile[BM * kStr];

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int m0 = blockIdx.x * BM;
  const int cr = r >> 3;                     // 16-byte k chunks per W row
  const int nb = blockIdx.y * ncols_wg;      // this workgroup's output columns
  const int ne = min(N, nb + ncols_wg);

  // NCOL / 2 one-KB copies per chunk (two W rows each); wave wv issues copies
  // wv, wv + 4, ...; slots whose logical chunk is past r copy the row's first
  // chunk and are never read
  auto issue_w = [&](int n0) {
    const int p = l & 31;
#pragma unroll 8
    for (int i = 0; i < NCOL / 8; ++i) {
      const int j = wv + 4 * i;
      const int row = 2 * j + (l >> 5);
      const int c = p ^ (row & 15);
      const long long n = min(n0 + row, N - 1);
      const char* g = reinterpret_cast<const char*>(W + n * ldw + wcol0) + (c < cr ? c : 0) * 16;
      dma16(g, __builtin_amdgcn_readfirstlane(lds_offset(wl) + j * 1024));
    }
  };
  issue_w(nb);

  // z mode: the row bias of every output this lane stores, fetched before the
  // LN phase so its latency hides behind the LN and MFMA work
  const int frow = l & 15;
  const int fq = l >> 4;
  float bias[TM][4][TN];
  auto load_bias = [&](int n0) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float* rb = row_bias + static_cast<long long>(min(m0 + a * 16 + fq * 4 + v, M - 1) / row_div) * N;
#pragma unroll
        for (int b = 0; b < TN; ++b) bias[a][v][b] = rb[min(n0 + wv * CW + b * 16 + frow, N - 1)];
      }
  };
  if constexpr (MODE == 1) load_bias(nb);

  // z mode pair states: this thread's item loaded now (every split, the
  // split index clamped so all loads issue unconditionally), added and
  // stored after the operand rows are normalised
  float4 pya[kPairMaxSplit], pyb[kPairMaxSplit];
  bool pok = false;
  long long pt = 0;
  if constexpr (PAIR == 2) {
    const int q4 = pa.rs >> 2;
    const int item = tid;
    const int p = static_cast<int>(blockIdx.x) * pa.ppw + item / q4;
    const int j = (item % q4) * 4;
    pok = item < pa.ppw * q4 && p < pa.P;
    const long long pp = pok ? p : 0;
    const long long nblk = pp / (pa.B - 1);
    const long long ml = nblk * pa.B + (pp - nblk * (pa.B - 1));   // left slot row; the right one is ml + 1
    const int jj = pok ? j : 0;
    const long long rows = static_cast<long long>(pa.P / (pa.B - 1)) * pa.B;
#pragma unroll
    for (int s2 = 0; s2 < kPairMaxSplit; ++s2) {
      const long long so = static_cast<long long>(min(s2, pa.split - 1)) * rows;
      pya[s2] = *reinterpret_cast<const float4*>(pa.y + (so + ml) * pa.ldy + pa.cl + jj);
      pyb[s2] = *reinterpret_cast<const float4*>(pa.y + (so + ml + 1) * pa.ldy + pa.cr + jj);
    }
    pt = pp * pa.rs + jj;
  }

  if constexpr (GATHER) {
    // ---- table rows of this wave's RPW operand rows: lanes 0-31 and 32-63
    // take two rows per load round, one 16-byte chunk each; every load is
    // issued (clamped row, clamped chunk) before the stores
    static_assert(RPW % 2 == 0, "two rows per round");
    const int ch = l & 31;
    const int ccl = ch < cr ? ch : 0;
    uint4 v[RPW / 2];
    bool keep[RPW / 2];
#pragma unroll
    for (int i = 0; i < RPW / 2; ++i) {
      const int q = 2 * i + (l >> 5);
      const int m = m0 + wv * RPW + q;
      int id = ga.ids[min(m, M - 1)];
      id = id < 0 ? 0 : (id > ga.idmax ? ga.idmax : id);
      v[i] = *reinterpret_cast<const uint4*>(ga.tab + static_cast<long long>(id) * r + ccl * 8);
      keep[i] = m < M;
    }
#pragma unroll
    for (int i = 0; i < RPW / 2; ++i) {
      const int q = 2 * i + (l >> 5);
      if (ch < cr)
        *reinterpret_cast<uint4*>(tile + (wv * RPW + q) * kStr + ch * 16) = keep[i] ? v[i] : make_uint4(0, 0, 0, 0);
    }
  } else {
    // ---- LayerNorm of rows m0 + wv * RPW + q into the tile (bf16)
    ln_rows_tile<RPW, SPLIT>(x, M, ldx, col0, r, eps, m0 + wv * RPW, tile + wv * RPW * kStr, kStr, l);
  }

  if constexpr (PAIR == 2) {
    if (pok) {
      float4 a = pya[0], b = pyb[0];
#pragma unroll
      for (int s2 = 1; s2 < kPairMaxSplit; ++s2) {
        if (s2 < pa.split) {
          a.x += pya[s2].x; a.y += pya[s2].y; a.z += pya[s2].z; a.w += pya[s2].w;
          b.x += pyb[s2].x; b.y += pyb[s2].y; b.z += pyb[s2].z; b.w += pyb[s2].w;
        }
      }
      store_pair_state(pa, pt, make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w));
    }
  }

  // ---- pair states of this workgroup's rows (loads in flight with the
  // weight copy; float4 items of (row, 4 columns), 1024 per batch)
  if constexpr (PAIR == 1) {
    // this column group's share of the pair-state columns (all of them when
    // the share would not be whole float4 items)
    const int groups = gridDim.y;
    const bool share = pa.rs % (4 * groups) == 0;
    const int q4 = share ? pa.rs / (4 * groups) : pa.rs / 4;
    const int jb = share ? static_cast<int>(blockIdx.y) * q4 * 4 : 0;
    const int items = (share || blockIdx.y == 0) ? BM * q4 : 0;
    for (int base = 0; base < items; base += 1024) {
      float4 sum[4];
      bool ok[4];
      long long t[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int item = base + k * 256 + tid;
        const int row = item / q4;
        const int j = jb + (item - row * q4) * 4;
        const int m = m0 + row;
        const int i = m % pa.B;
        ok[k] = item < items && m < M && i < pa.B - 1;
        // rows past the block's last pair read row 0 (always present) and are not stored
        const long long mm = ok[k] ? m : 0;
        const long long mr = ok[k] ? m + 1 : 0;
        const int jj = ok[k] ? j : 0;
        float4 a = *reinterpret_cast<const float4*>(x + mm * ldx + pa.cl + jj);
        float4 b = *reinterpret_cast<const float4*>(x + mr * ldx + pa.cr + jj);
#pragma unroll
        for (int s2 = 1; s2 < SPLIT; ++s2) {
          const float4 a2 = *reinterpret_cast<const float4*>(x + (s2 * static_cast<long long>(M) + mm) * ldx + pa.cl + jj);
          const float4 b2 = *reinterpret_cast<const float4*>(x + (s2 * static_cast<long long>(M) + mr) * ldx + pa.cr + jj);
          a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
          b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
        }
        sum[k] = make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
        t[k] = (static_cast<long long>(m / pa.B) * (pa.B - 1) + i) * pa.rs + j;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (ok[k]) store_pair_state(pa, t[k], sum[k]);
    }
  }

  for (int n0 = nb; n0 < ne; n0 += NCOL) {
    if (n0 > nb) {
      __syncthreads();                       // every wave is done with the last chunk
      issue_w(n0);
      if constexpr (MODE == 1) load_bias(n0);
    }
    wait_all_barrier();

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < r; k += 32) {
      const int c = (k >> 3) + fq;
      bf16x8_t fa[TM], fw[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a)
        fa[a] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    tile + (a * 16 + frow) * kStr + c * 16));
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int row = wv * CW + b * 16 + frow;
        fw[b] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    wl + row * kLgRowBytes + (c ^ (row & 15)) * 16));
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[a], fw[b], acc[a][b], 0, 0, 0);
    }

    // epilogue: lane l holds column l & 15 and rows 4 (l >> 4) + v of each tile
    int mrow[TM][4];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int v = 0; v < 4; ++v) mrow[a][v] = m0 + a * 16 + fq * 4 + v;
    if constexpr (MODE == 1) {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int n = n0 + wv * CW + b * 16 + frow;
            if (mrow[a][v] < M && n < ne)
              out_bf[static_cast<long long>(mrow[a][v]) * N + n] = bf16{f32_to_bf16(acc[a][b][v] + bias[a][v][b])};
          }
    } else {
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            const int n = n0 + wv * CW + b * 16 + frow;
            if (mrow[a][v] < M && n < ne) out_f32[static_cast<long long>(mrow[a][v]) * N + n] = acc[a][b][v];
          }
    }
  }
}

template <typename TO>
hipError_t launch_ln_t(const float* x, int split, int M, int ldx, int col0, int r, float eps, void* y,
                       hipStream_t st) {
  dim3 grid((M + 3) / 4);
  TO* yo = static_cast<TO*>(y);
  const int vpl = (r + kWave - 1) / kWave;
#define DCOCO_LN(V) hipLaunchKernelGGL((ln_rows_kernel<TO, V>), grid, dim3(256), 0, st, x, split, M, ldx, col0, r, eps, yo)
  if (vpl <= 1) DCOCO_LN(1);
  else if (vpl <= 2) DCOCO_LN(2);
  else if (vpl <= 4) DCOCO_LN(4);
  else if (vpl <= 8) DCOCO_LN(8);
  else if (vpl <= 16) DCOCO_LN(16);
  else DCOCO_LN(32);
#undef DCOCO_LN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_rows(const float* x, int split, int M, int ldx, int col0, int r, float eps,
                          void* y, int out_dtype, hipStream_t st) {
  if (out_dtype == kDtypeBf16) return launch_ln_t<bf16>(x, split, M, ldx, col0, r, eps, y, st);
  return launch_ln_t<float>(x, split, M, ldx, col0, r, eps, y, st);
}

namespace {

int ln_gemm_w_rows(int M) { return M >= 4096 ? 32 : 16; }

// the z-mode pair-state arguments, or false where the launch cannot carry them
bool z_pair_args(const PairStateArgs* ps, int M, PairArgs* pa) {
  if (ps == nullptr || ps->B < 2 || ps->P <= 0 || !ln_gemm_pairs_fit(M, ps->P, ps->rs) || ps->split < 1 ||
      ps->split > kPairMaxSplit)
    return false;
  const int grid = (M + ln_gemm_w_rows(M) - 1) / ln_gemm_w_rows(M);
  pa->B = ps->B; pa->cl = ps->cl; pa->cr = ps->cr; pa->rs = ps->rs;
  pa->s = ps->s; pa->s3 = static_cast<uint16_t*>(ps->s3);
  pa->total = static_cast<long long>(ps->P) * ps->rs;
  pa->y = ps->Y; pa->split = ps->split; pa->ldy = ps->ldy;
  pa->ppw = (ps->P + grid - 1) / grid; pa->P = ps->P;
  return true;
}

}  // namespace

// The z launch (one workgroup per ln_gemm_w_rows(M) rows) takes ceil(P /
// workgroups) pairs per workgroup, one float4 item per thread.
bool ln_gemm_pairs_fit(int M, int P, int rs) {
  if (M <= 0 || P <= 0 || rs <= 0 || rs % 4 != 0) return false;
  const long long grid = (M + ln_gemm_w_rows(M) - 1) / ln_gemm_w_rows(M);
  const long long ppw = (P + grid - 1) / grid;
  return ppw * (rs / 4) <= 256;
}

hipError_t launch_ln_gemm(const float* x, int split, int M, int ldx, int col0, int r, float eps,
                          const void* W, long long ldw, int wcol0, int N, float* out_f32, void* out_bf,
                          const float* row_bias, int row_div, hipStream_t st, const PairStateArgs* ps) {
  const bf16* Wb = static_cast<const bf16*>(W);
  bf16* ob = static_cast<bf16*>(out_bf);
  const bool bias = out_bf != nullptr;
  if (split != 1 && split != 2 && split != 4) return hipErrorInvalidValue;
  PairArgs pa{};
  const bool pairs = ps != nullptr;
  if (pairs && (!bias || r > 256 || !z_pair_args(ps, M, &pa))) return hipErrorInvalidValue;
  // tile rows: enough workgroups to cover the chip, LN width in registers
#define DCOCO_LNG(BMV, RM, SP, MD)                                                                      \
  hipLaunchKernelGGL((ln_gemm_kernel<BMV, RM, SP, MD>), dim3((M + BMV - 1) / BMV), dim3(256), 0, st, x, M, \
                     ldx, col0, r, eps, Wb, ldw, wcol0, N, out_f32, ob, row_bias, row_div)
#define DCOCO_LNG_SPLIT(BMV, RM, MD)                 \
  if (split == 1) DCOCO_LNG(BMV, RM, 1, MD);         \
  else if (split == 2) DCOCO_LNG(BMV, RM, 2, MD);    \
  else DCOCO_LNG(BMV, RM, 4, MD)
#define DCOCO_LNW(BMV, SP, MD, PR)                                                                      \
  hipLaunchKernelGGL((ln_gemm_w_kernel<BMV, SP, MD, PR>), dim3((M + BMV - 1) / BMV), dim3(256), 0, st, x, \
                     M, ldx, col0, r, eps, Wb, ldw, wcol0, N, out_f32, ob, row_bias, row_div, pa,          \
                     GatherArgs{}, N)
#define DCOCO_LNW_SPLIT(BMV, MD, PR)                 \
  if (split == 1) DCOCO_LNW(BMV, 1, MD, PR);         \
  else if (split == 2) DCOCO_LNW(BMV, 2, MD, PR);    \
  else DCOCO_LNW(BMV, 4, MD, PR)
  if (r <= 256) {
    if (M >= 4096) {
      if (pairs) { DCOCO_LNW_SPLIT(32, 1, 2); }
      else if (bias) { DCOCO_LNW_SPLIT(32, 1, 0); } else { DCOCO_LNW_SPLIT(32, 0, 0); }
    } else {
      if (pairs) { DCOCO_LNW_SPLIT(16, 1, 2); }
      else if (bias) { DCOCO_LNW_SPLIT(16, 1, 0); } else { DCOCO_LNW_SPLIT(16, 0, 0); }
    }
  } else if (r <= 512) {
    if (bias) { DCOCO_LNG_SPLIT(16, 512, 1); } else { DCOCO_LNG_SPLIT(16, 512, 0); }
  } else {
    if (bias) { DCOCO_LNG_SPLIT(16, 2048, 1); } else { DCOCO_LNG_SPLIT(16, 2048, 0); }
  }
#undef DCOCO_LNW_SPLIT
#undef DCOCO_LNW
#undef DCOCO_LNG_SPLIT
#undef DCOCO_LNG
  return hipGetLastError();
}

bool ln_gemm_pair_supported(int r, int rs) { return r <= 256 && rs % 4 == 0; }

hipError_t launch_ln_gemm_pair(const float* Y, int split, int M, int ldy, int r, float eps, const void* W,
                               long long ldw, int wcol0, int N, float* gf, int B, int cl, int cr, int rs, float* s,
                               void* s3, hipStream_t st) {
  if (!ln_gemm_pair_supported(r, rs) || (split != 1 && split != 2 && split != 4)) return hipErrorInvalidValue;
  PairArgs pa;
  pa.B = B; pa.cl = cl; pa.cr = cr; pa.rs = rs;
  pa.s = s; pa.s3 = static_cast<uint16_t*>(s3);
  pa.total = static_cast<long long>(M / B) * (B - 1) * rs;
  const bf16* Wb = static_cast<const bf16*>(W);
  // few rows: the output columns are spread over four workgroups of 64
#define DCOCO_LNP(SP)                                                                                             \
  hipLaunchKernelGGL((ln_gemm_w_kernel<16, SP, 0, 1, false, 64>), dim3((M + 15) / 16, (N + 63) / 64), dim3(256), \
                     0, st, Y, M, ldy, 0, r, eps, Wb, ldw, wcol0, N, gf, static_cast<bf16*>(nullptr),               \
                     static_cast<const float*>(nullptr), 1, pa, GatherArgs{}, 64)
  if (split == 1) DCOCO_LNP(1);
  else if (split == 2) DCOCO_LNP(2);
  else DCOCO_LNP(4);
#undef DCOCO_LNP
  return hipGetLastError();
}

hipError_t launch_ln_gemm_gf(const float* Y, int split, int M, int ldy, int r, float eps, const void* W,
                             long long ldw, int wcol0, int N, float* gf, hipStream_t st) {
  if (r > 256 || (split != 1 && split != 2 && split != 4)) return hipErrorInvalidValue;
  const bf16* Wb = static_cast<const bf16*>(W);
  // as launch_ln_gemm_pair, without the pair states
#define DCOCO_LNF(SP)                                                                                            \
  hipLaunchKernelGGL((ln_gemm_w_kernel<16, SP, 0, 0, false, 64>), dim3((M + 15) / 16, (N + 63) / 64), dim3(256), \
                     0, st, Y, M, ldy, 0, r, eps, Wb, ldw, wcol0, N, gf, static_cast<bf16*>(nullptr),              \
                     static_cast<const float*>(nullptr), 1, PairArgs{}, GatherArgs{}, 64)
  if (split == 1) DCOCO_LNF(1);
  else if (split == 2) DCOCO_LNF(2);
  else DCOCO_LNF(4);
#undef DCOCO_LNF
  return hipGetLastError();
}

bool gather_gemm_supported(int r) { return r <= 256 && r % 8 == 0; }

hipError_t launch_gather_gemm(const void* tab, const int32_t* ids, int idmax, int M, int r, const void* W,
                              long long ldw, int wcol0, int N, void* out_bf, const float* row_bias, int row_div,
                              hipStream_t st, const PairStateArgs* ps) {
  if (!gather_gemm_supported(r)) return hipErrorInvalidValue;
  PairArgs pa{};
  const bool pairs = ps != nullptr;
  if (pairs && !z_pair_args(ps, M, &pa)) return hipErrorInvalidValue;
  GatherArgs ga;
  ga.tab = static_cast<const uint16_t*>(tab);
  ga.ids = ids;
  ga.idmax = idmax;
  const bf16* Wb = static_cast<const bf16*>(W);
  bf16* ob = static_cast<bf16*>(out_bf);
#define DCOCO_LNG_G(BMV, PR)                                                                                  \
  hipLaunchKernelGGL((ln_gemm_w_kernel<BMV, 1, 1, PR, true>), dim3((M + BMV - 1) / BMV), dim3(256), 0, st,   \
                     static_cast<const float*>(nullptr), M, r, 0, r, 1.0f, Wb, ldw, wcol0, N,                \
                     static_cast<float*>(nullptr), ob, row_bias, row_div, pa, ga, N)
  if (M >= 4096) { if (pairs) { DCOCO_LNG_G(32, 2); } else { DCOCO_LNG_G(32, 0); } }
  else { if (pairs) { DCOCO_LNG_G(16, 2); } else { DCOCO_LNG_G(16, 0); } }
#undef DCOCO_LNG_G
  return hipGetLastError();
}

hipError_t launch_pair_state(const float* Y, int split, int N, int B, int ldy, int cl, int cr,
                             int rs, float* s, void* s3, hipStream_t st) {
  const long long total = static_cast<long long>(N) * (B - 1) * rs;
  if (total <= 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  dim3 grid(static_cast<unsigned>(blocks < 65535 ? blocks : 65535));
  hipLaunchKernelGGL(pair_state_kernel, grid, dim3(256), 0, st, Y, split, N, B, ldy, cl, cr, rs, s,
                     static_cast<uint16_t*>(s3));
  return hipGetLastError();
}

}  // namespace dcoco
