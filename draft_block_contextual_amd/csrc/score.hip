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
#include "wave.h"

namespace dcoco {

namespace {

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

struct GridDev {
  int N, B, K, H, P, nq;
  const float* AB;       // [N*B*K, 2H]: W1a z | W1b z
  const float* C;        // [nq, P, H]: parts of W1s s_p
  const void* b1;        // [H] or null
  const void* w2;        // [H]
  float b2;
  const float* cand_logits;
  float* S;
  int32_t* best;
};

// s -> three bf16 rows per pair (hi, mid, lo with s = hi + mid + lo exactly
// for normal values: each part takes the next 8 significand bits), the MFMA
// operand that keeps W1s s_p at fp32 accuracy on bf16 matrix cores.
__global__ void __launch_bounds__(256)
split3_kernel(const float* __restrict__ s, long long n, uint16_t* __restrict__ s3) {
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n; i += 256ll * gridDim.x) {
    const float x = s[i];
    const uint16_t hi = f32_to_bf16(x);
    const float r1 = x - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    const uint16_t lo = f32_to_bf16(r1 - bf16_to_f32(mid));
    s3[i] = hi;
    s3[n + i] = mid;
    s3[2 * n + i] = lo;
  }
}

// The K x K x H grid.  Inputs per pair (n, p): A = W1a z_{p,a} and
// B = W1b z_{p+1,b} (rows of the fp32 product AB = z [W1a; W1b]^T), and
// C_p = sum of nq rows of the fp32 product of the s operand with W1s.  With
// A' = -log2(e) A, B' = -log2(e) (B + C_p + b1) and w' = -ln2 w2, the term
// is  w2 SiLU(u) = w' (A' + B') / (1 + 2^A' 2^B').  The hidden units are
// processed in slabs staged in LDS as 2^A', w'A' (per candidate a) and
// 2^B', w'B' (per candidate b), so one grid element costs an fma, a rcp, an
// add and an fma.  If some |A'| in a slab exceeds 64 the factors could
// over/underflow where their product does not; that slab is staged again as
// A', B' and evaluated with 2^(A'+B') directly.
//
// One workgroup (4 waves) per pair; each wave takes a quarter of every slab's
// units.  A lane owns a TA x TA block of (a, b) outputs; the KR/TA x KR/TA
// lanes covering all outputs form a group, and a wave holds UPS groups that
// work on different runs of 4 units, so every 4 units a lane reads 4 TA
// values per array for 4 TA^2 elements.  The next slab's A and B rows are
// loaded into registers while the current slab is computed.  The partial
// sums of the 4 UPS lane groups are added in a fixed order at the end.
template <int KRV, int TAV>
struct GridShape {
  static constexpr int KR = KRV;                 // candidates, padded
  static constexpr int TA = TAV;                 // outputs per lane along a and b
  static constexpr int LPU = (KR / TA) * (KR / TA);   // lanes per group
  static constexpr int UPS = kWave / LPU;        // groups per wave
  static constexpr int HS = 4096 / KR;           // hidden units per slab
  static constexpr int STR = HS + 4;             // LDS row stride (floats)
  static constexpr int ARR = KR * STR;
  static constexpr int NLD = KR * HS / 4 / 256;  // float4 per thread per operand and slab
  static constexpr int kRed = 4 * UPS * KR * KR;  // partial sums to add at the end
  // LDS floats with partial sums of ACC_BYTES each (the reduction reuses the
  // slab arrays and the per-unit terms once the last slab is done)
  template <int ACC_BYTES>
  static constexpr int smem_floats() {
    return (4 * ARR > kRed * ACC_BYTES / 4 ? 4 * ARR : kRed * ACC_BYTES / 4) + 4 * HS;
  }
  static_assert(LPU * UPS == kWave && NLD * 1024 == KR * HS, "grid shape");
};

// The fp32 path adds its terms in fp64: a pair's terms can be hundreds of
// times larger than the score they sum to (large pre-activations of opposite
// signs), and fp32 running sums would then lose the score's low digits.  Each
// term is still formed in fp32.
template <typename T, typename GS>
__global__ void __launch_bounds__(256) grid_kernel(GridDev g) {
  using Acc = typename std::conditional<std::is_same<T, float>::value, double, float>::type;
  constexpr int KR = GS::KR;
  constexpr int TA = GS::TA;
  constexpr int HS = GS::HS;
  constexpr int STR = GS::STR;
  constexpr int NLD = GS::NLD;
  constexpr int UPS = GS::UPS;
  __shared__ __align__(16) float smem[GS::template smem_floats<sizeof(Acc)>()];
  __shared__ int s_slow[2];
  float* arr0 = smem;                 // 2^A'  (or A')
  float* arr1 = smem + GS::ARR;       // w'A'
  float* arr2 = smem + 2 * GS::ARR;   // 2^B'  (or B')
  float* arr3 = smem + 3 * GS::ARR;   // w'B'
  float* sCp = smem + 4 * GS::ARR;    // [2][HS] per unit: -log2(e) (C_p + b1)
  float* sWp = sCp + 2 * HS;          // [2][HS] per unit: w'

  const int np = blockIdx.x;
  const int Bm1 = g.B - 1;
  const int n = np / Bm1;
  const int p = np % Bm1;
  const int K = g.K;
  const int H = g.H;
  const long long ldab = 2ll * H;
  const float* Arow = g.AB + (static_cast<long long>(n) * g.B + p) * K * ldab;
  const float* Brow = g.AB + (static_cast<long long>(n) * g.B + p + 1) * K * ldab + H;
  const T* w2 = static_cast<const T*>(g.w2);
  const T* b1 = static_cast<const T*>(g.b1);

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int grp = l / GS::LPU;
  const int gi = l % GS::LPU;
  const int la = gi / (KR / TA);
  const int lb = gi % (KR / TA);

  // slab rows in registers: item k of thread tid is (row, 4 units) of the
  // slab's KR x HS block.  The loads are unconditional (row and unit clamped
  // into the pair's data) so none of them waits for another; rows >= K and
  // units past H are zeroed when the slab is staged.
  float4 pa[NLD], pb[NLD];
  auto fetch = [&](int hs0) {
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int idx = tid + 256 * k;
      const int row = min(idx / (HS / 4), K - 1);
      const int h = min(hs0 + (idx % (HS / 4)) * 4, H - 4);
      pa[k] = *reinterpret_cast<const float4*>(Arow + row * ldab + h);
      pb[k] = *reinterpret_cast<const float4*>(Brow + row * ldab + h);
    }
  };
  // per-unit terms of a slab; the loads are unconditional (clamped unit,
  // clamped part index) so they are all in flight before the first wait
  auto stage_c = [&](int hs0, int cb) {
    for (int h = tid; h < HS; h += 256) {
      const bool in = hs0 + h < H;
      const int hh = in ? hs0 + h : H - 1;
      float cq[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) cq[q] = g.C[(static_cast<long long>(min(q, g.nq - 1)) * g.P + np) * H + hh];
      const float bb = b1 ? Elem<T>::to_f32(b1[hh]) : 0.f;
      const float ww = Elem<T>::to_f32(w2[hh]);
      float c = cq[0];
      if (g.nq > 1) c += cq[1];
      if (g.nq > 2) c += cq[2];
      c += bb;
      sCp[cb * HS + h] = in ? kNegLog2e * c : 0.f;
      sWp[cb * HS + h] = in ? kNegLn2 * ww : 0.f;
    }
  };

  Acc acc[TA][TA];
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) acc[i][j] = 0;

  stage_c(0, 0);
  fetch(0);
  if (tid == 0) s_slow[0] = 0;
  __syncthreads();
  int cb = 0;
  for (int hs0 = 0; hs0 < H; hs0 += HS, cb ^= 1) {
    const int hlen = min(HS, H - hs0);
    const float* cp = sCp + cb * HS;
    const float* wp = sWp + cb * HS;
    // ---- stage the slab (fast form) from registers
    bool big = false;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int idx = tid + 256 * k;
      const int row = idx / (HS / 4);
      const int h = (idx % (HS / 4)) * 4;
      const float4 c4 = *reinterpret_cast<const float4*>(cp + h);
      const float4 w4 = *reinterpret_cast<const float4*>(wp + h);
      const bool ok = row < K && hs0 + h < H;
      float4 a = ok ? pa[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 b = ok ? pb[k] : make_float4(0.f, 0.f, 0.f, 0.f);
      a.x *= kNegLog2e; a.y *= kNegLog2e; a.z *= kNegLog2e; a.w *= kNegLog2e;
      b.x = fmaf(kNegLog2e, b.x, c4.x); b.y = fmaf(kNegLog2e, b.y, c4.y);
      b.z = fmaf(kNegLog2e, b.z, c4.z); b.w = fmaf(kNegLog2e, b.w, c4.w);
      big |= fabsf(a.x) > 64.f || fabsf(a.y) > 64.f || fabsf(a.z) > 64.f || fabsf(a.w) > 64.f;
      *reinterpret_cast<float4*>(arr1 + row * STR + h) = make_float4(w4.x * a.x, w4.y * a.y, w4.z * a.z, w4.w * a.w);
      *reinterpret_cast<float4*>(arr3 + row * STR + h) = make_float4(w4.x * b.x, w4.y * b.y, w4.z * b.z, w4.w * b.w);
      *reinterpret_cast<float4*>(arr0 + row * STR + h) =
          make_float4(__builtin_amdgcn_exp2f(a.x), __builtin_amdgcn_exp2f(a.y), __builtin_amdgcn_exp2f(a.z),
                      __builtin_amdgcn_exp2f(a.w));
      *reinterpret_cast<float4*>(arr2 + row * STR + h) =
          make_float4(__builtin_amdgcn_exp2f(b.x), __builtin_amdgcn_exp2f(b.y), __builtin_amdgcn_exp2f(b.z),
                      __builtin_amdgcn_exp2f(b.w));
    }
    if (big) s_slow[cb] = 1;
    // ---- next slab: rows into registers, per-unit terms into the other buffer
    if (hs0 + HS < H) {
      // the per-unit terms first: waiting for them must not wait for the rows
      stage_c(hs0 + HS, cb ^ 1);
      fetch(hs0 + HS);
    }
    if (tid == 0) s_slow[cb ^ 1] = 0;
    __syncthreads();
    const bool slow = s_slow[cb] != 0;
    if (slow) {
      // rare: stage A' and B' themselves (read again from memory)
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int idx = tid + 256 * k;
        const int row = idx / (HS / 4);
        const int h = (idx % (HS / 4)) * 4;
        const bool ok = row < K && hs0 + h < H;
        float4 a = ok ? *reinterpret_cast<const float4*>(Arow + row * ldab + hs0 + h) : make_float4(0.f, 0.f, 0.f, 0.f);
        float4 b = ok ? *reinterpret_cast<const float4*>(Brow + row * ldab + hs0 + h) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 c4 = *reinterpret_cast<const float4*>(cp + h);
        a.x *= kNegLog2e; a.y *= kNegLog2e; a.z *= kNegLog2e; a.w *= kNegLog2e;
        b.x = fmaf(kNegLog2e, b.x, c4.x); b.y = fmaf(kNegLog2e, b.y, c4.y);
        b.z = fmaf(kNegLog2e, b.z, c4.z); b.w = fmaf(kNegLog2e, b.w, c4.w);
        *reinterpret_cast<float4*>(arr0 + row * STR + h) = a;
        *reinterpret_cast<float4*>(arr2 + row * STR + h) = b;
      }
      __syncthreads();
    }
    // ---- this wave's quarter of the slab, runs of 4 units per lane group
    const int q4 = hlen / 4;
    const int h_end = wv * q4 + q4;
    if (!slow) {
      for (int h = wv * q4 + 4 * grp; h < h_end; h += 4 * UPS) {
        float4 ea[TA], wa[TA], eb[TA], wb[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          ea[i] = *reinterpret_cast<const float4*>(arr0 + (la * TA + i) * STR + h);
          wa[i] = *reinterpret_cast<const float4*>(arr1 + (la * TA + i) * STR + h);
          eb[i] = *reinterpret_cast<const float4*>(arr2 + (lb * TA + i) * STR + h);
          wb[i] = *reinterpret_cast<const float4*>(arr3 + (lb * TA + i) * STR + h);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < TA; ++i)
#pragma unroll
            for (int j = 0; j < TA; ++j) {
              const float den = fmaf(ea[i][c], eb[j][c], 1.0f);
              const float r = __builtin_amdgcn_rcpf(den);
              if constexpr (std::is_same<Acc, float>::value)
                acc[i][j] = fmaf(wa[i][c] + wb[j][c], r, acc[i][j]);
              else
                acc[i][j] += static_cast<Acc>((wa[i][c] + wb[j][c]) * r);
            }
      }
    } else {
      for (int h = wv * q4 + 4 * grp; h < h_end; h += 4 * UPS) {
        float4 av[TA], bv[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          av[i] = *reinterpret_cast<const float4*>(arr0 + (la * TA + i) * STR + h);
          bv[i] = *reinterpret_cast<const float4*>(arr2 + (lb * TA + i) * STR + h);
        }
        const float4 wq = *reinterpret_cast<const float4*>(wp + h);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int i = 0; i < TA; ++i)
#pragma unroll
            for (int j = 0; j < TA; ++j) {
              const float t = av[i][c] + bv[j][c];
              const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
              if constexpr (std::is_same<Acc, float>::value)
                acc[i][j] = fmaf(wq[c], t * r, acc[i][j]);
              else
                acc[i][j] += static_cast<Acc>(wq[c] * (t * r));
            }
      }
    }
    __syncthreads();
  }
  // ---- add the 4 UPS partial sums per output in a fixed order
  Acc* red = reinterpret_cast<Acc*>(smem);
  const int slot = wv * UPS + grp;
#pragma unroll
  for (int i = 0; i < TA; ++i)
#pragma unroll
    for (int j = 0; j < TA; ++j) red[(slot * KR + la * TA + i) * KR + lb * TA + j] = acc[i][j];
  __syncthreads();
  const float* lnext = g.cand_logits + (static_cast<long long>(n) * g.B + p + 1) * K;
  float* Sp = g.S + static_cast<long long>(np) * K * K;
  constexpr int kPerT = (KR * KR + 255) / 256;
  float sv[kPerT];
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < K * K) {
      const int a = idx / K;
      const int b = idx - a * K;
      const int o = a * KR + b;
      Acc sum = red[o];
      for (int sl = 1; sl < 4 * UPS; ++sl) sum += red[sl * KR * KR + o];
      sv[i] = lnext[b] + static_cast<float>(sum + static_cast<Acc>(g.b2));
      Sp[idx] = sv[i];
    }
  }
  if (g.best == nullptr) return;
  // the walk's step from each row a: argmax_b S_p(a, b) under the walk's rule
  // (largest order key, the lowest b among equal keys; NaN never wins)
  if constexpr (KR * KR <= 256) {
    if (K == KR) {
      // thread a K + b holds S_p(a, b) and each row fills an aligned group of
      // KR lanes: a max over (key, KR - 1 - b) within the group decides
      const int b = tid % KR;
      const bool valid = tid < K * K;
      uint64_t c = valid ? (static_cast<uint64_t>(order_key(sv[0])) << 32) | static_cast<uint32_t>(KR - 1 - b) : 0ull;
#pragma unroll
      for (int off = KR / 2; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(c, off, kWave);
        c = o > c ? o : c;
      }
      if (valid && b == 0) g.best[static_cast<long long>(np) * K + tid / KR] = KR - 1 - static_cast<int>(c & 0xffu);
      return;
    }
  }
  __syncthreads();                     // every thread is done reading red
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < K * K) smem[idx] = sv[i];
  }
  __syncthreads();
  if (tid < K) {
    const float* row = smem + tid * K;
    uint32_t bk = order_key(row[0]);
    int bb = 0;
    for (int b = 1; b < K; ++b) {
      const uint32_t k = order_key(row[b]);
      if (k > bk) {
        bk = k;
        bb = b;
      }
    }
    g.best[static_cast<long long>(np) * K + tid] = bb;
  }
}

constexpr int kWalkLds = 8192;   // floats of scores staged per batch
constexpr int kWalkIds = 1088;   // candidate ids staged per batch: (16 + 1) rows of 64

// argmax over lanes 0..K-1 of one wave: the largest order key, the lowest lane
// among equal keys (lanes >= K carry key 0, the NaN key, and sit above every
// valid lane, so they never win)
__device__ __forceinline__ int wave_argmax(float v, bool valid) {
  const uint32_t key = valid ? order_key(v) : 0u;
  const uint32_t m = wave_max_u32_dpp(key);
  return __builtin_ctzll(ballot(key == m));
}

// copy n 4-byte words global -> LDS with 256 threads; each thread issues up to
// four loads before it waits, so one batch costs about one memory latency
template <typename W, typename V>
__device__ __forceinline__ void walk_stage(W* dst, const W* src, int n, int tid) {
  constexpr int kPer = sizeof(V) / sizeof(W);
  const int nv = n / kPer;
  for (int b = tid; b < nv; b += 1024) {
    V v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (b + 256 * j < nv) v[j] = reinterpret_cast<const V*>(src)[b + 256 * j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (b + 256 * j < nv) reinterpret_cast<V*>(dst)[b + 256 * j] = v[j];
  }
  for (int i = nv * kPer + tid; i < n; i += 256) dst[i] = src[i];
}

// One workgroup per block.  Each batch of pairs stages its scores and the
// candidate ids of the slots it selects into LDS with one round of loads;
// wave 0 then walks the batch from LDS only, so the chain of dependent
// argmaxes never waits on global memory.
__global__ void __launch_bounds__(256)
walk_kernel(const float* __restrict__ S, const float* __restrict__ cl, const int32_t* __restrict__ ids,
            int B, int K, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_tok) {
  __shared__ __align__(16) float sS[kWalkLds];
  __shared__ __align__(16) int32_t sI[kWalkIds];
  __shared__ __align__(16) float sC[kWave + 4];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int per = K * K;
  const int Bm1 = B - 1;
  const int batch = max(1, min(kWalkLds / per, kWalkIds / K - 1));
  const float* Sn = S + static_cast<long long>(n) * Bm1 * per;
  const int32_t* idn = ids + static_cast<long long>(n) * B * K;
  int32_t* si = sel_idx ? sel_idx + static_cast<long long>(n) * B : nullptr;
  int32_t* stok = sel_tok + static_cast<long long>(n) * B;
  const bool vec = ((reinterpret_cast<uintptr_t>(Sn) & 15) == 0) && (per % 4 == 0) &&
                   ((reinterpret_cast<uintptr_t>(idn) & 15) == 0) && (K % 4 == 0);
  int k = 0;
  for (int p0 = 0;; p0 += batch) {
    const int cnt = max(0, min(batch, Bm1 - p0));
    __syncthreads();
    const float* src = Sn + static_cast<long long>(p0) * per;
    const int32_t* isrc = idn + static_cast<long long>(p0) * K;
    const int ns = cnt * per;
    const int ni = (cnt + 1) * K;
    if (vec && ns >= 4 && ns <= 4096 && ni <= 1024) {
      // one round: up to 4 float4 of scores, one int4 of ids and one logit per
      // thread.  The loads are unconditional (out-of-range threads re-read
      // element 0) so they are all in flight before the first wait.
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        v[j] = reinterpret_cast<const float4*>(src)[idx * 4 < ns ? idx : 0];
      }
      const int4 iv = reinterpret_cast<const int4*>(isrc)[tid * 4 < ni ? tid : 0];
      const float c0 = cl[static_cast<long long>(n) * B * K + (tid < K ? tid : 0)];
      // stores without branches: out-of-range threads write a spare slot
      // past the staged data (float4 1023: ns <= 4092 whenever some thread is
      // out of range; int4 271: ni <= 1024; sC[64])
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        reinterpret_cast<float4*>(sS)[idx * 4 < ns ? idx : 1023] = v[j];
      }
      reinterpret_cast<int4*>(sI)[tid * 4 < ni ? tid : kWalkIds / 4 - 1] = iv;
      sC[p0 == 0 && tid < K ? tid : kWave] = c0;
    } else {
      walk_stage<float, float>(sS, src, ns, tid);
      walk_stage<int32_t, int32_t>(sI, isrc, ni, tid);
      if (p0 == 0 && tid < K) sC[tid] = cl[static_cast<long long>(n) * B * K + tid];
    }
    __syncthreads();
    if (tid < kWave) {
      if (p0 == 0) {
        k = wave_argmax(l < K ? sC[l] : 0.f, l < K);
        if (l == 0) {
          if (si) si[0] = k;
          stok[0] = sI[k];
        }
      }
      for (int q = 0; q < cnt; ++q) {
        k = wave_argmax(l < K ? sS[q * per + k * K + l] : 0.f, l < K);
        if (l == 0) {
          if (si) si[p0 + q + 1] = k;
          stok[p0 + q + 1] = sI[(q + 1) * K + k];
        }
      }
    }
    if (p0 + batch >= Bm1) break;
  }
}

// The walk from the grid's argmax table: k_1 = argmax of the first slot's
// logits, then k_{p+1} = best_p(k_p).  One wave per block: the block's table is
// staged in LDS with its loads all in flight, one lane follows the chain
// (one LDS read per step), and the chosen ids are fetched in parallel.
constexpr int kWalkTab = 8192;    // table entries staged: (B - 1) K
constexpr int kWalkMaxB = 2048;   // slots per block

__global__ void __launch_bounds__(kWave)
walk_table_kernel(const int32_t* __restrict__ best, const float* __restrict__ cl, const int32_t* __restrict__ ids,
                  int B, int K, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_tok) {
  __shared__ int32_t sB[kWalkTab];
  __shared__ int32_t sK[kWalkMaxB];
  const int n = blockIdx.x;
  const int l = lane_id();
  const int nt = (B - 1) * K;
  const int32_t* bn = best + static_cast<long long>(n) * nt;
  for (int base = 0; base < nt; base += 8 * kWave) {
    int32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = bn[min(base + j * kWave + l, nt - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (base + j * kWave + l < nt) sB[base + j * kWave + l] = v[j];
  }
  const float c0 = cl[static_cast<long long>(n) * B * K + (l < K ? l : 0)];
  int k = wave_argmax(c0, l < K);
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
  if (l == 0) {
    sK[0] = k;
    for (int p = 0; p + 1 < B; ++p) {
      k = min(max(sB[p * K + k], 0), K - 1);   // in range by construction; kept so
      sK[p + 1] = k;                            // no table value can index outside
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
  for (int j = l; j < B; j += kWave) {
    const int kj = sK[j];
    const long long o = static_cast<long long>(n) * B + j;
    if (sel_idx) sel_idx[o] = kj;
    sel_tok[o] = ids[o * K + kj];
  }
}

constexpr int kPathLds = 12288;   // floats of scores staged per chunk of pairs
constexpr int kPathBp = 16384;    // bytes of back-pointers, one per (pair, candidate)
constexpr int kPathMaxB = 4096;   // slots per block: the chosen indices reuse the score buffer

// Whole-path rules, one workgroup per block.  The path score weights slot j
// (0-based) by lam^j; with U_{B-1} = 0 and, from the last pair back,
//   U_p(a) = max_b [S_p(a, b) + lam * U_{p+1}(b)],
// lam^(p+1) U_p(a) is the best weighted score of the slots after p given
// k_p = a.  Lane a of wave 0 holds U(a) in a register and reads U(b) with
// readlane; the lowest maximising b is kept as a back-pointer in LDS.  The
// forward pass takes k_0 = argmax_a [l_0(a) + lam U_0(a)] and follows the
// back-pointers, which walks the lexicographically smallest optimal path.
// NaN never wins a comparison, so a NaN term acts as -inf.
__global__ void __launch_bounds__(256)
path_kernel(const float* __restrict__ S, const float* __restrict__ cl, const int32_t* __restrict__ ids,
            int B, int K, float lam, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_tok) {
  __shared__ __align__(16) float sS[kPathLds];
  __shared__ uint8_t sBp[kPathBp];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int Bm1 = B - 1;
  const int per = K * K;
  const int KS = ((K + 3) & ~3) + 4;   // padded row stride in floats (16-byte rows)
  const int pstr = K * KS;              // floats per staged pair
  const int chunk = kPathLds / pstr;    // >= 2 for K <= 64
  const float* Sn = S + static_cast<long long>(n) * Bm1 * per;
  const bool vec = ((reinterpret_cast<uintptr_t>(Sn) & 15) == 0) && (K % 4 == 0);
  float u = 0.f;
  for (int hi = Bm1; hi > 0;) {
    const int lo = max(0, hi - chunk);
    const int ne = (hi - lo) * per;
    const float* src = Sn + static_cast<long long>(lo) * per;
    __syncthreads();   // the previous chunk has been consumed
    if (vec) {
      // 8 float4 per thread and round, loads unconditional (index clamped)
      const int nv = ne / 4;
      for (int e0 = 0; e0 < nv; e0 += 256 * 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = reinterpret_cast<const float4*>(src)[min(e0 + tid + 256 * j, nv - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = 4 * (e0 + tid + 256 * j);
          if (e < ne) {
            const int q = e / per;
            const int r = e - q * per;
            const int a = r / K;
            *reinterpret_cast<float4*>(sS + q * pstr + a * KS + (r - a * K)) = v[j];
          }
        }
      }
    } else {
      for (int e0 = 0; e0 < ne; e0 += 256 * 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[min(e0 + tid + 256 * j, ne - 1)];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = e0 + tid + 256 * j;
          if (e < ne) {
            const int q = e / per;
            const int r = e - q * per;
            const int a = r / K;
            sS[q * pstr + a * KS + (r - a * K)] = v[j];
          }
        }
      }
    }
    __syncthreads();
    if (tid < kWave) {
      for (int p = hi - 1; p >= lo; --p) {
        // lanes >= K work on row K-1 and their results are never read
        const float* row = sS + (p - lo) * pstr + min(l, K - 1) * KS;
        float best = -INFINITY;
        int bi = 0;
        for (int b4 = 0; b4 < K; b4 += 4) {
          const float4 r4 = *reinterpret_cast<const float4*>(row + b4);
          const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int b = b4 + t;
            if (b < K) {
              const float c = rv[t] + lam * read_lane(u, b);
              if (c > best) {
                best = c;
                bi = b;
              }
            }
          }
        }
        u = best;
        if (l < K) sBp[p * K + l] = static_cast<uint8_t>(bi);
      }
    }
    hi = lo;
  }
  __syncthreads();
  int32_t* sK = reinterpret_cast<int32_t*>(sS);   // the chosen index per slot
  if (tid < kWave) {
    const float c0 = cl[static_cast<long long>(n) * B * K + min(l, K - 1)] + lam * u;
    int k = wave_argmax(c0 == c0 ? c0 : -INFINITY, l < K);
    if (l == 0) {
      for (int j = 0; j < B; ++j) {
        sK[j] = k;
        if (j < Bm1) k = sBp[j * K + k];
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < B; j += 256) {
    const int k = sK[j];
    const long long o = static_cast<long long>(n) * B + j;
    if (sel_idx) sel_idx[o] = k;
    sel_tok[o] = ids[o * K + k];
  }
}

template <typename T>
hipError_t launch_grid_t(const GridProblem& q, hipStream_t st) {
  GridDev g;
  g.N = q.N; g.B = q.B; g.K = q.K; g.H = q.H; g.P = q.N * (q.B - 1); g.nq = q.nq;
  g.AB = q.AB; g.C = q.C; g.b1 = q.b1; g.w2 = q.w2; g.b2 = q.b2;
  g.cand_logits = q.cand_logits; g.S = q.S; g.best = q.best;
  const int blocks = q.N * (q.B - 1);
  if (blocks <= 0) return hipSuccess;
#define DCOCO_GRID(KRV, TAV) hipLaunchKernelGGL((grid_kernel<T, GridShape<KRV, TAV>>), dim3(blocks), dim3(256), 0, st, g)
  if (q.K <= 8) DCOCO_GRID(8, 2);
  else if (q.K <= 16) DCOCO_GRID(16, 4);
  else if (q.K <= 32) DCOCO_GRID(32, 4);
  else DCOCO_GRID(64, 8);
#undef DCOCO_GRID
  return hipGetLastError();
}

}  // namespace

bool path_supported(int B, int K) {
  return B >= 1 && K >= 1 && K <= 64 && B <= kPathMaxB && static_cast<long long>(B) * K <= kPathBp;
}

hipError_t launch_path(const float* S, const float* cand_logits, const int32_t* cand_ids, int N, int B, int K,
                       float lam, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st) {
  if (!path_supported(B, K)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(path_kernel, dim3(N), dim3(256), 0, st, S, cand_logits, cand_ids, B, K, lam, sel_idx,
                     sel_tok);
  return hipGetLastError();
}

hipError_t launch_grid(const GridProblem& q, hipStream_t st) {
  if (q.dtype == kDtypeBf16) return launch_grid_t<bf16>(q, st);
  return launch_grid_t<float>(q, st);
}

hipError_t launch_split3(const float* s, long long n, void* s3, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(split3_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, s, n,
                     static_cast<uint16_t*>(s3));
  return hipGetLastError();
}

hipError_t launch_walk(const float* S, const float* cand_logits, const int32_t* cand_ids, int N,
                       int B, int K, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st) {
  hipLaunchKernelGGL(walk_kernel, dim3(N), dim3(256), 0, st, S, cand_logits, cand_ids, B, K, sel_idx,
                     sel_tok);
  return hipGetLastError();
}

bool walk_table_supported(int B, int K) {
  return B >= 1 && K >= 1 && K <= kWave && B <= kWalkMaxB && static_cast<long long>(B - 1) * K <= kWalkTab;
}

hipError_t launch_walk_table(const int32_t* best, const float* cand_logits, const int32_t* cand_ids, int N,
                             int B, int K, int32_t* sel_idx, int32_t* sel_tok, hipStream_t st) {
  if (!walk_table_supported(B, K)) return hipErrorInvalidValue;
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(walk_table_kernel, dim3(N), dim3(kWave), 0, st, best, cand_logits, cand_ids, B, K, sel_idx,
                     sel_tok);
  return hipGetLastError();
}

}  // namespace dcoco
