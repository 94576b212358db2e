// Transition scoring with the per-candidate products formed on chip (bf16
// storage; review of arXiv 2610.12570, "Contextual Correction of Parallel
// Drafts for Speculative Decoding", part 1 of "New approach: DCOCO", paper
// Sec. 3.2; Two Delta, "Two Delta makes NVIDIA Nemotron 3.5 Super even faster
// with DCOCO", "Score neighboring candidates in parallel"):
//   S_p(a,b) = l_{p+1}(b) + b2 + sum_h w2_h SiLU(A_{p,a,h} + B_{p,b,h} + C_{p,h}),
//   A_{p,a} = W1a z_{p,a},  B_{p,b} = W1b z_{p+1,b},  C_p = W1s s_p + b1.
// W1s s_p comes either from memory (three parts, one per bf16 part of s_p)
// or, for chunks of at most five pairs, from the launch itself: the
// workgroup forms the parts of its chunk's pairs over its slab's units on
// MFMA in the prologue, exactly as the separate product would (same operand
// fragments, same k order), and adds them in the same order.
// The sum over hidden units is cut into slabs of 64 and a draft block's pairs
// into chunks.  A workgroup takes one (block, slab, chunk): each of its four
// waves keeps the W1a and W1b rows of 16 units of the slab in registers and
// walks the chunk's slots in order.  Slot t's candidate rows z_t are copied
// into LDS one slot ahead (direct global->LDS loads); A_t = W1a z_t and
// B_t = W1b z_t are formed on v_mfma_f32_16x16x32_bf16; B_t completes pair
// t-1, whose K x K grid over the wave's units is evaluated at once, and A_t
// is kept for pair t.  A and B never reach memory.  With A' = -log2(e) A,
// B' = -log2(e) (B + C_p) and w' = -ln(2) w2 a term is
// w2 SiLU(u) = w' (A' + B') / (1 + 2^A' 2^B'); a wave with some |A'| > 64 in
// a pair stages A', B' instead and evaluates 2^(A'+B') per element.  Each
// pair's sum over the slab (the four waves added in a fixed order) is stored
// per slab; pair_finish_kernel, or block_finish_walk_kernel for a whole block,
// adds the slabs in order, adds l_{p+1}(b) + b2 and takes each row's argmax
// for the walk.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "dma.h"
#include "kernels.h"
#include "wave.h"

namespace dcoco {

namespace {

constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;
constexpr int kUW = 16;                  // units per wave per slab
constexpr int kUS = 4 * kUW;             // units per slab
constexpr int kMaxKs = 8;                // 32-deep k steps of z (W1 fragments in registers): r_z <= 256
constexpr int kChipPairs = 5;            // pairs per chunk with the pair term formed on chip: 3 parts x 5 <= 16 rows

struct SlabDev {
  int N, B, K, H, P, rz, nq, nslab, pc, nchunk;
  const uint16_t* z;       // [N*B*K, rz]
  const uint16_t* W1;      // [H, ldw1]: columns [z_a | z_b | s]
  long long ldw1;
  const float* C;          // [nq, P, H]: parts of W1s s_p (summed); null when formed on chip
  const uint16_t* s3;      // [3, P, rs]: bf16 parts of s_p (on-chip pair term), else null
  long long s3_part;       // P rs
  int rs;
  const uint16_t* b1;      // [H] or null
  const uint16_t* w2;      // [H]
  float* part;             // [nslab, P, K, K]: each slab's sum
};

// KR candidates padded to whole 16-row MFMA tiles; a lane owns a TA x TA
// block of (a, b) outputs (TA = KR / 8, so the wave's 64 lanes cover the
// whole K x K grid) over all 16 of the wave's units: a lane's sums are the
// wave's, and no lane reduction is needed.  Each wave puts its sum of a pair
// in LDS; after the step's barrier the workgroup adds the four waves in order
// and stores the pair's slab sum.  For KR = 16 the sums are double-buffered
// (the pair finished at one step is added up at the next), so a chunk may hold
// any number of pairs; for KR = 32 a chunk is one pair.
template <int KRV, int NKSV>
struct SlabShape {
  static constexpr int KR = KRV;
  static constexpr int NKS = NKSV;                 // 32-deep k steps: r_z = 32 NKS
  static constexpr int TA = KR / 8;
  static constexpr int RT = KR / 16;
  static constexpr int STR = kUW + 4;              // LDS floats per staged candidate row
  static constexpr int ARR = KR * STR;             // floats per staged array
  static constexpr int WREG = 4 * ARR + kUW;       // a wave's region: 4 arrays + w' per unit
  static constexpr int STAGE = 4 * WREG;           // floats of the four waves' regions
  static constexpr int ZBUF = KR * NKS * 32 * 2;   // bytes of one slot's z rows
  static constexpr int NBUF = KR == 16 ? 2 : 1;      // pair-sum buffers (1: one pair per chunk)
  static constexpr int SUMS = NBUF * 4 * KR * KR;     // [buffer][wave][KR * KR] sums
  static_assert((KR / TA) * (KR / TA) == kWave, "one output block per lane");
  static_assert(NKS >= 2 && NKS <= kMaxKs, "r_z");
  static constexpr int CSUM = 4 * kChipPairs * kUW;  // on-chip pair term: [wave][pair][unit]
  // K <= 16: three workgroups per CU
  static_assert(2 * ZBUF + (STAGE + SUMS + CSUM) * 4 <= (KR == 16 ? 53 : 160) * 1024, "LDS");
  static_assert(2 * ARR >= 16 * kUW, "a wave's B-side arrays hold one 16 x 16 product tile");
  static_assert(SUMS * 4 >= 16 * 32 * kMaxKs * 2, "the pair-sum buffers hold 16 rows of s_p parts");
};

// the 16-byte chunk c of z row r sits at chunk position c ^ (r & 7) of its
// LDS row, so the 16 rows of one fragment read spread over the banks
__device__ __forceinline__ int zswz(int r, int c) { return c ^ (r & 7); }

// staged arrays: row r's float4 group g (units 4g .. 4g+3) sits at group
// g ^ ((r >> 3) & 1), so the eight rows one grid read touches fall on
// distinct banks
__device__ __forceinline__ int sidx(int r, int h) { return r * (kUW + 4) + (((h >> 2) ^ ((r >> 3) & 1)) << 2) + (h & 3); }

__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
}

template <typename SS, bool CHIP>
__global__ void __launch_bounds__(256, SS::KR == 16 ? 3 : 1) score_slab_kernel(SlabDev g) {
  constexpr int KR = SS::KR, TA = SS::TA, RT = SS::RT, ARR = SS::ARR, NBUF = SS::NBUF, NKS = SS::NKS;
  __shared__ __align__(1024) char zb0[SS::ZBUF];
  __shared__ __align__(1024) char zb1[SS::ZBUF];
  __shared__ __align__(16) float smem[SS::STAGE];
  __shared__ __align__(16) float sums[SS::SUMS];   // [pair p % NBUF][wave][KR * KR]
  __shared__ __align__(16) float csum[CHIP ? SS::CSUM : 4];   // [wave][pair - t0][unit]: W1s s_p summed

  const int tid = threadIdx.x;
  const int l = tid & 63;
  const int wv = tid >> 6;
  const int K = g.K;
  const int H = g.H;
  constexpr int rz = NKS * 32;
  const int B = g.B;
  const int Bm1 = B - 1;
  // workgroups are dealt to the 8 XCDs in turn (blockIdx % 8); when the
  // grid divides evenly, XCD x takes a contiguous run of the work items
  // (block, chunk, slab), slab fastest, so the slabs of one chunk share that
  // XCD's L2 copy of the chunk's z rows
  const int G = static_cast<int>(gridDim.x);
  int li = static_cast<int>(blockIdx.x);
  if (G % 8 == 0) li = (li % 8) * (G / 8) + li / 8;
  const int slab = li % g.nslab;
  li /= g.nslab;
  const int chunk = li % g.nchunk;
  const int n = li / g.nchunk;
  const int t0 = chunk * g.pc;                   // first slot: pair t0 is the chunk's first
  const int t1 = min(t0 + g.pc, Bm1);            // last slot: pair t1 - 1 is the chunk's last
  constexpr int rowb = rz * 2;                   // bytes of one z row

  // grid layout of this lane: outputs (la TA + i, lb TA + j)
  const int la = l / (KR / TA);
  const int lb = l % (KR / TA);
  // MFMA layout: unit fr of the wave's 16, candidate rows 4 fq + v of each
  // 16-row tile; fragment row fr, k chunk fq
  const int fr = l & 15;
  const int fq = l >> 4;

  float* wreg = smem + wv * SS::WREG;
  float* sEA = wreg;                 // 2^A' (or A')
  float* sWA = wreg + ARR;           // w'A'
  float* sEB = wreg + 2 * ARR;       // 2^B' (or B')
  float* sWB = wreg + 3 * ARR;       // w'B'
  float* sWq = wreg + 4 * ARR;       // w' per unit (per-element form)
  float* cs = csum + wv * kChipPairs * kUW;   // on-chip pair term, summed: [pair - t0][unit]

  // ---- this lane's unit
  const int u = slab * kUS + wv * kUW + fr;
  const int uc = min(u, H - 1);
  const bool uin = u < H;

  // ---- z rows of slot t into zb[t & 1] (KR rows; rows past K repeat row K-1)
  const long long zrow0 = static_cast<long long>(n) * B * K;
  const int ninst = KR * rowb / 1024;            // 1 KB direct loads per slot
  auto issue_z = [&](int t) {
    char* dst = (t & 1) ? zb1 : zb0;
    for (int j = wv; j < ninst; j += 4) {
      const int byte = j * 1024 + l * 16;
      const int r = byte / rowb;
      const int pc = (byte - r * rowb) >> 4;
      const int c = zswz(r, pc);
      const long long srow = zrow0 + static_cast<long long>(t) * K + min(r, K - 1);
      dma16(g.z + srow * rz + c * 8, __builtin_amdgcn_readfirstlane(lds_offset(dst) + j * 1024));
    }
  };

  // the parts of C_p for this lane's unit, pair p of the block (0 <= p < B - 1):
  // loaded unconditionally (part indices clamped to the parts there are) and
  // added only after the step's explicit wait, so no load is waited on early
  float cr[3];
  auto load_c = [&](int p) {
    const long long np = static_cast<long long>(n) * Bm1 + p;
#pragma unroll
    for (int q = 0; q < 3; ++q) cr[q] = g.C[(min(q, g.nq - 1) * static_cast<long long>(g.P) + np) * H + uc];
  };
  // C_p + b1, parts added in order (the loads have landed)
  auto sum_c = [&](float bb) -> float {
#pragma unroll
    for (int q = 0; q < 3; ++q) asm volatile("" : "+v"(cr[q]));
    float c = cr[0];
    if (g.nq > 1) c += cr[1];
    if (g.nq > 2) c += cr[2];
    return c + bb;
  };

  // every load of the prologue in flight at once: slot t0's rows, C of pair
  // t0, the W1a and W1b fragments of every k step, w2 and b1
  issue_z(t0);
  if constexpr (!CHIP) load_c(t0);
  // on chip: the chunk's bf16 parts of s_p, operand row r = (part q, pair
  // t0 + i) at q np + i (rows from 3 np on repeat row 0 and are never read),
  // copied once into the pair-sum buffers (first written at step t0 + 1);
  // 16-byte chunk c of row r at position c ^ (r & 7) when rows hold a
  // multiple of eight chunks
  const int np = t1 - t0;
  const int nks_s = g.rs >> 5;
  const int rowb_s = g.rs * 2;
  const int smask = (g.rs & 63) == 0 ? 7 : 0;
  if constexpr (CHIP) {
    for (int j = wv; j < nks_s; j += 4) {          // 16 rows x rs x 2 bytes = rs / 32 KB
      const int byte = j * 1024 + l * 16;
      const int r = byte / rowb_s;
      const int c = ((byte - r * rowb_s) >> 4) ^ (r & smask);
      const int rr = r < 3 * np ? r : 0;
      const int q = rr / np;
      const uint16_t* src = g.s3 + q * g.s3_part + (static_cast<long long>(n) * Bm1 + t0 + (rr - q * np)) * g.rs;
      dma16(src + c * 8, __builtin_amdgcn_readfirstlane(lds_offset(sums) + j * 1024));
    }
  }
  // W1a and W1b rows of the wave's 16 units, loaded with the four 16-byte
  // quarters of a unit's 64-byte slice of each k step in adjacent lanes
  // (lane 4 v + q: unit v, quarter q), so each group of four lanes reads one
  // contiguous segment; the fragments are moved into the MFMA layout below.
  // (Whole 128-byte lines per eight lanes measured slower.)  W1b is first
  // needed at step t0 + 1, so its loads are issued last and waited on at the
  // end of step t0.
  using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;
  u32x4 ra[NKS], rb[NKS];
  const uint16_t* wsrc = g.W1 + static_cast<long long>(min(slab * kUS + wv * kUW + (l >> 2), H - 1)) * g.ldw1 +
                         (l & 3) * 8;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) ra[ks] = *reinterpret_cast<const u32x4*>(wsrc + ks * 32);
  uint32_t w2b = g.w2[uc];
  uint32_t b1b = (g.b1 ? g.b1 : g.w2)[uc];
  // on chip: the W1s rows of the wave's units, as W1a (k steps past r_s
  // repeat the last)
  u32x4 rw[CHIP ? kMaxKs : 1];
  if constexpr (CHIP) {
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) rw[ks] = *reinterpret_cast<const u32x4*>(wsrc + 2 * rz + min(ks, nks_s - 1) * 32);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) rb[ks] = *reinterpret_cast<const u32x4*>(wsrc + rz + ks * 32);
  // every load but the W1b ones has landed (loads complete in issue order)
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(NKS) : "memory");
  // the compiler does not see the wait above: passing a loaded register
  // through an empty asm ends its tracking of that load there, so it never
  // waits on it again inside the loop (where that wait would also cover the
  // loads issued there)
  asm volatile("" : "+v"(w2b), "+v"(b1b));
  if constexpr (CHIP) {
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) asm volatile("" : "+v"(rw[ks]));
  }
  // MFMA B fragments: lane l holds unit l & 15, k chunk l >> 4 of each k
  // step, which lane 4 (l & 15) + (l >> 4) loaded
  bf16x8_t wa[NKS], wb[NKS];
  auto gather = [&](u32x4 (&r)[NKS], bf16x8_t (&w)[NKS]) {
    const int from = 4 * (4 * fr + fq);   // byte index of the source lane
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      asm volatile("" : "+v"(r[ks]));
      u32x4 x;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        x[d] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(r[ks][d])));
      w[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
  };
  gather(ra, wa);
  const float wq = uin ? kNegLn2 * bf16_to_f32(static_cast<uint16_t>(w2b)) : 0.f;
  const float bb = g.b1 ? bf16_to_f32(static_cast<uint16_t>(b1b)) : 0.f;
  if (l < kUW) sWq[l] = wq;          // lane l < 16 holds unit l of the wave's 16
  // C of the pair completed at the next step
  float c_prev = CHIP ? 0.f : sum_c(bb);
  bool slow_prev = false;            // that pair takes the per-element form (wave-uniform)
  __syncthreads();                   // slot t0's rows, the w' table (and the s_p parts) are in LDS
  if constexpr (CHIP) {
    // the parts of W1s s_p: one 16 x 16 tile (rows: part and pair; columns:
    // the wave's units) on MFMA, staged in the wave's B-side arrays (next
    // written by this wave's first grid), then added per pair and unit in
    // part order
    const char* sp = reinterpret_cast<const char*>(sums);
    f32x4_t accC = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int from = 4 * (4 * fr + fq);
#pragma unroll
    for (int ks = 0; ks < kMaxKs; ++ks) {
      if (ks < nks_s) {
        u32x4 x;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          x[d] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(rw[ks][d])));
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(sp + fr * rowb_s + (((ks * 4 + fq) ^ (fr & smask)) << 4)));
        accC = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, x), accC, 0, 0, 0);
      }
    }
    float* tc = sEB;
#pragma unroll
    for (int v = 0; v < 4; ++v) tc[(4 * fq + v) * kUW + fr] = accC[v];
    wave_lds_sync();
    for (int e = l; e < np * kUW; e += kWave) {
      const int i = e / kUW, uu = e % kUW;
      float c = tc[i * kUW + uu];
      c += tc[(np + i) * kUW + uu];
      c += tc[(2 * np + i) * kUW + uu];
      cs[e] = c;
    }
    wave_lds_sync();
    c_prev = cs[fr] + bb;
  }

  // the slab's sum of pair p: the four waves added in order
  const int kk = K * K;
  auto store_pair = [&](int p) {
    const float* sb = sums + (p % NBUF) * 4 * KR * KR;
    float* dst = g.part + (static_cast<long long>(slab) * g.P + static_cast<long long>(n) * Bm1 + p) * kk;
    for (int i = tid; i < kk; i += 256) {
      const int a = i / K;
      const int o = a * KR + (i - a * K);
      float sum = sb[o];
#pragma unroll
      for (int w = 1; w < 4; ++w) sum += sb[w * KR * KR + o];
      dst[i] = sum;
    }
  };

  // A_t = W1a z_t and / or B_t = W1b z_t for the wave's 16 units
  auto form = [&](auto DA, auto DB, const char* zt, f32x4_t (&accA)[RT], f32x4_t (&accB)[RT]) {
    constexpr bool kA = decltype(DA)::value, kB = decltype(DB)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      accA[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accB[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = rt * 16 + fr;
        const bf16x8_t x = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(zt + r * rowb + zswz(r, ks * 4 + fq) * 16));
        if constexpr (kA) accA[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, wa[ks], accA[rt], 0, 0, 0);
        if constexpr (kB) accB[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, wb[ks], accB[rt], 0, 0, 0);
      }
    }
  };

  // pair p: its successor side from B_{p+1} (cq = -log2(e) (C_p + b1)), then
  // its grid; the wave's sum is left in LDS for the workgroup to add up
  auto finish_pair = [&](int p, float cq, const f32x4_t (&accB)[RT]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float bp = fmaf(kNegLog2e, accB[rt][v], cq);
        const int o = sidx(rt * 16 + fq * 4 + v, fr);
        const float e = __builtin_amdgcn_exp2f(bp);
        sEB[o] = slow_prev ? bp : e;
        sWB[o] = wq * bp;
      }
    wave_lds_sync();
    float acc[TA][TA];
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
      for (int j = 0; j < TA; ++j) acc[i][j] = 0.f;
    if (!slow_prev) {
      for (int h = 0; h < kUW; h += 4) {
        float4 ea[TA], wa4[TA], eb[TA], wb4[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          ea[i] = *reinterpret_cast<const float4*>(sEA + sidx(la * TA + i, h));
          wa4[i] = *reinterpret_cast<const float4*>(sWA + sidx(la * TA + i, h));
          eb[i] = *reinterpret_cast<const float4*>(sEB + sidx(lb * TA + i, h));
          wb4[i] = *reinterpret_cast<const float4*>(sWB + sidx(lb * TA + i, h));
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int i = 0; i < TA; ++i)
#pragma unroll
            for (int j = 0; j < TA; ++j) {
              const float den = fmaf(ea[i][c4], eb[j][c4], 1.0f);
              const float r = __builtin_amdgcn_rcpf(den);
              acc[i][j] = fmaf(wa4[i][c4] + wb4[j][c4], r, acc[i][j]);
            }
      }
    } else {
      for (int h = 0; h < kUW; h += 4) {
        float4 av[TA], bv[TA];
#pragma unroll
        for (int i = 0; i < TA; ++i) {
          av[i] = *reinterpret_cast<const float4*>(sEA + sidx(la * TA + i, h));
          bv[i] = *reinterpret_cast<const float4*>(sEB + sidx(lb * TA + i, h));
        }
        const float4 w4 = *reinterpret_cast<const float4*>(sWq + h);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int i = 0; i < TA; ++i)
#pragma unroll
            for (int j = 0; j < TA; ++j) {
              const float tt = av[i][c4] + bv[j][c4];
              const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(tt));
              acc[i][j] = fmaf(w4[c4], tt * r, acc[i][j]);
            }
      }
    }
    float* ws = sums + ((p % NBUF) * 4 + wv) * KR * KR;
#pragma unroll
    for (int i = 0; i < TA; ++i)
#pragma unroll
      for (int j = 0; j < TA; ++j) ws[(la * TA + i) * KR + lb * TA + j] = acc[i][j];
  };

  // pair t: its predecessor side from A_t (and whether it takes the
  // per-element form)
  auto start_pair = [&](const f32x4_t (&accA)[RT]) {
    float ap[RT][4];
    bool big = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        ap[rt][v] = kNegLog2e * accA[rt][v];
        big |= fabsf(ap[rt][v]) > 64.f;
      }
    slow_prev = __builtin_amdgcn_ballot_w64(big) != 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = sidx(rt * 16 + fq * 4 + v, fr);
        const float e = __builtin_amdgcn_exp2f(ap[rt][v]);
        sEA[o] = slow_prev ? ap[rt][v] : e;
        sWA[o] = wq * ap[rt][v];
      }
  };

  using kYes = std::true_type;
  using kNo = std::false_type;
  // ---- step t0: A_t0 only (B_t0 would complete a pair outside the chunk);
  // every chunk has a pair, so slot t0 + 1 exists
  {
    issue_z(t0 + 1);
    f32x4_t accA[RT], accB[RT];
    form(kYes{}, kNo{}, (t0 & 1) ? zb1 : zb0, accA, accB);
    start_pair(accA);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // slot t0 + 1's rows, the W1b rows
    gather(rb, wb);
    __syncthreads();
  }
  // ---- steps t0 + 1 .. t1 - 1: B_t completes pair t - 1, A_t starts pair t
  for (int t = t0 + 1; t < t1; ++t) {
    const char* zt = (t & 1) ? zb1 : zb0;
    issue_z(t + 1);                  // the other buffer was last read at step t - 1
    // pair t - 2 was finished at step t - 1; its buffer is next written at step t + 1
    if (NBUF == 2 && t >= t0 + 2) store_pair(t - 2);
    const float cq = kNegLog2e * c_prev;   // pair t - 1
    if constexpr (!CHIP) load_c(t);        // pair t, used at step t + 1
    f32x4_t accA[RT], accB[RT];
    form(kYes{}, kYes{}, zt, accA, accB);
    finish_pair(t - 1, cq, accB);
    start_pair(accA);
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // slot t + 1's rows (this wave's share)
    c_prev = CHIP ? cs[(t - t0) * kUW + fr] + bb : sum_c(bb);
    __syncthreads();                                       // ... and every other wave's
  }
  // ---- step t1: B_t1 only (A_t1 would start a pair outside the chunk)
  {
    if (NBUF == 2 && t1 >= t0 + 2) store_pair(t1 - 2);
    const float cq = kNegLog2e * c_prev;   // pair t1 - 1
    f32x4_t accA[RT], accB[RT];
    form(kNo{}, kYes{}, (t1 & 1) ? zb1 : zb0, accA, accB);
    finish_pair(t1 - 1, cq, accB);
    __syncthreads();                 // every wave's sum of pair t1 - 1 is in LDS
  }
  // the last pair (and, with one buffer, the only one)
  store_pair(t1 - 1);
}

// S_p(a, b) = l_{p+1}(b) + (sum of the slabs' partial sums, in slab order) + b2,
// and best_p(a) = argmax_b S_p(a, b) (largest order key, the lowest b among
// equal keys; NaN never wins).  One workgroup per pair.
template <int KR>
__global__ void __launch_bounds__(256)
pair_finish_kernel(const float* __restrict__ part, int nslab, int P, int B, int K, float b2,
                   const float* __restrict__ cand_logits, float* __restrict__ S, int32_t* __restrict__ best) {
  constexpr int kPerT = (KR * KR + 255) / 256;
  __shared__ float sS[KR * KR];
  const int np = blockIdx.x;
  const int tid = threadIdx.x;
  const int Bm1 = B - 1;
  const int n = np / Bm1;
  const int p = np - n * Bm1;
  const int kk = K * K;
  const float* lnext = cand_logits + (static_cast<long long>(n) * B + p + 1) * K;
  float sum[kPerT];
#pragma unroll
  for (int i = 0; i < kPerT; ++i) sum[i] = 0.f;
  // four slabs' loads in flight at once (slab and index clamped, masked after)
  for (int s0 = 0; s0 < nslab; s0 += 4) {
    float v[4][kPerT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int idx = min(tid + 256 * i, kk - 1);
        v[q][i] = part[(static_cast<long long>(min(s0 + q, nslab - 1)) * P + np) * kk + idx];
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < kPerT; ++i)
        if (s0 + q < nslab) sum[i] = (s0 + q == 0) ? v[q][i] : sum[i] + v[q][i];
  }
  float* Sp = S + static_cast<long long>(np) * kk;
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < kk) {
      const int a = idx / K;
      const int b = idx - a * K;
      const float sv = lnext[b] + (sum[i] + b2);
      Sp[idx] = sv;
      sS[a * KR + b] = sv;
    }
  }
  if (best == nullptr) return;
  __syncthreads();
  if (tid < K) {
    const float* row = sS + tid * KR;
    uint32_t bk = order_key(row[0]);
    int bi = 0;
    for (int b = 1; b < K; ++b) {
      const uint32_t k2 = order_key(row[b]);
      if (k2 > bk) {
        bk = k2;
        bi = b;
      }
    }
    best[static_cast<long long>(np) * K + tid] = bi;
  }
}

// One workgroup per block: the finish of all its pairs, then the walk
// (review of arXiv 2610.12570, "Contextual Correction of Parallel Drafts for
// Speculative Decoding", part 2 of "New approach: DCOCO", paper Sec. 3.3),
// in one launch and without any workgroup waiting for another.  The threads
// take the block's outputs o = p K^2 + a K + b in groups of VEC (VEC = 4 when
// K^2 is a multiple of 4, so every group is one aligned 16-byte load per
// slab): S_p(a, b) = l_{p+1}(b) + (the slabs' sums in slab order) + b2 is
// stored and kept in LDS; then best_p(a) = argmax_b S_p(a, b) for every
// (p, a) (largest order key, lowest b among equal keys); then wave 0 follows
// k_0 = argmax_a l_0(a), k_{p+1} = best_p(k_p) and the chosen ids are written.
// The sums are the same, in the same order, as the per-pair finish above.
constexpr int kBlkThreads = 1024;
constexpr int kBlkSlabs = 8;         // slab loads in flight per group
constexpr int kBlkScores = 16384;    // scores of one block staged in LDS: (B - 1) K^2
constexpr int kBlkTab = 2048;        // walk table entries: (B - 1) K
// the staged rows are (K | 1) apart: at most (B - 1) K and B - 1 more entries
constexpr int kBlkScoresPad = kBlkScores + kBlkTab;
constexpr int kBlkTabPad = kBlkTab + 512;
constexpr int kBlkMaxB = 512;        // slots per block
constexpr int kBlkIds = kBlkTab + kWave;   // candidate ids of a block: B K <= (B - 1) K + K
constexpr int kBlkIdsPerT = (kBlkIds + kBlkThreads - 1) / kBlkThreads;
constexpr long long kBlkPartBytes = 256 * 1024;   // partial sums one workgroup reads

template <int VEC>
__device__ __forceinline__ void blk_load(const float* p, float (&v)[VEC]) {
  if constexpr (VEC == 4) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    v[0] = *p;
  }
}

template <int VEC>
__global__ void __launch_bounds__(kBlkThreads)
block_finish_walk_kernel(const float* __restrict__ part, int nslab, int P, int B, int K, float b2,
                         const float* __restrict__ cand_logits, const int32_t* __restrict__ cand_ids,
                         float* __restrict__ S, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_tok) {
  __shared__ float sS[kBlkScoresPad];
  __shared__ int32_t sT[kBlkTabPad];
  __shared__ int32_t sK[kBlkMaxB];
  __shared__ int32_t sId[kBlkIds];
  __shared__ float sC0[kWave];
  const int n = blockIdx.x;
  const int tid = threadIdx.x;
  const int Bm1 = B - 1;
  const int kk = K * K;
  const int tot = Bm1 * kk;   // this block's scores, a multiple of VEC
  const int srow = K | 1;     // LDS stride of a score row and a table row: odd
  const int ng = tot / VEC;
  const long long np0 = static_cast<long long>(n) * Bm1;
  const long long slab_stride = static_cast<long long>(P) * kk;
  const float* pb = part + np0 * kk;
  // the block's candidate ids and slot 0's logits are loaded now, with the
  // sums, and put in LDS once the sums are done (indices clamped)
  const int nid = B * K;
  const int32_t* idn = cand_ids + static_cast<long long>(n) * nid;
  int32_t idv[kBlkIdsPerT];
#pragma unroll
  for (int i = 0; i < kBlkIdsPerT; ++i) idv[i] = idn[min(tid + i * kBlkThreads, nid - 1)];
  const float c0v = cand_logits[static_cast<long long>(n) * nid + min(tid, K - 1)];
  for (int g = tid; g < ng; g += kBlkThreads) {
    float ln[VEC];   // l_{p+1}(b) of the group's outputs, loaded before the sums
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int o = g * VEC + i;
      ln[i] = cand_logits[(static_cast<long long>(n) * B + o / kk + 1) * K + o % K];
    }
    float sum[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) sum[i] = 0.f;
    for (int s0 = 0; s0 < nslab; s0 += kBlkSlabs) {
      float v[kBlkSlabs][VEC];
#pragma unroll
      for (int q = 0; q < kBlkSlabs; ++q)   // slab clamped, its value masked below
        blk_load<VEC>(pb + min(s0 + q, nslab - 1) * slab_stride + static_cast<long long>(g) * VEC, v[q]);
#pragma unroll
      for (int q = 0; q < kBlkSlabs; ++q)
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          if (s0 + q < nslab) sum[i] = (s0 + q == 0) ? v[q][i] : sum[i] + v[q][i];
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const int o = g * VEC + i;
      const float sv = ln[i] + (sum[i] + b2);
      S[np0 * kk + o] = sv;
      sS[(o / K) * srow + o % K] = sv;
    }
  }
#pragma unroll
  for (int i = 0; i < kBlkIdsPerT; ++i)
    if (tid + i * kBlkThreads < nid) sId[tid + i * kBlkThreads] = idv[i];
  if (tid < K) sC0[tid] = c0v;
  __syncthreads();
  // the walk's table: best_p(a) for every (p, a) of the block, one thread
  // per row (the odd row stride keeps the threads' reads on distinct banks)
  for (int r = tid; r < Bm1 * K; r += kBlkThreads) {
    const float* row = sS + r * srow;
    uint32_t bk = order_key(row[0]);
    int bi = 0;
    for (int b = 1; b < K; ++b) {
      const uint32_t k2 = order_key(row[b]);
      if (k2 > bk) {
        bk = k2;
        bi = b;
      }
    }
    sT[(r / K) * srow + r % K] = bi;
  }
  __syncthreads();
  if (tid < kWave) {
    const int l = tid;
    const uint32_t key = l < K ? order_key(sC0[l]) : 0u;   // lanes >= K carry the NaN key
    int k = __builtin_ctzll(ballot(key == wave_max_u32_dpp(key)));   // lowest index among the largest keys
    if (l == 0) {
      sK[0] = k;
      for (int p = 0; p < Bm1; ++p) {
        k = min(max(sT[p * srow + k], 0), K - 1);
        sK[p + 1] = k;
      }
    }
  }
  __syncthreads();
  for (int j = tid; j < B; j += kBlkThreads) {
    const int kj = sK[j];
    const long long o = static_cast<long long>(n) * B + j;
    if (sel_idx) sel_idx[o] = kj;
    sel_tok[o] = sId[j * K + kj];
  }
}

}  // namespace

constexpr long long kSlabSlots = 3 * 256;   // resident K <= 16 slab workgroups: three on each of 256 CUs

bool score_slab_supported(int dtype, int K, int rz, int H) {
  return dtype == kDtypeBf16 && K >= 1 && K <= 32 && (rz == 64 || rz == 128 || rz == 256) && H >= 16 &&
         H % 16 == 0;
}

int score_slab_count(int H) { return (H + kUS - 1) / kUS; }

// One workgroup holds a block's scores and table in LDS, and reads no more
// than kBlkPartBytes of partial sums: beyond that the per-pair finish, spread
// over every pair, and the separate walk finish first.
bool block_finish_walk_fits(int B, int K, int H) {
  const long long tot = static_cast<long long>(B - 1) * K * K;
  return B >= 2 && K >= 1 && K <= kWave && B <= kBlkMaxB && tot <= kBlkScores &&
         static_cast<long long>(B - 1) * K <= kBlkTab &&
         tot * score_slab_count(H) * static_cast<long long>(sizeof(float)) <= kBlkPartBytes;
}

// For K <= 16 the slab kernels scored faster than the A, B GEMM and the grid
// kernel at every block count measured (16 to 96 blocks of B = 16, K = 16,
// H = 512, r_z = 256: 130 against 133 us per call at 32 blocks, 326 against
// 352 at 96); they are taken while one chunk per block keeps the launch within
// one resident round (blocks x slabs <= 768), the largest count measured.
// For K > 16 (one pair per workgroup) up to about 40M grid elements
// (P K^2 H), as measured for the earlier K <= 16 form.
bool score_slab_preferred(int dtype, int N, int B, int K, int rz, int H) {
  if (!score_slab_supported(dtype, K, rz, H)) return false;
  if (K <= 16) return static_cast<long long>(N) * score_slab_count(H) <= kSlabSlots;
  const double elems = static_cast<double>(N) * (B - 1) * K * K * H;
  return elems <= 40.0e6;
}

size_t score_slab_part_bytes(int N, int B, int K, int H) {
  const long long P = static_cast<long long>(N) * (B - 1);
  return sizeof(float) * static_cast<size_t>(score_slab_count(H)) * static_cast<size_t>(P > 0 ? P : 0) *
         static_cast<size_t>(K) * static_cast<size_t>(K);
}

// pairs per chunk: for K <= 16 as many chunks as keep every resident
// workgroup slot busy for one round (three workgroups per CU), each at least
// one pair; for K > 16 one pair per chunk (one pair-sum buffer)
int score_slab_pairs_per_chunk(int N, int B, int K, int H) {
  const int Bm1 = B - 1;
  if (Bm1 < 1 || K > 16) return 1;
  const long long wg = static_cast<long long>(N) * score_slab_count(H);
  long long chunks = kSlabSlots / wg;
  if (chunks > Bm1) chunks = Bm1;
  if (chunks < 1) chunks = 1;
  return static_cast<int>((Bm1 + chunks - 1) / chunks);
}

// The pair term is formed inside the slab launch when every chunk has at
// most five pairs (its three bf16 parts per pair fill at most one 16-row
// MFMA tile) and r_s is a whole number of 32-deep k steps, at most 256.
bool score_slab_c_on_chip(int N, int B, int K, int H, int rs) {
  return B >= 2 && rs >= 32 && rs <= 32 * kMaxKs && rs % 32 == 0 &&
         score_slab_pairs_per_chunk(N, B, K, H) <= kChipPairs;
}

hipError_t launch_score_slab(const ScoreSlabProblem& q, hipStream_t st) {
  const int Bm1 = q.B - 1;
  const int P = q.N * Bm1;
  if (P <= 0) return hipSuccess;
  if (!score_slab_supported(kDtypeBf16, q.K, q.rz, q.H)) return hipErrorInvalidValue;
  const bool chip = q.s3 != nullptr;
  if (chip ? !score_slab_c_on_chip(q.N, q.B, q.K, q.H, q.rs) : q.C == nullptr) return hipErrorInvalidValue;
  SlabDev d;
  d.N = q.N; d.B = q.B; d.K = q.K; d.H = q.H; d.P = P; d.rz = q.rz; d.nq = q.nq;
  d.nslab = score_slab_count(q.H);
  d.pc = score_slab_pairs_per_chunk(q.N, q.B, q.K, q.H);
  d.nchunk = (Bm1 + d.pc - 1) / d.pc;
  d.z = static_cast<const uint16_t*>(q.z);
  d.W1 = static_cast<const uint16_t*>(q.W1);
  d.ldw1 = q.ldw1;
  d.C = chip ? nullptr : q.C;
  d.s3 = static_cast<const uint16_t*>(q.s3);
  d.s3_part = static_cast<long long>(P) * q.rs;
  d.rs = q.rs;
  d.b1 = static_cast<const uint16_t*>(q.b1);
  d.w2 = static_cast<const uint16_t*>(q.w2);
  d.part = q.part;
  const dim3 grid(static_cast<unsigned>(q.N) * d.nslab * d.nchunk);
#define DCOCO_SLAB_C(KRV, NKSV)                                                                         \
  if (chip) hipLaunchKernelGGL((score_slab_kernel<SlabShape<KRV, NKSV>, true>), grid, dim3(256), 0, st, d); \
  else hipLaunchKernelGGL((score_slab_kernel<SlabShape<KRV, NKSV>, false>), grid, dim3(256), 0, st, d)
#define DCOCO_SLAB(KRV)                        \
  if (q.rz == 64) { DCOCO_SLAB_C(KRV, 2); }     \
  else if (q.rz == 128) { DCOCO_SLAB_C(KRV, 4); } \
  else { DCOCO_SLAB_C(KRV, 8); }
  if (q.K <= 16) { DCOCO_SLAB(16) }
  else { DCOCO_SLAB(32) }
#undef DCOCO_SLAB
#undef DCOCO_SLAB_C
  if (q.sel_tok != nullptr) {
    // the finish of a whole block and its walk in one workgroup
    if (q.cand_ids == nullptr || !block_finish_walk_fits(q.B, q.K, q.H)) return hipErrorInvalidValue;
    if ((q.K * q.K) % 4 == 0)
      hipLaunchKernelGGL((block_finish_walk_kernel<4>), dim3(q.N), dim3(kBlkThreads), 0, st, q.part, d.nslab, P,
                         q.B, q.K, q.b2, q.cand_logits, q.cand_ids, q.S, q.sel_idx, q.sel_tok);
    else
      hipLaunchKernelGGL((block_finish_walk_kernel<1>), dim3(q.N), dim3(kBlkThreads), 0, st, q.part, d.nslab, P,
                         q.B, q.K, q.b2, q.cand_logits, q.cand_ids, q.S, q.sel_idx, q.sel_tok);
  } else if (q.K <= 16) {
    hipLaunchKernelGGL((pair_finish_kernel<16>), dim3(P), dim3(256), 0, st, q.part, d.nslab, P, q.B, q.K, q.b2,
                       q.cand_logits, q.S, q.best);
  } else {
    hipLaunchKernelGGL((pair_finish_kernel<32>), dim3(P), dim3(256), 0, st, q.part, d.nslab, P, q.B, q.K, q.b2,
                       q.cand_logits, q.S, q.best);
  }
  return hipGetLastError();
}

}  // namespace dcoco
