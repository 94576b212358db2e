// Top-K candidate extraction over logit rows ([P1] "Keep the leading
// candidates"; [P2] part 1, paper Sec. 3.2).  P1 = Two Delta, "Two Delta
// makes NVIDIA Nemotron 3.5 Super even faster with DCOCO"; P2 = review of
// arXiv 2610.12570, "Contextual Correction of Parallel Drafts for Speculative
// Decoding".
//
// Order: value descending under order_key() (-0 == +0, NaN below -inf), equal
// values to the lower id.  Every element carries a 64-bit composite
// (key << 32) | (0xffffffff - id); composites are unique, so "the K largest
// composites" is exactly the wanted set, whatever the ties.
//
// Design (HBM-bound scan; each logit is read once):
//   * a row is split into chunks of 4 wave segments; one workgroup (4 waves)
//     per (row, chunk).  A wave segment is 64 lanes x 8 x 16-byte vectors, read
//     with coalesced 16-byte loads and kept in registers as keys;
//   * each lane keeps the maximum key of G groups of its vectors.  The K-th
//     largest of those 64*G group maxima is a lower bound T0 of the segment's
//     K-th largest key (K distinct elements reach it), so only elements with
//     key >= T0 can be in the segment's top-K.  On random rows that leaves about
//     K + a few candidates, appended to LDS;
//   * an exact radix selection (bit by bit, ballot counts) over the few
//     candidates picks the segment's top-K; the 4 waves' results are merged the
//     same way and the workgroup writes K composites per chunk;
//   * if a segment has more than kCandCap candidates (long runs of equal
//     values), the wave selects exactly from its registers instead;
//   * a second kernel merges the chunks of a row, sorts the K winners and
//     writes ids and the original logit values.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace dcoco {

namespace {

constexpr int kTopkWaves = 4;
constexpr int kTopkThreads = kTopkWaves * kWave;
constexpr int kVecPerLane = 8;
constexpr int kCandCap = 256;   // candidates a wave may append before it falls back

template <typename T>
struct TopkShape {
  static constexpr int kVec = Elem<T>::kPer16B;
  static constexpr int kEPL = kVecPerLane * kVec;
  static constexpr int kSeg = kWave * kEPL;
  static constexpr int kChunk = kTopkWaves * kSeg;
  static constexpr int kKeyBits = sizeof(T) * 8;
};

__device__ __forceinline__ uint32_t comp_key(uint64_t c) { return static_cast<uint32_t>(c >> 32); }
__device__ __forceinline__ uint32_t comp_inv(uint64_t c) { return static_cast<uint32_t>(c); }
__device__ __forceinline__ uint64_t make_comp(uint32_t key, uint32_t id) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - id);
}

// Exact top-K of the composites c[0..Q) held by the lanes of one wave (0 =
// empty slot); KEYBITS is the width of the key half.  Marks the
// min(K, #non-empty) largest in sel[].
template <int Q, int KEYBITS>
__device__ void select_topk(const uint64_t (&c)[Q], int K, bool (&sel)[Q]) {
  uint32_t tk = 0;
  for (int bit = KEYBITS - 1; bit >= 0; --bit) {
    const uint32_t cand = tk | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) cnt += __popcll(ballot(c[q] != 0 && comp_key(c[q]) >= cand));
    if (cnt >= K) tk = cand;
  }
  int ngt = 0, neq = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const bool v = c[q] != 0;
    ngt += __popcll(ballot(v && comp_key(c[q]) > tk));
    neq += __popcll(ballot(v && comp_key(c[q]) == tk));
  }
  const int need = K - ngt;
  uint32_t ti = 0;
  if (neq > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = ti | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < Q; ++q)
        cnt += __popcll(ballot(c[q] != 0 && comp_key(c[q]) == tk && comp_inv(c[q]) >= cand));
      if (cnt >= need) ti = cand;
    }
  }
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint32_t k = comp_key(c[q]);
    sel[q] = c[q] != 0 && (k > tk || (k == tk && comp_inv(c[q]) >= ti));
  }
}

// Select the top-K of src[0..count) (count <= 64*Q) and write them, in any
// order, to dst[0..K) padded with zeros.  Executed by one whole wave.
template <int Q, int KEYBITS>
__device__ void select_to(const uint64_t* src, int count, int K, uint64_t* dst) {
  const int l = lane_id();
  uint64_t c[Q];
  bool sel[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = q * kWave + l;
    c[q] = i < count ? src[i] : 0ull;
  }
  select_topk<Q, KEYBITS>(c, K, sel);
  int base = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t m = ballot(sel[q]);
    if (sel[q]) dst[base + lanes_below(m)] = c[q];
    base += __popcll(m);
  }
  for (int i = base + l; i < K; i += kWave) dst[i] = 0ull;
}

template <int KEYBITS>
__device__ void select_small(const uint64_t* src, int count, int K, uint64_t* dst) {
  if (count <= kWave)
    select_to<1, KEYBITS>(src, count, K, dst);
  else if (count <= 2 * kWave)
    select_to<2, KEYBITS>(src, count, K, dst);
  else
    select_to<4, KEYBITS>(src, count, K, dst);
}

template <typename T, bool kVecLoad>
__global__ void __launch_bounds__(kTopkThreads)
topk_partial_kernel(const T* __restrict__ logits, int V, int K, int nchunks,
                    uint64_t* __restrict__ partial) {
  using S = TopkShape<T>;
  constexpr int kVec = S::kVec;
  const int chunk = blockIdx.x;
  const int row = blockIdx.y;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const T* rowp = logits + static_cast<size_t>(row) * V;

  __shared__ uint64_t s_cand[kTopkWaves][kCandCap];
  __shared__ uint64_t s_best[kTopkWaves * 64];
  __shared__ int s_cnt[kTopkWaves];

  const int seg0 = chunk * S::kChunk + w * S::kSeg;
  if (l == 0) s_cnt[w] = 0;

  uint64_t* wave_out = s_best + w * K;
  if (seg0 < V) {
    // ---- load the segment and turn it into keys (padding -> key 0, skipped)
    uint32_t key[kVecPerLane][kVec];
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i) {
      const int e0 = seg0 + (i * kWave + l) * kVec;
      if (kVecLoad && e0 + kVec <= V) {
        union { uint4 u; T t[kVec]; } v;
        v.u = *reinterpret_cast<const uint4*>(rowp + e0);
#pragma unroll
        for (int j = 0; j < kVec; ++j) key[i][j] = order_key(v.t[j]);
      } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) key[i][j] = (e0 + j < V) ? order_key(rowp[e0 + j]) : 0u;
      }
    }
    // ---- group maxima: G groups of kVecPerLane/G vectors per lane
    const int G = K <= 16 ? 1 : (K <= 32 ? 2 : 4);
    uint32_t gmax[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < kVec; ++j) m = max(m, key[i][j]);
      const int gi = (i * G) / kVecPerLane;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g == gi) gmax[g] = max(gmax[g], m);
    }
    // ---- T0 = K-th largest group maximum
    uint32_t t0 = 0;
    for (int bit = S::kKeyBits - 1; bit >= 0; --bit) {
      const uint32_t cand = t0 | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g < G) cnt += __popcll(ballot(gmax[g] >= cand));
      if (cnt >= K) t0 = cand;
    }
    // ---- append every real element with key >= T0 (LDS operations of one
    //      wave complete in order, so s_cnt[w] is already 0 here)
#pragma unroll
    for (int i = 0; i < kVecPerLane; ++i) {
#pragma unroll
      for (int j = 0; j < kVec; ++j) {
        const int e = seg0 + (i * kWave + l) * kVec + j;
        if (key[i][j] >= t0 && e < V) {
          const int pos = atomicAdd(&s_cnt[w], 1);
          if (pos < kCandCap) s_cand[w][pos] = make_comp(key[i][j], static_cast<uint32_t>(e));
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const int count = s_cnt[w];
    if (count <= kCandCap) {
      select_small<S::kKeyBits>(s_cand[w], count, K, wave_out);
    } else {
      // ---- exact fallback over the registers: key threshold, then the
      //      lowest ids among keys equal to it.
      uint32_t tk = 0;
      for (int bit = S::kKeyBits - 1; bit >= 0; --bit) {
        const uint32_t cand = tk | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < kVecPerLane; ++i)
#pragma unroll
          for (int j = 0; j < kVec; ++j) {
            const int e = seg0 + (i * kWave + l) * kVec + j;
            cnt += (key[i][j] >= cand && e < V) ? 1 : 0;
          }
        if (wave_sum_i(cnt) >= K) tk = cand;
      }
      // keys above tk: fewer than K of them, appended in any order
      if (l == 0) s_cnt[w] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < kVecPerLane; ++i)
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const int e = seg0 + (i * kWave + l) * kVec + j;
          if (key[i][j] > tk && e < V) {
            const int pos = atomicAdd(&s_cnt[w], 1);
            wave_out[pos] = make_comp(key[i][j], static_cast<uint32_t>(e));
          }
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      int have = s_cnt[w];
      // keys equal to tk, lowest ids first: vectors in index order
#pragma unroll
      for (int i = 0; i < kVecPerLane; ++i) {
        int mine = 0;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const int e = seg0 + (i * kWave + l) * kVec + j;
          mine += (key[i][j] == tk && e < V) ? 1 : 0;
        }
        const int incl = wave_prefix_incl(mine);
        int pos = have + incl - mine;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
          const int e = seg0 + (i * kWave + l) * kVec + j;
          if (key[i][j] == tk && e < V) {
            if (pos < K) wave_out[pos] = make_comp(tk, static_cast<uint32_t>(e));
            ++pos;
          }
        }
        have += __shfl(incl, kWave - 1, kWave);
      }
      for (int i = min(have, K) + l; i < K; i += kWave) wave_out[i] = 0ull;
    }
  } else {
    for (int i = l; i < K; i += kWave) wave_out[i] = 0ull;
  }
  __syncthreads();
  if (w == 0) {
    uint64_t* dst = partial + (static_cast<size_t>(row) * nchunks + chunk) * K;
    __shared__ uint64_t s_out[64];
    select_small<S::kKeyBits>(s_best, kTopkWaves * K, K, s_out);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    for (int i = l; i < K; i += kWave) dst[i] = s_out[i];
  }
}

// ---------------------------------------------------------------------------
// bf16 rows: the scan works on pairs of keys packed in 32-bit words.  The key
// of a bf16 pattern x is 0x8000 + |x| for x >= 0 and 0x8000 - |x| for x < 0
// (so -0 and +0 share 0x8000 and -inf maps to 0x0080); per 16-bit half that
// is  m = x >> 15 (arithmetic),  k = (x ^ (m | 0x8000)) - m,  three packed
// instructions per pair.  NaN patterns land above 0xff80 or below 0x0080; a
// wave that meets one re-derives exact keys (NaN -> 0, below -inf) and
// selects without the threshold shortcut.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_keys(uint32_t w) {
  const i16x2 x = __builtin_bit_cast(i16x2, w);
  const uint32_t m = __builtin_bit_cast(uint32_t, x >> (i16x2){15, 15});
  const u16x2 t = __builtin_bit_cast(u16x2, w ^ (m | 0x80008000u));
  return __builtin_bit_cast(uint32_t, t - __builtin_bit_cast(u16x2, m));
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}
// per half: saturate(a - b); nonzero iff the half of a exceeds that of b
__device__ __forceinline__ uint32_t pk_sub_sat(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a),
                                                                    __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t canon_half(uint32_t k) { return (k > 0xff80u || k < 0x0080u) ? 0u : k; }

// Exact key of one bf16 pattern (NaN -> 0).
__device__ __forceinline__ uint32_t exact_key16(uint32_t bits) {
  return canon_half((pack_keys(bits) & 0xffffu));
}

// Final step of a row: top-K of src[0..count) (count <= 64 * Q), sorted by
// composite (value desc, id asc); writes ids and the original logit values.
// Executed by one wave.
template <int Q, int KEYBITS, typename T>
__device__ void finish_row(const uint64_t* src, int count, int K, uint64_t* s_fin, const T* rowp,
                           int32_t* ids_row, float* vals_row) {
  const int l = lane_id();
  select_to<Q, KEYBITS>(src, count, K, s_fin);
  __builtin_amdgcn_wave_barrier();
  if (l < K) {
    const uint64_t mine = s_fin[l];
    int rank = 0;
    for (int j = 0; j < K; ++j) rank += s_fin[j] > mine ? 1 : 0;
    const uint32_t id = 0xffffffffu - comp_inv(mine);
    ids_row[rank] = static_cast<int32_t>(id);
    if constexpr (std::is_same<T, uint16_t>::value) vals_row[rank] = bf16_to_f32(rowp[id]);
    else vals_row[rank] = Elem<T>::to_f32(rowp[id]);
  }
}

// Exact top-K of the elements a wave owns (segments first_seg + r * seg_stride,
// r < rounds, each 64 lanes x nv vectors of 8), re-read from memory: the path
// for a wave that met a NaN or too many near-threshold keys.  Writes
// min(K, #elements) composites to out[0..K), zero padded.
__device__ __attribute__((noinline)) void exact_wave_bf16(const uint16_t* rowp, int V, int K, int first_seg,
                                                          int seg_stride, int rounds, int nv, int* cnt_slot,
                                                          uint64_t* out) {
  const int l = lane_id();
  const int seg_len = kWave * nv * 8;
  auto key_at = [&](int e) -> int { return e < V ? static_cast<int>(exact_key16(rowp[e])) : -1; };
  uint32_t tk = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const int cand = static_cast<int>(tk | (1u << bit));
    int cnt = 0;
    for (int rd = 0; rd < rounds; ++rd) {
      const int seg0 = (first_seg + rd * seg_stride) * seg_len;
      for (int i = 0; i < nv; ++i)
        for (int j = 0; j < 8; ++j) cnt += key_at(seg0 + (i * kWave + l) * 8 + j) >= cand ? 1 : 0;
    }
    if (wave_sum_i(cnt) >= K) tk = static_cast<uint32_t>(cand);
  }
  if (l == 0) *cnt_slot = 0;
  __builtin_amdgcn_wave_barrier();
  for (int rd = 0; rd < rounds; ++rd) {
    const int seg0 = (first_seg + rd * seg_stride) * seg_len;
    for (int i = 0; i < nv; ++i)
      for (int j = 0; j < 8; ++j) {
        const int e = seg0 + (i * kWave + l) * 8 + j;
        const int k = key_at(e);
        if (k > static_cast<int>(tk)) {
          const int pos = atomicAdd(cnt_slot, 1);
          out[pos] = make_comp(static_cast<uint32_t>(k), static_cast<uint32_t>(e));
        }
      }
  }
  __builtin_amdgcn_wave_barrier();
  int have = *cnt_slot;
  // keys equal to tk, lowest ids first: segments, vectors, lanes, then j
  for (int rd = 0; rd < rounds; ++rd) {
    const int seg0 = (first_seg + rd * seg_stride) * seg_len;
    for (int i = 0; i < nv; ++i) {
      int mine = 0;
      for (int j = 0; j < 8; ++j) mine += key_at(seg0 + (i * kWave + l) * 8 + j) == static_cast<int>(tk) ? 1 : 0;
      const int incl = wave_prefix_incl(mine);
      int pos = have + incl - mine;
      for (int j = 0; j < 8; ++j) {
        const int e = seg0 + (i * kWave + l) * 8 + j;
        if (key_at(e) == static_cast<int>(tk)) {
          if (pos < K) out[pos] = make_comp(tk, static_cast<uint32_t>(e));
          ++pos;
        }
      }
      have += __shfl(incl, kWave - 1, kWave);
    }
  }
  for (int i = min(have, K) + l; i < K; i += kWave) out[i] = 0ull;
}

// One workgroup (8 waves) per bf16 row; no cross-workgroup merge.  Wave w
// scans segments w, w+8, ... of 64 lanes x NV 16-byte vectors (8 bf16 each),
// all NV loads of a segment in flight at once, and keeps a running lower bound
// on its own K-th largest key: the K-th largest of a segment's 64*G group
// maxima.  Keys at or above it (about K + a few per segment on random rows)
// are appended to LDS.  Each wave then selects its top-K exactly and wave 0
// merges the 8 lists, sorts the K winners and writes ids and values.
constexpr int kRowWaves = 8;

template <int NV, int G, bool kVecLoad>
__global__ void __launch_bounds__(kRowWaves * kWave)
topk_bf16_row_kernel(const uint16_t* __restrict__ logits, int V, int K, int rounds, int32_t* __restrict__ ids,
                     float* __restrict__ vals) {
  constexpr int kWordsL = NV * 4;           // 32-bit words (bf16 pairs) per lane
  constexpr int kSegLen = kWave * NV * 8;
  static_assert(kWordsL <= 128, "candidate bitmask holds 128 words");
  const int row = blockIdx.x;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const uint16_t* rowp = logits + static_cast<size_t>(row) * V;

  __shared__ uint64_t s_cand[kRowWaves][kCandCap];
  __shared__ uint64_t s_best[kRowWaves * 64];
  __shared__ uint64_t s_fin[64];
  __shared__ int s_cnt[kRowWaves];

  if (l == 0) s_cnt[w] = 0;
  __builtin_amdgcn_wave_barrier();
  uint32_t t_run = 0;       // running lower bound on this wave's K-th largest key
  bool exact = false;
  int nseg = 0;
  for (int rd = 0; rd < rounds; ++rd) {
    const int seg0 = (rd * kRowWaves + w) * kSegLen;
    if (seg0 >= V) break;
    ++nseg;
    uint32_t kw[kWordsL];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e0 = seg0 + (i * kWave + l) * 8;
      if (kVecLoad && e0 + 8 <= V) {
        const uint4 v = *reinterpret_cast<const uint4*>(rowp + e0);
        kw[4 * i] = v.x; kw[4 * i + 1] = v.y; kw[4 * i + 2] = v.z; kw[4 * i + 3] = v.w;
      } else {
        // past the row end: -inf patterns (never appended: their ids are >= V)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = e0 + 2 * q < V ? rowp[e0 + 2 * q] : 0xff80u;
          const uint32_t hi = e0 + 2 * q + 1 < V ? rowp[e0 + 2 * q + 1] : 0xff80u;
          kw[4 * i + q] = lo | (hi << 16);
        }
      }
    }
    uint32_t gmx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) gmx[g] = 0u;
    uint32_t mn = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kWordsL; ++j) {
      kw[j] = pack_keys(kw[j]);
      const int g = (j * G) / kWordsL;
      gmx[g] = pk_max(gmx[g], kw[j]);
      mn = pk_min(mn, kw[j]);
    }
    uint32_t top = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      gmx[g] = max(gmx[g] & 0xffffu, gmx[g] >> 16);
      top = max(top, gmx[g]);
    }
    const bool lane_nan = top > 0xff80u || min(mn & 0xffffu, mn >> 16) < 0x0080u;
    if (ballot(lane_nan) != 0) {
      exact = true;
      break;
    }
    // this segment's bound: the K-th largest group maximum (all keys >= 0x0080)
    uint32_t t0 = 0;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = t0 | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) cnt += __popcll(ballot(gmx[g] >= cand));
      if (cnt >= K) t0 = cand;
    }
    t_run = max(t_run, t0);
    const uint32_t thr = (t_run - 1u) * 0x00010001u;
    // one bit per word holding a key >= t_run (words 0..63 and 64..)
    uint64_t mlo = 0, mhi = 0;
#pragma unroll
    for (int j = 0; j < kWordsL; ++j) {
      const uint64_t bit = pk_sub_sat(kw[j], thr) != 0u ? 1ull : 0ull;
      if (j < 64) mlo |= bit << j;
      else mhi |= bit << (j - 64);
    }
    while (mlo | mhi) {
      int j;
      if (mlo) {
        j = __builtin_ctzll(mlo);
        mlo &= mlo - 1ull;
      } else {
        j = 64 + __builtin_ctzll(mhi);
        mhi &= mhi - 1ull;
      }
      const int e = seg0 + ((j >> 2) * kWave + l) * 8 + (j & 3) * 2;
      if (e >= V) continue;   // padding only
      const uint32_t lo = rowp[e];
      const uint32_t hi = e + 1 < V ? rowp[e + 1] : 0xff80u;
      const uint32_t kk = pack_keys(lo | (hi << 16));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k = (kk >> (16 * h)) & 0xffffu;
        if (k >= t_run && e + h < V) {
          const int pos = atomicAdd(&s_cnt[w], 1);
          if (pos < kCandCap) s_cand[w][pos] = make_comp(k, static_cast<uint32_t>(e + h));
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (s_cnt[w] > kCandCap) {
      exact = true;
      break;
    }
  }
  uint64_t* wave_out = s_best + w * K;
  if (nseg == 0) {
    for (int i = l; i < K; i += kWave) wave_out[i] = 0ull;
  } else if (!exact) {
    select_small<16>(s_cand[w], s_cnt[w], K, wave_out);
  } else {
    int segs = 0;
    for (int rd = 0; rd < rounds; ++rd) segs += (rd * kRowWaves + w) * kSegLen < V ? 1 : 0;
    exact_wave_bf16(rowp, V, K, w, kRowWaves, segs, NV, &s_cnt[w], wave_out);
  }
  __syncthreads();
  if (w == 0) {
    const int count = kRowWaves * K;
    int32_t* ids_row = ids + static_cast<size_t>(row) * K;
    float* vals_row = vals + static_cast<size_t>(row) * K;
    if (count <= 2 * kWave) finish_row<2, 16>(s_best, count, K, s_fin, rowp, ids_row, vals_row);
    else if (count <= 4 * kWave) finish_row<4, 16>(s_best, count, K, s_fin, rowp, ids_row, vals_row);
    else finish_row<8, 16>(s_best, count, K, s_fin, rowp, ids_row, vals_row);
  }
}

template <typename T, int Q>
__global__ void __launch_bounds__(kWave)
topk_merge_kernel(const T* __restrict__ logits, int V, int K, int nchunks,
                  const uint64_t* __restrict__ partial, int32_t* __restrict__ ids,
                  float* __restrict__ vals) {
  constexpr int kKeyBits = sizeof(T) * 8;
  const int row = blockIdx.x;
  const int l = lane_id();
  const int count = nchunks * K;
  const uint64_t* src = partial + static_cast<size_t>(row) * count;
  __shared__ uint64_t s_sel[64];
  uint64_t c[Q];
  bool sel[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = q * kWave + l;
    c[q] = i < count ? src[i] : 0ull;
  }
  select_topk<Q, kKeyBits>(c, K, sel);
  int base = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const uint64_t m = ballot(sel[q]);
    if (sel[q]) s_sel[base + lanes_below(m)] = c[q];
    base += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  if (l < base) {
    const uint64_t mine = s_sel[l];
    int rank = 0;
    for (int j = 0; j < base; ++j) rank += s_sel[j] > mine ? 1 : 0;
    const uint32_t id = 0xffffffffu - comp_inv(mine);
    ids[static_cast<size_t>(row) * K + rank] = static_cast<int32_t>(id);
    vals[static_cast<size_t>(row) * K + rank] =
        Elem<T>::to_f32(logits[static_cast<size_t>(row) * V + id]);
  }
}

template <typename T>
int topk_nchunks(int V) {
  return (V + TopkShape<T>::kChunk - 1) / TopkShape<T>::kChunk;
}

template <typename T>
hipError_t launch_topk_t(const void* logits, int rows, int V, int K, uint64_t* partial,
                         int32_t* ids, float* vals, hipStream_t st) {
  const int nch = topk_nchunks<T>(V);
  const T* lg = static_cast<const T*>(logits);
  const bool vec = (static_cast<size_t>(V) * sizeof(T)) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(logits) % 16) == 0;
  dim3 g1(nch, rows);
  if constexpr (std::is_same<T, bf16>::value) {
    const uint16_t* lb = reinterpret_cast<const uint16_t*>(logits);
    const int G = K <= 16 ? 1 : (K <= 32 ? 2 : 4);
    // vectors per lane: the fewest rounds of 8 waves x 20 vectors, then the
    // smallest vector count (from 4, 8, 12, 16, 20) that covers the row
    const int per_round_max = kRowWaves * kWave * 20 * 8;
    const int rounds = (V + per_round_max - 1) / per_round_max;
    const int need = (V + rounds * kRowWaves * kWave * 8 - 1) / (rounds * kRowWaves * kWave * 8);
    const int nv = need <= 4 ? 4 : (need <= 8 ? 8 : (need <= 12 ? 12 : (need <= 16 ? 16 : 20)));
#define DCOCO_ROW(NVV, GG, VV)                                                                       \
  hipLaunchKernelGGL((topk_bf16_row_kernel<NVV, GG, VV>), dim3(rows), dim3(kRowWaves * kWave), 0, st, lb, V, \
                     K, rounds, ids, vals)
#define DCOCO_ROW_G(NVV, VV)                          \
  if (G == 1) DCOCO_ROW(NVV, 1, VV);                  \
  else if (G == 2) DCOCO_ROW(NVV, 2, VV);             \
  else DCOCO_ROW(NVV, 4, VV)
#define DCOCO_ROW_NV(VV)                              \
  if (nv == 4) { DCOCO_ROW_G(4, VV); }                \
  else if (nv == 8) { DCOCO_ROW_G(8, VV); }           \
  else if (nv == 12) { DCOCO_ROW_G(12, VV); }         \
  else if (nv == 16) { DCOCO_ROW_G(16, VV); }         \
  else { DCOCO_ROW_G(20, VV); }
    if (vec) { DCOCO_ROW_NV(true) } else { DCOCO_ROW_NV(false) }
#undef DCOCO_ROW_NV
#undef DCOCO_ROW_G
#undef DCOCO_ROW
    return hipGetLastError();
  } else {
    if (vec)
      hipLaunchKernelGGL((topk_partial_kernel<T, true>), g1, dim3(kTopkThreads), 0, st, lg, V, K, nch, partial);
    else
      hipLaunchKernelGGL((topk_partial_kernel<T, false>), g1, dim3(kTopkThreads), 0, st, lg, V, K, nch, partial);
  }
  const int count = nch * K;
  const int q = (count + kWave - 1) / kWave;
#define DCOCO_MERGE(QQ)                                                                     \
  hipLaunchKernelGGL((topk_merge_kernel<T, QQ>), dim3(rows), dim3(kWave), 0, st, lg, V, K, nch, \
                     partial, ids, vals)
  if (q <= 1) DCOCO_MERGE(1);
  else if (q <= 2) DCOCO_MERGE(2);
  else if (q <= 4) DCOCO_MERGE(4);
  else if (q <= 8) DCOCO_MERGE(8);
  else if (q <= 16) DCOCO_MERGE(16);
  else DCOCO_MERGE(32);
#undef DCOCO_MERGE
  return hipGetLastError();
}

}  // namespace

size_t topk_workspace_bytes(int dtype, int rows, int V, int K) {
  if (dtype == kDtypeBf16) return 0;   // one workgroup per row, no partials
  return static_cast<size_t>(rows) * topk_nchunks<float>(V) * K * sizeof(uint64_t);
}

bool topk_supported(int dtype, int V, int K) {
  if (dtype == kDtypeBf16) return true;
  return static_cast<long long>(topk_nchunks<float>(V)) * K <= 32 * kWave;
}

hipError_t launch_topk(int dtype, const void* logits, int rows, int V, int K, void* partial,
                       int32_t* ids, float* vals, hipStream_t st) {
  if (dtype == kDtypeBf16)
    return launch_topk_t<bf16>(logits, rows, V, K, static_cast<uint64_t*>(partial), ids, vals, st);
  return launch_topk_t<float>(logits, rows, V, K, static_cast<uint64_t*>(partial), ids, vals, st);
}

}  // namespace dcoco
