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
// bf16 rows (the drafter's logits) take one workgroup per row
// (topk_bf16_row_reg_kernel, described where it is defined): a sampled bound,
// a streamed screen, and an exact selection of the few survivors, with a
// running-list fallback for rows that defeat the bound.
//
// fp32 rows (HBM-bound scan; each logit is read once):
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
#include "gemm_tile.h"
#include "kernels.h"
#include "select.h"
#include "wave.h"

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
            if (pos < K) wave_out[pos] = make_comp(key[i][j], static_cast<uint32_t>(e));
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
// per half: signed 16-bit maximum
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, a),
                                                                __builtin_bit_cast(i16x2, b)));
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
__device__ void finish_row(const uint64_t* src, int count, int K, uint64_t* s_fin, const T* rowp, int V,
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
    // every id here is < V (a row holds at least K elements); the guard keeps
    // the value read inside the row regardless
    const uint32_t rid = id < static_cast<uint32_t>(V) ? id : 0u;
    if constexpr (std::is_same<T, uint16_t>::value) vals_row[rank] = bf16_to_f32(rowp[rid]);
    else vals_row[rank] = Elem<T>::to_f32(rowp[rid]);
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
          // fewer than K keys exceed tk when both passes read the same row;
          // the guard keeps a row that changes under the call (a caller's
          // race) from writing past the list
          const int pos = atomicAdd(cnt_slot, 1);
          if (pos < K) out[pos] = make_comp(static_cast<uint32_t>(k), static_cast<uint32_t>(e));
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
// scans segments w, w+8, ... of 64 lanes x NV 16-byte vectors (8 bf16 each).
//   1. A row-wide bound T on the K-th largest key: the K-th largest of the
//      maxima of G groups per lane over every wave's first segment (K
//      distinct elements reach it).
//   2. Streaming: every 16-byte vector is screened against T; the start of
//      each vector holding an element at or above T is recorded in a
//      per-wave LDS list.  On random rows that is about K times the ratio of
//      the row to the sampled part, spread over 8 waves.  The screen is a few
//      instructions per vector and never waits on memory, so the stream stays
//      ahead.
//   3. The flagged vectors are read again in one parallel round (the rows
//      were just streamed) and their elements at or above T become
//      candidates; each wave selects its top-K exactly and wave 0 merges the
//      8 lists, sorts the K winners and writes ids and values.
// In the aligned kernel a wave whose flags would overflow, or that meets a
// dense segment, keeps an exact running list instead (see list_merge); a NaN
// at or above the bound sends the wave to the exact path (a rescan).  The
// unaligned kernel sends every overflow there.
constexpr int kRowWaves = 8;
constexpr int kRowCap = 128;                // candidates per wave list
constexpr int kFlagCap = 128;               // flagged vectors per wave list

// group maxima of one segment's packed keys (raw bf16 pairs in kw)
template <int NV, int G>
__device__ __forceinline__ void group_max(const uint32_t (&kw)[NV * 4], uint32_t (&gmx)[G]) {
  constexpr int kWordsL = NV * 4;
#pragma unroll
  for (int g = 0; g < G; ++g) gmx[g] = 0u;
#pragma unroll
  for (int j = 0; j < kWordsL; ++j) {
    const int g = (j * G) / kWordsL;
    gmx[g] = pk_max(gmx[g], pack_keys(kw[j]));
  }
#pragma unroll
  for (int g = 0; g < G; ++g) gmx[g] = max(gmx[g] & 0xffffu, gmx[g] >> 16);
}

// Row-wide bound from every wave's group maxima (s_gm holds kRowWaves * G *
// 64 keys); called by all waves after a barrier, each computes the same T.
template <int G>
__device__ __forceinline__ uint32_t row_bound(const uint32_t* s_gm, int K, int l) {
  constexpr int Q = kRowWaves * G;
  uint32_t v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) v[q] = s_gm[q * kWave + l];
  uint32_t t = 0;
  for (int bit = 15; bit >= 0; --bit) {
    const uint32_t c = t | (1u << bit);
    int n = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) n += __popcll(ballot(v[q] >= c));
    if (n >= K) t = c;
  }
  return t;
}

// Screens one segment (raw bf16 pairs in kw) against the bound t and records
// the first element index of every vector holding an element at or above t.
//
// For a bound above the key of zero (t > 0x8000) the qualifying patterns are
// exactly the non-negative ones at or above the raw pattern of t, and read as
// signed 16-bit integers raw patterns order like their values on that side
// (negative patterns, -0 included, read as negative integers and never
// qualify), so a vector is screened with a packed signed max over its words
// and one compare.  Otherwise its words are packed into keys and compared.
// NaN patterns need no screening of their own: a positive NaN reads above
// every number and is always flagged, and a NaN that is not flagged ranks
// below at least K numbers of the row.
template <int NV>
__device__ __forceinline__ uint32_t row_vflags(const uint32_t (&kw)[NV * 4], uint32_t t) {
  uint32_t vflag = 0u;
  if (t > 0x8000u) {
    const uint32_t thr = ((t ^ 0x8000u) - 1u) * 0x00010001u;   // raw pattern of t, minus one
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t m = pk_max_i16(pk_max_i16(kw[4 * i], kw[4 * i + 1]), pk_max_i16(kw[4 * i + 2], kw[4 * i + 3]));
      vflag |= (pk_max_i16(m, thr) != thr ? 1u : 0u) << i;
    }
  } else {
    const uint32_t thr = (t - 1u) * 0x00010001u;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      uint32_t any = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) any |= pk_sub_sat(pack_keys(kw[4 * i + q]), thr);
      vflag |= (any != 0u ? 1u : 0u) << i;
    }
  }
  return vflag;
}

// Records the first element index of every flagged vector in the wave's list.
template <int NV>
__device__ __forceinline__ void row_append(uint32_t vflag, int seg0, int V, int l, int& nflag, int32_t* flags) {
  if (ballot(vflag != 0u) == 0ull) return;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e0 = seg0 + (i * kWave + l) * 8;
    const bool f = ((vflag >> i) & 1u) && e0 < V;
    const uint64_t m = ballot(f);
    if (m == 0ull) continue;
    const int pos = nflag + lanes_below(m);
    if (f && pos < kFlagCap) flags[pos] = e0;
    nflag += __popcll(m);
  }
}

template <int NV>
__device__ __forceinline__ void row_screen(const uint32_t (&kw)[NV * 4], int seg0, int V, int l, uint32_t t,
                                           int& nflag, int32_t* flags) {
  row_append<NV>(row_vflags<NV>(kw, t), seg0, V, l, nflag, flags);
}

// Reads the flagged vectors again (each lane one vector per pass) and appends
// their elements at or above t to cand, compacted with ballots.  Returns
// false when the wave must take the exact path (a NaN candidate, or more
// candidates than the list holds).
template <bool kVec>
__device__ __forceinline__ bool row_collect(const uint16_t* rowp, int V, uint32_t t, const int32_t* flags,
                                            int nflag, int l, uint64_t* cand, int& cnt) {
  bool bad = false;
  for (int b = 0; b < nflag; b += kWave) {
    const bool act = b + l < nflag;
    // flags hold vector starts e0 < V (e0 + 8 <= V on the vector path); the
    // clamp keeps every read inside the row whatever the list holds
    const int e0 = act ? min(max(flags[b + l], 0), kVec ? V - 8 : V - 1) : 0;
    uint32_t w4[4];
    if constexpr (kVec) {
      const uint4 v = *reinterpret_cast<const uint4*>(rowp + e0);
      w4[0] = v.x; w4[1] = v.y; w4[2] = v.z; w4[3] = v.w;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = e0 + 2 * q < V ? rowp[e0 + 2 * q] : 0xffffu;
        const uint32_t hi = e0 + 2 * q + 1 < V ? rowp[e0 + 2 * q + 1] : 0xffffu;
        w4[q] = lo | (hi << 16);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t kk = pack_keys(w4[q]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k = (kk >> (16 * h)) & 0xffffu;
        const int e = e0 + 2 * q + h;
        const bool c = act && k >= t && e < V;
        bad |= c && (k > 0xff80u || k < 0x0080u);
        const uint64_t m = ballot(c);
        const int pos = cnt + lanes_below(m);
        if (c && pos < kRowCap) cand[pos] = make_comp(k, static_cast<uint32_t>(e));
        cnt += __popcll(m);
      }
    }
  }
  return ballot(bad) == 0ull && cnt <= kRowCap;
}

// After the scan: each wave's exact top-K into s_best, then wave 0 sorts the
// row's K winners and writes ids and values.
template <int NV>
__device__ __forceinline__ void row_finish(const uint16_t* rowp, int V, int K, int rounds, int w, int l, int nseg,
                                           bool exact, int cnt, uint64_t (*s_cand)[kRowCap], uint64_t* s_best,
                                           uint64_t* s_fin, int* s_cnt, int32_t* ids_row, float* vals_row) {
  constexpr int kSegLen = kWave * NV * 8;
  uint64_t* wave_out = s_best + w * K;
  if (nseg == 0) {
    for (int i = l; i < K; i += kWave) wave_out[i] = 0ull;
  } else if (!exact) {
    select_small<16>(s_cand[w], cnt, K, wave_out);
  } else {
    int segs = 0;
    for (int rd = 0; rd < rounds; ++rd) segs += (rd * kRowWaves + w) * kSegLen < V ? 1 : 0;
    exact_wave_bf16(rowp, V, K, w, kRowWaves, segs, NV, &s_cnt[w], wave_out);
  }
  __syncthreads();
  if (w == 0) {
    const int count = kRowWaves * K;
    if (count <= 2 * kWave) finish_row<2, 16>(s_best, count, K, s_fin, rowp, V, ids_row, vals_row);
    else if (count <= 4 * kWave) finish_row<4, 16>(s_best, count, K, s_fin, rowp, V, ids_row, vals_row);
    else finish_row<8, 16>(s_best, count, K, s_fin, rowp, V, ids_row, vals_row);
  }
}

// Barrier for LDS traffic only: waits for this wave's LDS accesses, not for
// its vector-memory loads still in flight (a __syncthreads would drain those
// as well, and the register ring below keeps several segments in flight
// across the barriers of the bound computation).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

template <int NV>
__device__ __forceinline__ void row_load_regs(const uint16_t* rowp, int V, int seg0, int l, uint32_t (&kw)[NV * 4]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e0 = seg0 + (i * kWave + l) * 8;
    // clamped inside the row; non-temporal: the logits are read once, so they
    // should not push what other work keeps in L2 (the launch that also runs
    // the slot GEMM's tiles re-reads its weights from there)
    using u32x4 = __attribute__((ext_vector_type(4))) uint32_t;
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + min(e0, V - 8)));
    kw[4 * i] = v[0];
    kw[4 * i + 1] = v[1];
    kw[4 * i + 2] = v[2];
    kw[4 * i + 3] = v[3];
  }
}

// vectors past the row end become the padding pattern 0xffff
template <int NV>
__device__ __forceinline__ void row_pad(int seg0, int V, int l, uint32_t (&kw)[NV * 4]) {
  if (seg0 + kWave * NV * 8 > V) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool in = seg0 + (i * kWave + l) * 8 < V;
#pragma unroll
      for (int q = 0; q < 4; ++q) kw[4 * i + q] = in ? kw[4 * i + q] : 0xffffffffu;
    }
  }
}

// vectors per lane and segment (3: 3 KB per wave and segment), and register
// sets in the ring (4 segments in flight per wave).  Measured on the 32-stream
// workload: 4 vectors or 6 to 8 register sets were no faster, and more sets
// cost occupancy.
constexpr int kRegNV = 3;
constexpr int kRegD = 4;

// A wave's running top-K: one composite per lane (lanes < K, 0 = empty), and
// once it holds K entries the smallest key among them (kmin).  An element
// whose key is below kmin, or equal to it with a larger id than every entry,
// cannot be in the wave's top-K; elements streamed later have larger ids than
// every entry, so the screen may use kmin + 1.
struct RunList {
  uint64_t c = 0ull;
  int n = 0;
  uint32_t kmin = 0u;
  bool bad = false;   // a NaN at or above the threshold: the bound may not hold
};

// Merges the 8 elements of one 16-byte vector per lane (raw bf16 words w4,
// first element id e0, act false for an idle lane) into the running list:
// elements with exact key >= max(t0, kmin) (NaN keys are 0) join the list's
// composites, and the list becomes the top K of both.  s_tmp holds 64
// composites of this wave's LDS for the compaction.
__device__ __forceinline__ void list_merge(const uint32_t (&w4)[4], int e0, bool act, int V, int K, int l,
                                           uint32_t t0, RunList& L, uint64_t* s_tmp) {
  const uint32_t thr = L.n >= K ? max(t0, L.kmin) : t0;
  uint64_t c[9];
  bool any = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t kk = pack_keys(w4[q]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t raw = (kk >> (16 * h)) & 0xffffu;
      const uint32_t k = canon_half(raw);
      const int e = e0 + 2 * q + h;
      const bool live = act && e < V;
      const bool in = live && k >= thr;
      L.bad |= live && raw >= thr && k != raw;
      c[2 * q + h] = in ? make_comp(k, static_cast<uint32_t>(e)) : 0ull;
      any |= in;
    }
  }
  if (ballot(any) == 0ull) return;
  c[8] = L.c;
  bool sel[9];
  select_topk<9, 16>(c, K, sel, 32 - __clz(static_cast<unsigned>(V)));   // ids < V
  int base = 0;
#pragma unroll
  for (int q = 0; q < 9; ++q) {
    const uint64_t m = ballot(sel[q]);
    if (sel[q]) s_tmp[base + lanes_below(m)] = c[q];
    base += __popcll(m);
  }
  // one wave: its LDS accesses complete in order; wait for the stores only
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
  L.c = l < base ? s_tmp[l] : 0ull;
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
  L.n = base;
  if (base >= K) L.kmin = ~wave_max_u32_dpp(l < K ? ~comp_key(L.c) : 0u);
}

// Merges the flagged vectors (read again from the row) into the running list.
__device__ __forceinline__ void list_flush(const uint16_t* rowp, int V, int K, int l, uint32_t t0,
                                           const int32_t* flags, int& nflag, RunList& L, uint64_t* s_tmp) {
  for (int b = 0; b < nflag; b += kWave) {
    const bool act = b + l < nflag;
    // flagged vector starts satisfy e0 + 8 <= V; clamped so that every read
    // stays inside the row whatever the list holds
    const int e0 = act ? min(max(flags[b + l], 0), V - 8) : 0;
    const uint4 v = *reinterpret_cast<const uint4*>(rowp + e0);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    list_merge(w4, e0, act, V, K, l, t0, L, s_tmp);
  }
  nflag = 0;
}

// ---- on-chip finish of a row (register-ring kernel) --------------------
// A wave reading LDS that its own lanes just wrote: the wave's LDS accesses
// complete in order, so waiting for its stores and stopping the compiler from
// moving accesses across is enough.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
  __builtin_amdgcn_wave_barrier();
}

// The r-th largest of src[0..n) (unique composites, 0 = empty) goes to dst[r]
// for r < K, dst[#non-empty..K) is cleared.  Each lane ranks Q entries by
// counting the larger ones over broadcast LDS reads, so the list comes out
// sorted (value desc, id asc) without ballot chains.  n <= 64 Q; src and dst
// must not overlap.
template <int Q>
__device__ __forceinline__ void rank_top(const uint64_t* src, int n, int K, uint64_t* dst, int l) {
  uint64_t c[Q];
  int r[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int i = q * kWave + l;
    c[q] = i < n ? src[i] : 0ull;
    r[q] = 0;
  }
#pragma unroll 4
  for (int j = 0; j < n; ++j) {
    const uint64_t v = src[j];
#pragma unroll
    for (int q = 0; q < Q; ++q) r[q] += v > c[q] ? 1 : 0;
  }
  int nz = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    nz += __popcll(ballot(c[q] != 0ull));
    if (c[q] != 0ull && r[q] < K) dst[r[q]] = c[q];
  }
  for (int i = nz + l; i < K; i += kWave) dst[i] = 0ull;
}

// row_append that also keeps each flagged vector's four words in vecs[], so
// the candidates can later be collected from LDS instead of memory.
template <int NV>
__device__ __forceinline__ void row_append_keep(uint32_t vflag, const uint32_t (&kw)[NV * 4], int seg0, int V, int l,
                                                int& nflag, int32_t* flags, uint4* vecs) {
  if (ballot(vflag != 0u) == 0ull) return;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e0 = seg0 + (i * kWave + l) * 8;
    const bool f = ((vflag >> i) & 1u) && e0 < V;
    const uint64_t m = ballot(f);
    if (m == 0ull) continue;
    const int pos = nflag + lanes_below(m);
    if (f && pos < kFlagCap) {
      flags[pos] = e0;
      vecs[pos] = make_uint4(kw[4 * i], kw[4 * i + 1], kw[4 * i + 2], kw[4 * i + 3]);
    }
    nflag += __popcll(m);
  }
}

// row_collect over the kept vectors (nflag <= kFlagCap): the elements at or
// above t become candidates; false if one of them is a NaN pattern or the
// list overflows (the caller then takes another path).
__device__ __forceinline__ bool row_collect_kept(const int32_t* flags, const uint4* vecs, int nflag, int V, uint32_t t,
                                                 int l, uint64_t* cand, int& cnt) {
  bool bad = false;
  for (int b = 0; b < nflag; b += kWave) {
    const bool act = b + l < nflag;
    const int e0 = act ? flags[b + l] : 0;
    const uint4 v = vecs[act ? b + l : 0];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t kk = pack_keys(w4[q]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t k = (kk >> (16 * h)) & 0xffffu;
        const int e = e0 + 2 * q + h;
        const bool c = act && k >= t && e < V;
        bad |= c && (k > 0xff80u || k < 0x0080u);
        const uint64_t m = ballot(c);
        const int pos = cnt + lanes_below(m);
        if (c && pos < kRowCap) cand[pos] = make_comp(k, static_cast<uint32_t>(e));
        cnt += __popcll(m);
      }
    }
  }
  return ballot(bad) == 0ull && cnt <= kRowCap;
}

// All waves at once, after each has written its sorted list of K to
// lists[w K ..]: an entry's rank in the row is its position in its own list
// plus, for every other list, the number of that list's entries above it
// (counted with independent LDS reads, which pipeline, rather than a binary
// search, whose reads depend on each other).  With KP = K rounded up to a
// power of two, the 64 / KP lanes of one entry split the other lists between
// them and add their counts.  Entries of rank < K go to out[rank].
__device__ __forceinline__ void merge_sorted_lists(const uint64_t* lists, int K, int w, int l, uint64_t* out) {
  int KP = 1;
  while (KP < K) KP <<= 1;                   // K <= 64
  const int G = kWave / KP;                  // lanes per entry
  const int c = l % KP;
  const int g = l / KP;
  const uint64_t x = c < K ? lists[w * K + c] : 0ull;
  int rank = 0;
  for (int j = g; j < kRowWaves; j += G) {
    if (j == w) {
      rank += c;
      continue;
    }
    const uint64_t* lst = lists + j * K;
#pragma unroll 8
    for (int i = 0; i < K; ++i) rank += lst[i] > x ? 1 : 0;
  }
  for (int off = KP; off < kWave; off <<= 1) rank += __shfl_xor(rank, off, kWave);
  if (g == 0 && x != 0ull && rank < K) out[rank] = x;
}

// The bf16 pattern of an order key (the inverse of pack_keys on one half);
// 0x8000 stands for both zeros and 0 for a NaN, so those two read the row.
__device__ __forceinline__ bool key_is_exact_bf16(uint32_t k) { return k != 0u && k != 0x8000u; }
__device__ __forceinline__ uint32_t key_to_bf16(uint32_t k) {
  return k >= 0x8000u ? (k ^ 0x8000u) : ((0x10000u - k) & 0xffffu);
}

// Rows whose length is a multiple of 8 and that start 16-byte aligned.  Each
// wave streams its segments through a ring of D register sets: D segments per
// wave in flight, plain 16-byte vector loads (the compiler's waits follow the
// issue order).  Loads are unconditional; a vector past the row end reads a
// clamped address inside the row and is replaced by padding, the pattern
// 0xffff (a NaN whose packed key is 1, below every real key but the NaNs that
// also sit below -inf): groups of padding never lift the bound, and padding
// never joins a list (its ids are >= V).
//   Each wave keeps an exact running top-K.  A segment whose screen flags
// more than kDense vectors (ties at the bound, rising rows) is merged into it
// straight from registers, one vector per lane at a time; sparse flags are
// recorded and merged in batches (when the list would overflow, and at the
// end).  Every merge lifts the screen to one above the list's smallest key,
// so a row of equal or ascending values costs a few merges per segment, not
// a rescan.
//   The finish stays on chip.  A flagged vector's 16 bytes are kept in LDS
// when it is flagged, so the candidates are collected without reading the row
// again; each wave ranks its candidates into a sorted list of K; all waves
// then rank their own entries across the eight lists, and the values are
// decoded from the keys (only a zero or NaN key reads the row).
constexpr int kDense = 24;

// The LDS of one row's workgroup: the row kernel below declares the arrays;
// the launch that runs rows beside GEMM tiles carves them from one buffer.
template <int G>
struct RowLds {
  uint32_t* s_gm;                 // [kRowWaves * G * kWave]
  int32_t (*s_flag)[kFlagCap];    // [kRowWaves][kFlagCap]
  uint4 (*s_vec)[kFlagCap];       // [kRowWaves][kFlagCap]
  uint64_t (*s_tmp)[kWave];       // [kRowWaves][kWave]
  uint64_t (*s_cand)[kRowCap];    // [kRowWaves][kRowCap]
  uint64_t* s_best;               // [kRowWaves * 64]
  uint64_t* s_fin;                // [64]
  int* s_cnt;                     // [kRowWaves]

  // parts in decreasing alignment; bytes of the whole
  static constexpr size_t kVec = sizeof(uint4) * kRowWaves * kFlagCap;
  static constexpr size_t kTmp = sizeof(uint64_t) * kRowWaves * kWave;
  static constexpr size_t kCand = sizeof(uint64_t) * kRowWaves * kRowCap;
  static constexpr size_t kBest = sizeof(uint64_t) * kRowWaves * 64;
  static constexpr size_t kFin = sizeof(uint64_t) * 64;
  static constexpr size_t kGm = sizeof(uint32_t) * kRowWaves * G * kWave;
  static constexpr size_t kFlag = sizeof(int32_t) * kRowWaves * kFlagCap;
  static constexpr size_t kCnt = sizeof(int) * kRowWaves;
  static constexpr size_t kBytes = kVec + kTmp + kCand + kBest + kFin + kGm + kFlag + kCnt;
  static_assert(kVec % 16 == 0 && kTmp % 16 == 0 && kCand % 16 == 0 && kBest % 16 == 0 && kFin % 16 == 0 &&
                kGm % 16 == 0 && kFlag % 16 == 0, "16-byte aligned parts");

  // base 16-byte aligned
  __device__ static RowLds carve(char* base) {
    RowLds S;
    char* p = base;
    S.s_vec = reinterpret_cast<uint4 (*)[kFlagCap]>(p); p += kVec;
    S.s_tmp = reinterpret_cast<uint64_t (*)[kWave]>(p); p += kTmp;
    S.s_cand = reinterpret_cast<uint64_t (*)[kRowCap]>(p); p += kCand;
    S.s_best = reinterpret_cast<uint64_t*>(p); p += kBest;
    S.s_fin = reinterpret_cast<uint64_t*>(p); p += kFin;
    S.s_gm = reinterpret_cast<uint32_t*>(p); p += kGm;
    S.s_flag = reinterpret_cast<int32_t (*)[kFlagCap]>(p); p += kFlag;
    S.s_cnt = reinterpret_cast<int*>(p);
    return S;
  }
};

// top-K of one row by one workgroup of kRowWaves waves (threadIdx.x < 512)
// One row rowp[0, V) (or one segment of a longer row) per workgroup.  Writes
// the K ids and values to ids[0, K) and vals[0, K), or, with part given, the
// K composites to part[0, K) with id_off added to every id (the segment's
// first column), for a merge across the row's segments.
template <int NV, int G, int D>
__device__ __forceinline__ void topk_row_reg(const uint16_t* __restrict__ rowp, int V, int K, int rounds,
                                             int32_t* __restrict__ ids, float* __restrict__ vals,
                                             uint64_t* __restrict__ part, uint32_t id_off,
                                             const RowLds<G>& S) {
  constexpr int kSegLen = kWave * NV * 8;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  uint32_t* const s_gm = S.s_gm;
  int32_t (*const s_flag)[kFlagCap] = S.s_flag;
  uint4 (*const s_vec)[kFlagCap] = S.s_vec;
  uint64_t (*const s_tmp)[kWave] = S.s_tmp;
  uint64_t (*const s_cand)[kRowCap] = S.s_cand;
  uint64_t* const s_best = S.s_best;
  uint64_t* const s_fin = S.s_fin;
  int* const s_cnt = S.s_cnt;

  uint32_t ring[D][NV * 4];
#pragma unroll
  for (int r = 0; r < D; ++r) row_load_regs<NV>(rowp, V, (r * kRowWaves + w) * kSegLen, l, ring[r]);

  // row-wide bound from the first segments (all padding for a wave past the end)
  {
    uint32_t kw[NV * 4];
#pragma unroll
    for (int j = 0; j < NV * 4; ++j) kw[j] = ring[0][j];
    row_pad<NV>(w * kSegLen, V, l, kw);
    uint32_t gmx[G];
    group_max<NV, G>(kw, gmx);
#pragma unroll
    for (int g = 0; g < G; ++g) s_gm[(w * G + g) * kWave + l] = gmx[g];
  }
  lds_barrier();
  const uint32_t t0 = row_bound<G>(s_gm, K, l);

  // Until a wave meets a dense segment or fills its flag list it only records
  // flags (the common case); then it leaves the streaming loop for a loop
  // that keeps the running list (the segments still in flight are read again).
  RunList L;
  int nflag = 0;
  int rd_slow = rounds;                     // first round the slow loop takes
  for (int rd0 = 0; rd0 < rounds && rd_slow == rounds; rd0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int rd = rd0 + j;
      if (rd < rounds && rd_slow == rounds) {
        const int seg0 = (rd * kRowWaves + w) * kSegLen;
        uint32_t kw[NV * 4];
#pragma unroll
        for (int q = 0; q < NV * 4; ++q) kw[q] = ring[j][q];
        if (rd + D < rounds) row_load_regs<NV>(rowp, V, ((rd + D) * kRowWaves + w) * kSegLen, l, ring[j]);
        if (seg0 < V) {
          row_pad<NV>(seg0, V, l, kw);
          const uint32_t vf = row_vflags<NV>(kw, t0);
          if (ballot(vf != 0u) != 0ull) {
            int nf = 0;
#pragma unroll
            for (int i = 0; i < NV; ++i)
              nf += __popcll(ballot(((vf >> i) & 1u) && seg0 + (i * kWave + l) * 8 < V));
            if (nf > kDense || nflag + nf > kFlagCap) rd_slow = rd;
            else row_append_keep<NV>(vf, kw, seg0, V, l, nflag, s_flag[w], s_vec[w]);
          }
        }
      }
    }
  }
  const bool refining = rd_slow < rounds;
  if (refining) {
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // the ring's loads are not used
    list_flush(rowp, V, K, l, t0, s_flag[w], nflag, L, s_tmp[w]);
    uint32_t nxt[NV * 4];
    row_load_regs<NV>(rowp, V, (rd_slow * kRowWaves + w) * kSegLen, l, nxt);
    for (int rd = rd_slow; rd < rounds; ++rd) {
      const int seg0 = (rd * kRowWaves + w) * kSegLen;
      if (seg0 >= V) break;
      uint32_t kw[NV * 4];
#pragma unroll
      for (int q = 0; q < NV * 4; ++q) kw[q] = nxt[q];
      if (rd + 1 < rounds) row_load_regs<NV>(rowp, V, ((rd + 1) * kRowWaves + w) * kSegLen, l, nxt);
      row_pad<NV>(seg0, V, l, kw);
      const uint32_t ts = L.n >= K ? max(t0, L.kmin + 1u) : t0;
      const uint32_t vf = ts > 0xffffu ? 0u : row_vflags<NV>(kw, ts);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (ballot((vf >> i) & 1u) == 0ull) continue;
        const uint32_t w4[4] = {kw[4 * i], kw[4 * i + 1], kw[4 * i + 2], kw[4 * i + 3]};
        list_merge(w4, seg0 + (i * kWave + l) * 8, true, V, K, l, t0, L, s_tmp[w]);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  // Each wave leaves its K best, sorted, in s_best[w K ..]; then all waves
  // rank their entries across the lists and wave 0 writes the row.  Nothing
  // here reads memory except the exact path and values whose key stands for
  // two patterns (zeros) or none (NaN).
  uint64_t* mine = s_best + w * K;
  bool exact = false;
  bool listed = false;                       // the running list holds the wave's K best
  if (refining) {
    list_flush(rowp, V, K, l, t0, s_flag[w], nflag, L, s_tmp[w]);
    exact = ballot(L.bad) != 0ull;
    listed = !exact;
  } else {
    // the common case: the kept vectors' elements at or above t0 become
    // candidates (a NaN candidate takes the exact path; more candidates than
    // the list holds, the running list)
    int cnt = 0;
    exact = !row_collect_kept(s_flag[w], s_vec[w], nflag, V, t0, l, s_cand[w], cnt);
    if (!exact) {
      wave_lds_fence();
      if (cnt <= kWave) rank_top<1>(s_cand[w], cnt, K, mine, l);
      else rank_top<kRowCap / kWave>(s_cand[w], cnt, K, mine, l);
    } else if (cnt > kRowCap) {
      list_flush(rowp, V, K, l, t0, s_flag[w], nflag, L, s_tmp[w]);
      exact = ballot(L.bad) != 0ull;
      listed = !exact;
    }
  }
  if (listed) {
    if (l < K) s_tmp[w][l] = L.c;
    wave_lds_fence();
    rank_top<1>(s_tmp[w], K, K, mine, l);
  }
  if (exact) {
    int segs = 0;
    for (int rd = 0; rd < rounds; ++rd) segs += (rd * kRowWaves + w) * kSegLen < V ? 1 : 0;
    exact_wave_bf16(rowp, V, K, w, kRowWaves, segs, NV, &s_cnt[w], s_tmp[w]);
    wave_lds_fence();
    rank_top<1>(s_tmp[w], K, K, mine, l);
  }
  if (w == 0 && l < K) s_fin[l] = 0ull;
  lds_barrier();
  merge_sorted_lists(s_best, K, w, l, s_fin);
  lds_barrier();
  if (w == 0 && l < K) {
    const uint64_t x = s_fin[l];
    const uint32_t id = 0xffffffffu - comp_inv(x);
    const uint32_t k = comp_key(x);
    if (part) {
      part[l] = x == 0ull ? 0ull : make_comp(k, id + id_off);
    } else {
      const uint32_t rid = id < static_cast<uint32_t>(V) ? id : 0u;
      const uint32_t bits = key_is_exact_bf16(k) ? key_to_bf16(k) : static_cast<uint32_t>(rowp[rid]);
      ids[l] = static_cast<int32_t>(id);
      vals[l] = bf16_to_f32(static_cast<uint16_t>(bits));
    }
  }
}

// Rows cut into nseg segments of seg_len columns (the last one shorter):
// workgroup b takes segment b % nseg of row b / nseg.  With nseg == 1 it
// takes the whole row and writes its ids and values; otherwise it writes the
// segment's K composites to part[(row nseg + seg) K ..] for topk_merge_kernel.
template <int NV, int G, int D>
__device__ __forceinline__ void topk_row_seg(const uint16_t* __restrict__ logits, int V, int K, int rounds,
                                             int32_t* __restrict__ ids, float* __restrict__ vals, int nseg,
                                             int seg_len, uint64_t* __restrict__ part, int b, const RowLds<G>& S) {
  if (nseg == 1) {
    topk_row_reg<NV, G, D>(logits + static_cast<size_t>(b) * V, V, K, rounds, ids + static_cast<size_t>(b) * K,
                           vals + static_cast<size_t>(b) * K, nullptr, 0u, S);
    return;
  }
  constexpr int kRound = kRowWaves * kWave * NV * 8;
  const int row = b / nseg;
  const int seg = b - row * nseg;
  const int c0 = seg * seg_len;
  const int vn = min(seg_len, V - c0);
  topk_row_reg<NV, G, D>(logits + static_cast<size_t>(row) * V + c0, vn, K, (vn + kRound - 1) / kRound, nullptr,
                         nullptr, part + static_cast<size_t>(b) * K, static_cast<uint32_t>(c0), S);
}

template <int NV, int G, int D>
__global__ void __launch_bounds__(kRowWaves * kWave, 4)   // two workgroups per CU
topk_bf16_row_reg_kernel(const uint16_t* __restrict__ logits, int V, int K, int rounds, int32_t* __restrict__ ids,
                         float* __restrict__ vals, int nseg, int seg_len, uint64_t* __restrict__ part) {
  __shared__ uint32_t s_gm[kRowWaves * G * kWave];
  __shared__ int32_t s_flag[kRowWaves][kFlagCap];
  __shared__ uint4 s_vec[kRowWaves][kFlagCap];
  __shared__ uint64_t s_tmp[kRowWaves][kWave];
  __shared__ uint64_t s_cand[kRowWaves][kRowCap];
  __shared__ uint64_t s_best[kRowWaves * 64];
  __shared__ uint64_t s_fin[64];
  __shared__ int s_cnt[kRowWaves];
  const RowLds<G> S{s_gm, s_flag, s_vec, s_tmp, s_cand, s_best, s_fin, s_cnt};
  topk_row_seg<NV, G, D>(logits, V, K, rounds, ids, vals, nseg, seg_len, part, blockIdx.x, S);
}

// Top-K rows and the tiles of one small GEMM (fp32 split-K partials, no
// gather) in one launch, the GEMM's workgroups first: the rows stream the
// logits at the HBM rate while the GEMM, held back by its loads' latency, runs
// on the workgroup slots the rows leave (three workgroups per CU).  Each GEMM
// workgroup takes one 64 x 64 tile of one k range with eight waves.
constexpr int kFuseStages = 3;
using FuseTile = DmaTile<64, 64, 2, 4, kFuseStages>;
constexpr size_t kFuseLds = RowLds<1>::kBytes > static_cast<size_t>(FuseTile::kStage) * kFuseStages
                                ? RowLds<1>::kBytes
                                : static_cast<size_t>(FuseTile::kStage) * kFuseStages;

template <int NV, int D>
__global__ void __launch_bounds__(kRowWaves * kWave, 6)   // three workgroups per CU
topk_gemm_kernel(const uint16_t* __restrict__ logits, int V, int K, int rounds, int32_t* __restrict__ ids,
                 float* __restrict__ vals, GemmDev p, int tiles_m, int tiles_n, int n_gemm, int cm, int cn,
                 int nseg, int seg_len, uint64_t* __restrict__ part) {
  __shared__ __align__(1024) char arena[kFuseLds];
  const int bid = blockIdx.x;
  if (bid < n_gemm) {
    constexpr int MW = FuseTile::MW, NWB = FuseTile::NWB, TM = FuseTile::TM, TN = FuseTile::TN;
    constexpr int kStage = FuseTile::kStage;
    // workgroups are dealt to the 8 XCDs in turn (blockIdx % 8).  With a
    // block shape (cm, cn), the cm cn XCDs of one k split each take a
    // (tiles_m / cm) x (tiles_n / cn) block of tiles, so the rows of A and of
    // W an XCD reads stay few next to the logits streaming through its L2;
    // otherwise, when the tiles divide evenly, XCD x takes a contiguous run
    // of (split, tm, tn)
    int tn, tm, zs;
    if (cm > 0) {
      const int x = bid % 8, j = bid / 8;
      const int bm = tiles_m / cm, bn = tiles_n / cn;
      const int q = x % (cm * cn);
      zs = x / (cm * cn);
      tm = (q / cn) * bm + j / bn;
      tn = (q % cn) * bn + j % bn;
    } else {
      int b = bid;
      if (n_gemm % 8 == 0) b = (bid % 8) * (n_gemm / 8) + bid / 8;
      tn = b % tiles_n;
      b /= tiles_n;
      tm = b % tiles_m;
      zs = b / tiles_m;
    }
    const int n0 = tn * 64;
    const int m0 = tm * 64;
    const int kbeg = zs * p.ksplit;
    const int kend = min(p.Kd, kbeg + p.ksplit);
    f32x4_t acc[TM][TN];
    dma_tile_mainloop<64, 64, 2, 4, kFuseStages>(p, m0, n0, kbeg, kend, arena, arena + kStage, arena + 2 * kStage,
                                                  arena, acc);
    const int l = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int wm = wv / 4;
    const int wn = wv % 4;
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int c = 0; c < TN; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm * MW + a * 16 + (l >> 4) * 4 + v;
          const int n = n0 + wn * NWB + c * 16 + (l & 15);
          if (m < p.M && n < p.N) p.out_f32[(static_cast<long long>(zs) * p.M + m) * p.ldo + n] = acc[a][c][v];
        }
    return;
  }
  const RowLds<1> S = RowLds<1>::carve(arena);
  topk_row_seg<NV, 1, D>(logits, V, K, rounds, ids, vals, nseg, seg_len, part, bid - n_gemm, S);
}

// Any other bf16 row: element loads, one segment at a time.
template <int NV, int G>
__global__ void __launch_bounds__(kRowWaves * kWave)
topk_bf16_row_unaligned_kernel(const uint16_t* __restrict__ logits, int V, int K, int rounds,
                               int32_t* __restrict__ ids, float* __restrict__ vals) {
  constexpr int kSegLen = kWave * NV * 8;
  const int row = blockIdx.x;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const uint16_t* rowp = logits + static_cast<size_t>(row) * V;

  static_assert(kRowWaves * G * kWave * 4 <= kRowWaves * kRowCap * 8, "group maxima fit the lists");
  __shared__ uint64_t s_cand[kRowWaves][kRowCap];
  __shared__ int32_t s_flag[kRowWaves][kFlagCap];
  __shared__ uint64_t s_best[kRowWaves * 64];
  __shared__ uint64_t s_fin[64];
  __shared__ int s_cnt[kRowWaves];
  uint32_t* s_gm = reinterpret_cast<uint32_t*>(&s_cand[0][0]);

  auto load = [&](int rd, uint32_t (&kw)[NV * 4]) {
    const int seg0 = (rd * kRowWaves + w) * kSegLen;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e0 = seg0 + (i * kWave + l) * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = e0 + 2 * q < V ? rowp[e0 + 2 * q] : 0xffffu;
        const uint32_t hi = e0 + 2 * q + 1 < V ? rowp[e0 + 2 * q + 1] : 0xffffu;
        kw[4 * i + q] = lo | (hi << 16);
      }
    }
  };
  {
    uint32_t kw[NV * 4];
    load(0, kw);
    uint32_t gmx[G];
    group_max<NV, G>(kw, gmx);
#pragma unroll
    for (int g = 0; g < G; ++g) s_gm[(w * G + g) * kWave + l] = gmx[g];
  }
  __syncthreads();
  const uint32_t t = row_bound<G>(s_gm, K, l);
  __syncthreads();

  int nseg = 0;
  int nflag = 0;
  for (int rd = 0; rd < rounds; ++rd) {
    const int seg0 = (rd * kRowWaves + w) * kSegLen;
    if (seg0 >= V) break;
    ++nseg;
    uint32_t kw[NV * 4];
    load(rd, kw);
    row_screen<NV>(kw, seg0, V, l, t, nflag, s_flag[w]);
  }
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
  const bool exact = nflag > kFlagCap || !row_collect<false>(rowp, V, t, s_flag[w], nflag, l, s_cand[w], cnt);
  row_finish<NV>(rowp, V, K, rounds, w, l, nseg, exact, cnt, s_cand, s_best, s_fin, s_cnt,
                 ids + static_cast<size_t>(row) * K, vals + static_cast<size_t>(row) * K);
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

// At most 32 rows (one or two draft blocks of 16 slots) leave most of the
// chip idle with a workgroup per row, each streaming its whole row: rows are
// then cut into up to 8 column segments (at most 256 workgroups in all; each
// segment at least 4096 columns, so it holds more than K), and a merge launch
// ranks each row's segment results.  Measured at 16 rows of 151936, the
// whole-path call took 43.0 us with 8 segments against 43.5 with 4, 44.3
// with 16 and 46.8 with whole rows.  From 64 rows on, the extra launch and
// the segments' finishing work cost more than the shorter streams save (a
// whole-path call at 64 to 256 rows was 2.4 to 4.6 us slower with segments),
// so those rows stay whole.
int topk_row_segments(int rows, int V) {
  if (rows <= 0 || rows > 32) return 1;
  const int s = std::min(std::min((256 + rows - 1) / rows, 8), V / 4096);
  return std::max(s, 1);
}

int topk_seg_len(int V, int nseg) { return ((V + nseg - 1) / nseg + 7) / 8 * 8; }

template <typename T>
int topk_nchunks(int V) {
  return (V + TopkShape<T>::kChunk - 1) / TopkShape<T>::kChunk;
}

// Each row's K best of its nch * K partial composites, sorted, values read
// back from the logits.
template <typename T>
hipError_t launch_topk_merge(const T* lg, int rows, int V, int K, int nch, const uint64_t* partial, int32_t* ids,
                             float* vals, hipStream_t st) {
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
    // aligned rows: kRegNV vectors per lane and segment, kRegD segments in
    // flight per wave; other rows: 8 vectors per lane, element loads
    if (vec) {
      const int rounds = (V + kRowWaves * kWave * kRegNV * 8 - 1) / (kRowWaves * kWave * kRegNV * 8);
      const int nseg = topk_row_segments(rows, V);
      const int seg_len = topk_seg_len(V, nseg);
#define DCOCO_ROW(GG)                                                                                   \
  hipLaunchKernelGGL((topk_bf16_row_reg_kernel<kRegNV, GG, kRegD>), dim3(rows * nseg), dim3(kRowWaves * kWave), 0, \
                     st, lb, V, K, rounds, ids, vals, nseg, seg_len, partial)
      if (G == 1) DCOCO_ROW(1);
      else if (G == 2) DCOCO_ROW(2);
      else DCOCO_ROW(4);
#undef DCOCO_ROW
      if (nseg > 1) return launch_topk_merge<T>(lg, rows, V, K, nseg, partial, ids, vals, st);
    } else {
      const int rounds = (V + kRowWaves * kWave * 8 * 8 - 1) / (kRowWaves * kWave * 8 * 8);
#define DCOCO_ROW(GG)                                                                                 \
  hipLaunchKernelGGL((topk_bf16_row_unaligned_kernel<8, GG>), dim3(rows), dim3(kRowWaves * kWave), 0, st, lb, \
                     V, K, rounds, ids, vals)
      if (G == 1) DCOCO_ROW(1);
      else if (G == 2) DCOCO_ROW(2);
      else DCOCO_ROW(4);
#undef DCOCO_ROW
    }
    return hipGetLastError();
  } else {
    if (vec)
      hipLaunchKernelGGL((topk_partial_kernel<T, true>), g1, dim3(kTopkThreads), 0, st, lg, V, K, nch, partial);
    else
      hipLaunchKernelGGL((topk_partial_kernel<T, false>), g1, dim3(kTopkThreads), 0, st, lg, V, K, nch, partial);
  }
  return launch_topk_merge<T>(lg, rows, V, K, nch, partial, ids, vals, st);
}

}  // namespace

bool topk_gemm_supported(int V, int K, const void* logits, const GemmProblem& q) {
  const bool vec = (static_cast<size_t>(V) * sizeof(uint16_t)) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(logits) % 16) == 0;
  return vec && K >= 1 && K <= 16 && q.a_dtype == kDtypeBf16 && q.w_dtype == kDtypeBf16 && q.a_rows == nullptr &&
         q.out == nullptr && q.out_f32 != nullptr && q.Kd % 64 == 0 && q.M >= 1 && q.N >= 1 && q.split >= 1;
}

int topk_gemm_workgroups(const GemmProblem& q) {
  return ((q.M + 63) / 64) * ((q.N + 63) / 64) * q.split;
}

int topk_gemm_row_workgroups(int rows, int V) { return rows * topk_row_segments(rows, V); }

hipError_t launch_topk_gemm(const void* logits, int rows, int V, int K, int32_t* ids, float* vals,
                            const GemmProblem& q, void* partial, hipStream_t st) {
  if (!topk_gemm_supported(V, K, logits, q)) return hipErrorInvalidValue;
  if (rows <= 0) return hipSuccess;
  const GemmDev p = gemm_dev(q, 64);
  const int tiles_m = (q.M + 63) / 64;
  const int tiles_n = (q.N + 63) / 64;
  const int n_gemm = tiles_m * tiles_n * q.split;
  const int rounds = (V + kRowWaves * kWave * kRegNV * 8 - 1) / (kRowWaves * kWave * kRegNV * 8);
  // the block shape with the fewest A and W rows per XCD: the 8 / split XCDs
  // of a k split factored as cm x cn, dividing the tile grid evenly
  int cm = 0, cn = 0;
  if (8 % q.split == 0) {
    const int c = 8 / q.split;
    int best = 1 << 30;
    for (int f = 1; f <= c; ++f) {
      if (c % f || tiles_m % f || tiles_n % (c / f)) continue;
      const int rows_x = tiles_m / f + tiles_n / (c / f);
      if (rows_x < best) { best = rows_x; cm = f; cn = c / f; }
    }
  }
  const int nseg = topk_row_segments(rows, V);
  const int seg_len = topk_seg_len(V, nseg);
  uint64_t* part = static_cast<uint64_t*>(partial);
  hipLaunchKernelGGL((topk_gemm_kernel<kRegNV, kRegD>), dim3(n_gemm + rows * nseg), dim3(kRowWaves * kWave), 0, st,
                     static_cast<const uint16_t*>(logits), V, K, rounds, ids, vals, p, tiles_m, tiles_n, n_gemm, cm,
                     cn, nseg, seg_len, part);
  if (nseg > 1)
    return launch_topk_merge<bf16>(static_cast<const bf16*>(logits), rows, V, K, nseg, part, ids, vals, st);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int dtype, int rows, int V, int K) {
  if (dtype == kDtypeBf16) {   // segment composites when the rows are cut (aligned rows only use them)
    const int nseg = topk_row_segments(rows, V);
    return nseg > 1 ? static_cast<size_t>(rows) * nseg * K * sizeof(uint64_t) : 0;
  }
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
