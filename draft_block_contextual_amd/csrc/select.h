// Exact top-K selection over 64-bit composites held by one wave, shared by
// the top-K kernels and the fused LM-head top-K.  A composite is
// (key << 32) | (0xffffffff - id): larger keys first, equal keys to the lower
// id; composites are unique, so "the K largest" is a set without ties.
#pragma once
#include "common.h"

namespace dcoco {

__device__ __forceinline__ uint32_t comp_key(uint64_t c) { return static_cast<uint32_t>(c >> 32); }
__device__ __forceinline__ uint32_t comp_inv(uint64_t c) { return static_cast<uint32_t>(c); }
__device__ __forceinline__ uint64_t make_comp(uint32_t key, uint32_t id) {
  return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xffffffffu - id);
}

// Exact top-K of the composites c[0..Q) held by the lanes of one wave (0 =
// empty slot); KEYBITS is the width of the key half.  Marks the
// min(K, #non-empty) largest in sel[].  idbits bounds the ids (id < 2^idbits),
// so the inverted ids share their top 32 - idbits bits (all ones) and the
// tie-break search starts below them.
template <int Q, int KEYBITS>
__device__ void select_topk(const uint64_t (&c)[Q], int K, bool (&sel)[Q], int idbits = 32) {
  uint32_t tk = 0;
  for (int bit = KEYBITS - 1; bit >= 0; --bit) {
    const uint32_t cand = tk | (1u << bit);
    int cnt = 0;
    // an empty slot has key 0, below every candidate bound (cand >= 1)
#pragma unroll
    for (int q = 0; q < Q; ++q) cnt += __popcll(ballot(comp_key(c[q]) >= cand));
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
  uint32_t ti = idbits >= 32 ? 0u : (0xffffffffu << idbits);
  if (neq > need) {
    for (int bit = min(idbits, 32) - 1; bit >= 0; --bit) {
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

}  // namespace dcoco
