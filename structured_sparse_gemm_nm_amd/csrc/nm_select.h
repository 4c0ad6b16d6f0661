// Magnitude selection of N survivors per group of M on one 16-byte chunk
// (eight 16-bit weights): shared by the N:M pack and the hybrid-tile pack, so
// both keep exactly the same weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nm {

// Composite key of element i (0..7) of a chunk held in w[4]: the magnitude
// key (the 16-bit pattern with the sign cleared) above the tie-break
// M-1-(i mod M).  Keys of one group are distinct and a larger composite key
// wins: larger magnitude first, then the lower position.
template <int M>
__device__ inline uint32_t ckey(const uint32_t (&w)[4], int i) {
  const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : w[i >> 1];
  return ((h & 0x7FFFu) << 3) | uint32_t(M - 1 - (i % M));
}

// Position (0..M-1) encoded in a composite key.
template <int M>
__device__ inline uint32_t ckey_pos(uint32_t k) { return uint32_t(M - 1) - (k & 7u); }

// Byte selector for v_perm picking element p (0..3) of the dword pair
// {hi, lo} into the low half and element q into the high half.
__device__ inline uint32_t pick2(uint32_t p, uint32_t q) {
  return (p * 0x0202u + 0x0100u) | ((q * 0x0202u + 0x0100u) << 16);
}

// The chunk's survivors, pushed left (vals: SPL halves, two per dword) and
// their in-group positions in survivor order (BPL bits).  Selection works on
// the composite keys with min / max; survivors come out in ascending
// position order.
template <int N, int M>
__device__ inline void select_chunk(const uint32_t (&w)[4], uint32_t (&vals)[2], uint32_t& lane_idx) {
  if constexpr (N == 2 && M == 4) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t a = ckey<4>(w, 4 * g), b = ckey<4>(w, 4 * g + 1);
      const uint32_t c = ckey<4>(w, 4 * g + 2), d = ckey<4>(w, 4 * g + 3);
      const uint32_t hi1 = max(a, b), lo1 = min(a, b), hi2 = max(c, d), lo2 = min(c, d);
      const uint32_t k1 = max(hi1, hi2);                       // largest
      const uint32_t k2 = max(min(hi1, hi2), max(lo1, lo2));   // second largest
      const uint32_t p1 = ckey_pos<4>(k1), p2 = ckey_pos<4>(k2);
      const uint32_t pl = min(p1, p2), ph = max(p1, p2);
      vals[g] = __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], pick2(pl, ph));
      lane_idx |= (pl | (ph << 2)) << (4 * g);
    }
  } else if constexpr (N == 1 && M == 4) {
    uint32_t v[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint32_t k = max(max(ckey<4>(w, 4 * g), ckey<4>(w, 4 * g + 1)),
                             max(ckey<4>(w, 4 * g + 2), ckey<4>(w, 4 * g + 3)));
      const uint32_t p = ckey_pos<4>(k);
      v[g] = __builtin_amdgcn_perm(w[2 * g + 1], w[2 * g], pick2(p, p));
      lane_idx |= p << (2 * g);
    }
    vals[0] = (v[0] & 0xFFFFu) | (v[1] << 16);
    vals[1] = 0u;
  } else {
    static_assert(N == 1 && M == 8, "2:4, 1:4 or 1:8");
    uint32_t k = ckey<8>(w, 0);
#pragma unroll
    for (int i = 1; i < 8; ++i) k = max(k, ckey<8>(w, i));
    const uint32_t p = ckey_pos<8>(k);
    const uint32_t q = p & 3u;
    const uint32_t lo = __builtin_amdgcn_perm(w[1], w[0], pick2(q, q));
    const uint32_t hi = __builtin_amdgcn_perm(w[3], w[2], pick2(q, q));
    vals[0] = (p < 4 ? lo : hi) & 0xFFFFu;
    vals[1] = 0u;
    lane_idx = p;
  }
}

}  // namespace nm
