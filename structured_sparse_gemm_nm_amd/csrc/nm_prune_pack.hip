// Prune + pack and decompress kernels for N:M structured sparsity (gfx950).
//
// Prune rule: "M:N sparsity on NVIDIA tensor cores" (COE-592 lecture 04-2),
// section "The recipe", step 2 -- in every group of M weights along a row keep
// the N with the largest absolute value.  Magnitude is compared on the stored
// 16-bit pattern with the sign cleared; equal magnitudes go to the lower
// position.  Storage (same page, "Where this sits among the three case
// studies"): survivors pushed left into contiguous values; each survivor's
// in-group position stored as a b-bit field of an LSB-first per-row bitstream
// padded to whole 32-bit words.
//
// Thread mapping (2:4).  A lane position owns one 16-byte chunk (8
// consecutive weights) of a row, so a wavefront reads 1 KiB of W
// contiguously.  A workgroup covers 256 chunk positions of kRows consecutive
// rows: each thread issues the loads of its position in all kRows rows before
// selecting, and row and position come from the workgroup coordinates (no
// division).  A lane produces 8*N/M survivors and BPL = 8*N/M*b index bits.
// The smallest run of lanes whose bits fill whole words (L = 32 / gcd(BPL, 32)
// lanes -> L*BPL/32 words) assembles its words with an OR-reduction over
// cross-lane shuffles; rows are padded to a multiple of L lanes so a run never
// spans two rows.
//
// 1:4 and 1:8 carry only 4 or 3 index bits per chunk, so one chunk per lane
// would take runs of 8 or 32 lanes (3 or 5 shuffle stages per word).  There
// the workgroup stages its chunks in LDS after the same coalesced loads, and
// a thread selects kQ = 4 consecutive chunks of one row: 16 or 12 bits per
// thread, runs of 2 or 8 threads, and one 16- or 8-byte value store per run
// (measured on 4096 x 4096 fp16: 1:8 10.1 -> 7.7 us, 1:4 8.1 -> 7.8 us; 2:4
// keeps one chunk per lane, where the LDS round trip costs more than its two
// shuffle stages).
#include "nm_internal.h"
#include "nm_select.h"

namespace nm {
namespace {

template <int N, int M>
struct PackShape {
  static constexpr int B = (M <= 2) ? 1 : (M <= 4) ? 2 : 3;      // index bits
  static constexpr int GPL = 8 / M;                              // groups per lane
  static constexpr int SPL = GPL * N;                            // survivors per lane
  static constexpr int BPL = SPL * B;                            // index bits per lane
  static constexpr int GCD = (BPL % 32 == 0) ? 32 : (BPL % 16 == 0) ? 16 : (BPL % 8 == 0) ? 8
                             : (BPL % 4 == 0) ? 4 : (BPL % 2 == 0) ? 2 : 1;
  static constexpr int L = 32 / GCD;                             // lanes per word run
  static constexpr int WPR = L * BPL / 32;                       // words per run
};

constexpr int kQ = 4;      // consecutive chunks a thread selects from

template <int N, int M>
struct RunShape {
  static constexpr int B = (M <= 2) ? 1 : (M <= 4) ? 2 : 3;      // index bits
  static constexpr int GPC = 8 / M;                              // groups per chunk
  static constexpr int SPC = GPC * N;                            // survivors per chunk
  static constexpr int BPC = SPC * B;                            // index bits per chunk
  static constexpr int BPL = kQ * BPC;                           // index bits per thread
  static constexpr int GCD = (BPL % 32 == 0) ? 32 : (BPL % 16 == 0) ? 16 : (BPL % 8 == 0) ? 8
                             : (BPL % 4 == 0) ? 4 : (BPL % 2 == 0) ? 2 : 1;
  static constexpr int L = 32 / GCD;                             // threads per word run
  static constexpr int WPR = L * BPL / 32;                       // words per run
  static_assert(BPL <= 32, "a thread's index bits fit one register");
};

constexpr int kRows = 4;   // rows per workgroup (chunks per thread)

// Prune and pack chunk c of row r (loaded into w).
template <int N, int M>
__device__ inline void pack_chunk(const uint32_t (&w)[4], int64_t r, int64_t c, int64_t R, int64_t K,
                                  uint16_t* __restrict__ values, uint32_t* __restrict__ idx,
                                  int64_t idx_row_words) {
  using PS = PackShape<N, M>;
  const int64_t chunks = K / 8;
  const bool live = (r < R) && (c < chunks);
  uint32_t lane_idx = 0;        // this lane's BPL index bits, survivor order
  uint32_t kept[2];
  select_chunk<N, M>(w, kept, lane_idx);

  // Values: SPL consecutive halves at survivor offset c*SPL of the row.
  if (live) {
    const int64_t S = K / M * N;
    uint16_t* dst = values + r * S + c * PS::SPL;
    if constexpr (PS::SPL == 4) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(kept[0], kept[1]);
    } else if constexpr (PS::SPL == 2) {
      *reinterpret_cast<uint32_t*>(dst) = kept[0];
    } else {
      *dst = uint16_t(kept[0]);
    }
  }

  // Index words: OR-reduce each word's contributions over the L-lane run.
  const int li = int(c % PS::L);           // lane position inside its run
  const int off = li * PS::BPL;            // bit offset inside the run
  const uint32_t mine = live ? lane_idx : 0u;
#pragma unroll
  for (int wd = 0; wd < PS::WPR; ++wd) {
    const int sh = off - 32 * wd;
    uint32_t part = 0;
    if (sh >= 0 && sh < 32) part = mine << sh;
    else if (sh < 0 && sh > -PS::BPL) part = mine >> (-sh);
#pragma unroll
    for (int d = 1; d < PS::L; d <<= 1) part |= uint32_t(__shfl_xor(int(part), d, 64));
    if (li == wd && r < R) {
      const int64_t word = (c - li) * PS::BPL / 32 + wd;
      if (word < idx_row_words) idx[r * idx_row_words + word] = part;
    }
  }
}

// A row takes 2^shift chunk positions: shift 8 when it has 256 chunks or
// more (position c = 256 blockIdx.x + threadIdx.x); shorter rows are padded to
// a power of two (at least L) and 256 >> shift of them share a workgroup, in
// row slots threadIdx.x >> shift.  The workgroup walks the row groups
// blockIdx.y, + gridDim.y, ... (kRows row slots each).  Positions past the
// row's chunks (or rows past R) load nothing but still take part in the
// cross-lane reductions; a row's positions start on a multiple of L, so every
// L-lane run stays inside one row.
template <int N, int M>
__global__ __launch_bounds__(256) void prune_pack_kernel(const uint16_t* __restrict__ W, int64_t R,
                                                         int64_t K, int64_t ldw, int shift,
                                                         uint16_t* __restrict__ values,
                                                         uint32_t* __restrict__ idx,
                                                         int64_t idx_row_words) {
  const int per_wg = 256 >> shift;                      // rows side by side in a workgroup
  const int64_t c = int64_t(blockIdx.x) * 256 + (threadIdx.x & ((1 << shift) - 1));
  const int sub = threadIdx.x >> shift;
  const int64_t chunks = K / 8;
  for (int64_t g = blockIdx.y; g * kRows * per_wg < R; g += gridDim.y) {
    const int64_t r0 = g * kRows * per_wg + sub;
    uint32_t w[kRows][4];
#pragma unroll
    for (int p = 0; p < kRows; ++p) {
      const int64_t r = r0 + int64_t(p) * per_wg;
      w[p][0] = w[p][1] = w[p][2] = w[p][3] = 0u;
      if (r < R && c < chunks) {
        const uint4 v = *reinterpret_cast<const uint4*>(W + r * ldw + c * 8);
        w[p][0] = v.x; w[p][1] = v.y; w[p][2] = v.z; w[p][3] = v.w;
      }
    }
#pragma unroll
    for (int p = 0; p < kRows; ++p)
      pack_chunk<N, M>(w[p], r0 + int64_t(p) * per_wg, c, R, K, values, idx, idx_row_words);
  }
}

// Prune and pack chunks c .. c+kQ-1 of row r (w[q] holds chunk c+q).
template <int N, int M>
__device__ inline void pack_run(const uint32_t (&w)[kQ][4], int64_t r, int64_t c, int64_t R, int64_t K,
                                uint16_t* __restrict__ values, uint32_t* __restrict__ idx,
                                int64_t idx_row_words) {
  using PS = RunShape<N, M>;
  const int64_t chunks = K / 8;
  const bool row_live = r < R;
  uint32_t bits = 0;            // this thread's BPL index bits, survivor order
  uint32_t kept[kQ][2];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    uint32_t lane_idx = 0;
    select_chunk<N, M>(w[q], kept[q], lane_idx);
    if (row_live && c + q < chunks) bits |= lane_idx << (q * PS::BPC);
  }

  // Values: kQ*SPC consecutive halves at survivor offset c*SPC of the row.
  if (row_live && c < chunks) {
    const int64_t S = K / M * N;
    uint16_t* dst = values + r * S + c * PS::SPC;
    // one store for the whole run when it is aligned for it (1:4 and 1:8 rows
    // start only 8- / 4-byte aligned when K % 32 == 16)
    constexpr uintptr_t kRunBytes = kQ * PS::SPC * 2;
    constexpr uintptr_t kAlign = kRunBytes < 16 ? kRunBytes : 16;
    if (c + kQ <= chunks && (reinterpret_cast<uintptr_t>(dst) & (kAlign - 1)) == 0) {
      if constexpr (PS::SPC == 4) {
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(kept[0][0], kept[0][1], kept[1][0], kept[1][1]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(kept[2][0], kept[2][1], kept[3][0], kept[3][1]);
      } else if constexpr (PS::SPC == 2) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(kept[0][0], kept[1][0], kept[2][0], kept[3][0]);
      } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2((kept[0][0] & 0xFFFFu) | (kept[1][0] << 16),
                                                    (kept[2][0] & 0xFFFFu) | (kept[3][0] << 16));
      }
    } else {
      // the row ends inside the run, or the run is not aligned for one store
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (c + q >= chunks) break;
        if constexpr (PS::SPC == 4) {
          *reinterpret_cast<uint2*>(dst + q * 4) = make_uint2(kept[q][0], kept[q][1]);
        } else if constexpr (PS::SPC == 2) {
          *reinterpret_cast<uint32_t*>(dst + q * 2) = kept[q][0];
        } else {
          dst[q] = uint16_t(kept[q][0]);
        }
      }
    }
  }

  // Index words: OR-reduce each word's contributions over the L-thread run.
  const int li = int((c / kQ) % PS::L);    // thread position inside its run
  const int off = li * PS::BPL;            // bit offset inside the run
#pragma unroll
  for (int wd = 0; wd < PS::WPR; ++wd) {
    const int sh = off - 32 * wd;
    uint32_t part = 0;
    if (sh >= 0 && sh < 32) part = bits << sh;
    else if (sh < 0 && sh > -PS::BPL) part = bits >> (-sh);
#pragma unroll
    for (int d = 1; d < PS::L; d <<= 1) part |= uint32_t(__shfl_xor(int(part), d, 64));
    if (li == wd && row_live) {
      const int64_t word = (c / kQ - li) * PS::BPL / 32 + wd;
      if (word < idx_row_words) idx[r * idx_row_words + word] = part;
    }
  }
}

// 1:4 and 1:8.  A row takes 2^shift chunk positions: shift 8 when it has 256
// chunks or more (position c = 256 blockIdx.x + lane position); shorter rows
// are padded to a power of two (at least kQ*L) and 256 >> shift of them share
// a workgroup, in row slots t >> shift.  The workgroup walks the row groups
// blockIdx.y, + gridDim.y, ... (kRows row slots each): every thread loads its
// position in the kRows rows into LDS, then thread t selects positions
// 4(t % 64) .. +3 of row slot t / 64 of the tile.  Positions past the row's
// chunks (or rows past R) load zeros and store nothing but still take part in
// the cross-lane reductions; a row's positions start on a multiple of kQ*L,
// so every L-thread run stays inside one row.
template <int N, int M>
__global__ __launch_bounds__(256) void prune_pack_run_kernel(const uint16_t* __restrict__ W, int64_t R,
                                                         int64_t K, int64_t ldw, int shift,
                                                         uint16_t* __restrict__ values,
                                                         uint32_t* __restrict__ idx,
                                                         int64_t idx_row_words) {
  __shared__ uint4 tile[kRows * 256];                  // [row slot p][position]
  const int per_wg = 256 >> shift;                      // rows side by side in a workgroup
  const int mask = (1 << shift) - 1;
  const int t = threadIdx.x;
  const int64_t chunks = K / 8;
  // loads: position t of each row slot
  const int64_t lc = int64_t(blockIdx.x) * 256 + (t & mask);
  const int lsub = t >> shift;
  // selection: positions 4j .. 4j+3 of row slot p
  const int p_sel = t >> 6, j = t & 63;
  const int64_t sc = int64_t(blockIdx.x) * 256 + ((kQ * j) & mask);
  const int ssub = (kQ * j) >> shift;
  for (int64_t g = blockIdx.y; g * kRows * per_wg < R; g += gridDim.y) {
    const int64_t base = g * kRows * per_wg;
    uint4 v[kRows];
#pragma unroll
    for (int p = 0; p < kRows; ++p) {
      const int64_t r = base + lsub + int64_t(p) * per_wg;
      v[p] = make_uint4(0u, 0u, 0u, 0u);
      if (r < R && lc < chunks) v[p] = *reinterpret_cast<const uint4*>(W + r * ldw + lc * 8);
    }
    __syncthreads();  // the previous row group's selection is done with the tile
#pragma unroll
    for (int p = 0; p < kRows; ++p) tile[p * 256 + t] = v[p];
    __syncthreads();
    uint32_t w[kQ][4];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const uint4 x = tile[p_sel * 256 + kQ * j + q];
      w[q][0] = x.x; w[q][1] = x.y; w[q][2] = x.z; w[q][3] = x.w;
    }
    pack_run<N, M>(w, base + ssub + int64_t(p_sel) * per_wg, sc, R, K, values, idx, idx_row_words);
  }
}

// Decompress: one lane writes one 16-byte chunk (8 dense positions).
template <int N, int M>
__global__ __launch_bounds__(256) void decompress_kernel(const uint16_t* __restrict__ values,
                                                         const uint32_t* __restrict__ idx, int64_t R,
                                                         int64_t K, int64_t idx_row_words,
                                                         uint16_t* __restrict__ Wout, int64_t ldw) {
  using PS = PackShape<N, M>;
  const int64_t chunks = K / 8;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t r = gid / chunks;
  const int64_t c = gid - r * chunks;
  if (r >= R) return;
  const int64_t S = K / M * N;
  const uint32_t* irow = idx + r * idx_row_words;
  const int64_t bit0 = c * PS::BPL;
  const int64_t wi = bit0 >> 5;
  const int sh = int(bit0 & 31);
  uint64_t both = irow[wi];
  if (sh + PS::BPL > 32 && wi + 1 < idx_row_words) both |= uint64_t(irow[wi + 1]) << 32;
  const uint32_t lane_idx = uint32_t(both >> sh);
  uint32_t outv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < PS::SPL; ++s) {
    const int g = s / N;
    const int p = int((lane_idx >> (s * PS::B)) & ((1u << PS::B) - 1));
    const uint32_t v = values[r * S + c * PS::SPL + s];
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (p == i) outv[g * M + i] = v;
  }
  uint4 o;
  o.x = outv[0] | (outv[1] << 16);
  o.y = outv[2] | (outv[3] << 16);
  o.z = outv[4] | (outv[5] << 16);
  o.w = outv[6] | (outv[7] << 16);
  *reinterpret_cast<uint4*>(Wout + r * ldw + c * 8) = o;
}

template <int N, int M>
hipError_t prune_pack_t(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, uint16_t* values,
                        uint32_t* idx, int64_t idx_row_words, hipStream_t s) {
  constexpr bool kRun = !(N == 2 && M == 4);
  // chunk positions one word run covers
  constexpr int RUN = kRun ? kQ * RunShape<N, M>::L : PackShape<N, M>::L;
  static_assert(256 % RUN == 0, "runs inside a segment");
  const int64_t chunks = K / 8;
  const int64_t segs = (chunks + 255) / 256;
  if (segs > 0x7FFFFFFF) return hipErrorInvalidValue;
  // positions per row: 2^shift, the least power of two >= chunks and >= RUN, at most 256
  int shift = 8;
  while (shift > 0 && (int64_t(1) << (shift - 1)) >= chunks && (1 << (shift - 1)) >= RUN) --shift;
  const int64_t rows_per_group = int64_t(kRows) * (256 >> shift);
  const int64_t groups = (R + rows_per_group - 1) / rows_per_group;
  const unsigned gy = unsigned(groups < 65535 ? groups : 65535);   // grid-stride beyond
  if constexpr (kRun)
    hipLaunchKernelGGL((prune_pack_run_kernel<N, M>), dim3(unsigned(segs), gy), dim3(256), 0,
                       s, W, R, K, ldw, shift, values, idx, idx_row_words);
  else
    hipLaunchKernelGGL((prune_pack_kernel<N, M>), dim3(unsigned(segs), gy), dim3(256), 0,
                       s, W, R, K, ldw, shift, values, idx, idx_row_words);
  return hipGetLastError();
}

template <int N, int M>
hipError_t decompress_t(const uint16_t* values, const uint32_t* idx, int64_t R, int64_t K,
                        int64_t idx_row_words, uint16_t* W, int64_t ldw, hipStream_t s) {
  const int64_t threads = R * (K / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decompress_kernel<N, M>), dim3(unsigned(blocks)), dim3(256), 0, s, values, idx,
                     R, K, idx_row_words, W, ldw);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prune_pack(const uint16_t* W, int64_t R, int64_t K, int64_t ldw, int n, int m,
                             uint16_t* values, uint32_t* idx, int64_t idx_row_words,
                             hipStream_t s) {
  if (n == 2 && m == 4) return prune_pack_t<2, 4>(W, R, K, ldw, values, idx, idx_row_words, s);
  if (n == 1 && m == 4) return prune_pack_t<1, 4>(W, R, K, ldw, values, idx, idx_row_words, s);
  if (n == 1 && m == 8) return prune_pack_t<1, 8>(W, R, K, ldw, values, idx, idx_row_words, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decompress(const uint16_t* values, const uint32_t* idx, int64_t R, int64_t K,
                             int n, int m, int64_t idx_row_words, uint16_t* W, int64_t ldw,
                             hipStream_t s) {
  if (n == 2 && m == 4) return decompress_t<2, 4>(values, idx, R, K, idx_row_words, W, ldw, s);
  if (n == 1 && m == 4) return decompress_t<1, 4>(values, idx, R, K, idx_row_words, W, ldw, s);
  if (n == 1 && m == 8) return decompress_t<1, 8>(values, idx, R, K, idx_row_words, W, ldw, s);
  return hipErrorInvalidValue;
}

}  // namespace nm
