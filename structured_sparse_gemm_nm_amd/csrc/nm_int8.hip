// INT8 2:4: prune + pack, decompress, and the sparse GEMM on
// v_smfmac_i32_16x16x128_i8.
//
// The 2:4 pattern is also offered for INT8 weights; the index stays 2 bits per
// stored value (a 20-bit group, 37.5% smaller than dense) and the reduction
// length must be a multiple of 32 (COE-592 lecture 04-2, "M:N sparsity on
// NVIDIA tensor cores": opening section, and section "Where this sits among
// the three case studies").  Packed layout as for 16-bit weights: survivors of
// a row pushed left (one byte each), positions in a per-row LSB-first 2-bit
// stream of 32-bit words.  Magnitude is |w| as an integer (-128 ranks above
// 127), equal magnitudes go to the lower position; the product accumulates
// in int32 and is exact.
//
// Operand layout of v_smfmac_i32_16x16x128_i8 (lane l, li = l & 15,
// lq = l >> 4; found by running the instruction on random 2:4 data under each
// candidate layout and comparing with the exact product):
//   A  row li, survivors 16 lq .. 16 lq + 15 of the 128-wide K step (16
//      bytes), and its index register holds their 2-bit positions LSB-first:
//      exactly word 4 s + lq of the row's stored stream for step s;
//   B  token li, K 16 lq .. 16 lq + 15 and 64 + 16 lq .. 64 + 16 lq + 15;
//   D  element e is the product's row 4 lq + e, token li.
// So every operand is a plain 16- or 4-byte load of the stored data.
#include "nm_internal.h"

namespace nm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One group of four int8 weights (byte p = position p): the two kept
// positions, ascending, with their bytes.  Composite keys put |w| above the
// tie-break (the lower position wins), so they are distinct and a position is
// kept when fewer than two keys exceed its own.
__device__ inline void top2_of_4(uint32_t g, uint32_t& p0, uint32_t& p1, uint32_t& v0, uint32_t& v1) {
  uint32_t key[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int w = int(int8_t(uint8_t(g >> (8 * p))));
    key[p] = (uint32_t(w < 0 ? -w : w) << 2) | uint32_t(3 - p);
  }
  uint32_t kept = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int above = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) above += key[q] > key[p];
    kept |= uint32_t(above < 2) << p;
  }
  p0 = __builtin_ctz(kept);
  p1 = 31 - __builtin_clz(kept);
  v0 = (g >> (8 * p0)) & 0xFFu;
  v1 = (g >> (8 * p1)) & 0xFFu;
}

// One thread per 16-byte chunk of a row (four groups): 8 value bytes and the
// chunk's 16 index bits, which sit at byte 2c of the row's stream.
__global__ __launch_bounds__(256) void prune_pack_i8_kernel(const uint8_t* __restrict__ W, int64_t R,
                                                            int64_t K, int64_t ldw,
                                                            uint8_t* __restrict__ values,
                                                            uint32_t* __restrict__ idx, int64_t words) {
  const int64_t cpr = K >> 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= R * cpr) return;
  const int64_t r = i / cpr, c = i - r * cpr;
  const uint4 w = *reinterpret_cast<const uint4*>(W + r * ldw + c * 16);
  const uint32_t g4[4] = {w.x, w.y, w.z, w.w};
  uint32_t v[2] = {0u, 0u}, bits = 0u;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t p0, p1, v0, v1;
    top2_of_4(g4[g], p0, p1, v0, v1);
    v[g >> 1] |= (v0 | (v1 << 8)) << (16 * (g & 1));
    bits |= (p0 | (p1 << 2)) << (4 * g);
  }
  *reinterpret_cast<uint2*>(values + r * (K >> 1) + c * 8) = make_uint2(v[0], v[1]);
  *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(idx) + r * words * 4 + c * 2) = uint16_t(bits);
}

__global__ __launch_bounds__(256) void decompress_i8_kernel(const uint8_t* __restrict__ values,
                                                            const uint32_t* __restrict__ idx, int64_t R,
                                                            int64_t K, int64_t words,
                                                            uint8_t* __restrict__ W, int64_t ldw) {
  const int64_t cpr = K >> 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= R * cpr) return;
  const int64_t r = i / cpr, c = i - r * cpr;
  const uint2 v = *reinterpret_cast<const uint2*>(values + r * (K >> 1) + c * 8);
  const uint32_t bits =
      *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(idx) + r * words * 4 + c * 2);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t vv = (g < 2 ? v.x : v.y) >> (16 * (g & 1));
    const uint32_t p0 = (bits >> (4 * g)) & 3u, p1 = (bits >> (4 * g + 2)) & 3u;
    out[g] = ((vv & 0xFFu) << (8 * p0)) | (((vv >> 8) & 0xFFu) << (8 * p1));
  }
  *reinterpret_cast<uint4*>(W + r * ldw + c * 16) = make_uint4(out[0], out[1], out[2], out[3]);
}

// 128 x 128 tiles (rows x tokens), 4 waves as 2 x 2, each 64 x 64 = 4 x 4
// fragments; one 128-wide K step per instruction.  Operands go straight from
// global memory to registers (a lane's share of each is contiguous, see
// above), one step ahead in a second register set.  Rows and tokens past the
// edge reread the last one and are not stored; a lane's K range past K (K is
// a multiple of 32, so a range is wholly in or out) loads zeros.
constexpr int kBR8 = 128, kBT8 = 128;

__global__ __launch_bounds__(256) void spmm_i8_kernel(const uint8_t* __restrict__ values,
                                                      const uint32_t* __restrict__ idx, int R, int K,
                                                      int words, const uint8_t* __restrict__ act, int T,
                                                      int64_t ldx, int32_t* __restrict__ Y, int64_t ldy,
                                                      int tilesT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int R0 = (int(blockIdx.x) / tilesT) * kBR8 + (wave >> 1) * 64;
  const int T0 = (int(blockIdx.x) % tilesT) * kBT8 + (wave & 1) * 64;
  const int64_t S = K >> 1;
  const int nsteps = (K + 127) >> 7;

  const uint8_t* arow[4];
  const uint32_t* irow[4];
  const uint8_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(R0 + i * 16 + li, R - 1);
    arow[i] = values + int64_t(r) * S + 16 * lq;
    irow[i] = idx + int64_t(r) * words + lq;
    const int t = min(T0 + i * 16 + li, T - 1);
    brow[i] = act + int64_t(t) * ldx + 16 * lq;
  }

  auto load = [&](int s, i32x4 (&a)[4], uint32_t (&x)[4], i32x8 (&b)[4]) {
    const bool a_in = s * 128 + 32 * lq + 32 <= K;
    const bool b0_in = s * 128 + 16 * lq + 16 <= K;
    const bool b1_in = s * 128 + 64 + 16 * lq + 16 <= K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = a_in ? *reinterpret_cast<const i32x4*>(arow[i] + s * 64) : i32x4{0, 0, 0, 0};
      x[i] = a_in ? irow[i][s * 4] : 0u;
      const i32x4 lo = b0_in ? *reinterpret_cast<const i32x4*>(brow[i] + s * 128) : i32x4{0, 0, 0, 0};
      const i32x4 hi = b1_in ? *reinterpret_cast<const i32x4*>(brow[i] + s * 128 + 64) : i32x4{0, 0, 0, 0};
      b[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };

  i32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = i32x4{0, 0, 0, 0};
  auto mma = [&](const i32x4 (&a)[4], const uint32_t (&x)[4], const i32x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[i], b[j], acc[i][j], int(x[i]), 0, 0);
  };

  i32x4 a0[4], a1[4];
  uint32_t x0[4], x1[4];
  i32x8 b0[4], b1[4];
  load(0, a0, x0, b0);
  for (int s = 0; s < nsteps; s += 2) {
    if (s + 1 < nsteps) load(s + 1, a1, x1, b1);
    mma(a0, x0, b0);
    if (s + 1 < nsteps) {
      if (s + 2 < nsteps) load(s + 2, a0, x0, b0);
      mma(a1, x1, b1);
    }
  }

  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = R0 + i * 16 + 4 * lq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = T0 + j * 16 + li;
      if (t >= T || r >= R) continue;
      int32_t* y = Y + int64_t(t) * ldy + r;
      if (vec_ok && r + 3 < R) {
        *reinterpret_cast<i32x4*>(y) = acc[i][j];
      } else {
        for (int e = 0; e < 4 && r + e < R; ++e) y[e] = acc[i][j][e];
      }
    }
  }
}

}  // namespace

hipError_t launch_prune_pack_i8(const uint8_t* W, int64_t R, int64_t K, int64_t ldw, uint8_t* values,
                                uint32_t* idx, int64_t idx_row_words, hipStream_t s) {
  const int64_t chunks = R * (K >> 4);
  if (chunks <= 0) return hipSuccess;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(prune_pack_i8_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, W, R, K, ldw, values,
                     idx, idx_row_words);
  return hipGetLastError();
}

hipError_t launch_decompress_i8(const uint8_t* values, const uint32_t* idx, int64_t R, int64_t K,
                                int64_t idx_row_words, uint8_t* W, int64_t ldw, hipStream_t s) {
  const int64_t chunks = R * (K >> 4);
  if (chunks <= 0) return hipSuccess;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decompress_i8_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, values, idx, R, K,
                     idx_row_words, W, ldw);
  return hipGetLastError();
}

hipError_t launch_spmm_i8(const SpmmArgs& a, hipStream_t s) {
  const int64_t tilesR = (a.R + kBR8 - 1) / kBR8;
  const int64_t tilesT = (a.T + kBT8 - 1) / kBT8;
  if (tilesR * tilesT > 0x7FFFFFFF || a.R > 0x7FFFFFFF || a.T > 0x7FFFFFFF || a.K > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(spmm_i8_kernel, dim3(unsigned(tilesR * tilesT)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(a.values), a.idx, int(a.R), int(a.K),
                     int(a.idx_row_words), reinterpret_cast<const uint8_t*>(a.act), int(a.T), a.ldx,
                     static_cast<int32_t*>(a.Y), a.ldy, int(tilesT));
  return hipGetLastError();
}

}  // namespace nm
