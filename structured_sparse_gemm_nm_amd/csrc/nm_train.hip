// Training-side products of an N:M layer on gfx950.
//
// Source: COE-592 lecture 04-2, "M:N sparsity on NVIDIA tensor cores",
// section "The recipe", step 3 (retrain with the zeros held fixed, so the
// pattern survives), and the RNM-TD3 abstract of thelatestinai.com's
// "Structured Sparsity" cards (row-wise N:M kept throughout training).  With
// G = dL/dYt [T, R] (the forward output's layout):
//   dX[T, K]  = G W_nm                          (nm_spmm_dx, this file);
//   dW[R, S]  = sum_t G[t, r] act[t, k(r, s)]   (nm_spmm_dw), the gradient of
//               each stored survivor, in the packed layout.
// In dX the reduction runs over R, across the rows of W, so the N:M groups
// (which run along K) give the instruction nothing to skip: the product is
// dense on the MFMA and what the packed form saves is the weight bytes read.
//
// LDS transpose reads.  ds_read_b64_tr_b16 reads 4 halves per lane like a
// plain 64-bit read and then exchanges them within each group of 16 lanes:
// lane 16g + 4a + b receives element b of what lane 16g + 4j + a read, for
// j = 0..3 (measured on the MI355X with a probe of the instruction).  So
// when lane 16g + 4j + a points at row 8g + j (plus 4 for a second read),
// columns 4a..4a+3, of a tile stored reduction-major (rows = reduction),
// lane 16g + 4a + b gets rows 8g..8g+7 of column 4a + b: the 8 consecutive
// reduction elements of one column that a v_mfma_f32_16x16x32 operand lane
// (column 4a + b, quarter g) holds.  Tiles that arrive reduction-major (the
// decompressed W for dX, G and act for dW) feed the MFMA through two such
// reads per operand, without a transposing copy.
#include "nm_device.h"
#include "nm_internal.h"

#include <algorithm>
#include <type_traits>

namespace nm {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ inline u32x2 lds_read_tr(const unsigned char* p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(u32x2, v);
}

constexpr int pat_n(int P) { return P == 0 ? 2 : 1; }
constexpr int pat_m(int P) { return P == 2 ? 8 : 4; }

// ---------------------------------------------------------------------------
// dX = G W_nm, computed as dX^T tiles: D[k][t] = sum_r W[r][k] G[t][r].
//
// A workgroup (4 waves, 2 x 2) owns 128 k x 128 t; a wave 64 x 64 (4 x 4
// fragments).  R is walked in chunks of 64 rows, each staged in LDS:
//   * G's tile (128 tokens x 64 r, 16 KB), 4 16-byte pieces per thread,
//     loaded into registers two chunks ahead and written to a double-buffered
//     stage, slot (token, 16-byte chunk c) at token*8 + (c ^ (token & 7)); a
//     B operand lane (token i, quarter q) reads chunk 4h + q of sub-step h
//     (r 32h + 8q ..) with one 16-byte read;
//   * W's chunk (64 rows x 128 columns) is decompressed by the workgroup's
//     256 threads, each one row and 32 columns, from packed values and index
//     bits it loaded into registers two chunks earlier, into a dense
//     double-buffered tile [64 r][128 k] (rows padded to 288 bytes); the A
//     operands (k rows, r reduction) come out of it by transpose reads.
// The stages are filled from registers, not by direct global->LDS loads: the
// compiler cannot tell which LDS bytes a transpose read touches, so after a
// direct load it would hold every transpose read until that load landed.
// One barrier per chunk publishes the chunk's stage and tile (written in the
// previous step) and retires the ones the step then refills.  At 68 KB of
// LDS two workgroups share a compute unit, each covering the other's barrier
// and epilogue.
// ---------------------------------------------------------------------------
constexpr int kDxBK = 128, kDxBT = 128, kDxRC = 64;
constexpr int kDxGStage = kDxBT * kDxRC * 2;     // 16 KB
constexpr int kDxWRow = kDxBK * 2 + 32;          // 288 bytes: padded row of the W tile
constexpr int kDxWTile = kDxRC * kDxWRow;        // 18 KB
constexpr int kDxLds = 2 * kDxGStage + 2 * kDxWTile;

// One thread's packed share of a chunk: values of 32 columns of one row
// (2:4 16 values, 1:4 8, 1:8 4) and the two index words holding its bits.
struct DxPack {
  u32x4 v0, v1;
  uint32_t i0, i1;
};

// Offset that no descriptor here covers: a load from it returns zeros.
constexpr uint32_t kDeadOff = 0xFFFFFFF0u;

template <int P>
__device__ inline void dx_load(DxPack& d, __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t ri, uint32_t voff,
                               uint32_t ioff0, uint32_t ioff1) {
  if constexpr (P == 0) {
    d.v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
    // a dead share stays dead: kDeadOff + 16 would wrap to offset 0, and row
    // 0's values with zero index bits expand (two halves OR'ed into one
    // position) into arbitrary bits, Inf and NaN among them
    const uint32_t voff1 = voff == kDeadOff ? kDeadOff : voff + 16u;
    d.v1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff1, 0, 0));
  } else if constexpr (P == 1) {
    d.v0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, 0, 0));
  } else {
    const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff, 0, 0));
    d.v0 = u32x4{t[0], t[1], 0u, 0u};
  }
  d.i0 = __builtin_amdgcn_raw_buffer_load_b32(ri, ioff0, 0, 0);
  d.i1 = __builtin_amdgcn_raw_buffer_load_b32(ri, ioff1, 0, 0);
}

// The 32 dense halves (16 dwords) of a thread's row segment from its packed
// share; ishift is the position of its first index bit in word i0.
template <int P>
__device__ inline void dx_expand(const DxPack& d, uint32_t ishift, uint32_t (&o)[16]) {
  const uint64_t bits = (uint64_t(d.i1) << 32 | d.i0) >> ishift;
  if constexpr (P == 0) {  // 8 groups of 4, two values each
    const uint32_t v[8] = {d.v0[0], d.v0[1], d.v0[2], d.v0[3], d.v1[0], d.v1[1], d.v1[2], d.v1[3]};
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t p0 = uint32_t(bits >> (4 * g)) & 3u, p1 = uint32_t(bits >> (4 * g + 2)) & 3u;
      const uint64_t w = (uint64_t(v[g] & 0xFFFFu) << (16 * p0)) | (uint64_t(v[g] >> 16) << (16 * p1));
      o[2 * g] = uint32_t(w);
      o[2 * g + 1] = uint32_t(w >> 32);
    }
  } else if constexpr (P == 1) {  // 8 groups of 4, one value each
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t h = (d.v0[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
      const uint32_t p = uint32_t(bits >> (2 * g)) & 3u;
      const uint64_t w = uint64_t(h) << (16 * p);
      o[2 * g] = uint32_t(w);
      o[2 * g + 1] = uint32_t(w >> 32);
    }
  } else {  // 4 groups of 8, one value each
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t h = (d.v0[g >> 1] >> (16 * (g & 1))) & 0xFFFFu;
      const uint32_t p = uint32_t(bits >> (3 * g)) & 7u;
      const uint32_t x = h << (16 * (p & 1));
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * g + e] = (p >> 1) == uint32_t(e) ? x : 0u;
    }
  }
}

template <int P, int DT, int OUT>
__global__ __launch_bounds__(256, 2) void spmm_dx_kernel(const uint16_t* __restrict__ values, uint32_t values_bytes,
                                                      const uint32_t* __restrict__ idx, uint32_t idx_bytes, int R,
                                                      int K, int idx_row_words, const uint16_t* __restrict__ G,
                                                      int T, int64_t ldg, void* __restrict__ dX, int64_t lddx,
                                                      int tilesK, int tilesT, int group) {
  constexpr int N = pat_n(P), M = pat_m(P);
  constexpr int B = P == 2 ? 3 : 2;  // index bits per survivor
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* gbuf = smem;                          // [2][16 KB]
  unsigned char* wbuf = smem + 2 * kDxGStage;          // [2][64][288 B]

  int tk, tt;
  grouped_tile(xcd_tile(blockIdx.x, gridDim.x), tilesK, tilesT, group, tk, tt);
  const int K0 = tk * kDxBK, T0 = tt * kDxBT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 1, wt = wave & 1;
  const int li = lane & 15, lq = lane >> 4;
  const int nchunks = (R + kDxRC - 1) / kDxRC;
  const int64_t S = int64_t(K) * N / M;

  // G: descriptor over the tile's token rows (rows past T reread row T - 1;
  // their outputs are dropped).  R % 8 == 0, so a 16-byte piece of a row lies
  // wholly before R or wholly past it; pieces past R read zeros, which meet
  // the zero rows of W's tile past R.
  const int tlast = min(T0 + kDxBT, T) - 1;
  const __amdgpu_buffer_rsrc_t rg =
      make_rsrc(G + int64_t(T0) * ldg, uint32_t((int64_t(tlast - T0) * ldg + R) * 2));
  // this thread's 4 pieces of a chunk: LDS slot gslot[j] = (wave*4 + j)*64 +
  // lane, holding (token, 16-byte chunk c) of the tile
  uint32_t goff[4];
  int gcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int tok = slot >> 3;
    const int c = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1) - T0;
    goff[j] = uint32_t(t) * uint32_t(ldg) * 2u + uint32_t(c) * 16u;
    gcol[j] = c * 8;
  }
  auto load_g = [&](int chunk, u32x4 (&gr)[4]) {
    const int r0 = chunk * kDxRC;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // a piece past R (or of a chunk past the last) reads zeros
      const bool live = chunk < nchunks && r0 + gcol[j] < R;
      gr[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, live ? goff[j] + uint32_t(r0) * 2u : kDeadOff, 0, 0));
    }
  };
  auto write_g = [&](int stage, const u32x4 (&gr)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(gbuf + stage * kDxGStage + ((wave * 4 + j) * 64 + lane) * 16) = gr[j];
  };

  // W: this thread decompresses row (tid >> 2) of the chunk, columns
  // K0 + 32 (tid & 3) .. +31
  const int wr = tid >> 2, wc = tid & 3;
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx, idx_bytes);
  const int kc = K0 + 32 * wc;                      // first column of the segment
  const int64_t s0 = int64_t(kc) * N / M;           // its first survivor in the row
  const int64_t bit0 = s0 * B;                      // its first index bit in the row
  const uint32_t ishift = uint32_t(bit0 & 31);
  // the word holding the first bit and the next one, clamped to the row (the
  // row's last word then holds every bit the segment needs)
  const int64_t w0 = bit0 >> 5, w1 = min(w0 + 1, int64_t(idx_row_words) - 1);
  auto pack_offsets = [&](int chunk, uint32_t& voff, uint32_t& ioff0, uint32_t& ioff1) {
    const int64_t row = int64_t(chunk) * kDxRC + wr;
    const bool live = chunk < nchunks && row < R && kc < K;
    voff = live ? uint32_t((row * S + s0) * 2) : kDeadOff;
    ioff0 = live ? uint32_t((row * idx_row_words + w0) * 4) : kDeadOff;
    ioff1 = live ? uint32_t((row * idx_row_words + w1) * 4) : kDeadOff;
  };
  auto decompress = [&](const DxPack& d, int buf) {
    uint32_t o[16];
    dx_expand<P>(d, ishift, o);
    unsigned char* dst = wbuf + buf * kDxWTile + wr * kDxWRow + wc * 64;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(dst + 16 * q) = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A operand addresses in the W tile: lane L = 16g + 4j + a reads row
  // 8g + j (+4) of the sub-step, columns 4a.. of fragment kf
  const int tr_row = 8 * (lane >> 4) + ((lane >> 2) & 3), tr_col = 4 * (lane & 3);
  auto read_a = [&](int buf, int h, int kf) {
    const unsigned char* base =
        wbuf + buf * kDxWTile + (32 * h + tr_row) * kDxWRow + (wk * 64 + kf * 16 + tr_col) * 2;
    const u32x2 lo = lds_read_tr(base), hi = lds_read_tr(base + 4 * kDxWRow);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto read_b = [&](int slot, int h, int tf) {
    const int tok = wt * 64 + tf * 16 + li;
    const int c = 4 * h + lq;
    return *reinterpret_cast<const u32x4*>(gbuf + slot * kDxGStage + (tok * 8 + (c ^ (tok & 7))) * 16);
  };

  // ---- prologue: chunks 0 and 1 in registers, chunk 0 staged and
  // decompressed, chunk 2 in registers
  DxPack pk[2];
  u32x4 gs[2][4];
  auto load_pack = [&](int chunk, DxPack& d) {
    uint32_t vo, i0, i1;
    pack_offsets(chunk, vo, i0, i1);
    dx_load<P>(d, rv, ri, vo, i0, i1);
  };
  load_g(0, gs[0]);
  load_pack(0, pk[0]);
  load_g(1, gs[1]);
  load_pack(1, pk[1]);
  decompress(pk[0], 0);
  write_g(0, gs[0]);
  load_g(2, gs[0]);
  load_pack(2, pk[0]);

  // Step c (parity PAR = c & 1, a compile-time constant: the loop is unrolled
  // by two so the register sets alternate without copies): the barrier
  // publishes G stage PAR and W tile PAR, written in step c-1 (or the
  // prologue), and retires stage and tile PAR ^ 1, read in step c-1.  The step
  // multiplies chunk c, then stages chunk c+1 from register sets (c+1) & 1
  // into stage and tile PAR ^ 1 and loads chunk c+3 into those sets.  Past the
  // last chunk the loads read zeros (dead offsets).
  auto step = [&](auto par_c, int c) {
    constexpr int PAR = decltype(par_c)::value;
    DxPack& nextp = pk[PAR ^ 1];
    u32x4 (&nextg)[4] = gs[PAR ^ 1];
    wait_lgkm0();
    barrier_no_fence();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 a[4], b[4];
#pragma unroll
      for (int kf = 0; kf < 4; ++kf) a[kf] = read_a(PAR, h, kf);
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) b[tf] = read_b(PAR, h, tf);
#pragma unroll
      for (int kf = 0; kf < 4; ++kf)
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) acc[kf][tf] = mfma32<DT>(a[kf], b[tf], acc[kf][tf]);
    }
    if (c + 1 < nchunks) {
      decompress(nextp, PAR ^ 1);
      write_g(PAR ^ 1, nextg);
    }
    load_g(c + 3, nextg);
    load_pack(c + 3, nextp);
  };
  // whole pairs in the loop and an odd last chunk after it: a pair cut short
  // inside the loop would give the back edge a path on which the other
  // register set holds the newest loads, and the compiler's waits before
  // every later write of a set would then drain both sets
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(std::integral_constant<int, 0>{}, c);
    step(std::integral_constant<int, 1>{}, c + 1);
  }
  if (c < nchunks) step(std::integral_constant<int, 0>{}, c);
  wait_vmcnt<0>();

  // ---- epilogue: lane (t = li, quarter q) holds rows 4q..4q+3 (k) of
  // column t of each fragment: 16 (fp32) or 8 (half) contiguous bytes of dX
  const bool vec_ok = OUT == NM_F32 ? (lddx & 3) == 0 : (lddx & 3) == 0;
#pragma unroll
  for (int kf = 0; kf < 4; ++kf) {
    const int k = K0 + wk * 64 + kf * 16 + lq * 4;
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) {
      const int t = T0 + wt * 64 + tf * 16 + li;
      if (t >= T || k >= K) continue;
      const f32x4 v = acc[kf][tf];
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(dX) + int64_t(t) * lddx + k;
        if (vec_ok && k + 3 < K) {
          *reinterpret_cast<f32x4*>(y) = v;
        } else {
          for (int e = 0; e < 4 && k + e < K; ++e) y[e] = v[e];
        }
      } else {
        uint16_t* y = static_cast<uint16_t*>(dX) + int64_t(t) * lddx + k;
        const uint32_t p0 = pack_half2<DT>(v[0], v[1]), p1 = pack_half2<DT>(v[2], v[3]);
        if (vec_ok && k + 3 < K) {
          *reinterpret_cast<uint2*>(y) = make_uint2(p0, p1);
        } else {
          const uint16_t hh[4] = {uint16_t(p0), uint16_t(p0 >> 16), uint16_t(p1), uint16_t(p1 >> 16)};
          for (int e = 0; e < 4 && k + e < K; ++e) y[e] = hh[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dW[r, s] = sum_t G[t, r] act[t, k(r, s)], computed as dense dW^T tiles
// D[k][r] = sum_t act[t][k] G[t][r] of which each lane keeps the stored
// entries.  A workgroup (4 waves, 2 x 2) owns 256 k x 128 r; a wave 128 k x
// 64 r (8 x 4 fragments), so one LDS byte feeds 43 MACs on average against
// 32 at 64 x 64.  T is walked in chunks of 32 tokens (one MFMA K step): act's
// [32 t][256 k] and G's [32 t][128 r] tiles are loaded into registers two
// chunks ahead (6 16-byte pieces per thread) and written to a double-buffered
// stage after the previous chunk's MFMAs; both operands come out by transpose
// reads (an operand lane needs 8 consecutive tokens of one column).  Staging
// from registers rather than by direct global->LDS loads keeps the compiler
// from holding each transpose read until every direct load in flight has
// landed.  Token row t of a tile starts at byte P t + 128 (((t >> 3) & 1) + (t
// >> 4)), P = 544 (act, 512-byte rows) or 288 (G, 256-byte rows): the 8-byte
// transpose reads of 32 lanes (rows 8g + j, g = 0, 1, j = 0..3) fall in
// distinct banks (64 banks of 4 bytes), the lanes writing one row write its
// bytes contiguously, and every fragment's address is a base register plus
// a constant.  At 2 x 27 KB of LDS two workgroups share a compute unit.
// A result lane (column r, quarter q) holds rows 4q..4q+3 of D, four
// consecutive columns k of W's row r: a whole group of four, or half of one
// of eight, whose stored positions it reads from the index bits and whose
// survivors it writes to the packed gradient.
// ---------------------------------------------------------------------------
constexpr int kDwBK = 256, kDwBR = 128, kDwTC = 32;
constexpr int kDwFK = 8, kDwFR = 4;                    // fragments per wave along k and r

__host__ __device__ constexpr int dw_row(int t, int pitch) {
  return t * pitch + (((t >> 3) & 1) + (t >> 4)) * 128;
}
constexpr int kDwActTile = dw_row(kDwTC - 1, 544) + 512;   // 17632 bytes
constexpr int kDwGTile = dw_row(kDwTC - 1, 288) + 256;     // 9440 bytes
constexpr int kDwStage = kDwActTile + kDwGTile;
constexpr int kDwLds = 2 * kDwStage;
static_assert(kDwActTile % 16 == 0 && kDwGTile % 16 == 0, "16-byte aligned tiles");

template <int P, int DT, int OUT>
__global__ __launch_bounds__(256, 2) void spmm_dw_kernel(const uint32_t* __restrict__ idx, uint32_t idx_bytes, int R,
                                                      int K, int idx_row_words, const uint16_t* __restrict__ G,
                                                      int T, int64_t ldg, const uint16_t* __restrict__ act,
                                                      int64_t ldx, void* __restrict__ dW, int tilesK, int tilesR,
                                                      int group) {
  constexpr int N = pat_n(P), M = pat_m(P);
  constexpr int B = P == 2 ? 3 : 2;
  extern __shared__ __align__(16) unsigned char smem[];

  int tk, tr;
  grouped_tile(xcd_tile(blockIdx.x, gridDim.x), tilesK, tilesR, group, tk, tr);
  const int K0 = tk * kDwBK, R0 = tr * kDwBR;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave >> 1, wr = wave & 1;
  const int li = lane & 15, lq = lane >> 4;
  const int nchunks = (T + kDwTC - 1) / kDwTC;
  const int64_t S = int64_t(K) * N / M;

  // A thread's pieces of a chunk: act rows (tid / 32) + 8 j, piece tid % 32
  // (j = 0..3), and G rows (tid / 16) + 16 j, piece tid % 16 (j = 0, 1).
  // Tokens past T read zeros, so they add nothing; columns past K or R are
  // whatever the descriptor allows and only reach outputs that are dropped
  // (with T == 0 nothing is read: the descriptors cover no bytes).
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(act + K0, T > 0 ? uint32_t(((int64_t(T) - 1) * ldx + (K - K0)) * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rg =
      make_rsrc(G + R0, T > 0 ? uint32_t(((int64_t(T) - 1) * ldg + (R - R0)) * 2) : 0u);
  int arow[4], grow[2];
  uint32_t aoff[4], goff[2], aloff[4], gloff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    arow[j] = (tid >> 5) + 8 * j;
    aoff[j] = uint32_t(arow[j]) * uint32_t(ldx) * 2u + uint32_t(tid & 31) * 16u;
    aloff[j] = uint32_t(dw_row(arow[j], 544) + (tid & 31) * 16);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    grow[j] = (tid >> 4) + 16 * j;
    goff[j] = uint32_t(grow[j]) * uint32_t(ldg) * 2u + uint32_t(tid & 15) * 16u;
    gloff[j] = uint32_t(kDwActTile + dw_row(grow[j], 288) + (tid & 15) * 16);
  }
  auto load_chunk = [&](int chunk, u32x4 (&v)[6]) {
    const int t0 = chunk * kDwTC;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool live = t0 + arow[j] < T;      // false for every chunk past the last
      v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           ra, live ? aoff[j] + uint32_t(t0) * uint32_t(ldx) * 2u : kDeadOff, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool live = t0 + grow[j] < T;
      v[4 + j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rg, live ? goff[j] + uint32_t(t0) * uint32_t(ldg) * 2u : kDeadOff, 0, 0));
    }
  };
  auto write_chunk = [&](int stage, const u32x4 (&v)[6]) {
    unsigned char* st = smem + stage * kDwStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(st + aloff[j]) = v[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(st + gloff[j]) = v[4 + j];
  };

  // transpose reads: lane L = 16g + 4j + a reads token rows 8g + j and
  // 8g + j + 4, columns 4a.. of a 16-column fragment
  const int tr_row = 8 * (lane >> 4) + ((lane >> 2) & 3), tr_a = lane & 3;
  const int a_lo = dw_row(tr_row, 544) + 8 * tr_a, a_hi = dw_row(tr_row + 4, 544) + 8 * tr_a;
  const int g_lo = kDwActTile + dw_row(tr_row, 288) + 8 * tr_a, g_hi = kDwActTile + dw_row(tr_row + 4, 288) + 8 * tr_a;
  auto read_tr = [&](const unsigned char* st, int lo, int hi, int col0) {
    const u32x2 l = lds_read_tr(st + lo + col0 * 2);
    const u32x2 h = lds_read_tr(st + hi + col0 * 2);
    return u32x4{l[0], l[1], h[0], h[1]};
  };

  f32x4 acc[kDwFK][kDwFR];
#pragma unroll
  for (int i = 0; i < kDwFK; ++i)
#pragma unroll
    for (int j = 0; j < kDwFR; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk 0 staged, chunks 1 and 2 in registers; step c (parity PAR, the loop
  // unrolled by two): the barrier publishes stage PAR and retires stage
  // PAR ^ 1; the step multiplies chunk c, stages chunk c+1 from register set
  // PAR ^ 1 and loads chunk c+3 into it (past the last chunk, zeros)
  u32x4 vs[2][6];
  load_chunk(0, vs[0]);
  load_chunk(1, vs[1]);
  write_chunk(0, vs[0]);
  load_chunk(2, vs[0]);
  auto step = [&](auto par_c, int c) {
    constexpr int PAR = decltype(par_c)::value;
    u32x4 (&nextv)[6] = vs[PAR ^ 1];
    wait_lgkm0();
    barrier_no_fence();
    const unsigned char* st = smem + PAR * kDwStage;
    u32x4 a[kDwFK];
#pragma unroll
    for (int kf = 0; kf < kDwFK; ++kf) a[kf] = read_tr(st, a_lo, a_hi, wk * 128 + kf * 16);
#pragma unroll
    for (int rf = 0; rf < kDwFR; ++rf) {
      const u32x4 b = read_tr(st, g_lo, g_hi, wr * 64 + rf * 16);
#pragma unroll
      for (int kf = 0; kf < kDwFK; ++kf) acc[kf][rf] = mfma32<DT>(a[kf], b, acc[kf][rf]);
    }
    if (c + 1 < nchunks) write_chunk(PAR ^ 1, nextv);
    load_chunk(c + 3, nextv);
  };
  // whole pairs in the loop and an odd last chunk after it: a pair cut short
  // inside the loop would give the back edge a path on which the other
  // register set holds the newest loads, and the compiler's waits before
  // every later write of a set would then drain both sets
  int c = 0;
  for (; c + 1 < nchunks; c += 2) {
    step(std::integral_constant<int, 0>{}, c);
    step(std::integral_constant<int, 1>{}, c + 1);
  }
  if (c < nchunks) step(std::integral_constant<int, 0>{}, c);
  wait_vmcnt<0>();

  // ---- epilogue: lane (r = li of the fragment, quarter q) holds D rows
  // 4q..4q+3, columns k..k+3 of W's row r
#pragma unroll
  for (int rf = 0; rf < kDwFR; ++rf) {
    const int r = R0 + wr * 64 + rf * 16 + li;
#pragma unroll
    for (int kf = 0; kf < kDwFK; ++kf) {
      const int k = K0 + wk * 128 + kf * 16 + lq * 4;
      if (r >= R || k >= K) continue;
      const f32x4 v = acc[kf][rf];
      const int g = k / M;                          // the group holding k .. k+3
      const int64_t sg = int64_t(g) * N;            // its first survivor
      const int64_t bit = sg * B;
      const uint32_t* irow = idx + int64_t(r) * idx_row_words;
      const int64_t w = bit >> 5;
      const uint64_t pair = uint64_t(irow[w]) |
                            (w + 1 < idx_row_words ? uint64_t(irow[w + 1]) << 32 : uint64_t(0));
      const uint32_t bits = uint32_t(pair >> (bit & 31));
      auto pick = [&](uint32_t p) {   // D value at in-lane column p (0..3)
        return p == 0 ? v[0] : p == 1 ? v[1] : p == 2 ? v[2] : v[3];
      };
      const int64_t o = int64_t(r) * S + sg;
      if constexpr (P == 0) {
        const float x0 = pick(bits & 3u), x1 = pick((bits >> 2) & 3u);
        if constexpr (OUT == NM_F32) {
          float* y = static_cast<float*>(dW) + o;
          y[0] = x0;
          y[1] = x1;
        } else {
          *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(dW) + o) = pack_half2<DT>(x0, x1);
        }
      } else {
        const uint32_t pos = bits & (M - 1);
        // 1:8: the survivor is in this lane's half of the group of eight only
        // when its position's high bit matches the half
        const bool mine = P == 1 || int(pos >> 2) == ((k % M) >> 2);
        if (mine) {
          const float x = pick(pos & 3u);
          if constexpr (OUT == NM_F32) {
            static_cast<float*>(dW)[o] = x;
          } else {
            static_cast<uint16_t*>(dW)[o] = uint16_t(pack_half2<DT>(x, 0.f));
          }
        }
      }
    }
  }
}

// Group size for grouped_tile.  An XCD's run of about tiles / 8 tiles covers
// some bands of the grouped operand (at least min(group, run), more once the
// run spans several groups) and ceil(run / group) bands of the other, up to
// their counts; with band bytes in proportion band_a : band_b, the power of two
// with the fewest bytes is taken, so the XCD's L2 serves the rest.
int pick_group(int64_t tiles_a, int64_t tiles_b, double band_a, double band_b) {
  const int64_t run = (tiles_a * tiles_b + 7) / 8;
  int best = 1;
  double best_bytes = 0.0;
  for (int64_t g = 1; g <= tiles_a; g *= 2) {
    const int64_t na = std::min(tiles_a, std::max(std::min(g, run), (run + tiles_b - 1) / tiles_b));
    const int64_t nb = std::min(tiles_b, (run + g - 1) / g);
    const double bytes = double(na) * band_a + double(nb) * band_b;
    if (g == 1 || bytes < best_bytes) best = int(g), best_bytes = bytes;
  }
  return best;
}

template <int P, int DT, int OUT>
hipError_t launch_dw_cfg(const TrainArgs& a, hipStream_t s) {
  const int64_t tilesK = (a.K + kDwBK - 1) / kDwBK, tilesR = (a.R + kDwBR - 1) / kDwBR;
  if (tilesK * tilesR > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto kern = spmm_dw_kernel<P, DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), kDwLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tilesK * tilesR)), dim3(256), kDwLds, s, a.idx, uint32_t(a.idx_bytes),
                     int(a.R), int(a.K), int(a.idx_row_words), a.G, int(a.T), a.ldg, a.act, a.ldx, a.out,
                     int(tilesK), int(tilesR), pick_group(tilesK, tilesR, 2.0, 1.0));
  return hipGetLastError();
}

template <int P, int DT>
hipError_t launch_dw_out(const TrainArgs& a, hipStream_t s) {
  return a.out_dtype == NM_F32 ? launch_dw_cfg<P, DT, NM_F32>(a, s) : launch_dw_cfg<P, DT, DT>(a, s);
}

template <int P>
hipError_t launch_dw_dt(const TrainArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? launch_dw_out<P, NM_F16>(a, s) : launch_dw_out<P, NM_BF16>(a, s);
}

template <int P, int DT, int OUT>
hipError_t launch_dx_cfg(const TrainArgs& a, hipStream_t s) {
  const int64_t tilesK = (a.K + kDxBK - 1) / kDxBK, tilesT = (a.T + kDxBT - 1) / kDxBT;
  if (tilesK * tilesT > 0x7FFFFFFF) return hipErrorInvalidValue;
  auto kern = spmm_dx_kernel<P, DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), kDxLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tilesK * tilesT)), dim3(256), kDxLds, s, a.values,
                     uint32_t(a.values_bytes), a.idx, uint32_t(a.idx_bytes), int(a.R), int(a.K),
                     int(a.idx_row_words), a.G, int(a.T), a.ldg, a.out, a.ldo, int(tilesK), int(tilesT),
                     pick_group(tilesK, tilesT, double(pat_n(P)) / pat_m(P), 1.0));
  return hipGetLastError();
}

template <int P, int DT>
hipError_t launch_dx_out(const TrainArgs& a, hipStream_t s) {
  return a.out_dtype == NM_F32 ? launch_dx_cfg<P, DT, NM_F32>(a, s) : launch_dx_cfg<P, DT, DT>(a, s);
}

template <int P>
hipError_t launch_dx_dt(const TrainArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? launch_dx_out<P, NM_F16>(a, s) : launch_dx_out<P, NM_BF16>(a, s);
}

}  // namespace

hipError_t launch_spmm_dw(const TrainArgs& a, hipStream_t s) {
  if (a.n == 2 && a.m == 4) return launch_dw_dt<0>(a, s);
  if (a.n == 1 && a.m == 4) return launch_dw_dt<1>(a, s);
  if (a.n == 1 && a.m == 8) return launch_dw_dt<2>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_spmm_dx(const TrainArgs& a, hipStream_t s) {
  if (a.n == 2 && a.m == 4) return launch_dx_dt<0>(a, s);
  if (a.n == 1 && a.m == 4) return launch_dx_dt<1>(a, s);
  if (a.n == 1 && a.m == 8) return launch_dx_dt<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nm
