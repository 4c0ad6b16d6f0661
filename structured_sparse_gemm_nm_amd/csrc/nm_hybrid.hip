// Hybrid dense / 2:4 weight tiles on gfx950.
//
// Source: thelatestinai.com "Structured Sparsity" topic cards, the PATCH
// abstract: the weight matrix is cut into tiles, each kept dense or made 2:4
// sparse, which puts the fraction of zeros anywhere from 0 to 50%.  Tiles are
// tile_rows x tile_cols blocks (both multiples of 64 here); a row stores its
// tiles in column order, a dense tile as its tile_cols values (each block of
// 16 as the values at positions 0 and 1 of its four groups, then those at 2
// and 3), a 2:4 tile as its tile_cols/2 survivors plus tile_cols/8 index
// bytes (2 bits per survivor, LSB first), and the layout tables give each
// tile-row's row lengths and starting offsets (nmsparse.h, nm_hybrid_layout).
//
// Pack: one thread per 16-byte chunk (eight weights) of a row: a dense tile's
// chunk takes its half of its block's reordered values, a 2:4 tile's chunk
// gives its four survivors and its index byte with the selection nm_compress
// uses (same largest-magnitude rule).
//
// Product: a workgroup of 8 waves owns 256 x 128 (or 128 x 64) of Y^T;
// activations and weights go through an LDS ring of direct global->LDS loads,
// each wave multiplying one of four 64- (32-) row weight slices by half of the
// workgroup's tokens.  A 64-wide K step of a 2:4 tile is one
// v_smfmac_f32_16x16x64 per fragment pair, of a dense tile two: one with the
// values at positions 0 and 1 of every group and one with those at 2 and 3,
// each with fixed index bits.  Both kinds read the same activation fragments
// and accumulate in place.
// Tile-rows are multiples of 64 rows, so a wave's rows share one flag per
// step and the choice is one uniform branch per step.  Weight reads go
// through buffer descriptors bounded by the arrays' sizes: offsets from a
// wrong layout table read zeros instead of memory outside the arrays, and the
// pack's stores are bounded the same way.
#include "nm_device.h"
#include "nm_internal.h"
#include "nm_select.h"

namespace nm {
namespace {

// A byte offset into a buffer of `bytes` bytes, or one the buffer refuses.
__device__ inline uint32_t bounded(int64_t off, uint32_t bytes) {
  return (off >= 0 && off < int64_t(bytes)) ? uint32_t(off) : 0xFFFFFFFFu;
}

__global__ __launch_bounds__(256) void hybrid_pack_kernel(
    const uint16_t* __restrict__ W, int64_t R, int64_t K, int64_t ldw, int tile_rows, int tile_cols, int KB,
    const int64_t* __restrict__ tile_meta, const int64_t* __restrict__ row_meta, uint16_t* values,
    uint32_t values_bytes, uint8_t* idx, uint32_t idx_bytes) {
  const int64_t cpr = K >> 3;  // 16-byte chunks per row
  const int64_t g = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= R * cpr) return;
  const int64_t r = g / cpr;
  const int k0 = int(g - r * cpr) * 8;
  const int j = k0 / tile_cols, kin = k0 - j * tile_cols;
  const int64_t b = r / tile_rows, rr = r - b * tile_rows;
  const int64_t v0 = tile_meta[(b * KB + j) * 2], i0 = tile_meta[(b * KB + j) * 2 + 1];
  const int64_t Lv = row_meta[b * 4], Li = row_meta[b * 4 + 1];
  const u32x4 w = *reinterpret_cast<const u32x4*>(W + r * ldw + k0);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  if (i0 < 0) {
    // dense tile: a block of 16 values is stored as its values at positions 0
    // and 1 of each group of four (dwords 0 and 2 of both its chunks), then
    // those at positions 2 and 3 (dwords 1 and 3); this thread writes half
    // kin / 8 & 1 of its block, from its own chunk and its partner's
    const u32x4 p = *reinterpret_cast<const u32x4*>(W + r * ldw + (k0 ^ 8));
    const bool second = (kin >> 3) & 1;
    const u32x4 lo = second ? p : w, hi = second ? w : p;  // chunks 0 and 1 of the block
    const u32x4 o = second ? u32x4{lo[1], lo[3], hi[1], hi[3]} : u32x4{lo[0], lo[2], hi[0], hi[2]};
    __builtin_amdgcn_raw_buffer_store_b128(o, rv, bounded((v0 + rr * Lv + kin) * 2, values_bytes), 0, 0);
  } else {       // 2:4 tile: four survivors and their index byte
    const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
    uint32_t kept[2];
    uint32_t bits = 0;
    select_chunk<2, 4>(ww, kept, bits);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{kept[0], kept[1]}, rv,
                                          bounded((v0 + rr * Lv + kin / 2) * 2, values_bytes), 0, 0);
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx, idx_bytes);
    __builtin_amdgcn_raw_buffer_store_b8(uint8_t(bits), ri, bounded(i0 + rr * Li + kin / 8, idx_bytes), 0, 0);
  }
}

constexpr int kMaxFlagWords = 256;  // tile-columns per row up to 32 * 256

// Positions of a dense step's two 2:4 products: 0 and 1 in every group of
// four (low half, 0x4444), 2 and 3 (high half, 0xEEEE); two bits per value,
// the value's position in its group.
constexpr uint32_t kDensePositions = 0xEEEE4444u;

// Product.  A workgroup (8 waves, two per SIMD) owns BR x BT of Y^T in four
// row slices of WROWS = BR/4 rows; wave w multiplies slice w % 4 by token half
// w / 4.  The tile-rows are multiples of 64 rows, so a slice's rows share one
// flag per K step.  Stages form an NS-deep ring; stage = the BT tokens'
// activations (slot (token, chunk c) at token*8 + (c ^ (token & 7))) plus one
// weight slice per row slice of WROWS x 128 bytes:
//   dense step  the rows' 128 bytes of (reordered) values, slot (row,
//               chunk c) at row*8 + (c ^ ((row >> 1) & 7));
//   2:4 step    the rows' 64 bytes of survivors, slot (row, chunk c) at
//               row*4 + (c ^ ((row >> 1) & 3)), and from the slice's middle
//               each row's aligned 16-byte index block holding its 8 index
//               bytes of the step (16 bytes per row).
// A slice's AL direct loads are split between its two waves, AL/2 each, for
// both kinds of step (a 2:4 step gives the survivors to the first wave, the
// index blocks and loads the descriptor refuses, which write zeros into slots
// nothing reads, to the second), so the counted waits are fixed; the barrier
// of each step publishes every wave's loads to the others.
template <int DT, int OUT, int BR, int BT, int NS>
__global__ __launch_bounds__(512) void hybrid_gemm_kernel(
    const uint16_t* __restrict__ values, uint32_t values_bytes, const uint8_t* __restrict__ idx,
    uint32_t idx_bytes, const int64_t* __restrict__ tile_meta, const int64_t* __restrict__ row_meta, int R,
    int K, int tile_rows, int tile_cols, int KB, const uint16_t* __restrict__ act, int T, int64_t ldx,
    void* __restrict__ Y, int64_t ldy, int tilesR, int tilesT, int group_r) {
  constexpr int WROWS = BR / 4;          // rows per slice
  constexpr int TW = BT / 2;             // tokens per wave
  constexpr int FR = WROWS / 16;         // 16-row fragments per wave
  constexpr int FT = TW / 16;            // 16-token fragments per wave
  constexpr int SB = WROWS * 128;        // bytes of one weight slice
  constexpr int STAGE_B = BT * 128;      // activations of one stage
  constexpr int STAGE = STAGE_B + 4 * SB;
  constexpr int BL = BT / 64;            // activation loads per wave per step
  constexpr int AL = SB / 1024;          // weight loads per slice per step
  constexpr int AH = AL / 2;             // ... per wave
  constexpr int PER_STEP = BL + AH;
  static_assert((NS - 2) * PER_STEP < 64, "vmcnt range");
  static_assert(WROWS <= 64 && AL >= 2, "a 2:4 step's index blocks take one load");
  extern __shared__ __align__(16) unsigned char smem[];  // [NS][STAGE], then the flag words
  uint32_t* flag_words = reinterpret_cast<uint32_t*>(smem + NS * STAGE);  // [8][kMaxFlagWords]

  // ---- tile: XCD-aware remap, then groups of group_r row tiles
  const int ntiles = tilesR * tilesT;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int per_group = group_r * tilesT;
  const int grp = bid / per_group;
  const int rem = bid - grp * per_group;
  const int rows_in_grp = min(group_r, tilesR - grp * group_r);
  const int R0 = (grp * group_r + rem % rows_in_grp) * BR;
  const int T0 = (rem / rows_in_grp) * BT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rs = wave & 3, th = wave >> 2;  // row slice, token half
  const int li = lane & 15, lq = lane >> 4;
  const int nsteps = K >> 6;
  const int spt = tile_cols >> 6;  // K steps per tile-column

  // ---- the slice's tile-row (rows past R read row R - 1, in the last one)
  const int srow0 = R0 + rs * WROWS;
  const int b = __builtin_amdgcn_readfirstlane(min(srow0, R - 1) / tile_rows);
  const int64_t Lv = row_meta[b * 4], Li = row_meta[b * 4 + 1];
  const int64_t VB = row_meta[b * 4 + 2], IB = row_meta[b * 4 + 3];
  uint32_t* wflags = flag_words + wave * kMaxFlagWords;
  for (int j0 = 0; j0 < KB; j0 += 64) {
    const int j = j0 + lane;
    const bool dense = j < KB && tile_meta[(int64_t(b) * KB + j) * 2 + 1] < 0;
    const uint64_t m = __builtin_amdgcn_ballot_w64(dense);
    if (lane == 0) {
      wflags[j0 >> 5] = uint32_t(m);
      if (j0 + 32 < KB) wflags[(j0 >> 5) + 1] = uint32_t(m >> 32);
    }
  }
  // Byte offsets of slice row q's values and index bytes (rows past R lie past
  // the end of the arrays: the descriptors return zeros for them, and their
  // outputs are dropped).
  const int64_t rq0 = int64_t(srow0) - int64_t(b) * tile_rows;  // first slice row in its tile-row
  auto vrow_bytes = [&](int q) { return uint32_t((VB + (rq0 + q) * Lv) * 2); };
  auto irow_bytes = [&](int q) { return uint32_t(IB + (rq0 + q) * Li); };
  // per-lane parts of this wave's weight loads (loads j = th*AH .. th*AH+AH-1
  // of the slice): dense load j covers slice rows [8j, 8j+8) (lane: row
  // 8j + l/8, position l%8), 2:4 survivor load j rows [16j, 16j+16) (row
  // 16j + l/4, position l%4), the index load row l % WROWS
  uint32_t doff[AH], soff[AH];
#pragma unroll
  for (int jj = 0; jj < AH; ++jj) {
    const int j = th * AH + jj;
    const int q = j * 8 + (lane >> 3);
    doff[jj] = vrow_bytes(q) + uint32_t((lane & 7) ^ ((q >> 1) & 7)) * 16u;
    const int q2 = jj * 16 + (lane >> 2);
    soff[jj] = vrow_bytes(q2) + uint32_t((lane & 3) ^ ((q2 >> 1) & 3)) * 16u;
  }
  const uint32_t ioff = irow_bytes(lane % WROWS);
  // for the fragment reads: bit 3 of each fragment row's index-row start
  uint32_t ihalf = 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) ihalf |= ((irow_bytes(i * 16 + li) >> 3) & 1u) << i;
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx, idx_bytes);

  // activations: descriptor over the tile's token rows (rows past T reread
  // row T - 1, whose outputs are dropped)
  const int tlast = min(T0 + BT, T) - 1;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(act + int64_t(T0) * ldx, uint32_t((int64_t(tlast - T0) * ldx + K) * 2));
  uint32_t boff[BL];
#pragma unroll
  for (int j = 0; j < BL; ++j) {
    const int slot = (wave * BL + j) * 64 + lane;
    const int tok = slot >> 3;
    const int chunk = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1) - T0;
    boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(chunk) * 16u;
  }

  // The weight stream walks the row's tiles in order: lv / lio are the next
  // step's value / index-byte positions along a row of the tile-row, jt and
  // kt its tile-column and step within it.  Past the last step every load
  // reads zeros (offsets the descriptors refuse), so those steps add zero.
  uint32_t lv = 0, lio = 0;
  int jt = 0, kt = 0;
  uint32_t sdense = 0, shalf = 0;  // bit u: stage u's step is dense / reads its index block at +8
  auto issue = [&](int u, int step) {
    unsigned char* st = smem + u * STAGE;
    const uint32_t so = step < nsteps ? uint32_t(step) * 128u : 0x80000000u;
#pragma unroll
    for (int j = 0; j < BL; ++j) dma16(rb, boff[j], so, st + (wave * BL + j) * 1024);
    const int jc = min(jt, KB - 1);
    const uint32_t dense = (__builtin_amdgcn_readfirstlane(wflags[jc >> 5]) >> (jc & 31)) & 1u;
    const bool live = step < nsteps;
    const uint32_t v2 = lv * 2u, io = lio;
    unsigned char* sl = st + STAGE_B + rs * SB;
#pragma unroll
    for (int jj = 0; jj < AH; ++jj) {
      // 2:4: the first wave loads the survivors (AH loads), the second the
      // index blocks (its load 0) and zeros
      uint32_t o2 = th == 0 ? soff[jj] + v2 : (jj == 0 ? (ioff + io) & ~15u : 0xFFFFFFF0u);
      const __amdgpu_buffer_rsrc_t r = (dense || th == 0 || jj != 0) ? rv : ri;
      const uint32_t o = dense ? doff[jj] + v2 : o2;
      dma16(r, live ? o : 0xFFFFFFF0u, 0u, sl + (th * AH + jj) * 1024);
    }
    sdense = (sdense & ~(1u << u)) | (dense << u);
    shalf = (shalf & ~(1u << u)) | (((io >> 3) & 1u) << u);
    lv += dense ? 64u : 32u;
    lio += dense ? 0u : 8u;
    const int nk = kt + 1;
    jt += nk == spt ? 1 : 0;
    kt = nk == spt ? 0 : nk;
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: steps 0 .. NS-2 in flight.  Every step then issues the
  // same loads (past the last step, zeros nothing reads), so the waits are
  // fixed counts; the stage index is a run-time value, so one copy of the
  // step's code (and of its per-lane offsets) serves every stage, and the
  // loop's only branch is the uniform dense / 2:4 choice.
  for (int p = 0; p < NS - 1; ++p) issue(p, p);

  int u = 0, un = NS - 1;  // stages of step s and of step s + NS - 1
  for (int s = 0; s < nsteps; ++s) {
    {
      // step s has landed once at most the later steps' loads remain; the
      // barrier publishes every wave's loads and retires the slot the new
      // loads reuse
      wait_vmcnt<(NS - 2) * PER_STEP>();
      barrier_no_fence();
      issue(un, s + NS - 1);
      const unsigned char* st = smem + u * STAGE;
      const unsigned char* sl = st + STAGE_B + rs * SB;
      u32x8 bf[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int tok = th * TW + j * 16 + li;
        const int sw = tok & 7;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(st + (tok * 8 + (lq ^ sw)) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(st + (tok * 8 + ((lq + 4) ^ sw)) * 16);
        bf[j] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // A dense step is two 2:4 products with fixed positions: the values at
      // positions 0 and 1 of every group of four (index 0x4444), then those at
      // 2 and 3 (0xEEEE).  A lane's 16 dense values of row q are chunks 2 lq
      // and 2 lq + 1 of the row; the first product takes dwords 0 and 2 of
      // each chunk, the second dwords 1 and 3.  A 2:4 step is one product with
      // the stored values and positions.  Both kinds accumulate in place, so
      // the accumulators stay in the same registers whichever kind a step is.
      // A dense step is two 2:4 products with fixed positions: a block of 16
      // values is stored as those at positions 0 and 1 of its groups of four
      // (for this lane, chunk 2 lq of the row), then 2 and 3 (chunk 2 lq + 1),
      // so each chunk is one product's A operand as it stands.  The first
      // product (a 2:4 step's only one) is shared by both kinds of step and
      // the dense step's second one follows under a uniform branch: every
      // product accumulates in place and no operand outlives its branch, so
      // the accumulators stay in the same registers whatever the step.
      const bool dense_step = (sdense >> u) & 1u;
      u32x4 x[FR];
      uint32_t ix[FR];
      if (dense_step) {
#pragma unroll
        for (int i = 0; i < FR; ++i) {
          const int q = i * 16 + li;
          x[i] = *reinterpret_cast<const u32x4*>(sl + (q * 8 + ((2 * lq) ^ ((q >> 1) & 7))) * 16);
          ix[i] = kDensePositions;
        }
      } else {
        const uint32_t sh = (shalf >> u) & 1u;
#pragma unroll
        for (int i = 0; i < FR; ++i) {
          const int q = i * 16 + li;
          x[i] = *reinterpret_cast<const u32x4*>(sl + (q * 4 + (lq ^ ((q >> 1) & 3))) * 16);
          // this lane's two index bytes: the row's start and the step's
          // position put them at byte 8*((row bit + step bit) & 1) + 2*lq
          const uint32_t pos = ((((ihalf >> i) & 1u) ^ sh) << 3) + uint32_t(lq) * 2u;
          ix[i] = *reinterpret_cast<const uint16_t*>(sl + SB / 2 + q * 16 + pos);
        }
      }
#pragma unroll
      for (int j = 0; j < FT; ++j)
#pragma unroll
        for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT, 0>(x[i], bf[j], acc[i][j], ix[i]);
      if (dense_step) {
#pragma unroll
        for (int i = 0; i < FR; ++i) {
          const int q = i * 16 + li;
          x[i] = *reinterpret_cast<const u32x4*>(sl + (q * 8 + ((2 * lq + 1) ^ ((q >> 1) & 7))) * 16);
        }
#pragma unroll
        for (int j = 0; j < FT; ++j)
#pragma unroll
          for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT, 1>(x[i], bf[j], acc[i][j], kDensePositions);
      }
    }
    u = u + 1 == NS ? 0 : u + 1;
    un = un + 1 == NS ? 0 : un + 1;
  }
  // the loads past the last step are still landing: the workgroup ends only
  // once no direct load is writing LDS
  wait_vmcnt<0>();

  // ---- epilogue
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = srow0 + i * 16 + lq * 4;
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      const int t = T0 + th * TW + j * 16 + li;
      if (t >= T || r >= R) continue;
      const f32x4 v = acc[i][j];
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok && r + 3 < R) {
          *reinterpret_cast<f32x4*>(y) = v;
        } else {
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = v[e];
        }
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint32_t p0 = pack_half2<DT>(v[0], v[1]), p1 = pack_half2<DT>(v[2], v[3]);
        if (vec_ok && r + 3 < R) {
          *reinterpret_cast<uint2*>(y) = make_uint2(p0, p1);
        } else {
          const uint16_t hh[4] = {uint16_t(p0), uint16_t(p0 >> 16), uint16_t(p1), uint16_t(p1 >> 16)};
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = hh[e];
        }
      }
    }
  }
}

template <int DT, int OUT, int BR, int BT, int NS>
hipError_t launch_hybrid_cfg(const HybridArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + BR - 1) / BR);
  const int tilesT = int((a.T + BT - 1) / BT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int group_r = tilesR < 4 ? tilesR : 4;
  constexpr int lds = NS * (BT * 128 + BR * 128) + 8 * kMaxFlagWords * 4;
  auto kern = hybrid_gemm_kernel<DT, OUT, BR, BT, NS>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(512), lds, s, a.values, uint32_t(a.values_bytes), a.idx,
                     uint32_t(a.idx_bytes), a.tile_meta, a.row_meta, int(a.R), int(a.K), int(a.tile_rows),
                     int(a.tile_cols), int(a.K / a.tile_cols), a.act, int(a.T), a.ldx, a.Y, a.ldy, tilesR,
                     tilesT, group_r);
  return hipGetLastError();
}

template <int DT, int OUT>
hipError_t hybrid_tile(const HybridArgs& a, hipStream_t s) {
  // 256 x 128 tiles when they cover the chip's 256 CUs, else 128 x 64
  const int64_t big = ((a.R + 255) / 256) * ((a.T + 127) / 128);
  if (big >= 256) return launch_hybrid_cfg<DT, OUT, 256, 128, 3>(a, s);
  return launch_hybrid_cfg<DT, OUT, 128, 64, 6>(a, s);
}

}  // namespace

hipError_t launch_hybrid_pack(const HybridArgs& a, hipStream_t s) {
  const int64_t threads = a.R * (a.K / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(hybrid_pack_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, a.W, a.R, a.K, a.ldw,
                     int(a.tile_rows), int(a.tile_cols), int(a.K / a.tile_cols), a.tile_meta, a.row_meta,
                     a.values_out, uint32_t(a.values_bytes), a.idx_out, uint32_t(a.idx_bytes));
  return hipGetLastError();
}

hipError_t launch_hybrid_spmm(const HybridArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? hybrid_tile<NM_F16, NM_F32>(a, s) : hybrid_tile<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? hybrid_tile<NM_BF16, NM_F32>(a, s) : hybrid_tile<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
