// 2:4 sparse GEMM for prefill shapes with every operand staged through LDS
// by direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k] on
// v_smfmac_f32_16x16x64).  No lane loads fewer than 16 bytes and every load
// instruction reads 64- or 128-byte runs.  A direct load deposits lane l's 16
// bytes at slot base + l of LDS, so the LDS layout is chosen by which global
// address each lane reads.  The XOR swizzles below were picked by measuring
// the LDS bank-conflict counter for the exact fragment reads of this kernel;
// each layout reads without conflicts.  A lane reads just its own 2 index
// bytes of its row's step: they land in the low half of a register, which is
// the index operand the MFMA takes as it is (reading the row's 8 bytes and
// picking 2 with a byte permute cost ~8% more time: LDS traffic and VALU):
//
//   packed values  one K step per stage; slot (row, quarter q) at
//                  row*4 + (q ^ ((row >> 1) & 3)): a load covers 16 rows x 64 B;
//   activations    one K step per stage; slot (token, chunk c) at
//                  token*8 + (c ^ (token & 7)): 8 tokens x 128 B per load;
//   index bits     block = 8 K steps (64 bytes per row); slot (row, chunk) at
//                  row*4 + (chunk ^ ((row >> 2) & 3)).
//
// A workgroup (4 waves) computes 256 x 128 tiles; waves are 2 x 2, each owning
// 128 rows x 64 tokens (8 x 4 fragments: the fragment-read volume per MFMA is
// lowest for this split).  Stages form a 4-deep ring, so three K steps of
// loads are in flight while one is read.  Fragments go through two register
// sets: the LDS reads of step s+1 are issued between the MFMAs of step s.
// Each step waits (counted vmcnt) for exactly the loads of the step it is
// about to read and passes one fence-free barrier, which both publishes that
// step and retires the slot the new loads reuse.
//
// With more tiles than compute units one workgroup per CU walks the tiles,
// and the ring runs on from one tile into the next: the last steps of a tile
// already load and read the first steps of the following one, so neither the
// ring's fill nor the epilogue's stores leave the MFMAs idle between tiles.
#include "nm_device.h"
#include "nm_internal.h"

#include <type_traits>

namespace nm {
namespace {

constexpr int kBR = 256;
constexpr int kBT = 128;
constexpr int kNS = 4;                     // one-K-step stages in the ring
constexpr int kStageB = kBT * 128;         // activations, one step
constexpr int kStageA = kBR * 64;          // packed values, one step
constexpr int kBlockI = kBR * 64;          // index bits, 8 steps
constexpr int kLds = kNS * (kStageB + kStageA) + 2 * kBlockI;
constexpr int kPerStep = 8;                // direct loads per wave per step (4 B + 4 A)

// Where a workgroup's tiles are: tile i of the grid-stride sequence
// (blockIdx.x, + grid, ...) -> (row tile, token tile).  Within a full round of
// `grid` tiles the XCD-aware remap gives each XCD a contiguous run; tiles are
// then ordered in groups of group_r row tiles sharing activation columns.
// DPP control: each lane reads the lane 8 places further round its row of 16.
constexpr int kRowRotate8 = 0x128;

struct TileMap {
  int tilesR, tilesT, group_r, ntiles, grid;
  __device__ void rt(int i, int& R0, int& T0) const {
    const int round = i / grid, p = i - round * grid;
    int q = p;
    if ((grid & 7) == 0 && (round + 1) * grid <= ntiles) q = (p & 7) * (grid >> 3) + (p >> 3);
    const int b = round * grid + q;
    const int per_group = group_r * tilesT;
    const int grp = b / per_group;
    const int rem = b - grp * per_group;
    const int rows_in_grp = min(group_r, tilesR - grp * group_r);
    R0 = (grp * group_r + rem % rows_in_grp) * kBR;
    T0 = (rem / rows_in_grp) * kBT;
  }
};

template <int DT, int OUT>
__global__ __launch_bounds__(256, 1) void spmm_lds_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y, int64_t ldy,
    TileMap tm) {
  constexpr int FR = 8, FT = kBT / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* bbuf = smem;                              // [kNS][kStageB]
  unsigned char* abuf = smem + kNS * kStageB;              // [kNS][kStageA]
  unsigned char* ibuf = smem + kNS * (kStageB + kStageA);  // [2][kBlockI]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform: LDS destinations of the direct loads (M0) are then scalar sums
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int wr = wave >> 1, wt = wave & 1;
  const int nsteps = K >> 6;                 // even: K % 128 == 0 on this path
  const int nblocks = (nsteps + 7) >> 3;     // index blocks of 8 steps per tile
  const int S = K >> 1;                      // packed values per row
  const int irow_bytes = K >> 3;             // index bytes per row (2 bits per survivor)

  // Per-lane slot roles (instruction j of a wave fills slots [(wave*4 + j)*64,
  // +64); lane l takes slot base + l):
  //   activations, one step: slot (token, chunk) at token*8 + (c ^ (token & 7));
  //   packed values, one step: slot (row, quarter) at row*4 + (q ^ ((row >> 1) & 3));
  //   index bits, 8 steps: slot (row, chunk) at row*4 + (c ^ ((row >> 2) & 3)).
  int ichunk[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    ichunk[j] = (slot & 3) ^ ((slot >> 4) & 3);
  }

  // A tile's load sources: uniform buffer resources at the tile's corner and
  // per-lane 32-bit byte offsets (rows / tokens past the edge reread the last
  // one; the launcher checks that every offset fits).
  struct Src {
    __amdgpu_buffer_rsrc_t a, b, i;
    uint32_t boff[4], aoff[4], ioff[4];
  };
  auto make_src = [&](int R0, int T0, Src& o) {
    o.b = make_rsrc(act + int64_t(T0) * ldx);
    o.a = make_rsrc(values + int64_t(R0) * S);
    o.i = make_rsrc(reinterpret_cast<const unsigned char*>(idx) + int64_t(R0) * irow_bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int slot = (wave * 4 + j) * 64 + lane;
      const int tok = slot >> 3;
      const int c = (slot & 7) ^ (tok & 7);
      const int t = min(T0 + tok, T - 1) - T0;
      o.boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(c) * 16u;
      const int row = slot >> 2;
      const int q = (slot & 3) ^ ((row >> 1) & 3);
      const int r = min(R0 + row, R - 1) - R0;
      o.aoff[j] = uint32_t(r) * uint32_t(S) * 2u + uint32_t(q) * 16u;
      o.ioff[j] = uint32_t(r) * uint32_t(irow_bytes) + uint32_t(ichunk[j]) * 16u;
    }
  };

  // Load j (0..3 activations, 4..7 packed values) of step src of the current
  // tile (nt false) or the next one (nt true) into ring slot buf.  Fields are
  // selected by value (a reference to either source would put both on the
  // stack).
  auto issue_load = [&](const Src& c, const Src& n, bool nt, int j, int src, int buf) {
    if (j < 4)
      dma16(nt ? n.b : c.b, nt ? n.boff[j] : c.boff[j], uint32_t(src) * 128u,
            bbuf + buf * kStageB + (wave * 4 + j) * 1024);
    else
      dma16(nt ? n.a : c.a, nt ? n.aoff[j - 4] : c.aoff[j - 4], uint32_t(src) * 64u,
            abuf + buf * kStageA + (wave * 4 + j - 4) * 1024);
  };
  // Load j of a step whose per-lane offset was selected beforehand.
  auto issue_load_at = [&](__amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t ra, uint32_t off, int j,
                           int src, int buf) {
    if (j < 4)
      dma16(rb, off, uint32_t(src) * 128u, bbuf + buf * kStageB + (wave * 4 + j) * 1024);
    else
      dma16(ra, off, uint32_t(src) * 64u, abuf + buf * kStageA + (wave * 4 + j - 4) * 1024);
  };
  auto issue_step = [&](const Src& c, const Src& n, bool nt, int src, int buf) {
#pragma unroll
    for (int j = 0; j < kPerStep; ++j) issue_load(c, n, nt, j, src, buf);
  };
  // index block q of a tile into buffer ib
  auto issue_index = [&](const Src& o, int q, int ib) {
    const int steps_left = nsteps - 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // chunk c holds steps 2c, 2c+1 of the block (steps_left is even); past
      // the row's end the lane rereads chunk 0 of the block
      const uint32_t back = (2 * ichunk[j] < steps_left) ? 0u : uint32_t(ichunk[j]) * 16u;
      dma16(o.i, o.ioff[j] - back, uint32_t(q) * 64u, ibuf + ib * kBlockI + (wave * 4 + j) * 1024);
    }
  };

  // Fragment reads of a step from LDS into registers (ring slot sl, index
  // buffer ib, step u8 within its index block): row fragment i (packed values
  // and index bits) and one half (h: K 8q..8q+7 or 32+8q..) of token fragment j.
  auto read_av = [&](int sl, int i, u32x4& a) {
    const unsigned char* sa = abuf + sl * kStageA;
    const int row = wr * 128 + i * 16 + li;
    a = *reinterpret_cast<const u32x4*>(sa + (row * 4 + (lq ^ ((row >> 1) & 3))) * 16);
  };
  auto read_ix = [&](int ib, int u8, int i, uint32_t& ix) {
    const unsigned char* si = ibuf + ib * kBlockI;
    const int row = wr * 128 + i * 16 + li;
    // this lane's 2 index bytes of the step (bytes 2lq, 2lq+1 of the row's 8)
    const int ch = (u8 >> 1) ^ ((row >> 2) & 3);
    ix = *reinterpret_cast<const uint16_t*>(si + row * 64 + ch * 16 + (u8 & 1) * 8 + lq * 2);
  };
  auto read_b = [&](int sl, int j, int h, u32x8& bf) {
    const unsigned char* sb = bbuf + sl * kStageB;
    const int tok = wt * (kBT / 2) + j * 16 + li;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sb + (tok * 8 + ((lq + 4 * h) ^ (tok & 7))) * 16);
    bf[4 * h + 0] = v[0];
    bf[4 * h + 1] = v[1];
    bf[4 * h + 2] = v[2];
    bf[4 * h + 3] = v[3];
  };
  auto read_frags = [&](int sl, int ib, int u8, u32x4 (&a)[FR], uint32_t (&ix)[FR], u32x8 (&bf)[FT]) {
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      read_av(sl, i, a[i]);
      read_ix(ib, u8, i, ix[i]);
    }
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      read_b(sl, j, 0, bf[j]);
      read_b(sl, j, 1, bf[j]);
    }
  };

  f32x4 acc[FR][FT];
  // Two register sets: the fragments of step s+1 are read from LDS while the
  // MFMAs of step s run.  The loop is unrolled by two so the sets alternate
  // without copies.
  u32x4 a0[FR], a1[FR];
  uint32_t x0[FR], x1[FR];
  u32x8 b0[FT], b1[FT];

  // The workgroup walks tiles blockIdx.x, + grid, ...  The ring runs on
  // across tiles: in a tile's last steps the loads, index blocks and fragment
  // reads of the steps after it belong to the next tile, so a tile starts
  // with its first steps already in flight.
  int tile = blockIdx.x;
  int R0, T0, nR0 = 0, nT0 = 0;
  tm.rt(tile, R0, T0);
  Src cur, nxt;
  make_src(R0, T0, cur);
  bool has_next = tile + tm.grid < tm.ntiles;
  if (has_next) {
    tm.rt(tile + tm.grid, nR0, nT0);
    make_src(nR0, nT0, nxt);
  } else {
    nxt = cur;
  }
  int g = 0;    // ring position of the tile's step 0
  // The vector-memory counter retires loads and stores in issue order.  A
  // tile's epilogue issues its stores after the loads of the next tile's
  // steps 1 .. kNS-1, so the waits for those steps may leave the stores
  // outstanding: they drain under three steps of MFMAs instead of holding up
  // the first.  Only after a full tile, whose waves each issued at least
  // kStores stores (fewer would let such a wait pass early; half outputs
  // store 8 rows per lane, so half as many).
  constexpr int kStores = OUT == NM_F32 ? FR * FT : (FR / 2) * FT;
  bool stores_behind = false;
  int qb = 0;   // index-buffer parity of the tile's block 0

  // One step: make step s+1 visible, refill the slot step s used, read step
  // s+1, multiply step s.  Every step issues the same loads: past the last
  // step of the last tile a slot is refilled with that step again, into a slot
  // nothing reads any more.  So the wait counts are fixed and the loads, the
  // fragment reads and the MFMAs form one branch-free block the scheduler
  // interleaves (a burst of loads would hold up the MFMAs behind it).
  // MODE (compile time):
  //   -2  any step;
  //   -1  steps s+1 .. s+kNS lie inside the tile (every step but a tile's last
  //       kNS), so the loads come from this tile and nothing on them is
  //       selected at run time;
  //   0..7  as -1, and moreover s = 8m + MODE with the tile starting at a ring
  //       position that is a multiple of kNS: ring slots and the index bytes'
  //       place in their block are constants, and ibc / ibn are the index
  //       buffers of this step's block and of the next.
  auto body = [&](auto mode_c, int s, int ibc, int ibn, u32x4 (&ca)[FR], uint32_t (&cx)[FR],
                  u32x8 (&cb)[FT], u32x4 (&na)[FR], uint32_t (&nx)[FR], u32x8 (&nb)[FT]) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr bool IN = MODE != -2;
    constexpr bool FAST = MODE >= 0;
    // step s+1 has landed once at most the loads of steps s+2, s+3 remain (an
    // index block issued in between only makes the wait stricter), and, in a
    // tile's first kNS-1 steps, the previous tile's stores issued after them
    if (s < kNS - 1 && stores_behind)
      wait_vmcnt<2 * kPerStep + kStores>();
    else
      wait_vmcnt<2 * kPerStep>();
    wait_lgkm0();        // this wave's reads of step s are done
    barrier_no_fence();  // publishes step s+1; every wave is done reading step s
    // at a block's first step, the block after it: this tile's next, or the
    // next tile's first
    if constexpr (FAST) {
      if constexpr (MODE == 0) issue_index(cur, (s >> 3) + 1, ibn);  // s + 8 < nsteps here
    } else if ((s & 7) == 0) {
      const int ib = (qb + (s >> 3) + 1) & 1;
      if (s + 8 < nsteps) issue_index(cur, (s >> 3) + 1, ib);
      else if (has_next) issue_index(nxt, 0, ib);
    }
    // loads of the step 4 ahead into step s's slot
    const int buf = FAST ? (MODE & (kNS - 1)) : (g + s) & (kNS - 1);
    const bool in_tile = IN || s + kNS < nsteps;
    const bool ln = !in_tile && has_next;
    const int src = in_tile ? s + kNS : (has_next ? s + kNS - nsteps : nsteps - 1);
    // where step s+1 is read from
    const int rsl = FAST ? ((MODE + 1) & (kNS - 1)) : (g + s + 1) & (kNS - 1);
    const bool r_in = IN || s + 1 < nsteps;
    const int rib = FAST ? (MODE == 7 ? ibn : ibc) : (qb + (r_in ? ((s + 1) >> 3) : nblocks)) & 1;
    const int ru8 = FAST ? ((MODE + 1) & 7) : r_in ? ((s + 1) & 7) : 0;
    // The step's load offsets are worked out before its first MFMA: a VALU
    // result that an MFMA (or a load) waits for inside the chunks would stall
    // the matrix pipe every chunk.
    uint32_t lo[kPerStep];
    __amdgpu_buffer_rsrc_t lrb = cur.b, lra = cur.a;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = cur.boff[j];
      lo[4 + j] = cur.aoff[j];
    }
    if constexpr (!IN) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = ln ? nxt.boff[j] : lo[j];
        lo[4 + j] = ln ? nxt.aoff[j] : lo[4 + j];
      }
      lrb = ln ? nxt.b : lrb;
      lra = ln ? nxt.a : lra;
    }
    __builtin_amdgcn_sched_barrier(0);
    // Eight chunks, each: fragment reads of step s+1, then the 4 MFMAs of
    // row fragment k and one load.  The reads come early in the step, the
    // token fragments and index words (which the next step needs from its
    // first chunk on) before the row fragments, and the last chunk reads
    // nothing: when the next step starts its wait for them, they have long
    // landed.  Scheduling barriers keep the chunks, and the reads ahead of
    // the MFMAs within a chunk, in this order.
#pragma unroll
    for (int k = 0; k < FR; ++k) {
      if (k < FT) {
        read_b(rsl, k, 0, nb[k]);
        read_b(rsl, k, 1, nb[k]);
        read_ix(rib, ru8, 2 * k, nx[2 * k]);
        read_ix(rib, ru8, 2 * k + 1, nx[2 * k + 1]);
      } else {
#pragma unroll
        for (int i = 3 * (k - FT); i < 3 * (k - FT) + 3; ++i)
          if (i < FR) read_av(rsl, i, na[i]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < FT; ++j) acc[k][j] = smfmac<DT>(ca[k], cb[j], acc[k][j], cx[k]);
      issue_load_at(lrb, lra, lo[k], k, src, buf);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  static_assert(FR == kPerStep && FT * 2 == FR && 3 * (FR - FT) >= FR,
                "one load per chunk; token fragments in the first FT chunks, row fragments after");

  // ---- prologue: index block 0 and steps 0 .. kNS-2 of the first tile, then
  // step 0 into set 0
  issue_index(cur, 0, 0);
#pragma unroll
  for (int p = 0; p < kNS - 1; ++p) {
    const bool in_tile = p < nsteps;
    issue_step(cur, nxt, !in_tile && has_next, in_tile ? p : (has_next ? p - nsteps : nsteps - 1), p);
  }
  wait_vmcnt<2 * kPerStep>();
  barrier_no_fence();
  {
    const bool in_tile = kNS - 1 < nsteps;
    issue_step(cur, nxt, !in_tile && has_next,
               in_tile ? kNS - 1 : (has_next ? kNS - 1 - nsteps : nsteps - 1), kNS - 1);  // slot still unused
  }
  read_frags(0, 0, 0, a0, x0, b0);

  while (true) {
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Eight steps at a time while all eight stay in the tile and the tile
    // starts on a multiple of kNS in the ring; then pairs of in-tile steps;
    // then the last kNS steps (nsteps is even, so every loop runs whole pairs).
    using std::integral_constant;
    int s = 0;
    if ((g & (kNS - 1)) == 0) {
      for (; s + 8 + kNS - 1 < nsteps; s += 8) {
        const int ibc = (qb + (s >> 3)) & 1, ibn = ibc ^ 1;
        body(integral_constant<int, 0>{}, s, ibc, ibn, a0, x0, b0, a1, x1, b1);
        body(integral_constant<int, 1>{}, s + 1, ibc, ibn, a1, x1, b1, a0, x0, b0);
        body(integral_constant<int, 2>{}, s + 2, ibc, ibn, a0, x0, b0, a1, x1, b1);
        body(integral_constant<int, 3>{}, s + 3, ibc, ibn, a1, x1, b1, a0, x0, b0);
        body(integral_constant<int, 4>{}, s + 4, ibc, ibn, a0, x0, b0, a1, x1, b1);
        body(integral_constant<int, 5>{}, s + 5, ibc, ibn, a1, x1, b1, a0, x0, b0);
        body(integral_constant<int, 6>{}, s + 6, ibc, ibn, a0, x0, b0, a1, x1, b1);
        body(integral_constant<int, 7>{}, s + 7, ibc, ibn, a1, x1, b1, a0, x0, b0);
      }
    }
    for (; s + kNS < nsteps; s += 2) {
      body(integral_constant<int, -1>{}, s, 0, 0, a0, x0, b0, a1, x1, b1);
      body(integral_constant<int, -1>{}, s + 1, 0, 0, a1, x1, b1, a0, x0, b0);
    }
    for (; s < nsteps; s += 2) {
      body(integral_constant<int, -2>{}, s, 0, 0, a0, x0, b0, a1, x1, b1);
      body(integral_constant<int, -2>{}, s + 1, 0, 0, a1, x1, b1, a0, x0, b0);
    }

    // ---- epilogue
    stores_behind = R0 + kBR <= R && T0 + kBT <= T;
    if constexpr (OUT == NM_F32) {
      // fp32 Y is written in whole 128-byte lines with non-temporal stores.
      // Fragments i and i+1 hold rows 0..31 of a token as 8 runs of 16 bytes
      // (quarter q of fragment i: rows 4q..4q+3; of fragment i+1: 16+4q..).
      // The upper 8 lanes of each 16-lane row swap their fragment-i values for
      // the lower 8 lanes' fragment-(i+1) values (a rotate by 8 within the
      // row), so one store writes tokens 0..7 of the fragment pair and the
      // next tokens 8..15, each token's 32 rows by 8 lanes: whole lines.
      // Written past the caches, Y no longer evicts the packed weights and
      // activations the later tiles re-read from L2 (on a 3072 x 768 layer
      // over 12608 tokens, HBM reads 126 -> ~70 MB), and whole lines leave no
      // partial-line writes for the memory to merge.
      const bool vec_ok = (ldy & 3) == 0;
      const bool upper = li >= 8;
#pragma unroll
      for (int i = 0; i < FR; i += 2) {
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          f32x4 va, vb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[i][j][e], y = acc[i + 1][j][e];
            const float got = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                0, __builtin_bit_cast(int, upper ? x : y), kRowRotate8, 0xF, 0xF, false));
            va[e] = upper ? got : x;
            vb[e] = upper ? y : got;
          }
          const int r = R0 + wr * 128 + i * 16 + (upper ? 16 : 0) + lq * 4;
          const int tb = T0 + wt * (kBT / 2) + j * 16 + (li & 7);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = tb + 8 * h;
            const f32x4 v = h ? vb : va;
            if (t >= T || r >= R) continue;
            float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
            if (vec_ok && r + 3 < R) {
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(y));
            } else {
              for (int e = 0; e < 4 && r + e < R; ++e) y[e] = v[e];
            }
          }
        }
      }
    } else {
      // Half outputs, also whole 128-byte lines (64 rows) with non-temporal
      // stores.  First fragments i and i+1 (32 rows) are exchanged across lane
      // quarters so that quarter q holds rows 8q .. 8q+7 of the pair (16
      // contiguous bytes); then, as for fp32, the upper 8 lanes of each row of
      // 16 swap their first pair (rows 0..31) for the lower 8 lanes' second
      // pair (rows 32..63), so each store writes 8 tokens x 64 rows.
      const bool vec_ok = (ldy & 7) == 0;
      const bool upper = li >= 8;
      auto pair_rows = [&](int i, int j) {
        const uint32_t x0 = pack_half2<DT>(acc[i][j][0], acc[i][j][1]);
        const uint32_t x1 = pack_half2<DT>(acc[i][j][2], acc[i][j][3]);
        const uint32_t y0 = pack_half2<DT>(acc[i + 1][j][0], acc[i + 1][j][1]);
        const uint32_t y1 = pack_half2<DT>(acc[i + 1][j][2], acc[i + 1][j][3]);
        // lanes 32..63 of x <-> lanes 0..31 of y, then odd 16-lane rows of
        // x <-> even rows of y
        const auto s0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
        const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
        const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
        return u32x4{t0[0], t1[0], t0[1], t1[1]};  // rows 8 lq .. 8 lq + 7 of the pair
      };
#pragma unroll
      for (int i = 0; i < FR; i += 4) {
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const u32x4 p0 = pair_rows(i, j), p1 = pair_rows(i + 2, j);
          u32x4 va, vb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t got = uint32_t(__builtin_amdgcn_update_dpp(
                0, int(upper ? p0[e] : p1[e]), kRowRotate8, 0xF, 0xF, false));
            va[e] = upper ? got : p0[e];
            vb[e] = upper ? p1[e] : got;
          }
          const int r = R0 + wr * 128 + i * 16 + (upper ? 32 : 0) + lq * 8;
          const int tb = T0 + wt * (kBT / 2) + j * 16 + (li & 7);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int t = tb + 8 * h;
            const u32x4 v = h ? vb : va;
            if (t >= T || r >= R) continue;
            uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
            if (vec_ok && r + 7 < R) {
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y));
            } else {
              for (int e = 0; e < 8 && r + e < R; ++e) y[e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
            }
          }
        }
      }
    }
    // The next tile's loads, already in flight, stay in flight across the
    // epilogue.  The last tile waits for everything, so no direct load is
    // still writing LDS when the workgroup ends.
    if (!has_next) {
      wait_vmcnt<0>();
      break;
    }
    tile += tm.grid;
    R0 = nR0;
    T0 = nT0;
    cur = nxt;
    g += nsteps;
    qb += nblocks;
    has_next = tile + tm.grid < tm.ntiles;
    if (has_next) {
      tm.rt(tile + tm.grid, nR0, nT0);
      make_src(nR0, nT0, nxt);
    }
  }
}

template <int DT, int OUT>
hipError_t launch_lds(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + kBR - 1) / kBR);
  const int tilesT = int((a.T + kBT - 1) / kBT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int cus = device_cu_count();
  // One workgroup per CU walks the tiles (each CU holds one: 160 KB of LDS).
  // Running the ring on into the next tile needs the next tile's index block
  // issued at least four steps before its first step is read, i.e. a tile's
  // last index block at least four steps long (nsteps % 8 != 2) and nsteps >= 4;
  // otherwise every tile gets its own workgroup.
  const int64_t nsteps = a.K / 64;
  const bool walk = nsteps >= 4 && nsteps % 8 != 2;
  TileMap tm;
  tm.tilesR = tilesR;
  tm.tilesT = tilesT;
  // Row tiles sharing activation columns are grouped four at a time (per
  // XCD run, four row tiles x eight token tiles: the fewest unique bytes).
  // When the packed values fit an XCD's L2 (4 MB) they stay there across
  // rounds anyway, so all row tiles of a token tile are grouped and each
  // token tile's activations are fetched about once.
  tm.group_r = tilesR < 4 ? tilesR : 4;
  if (a.R * a.K <= (int64_t(4) << 20)) tm.group_r = tilesR;
  tm.ntiles = int(ntiles);
  tm.grid = int(walk && ntiles > cus ? cus : ntiles);
  auto kern = spmm_lds_kernel<DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), kLds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tm.grid)), dim3(256), kLds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.act, int(a.T), a.ldx, a.Y, a.ldy, tm);
  return hipGetLastError();
}

}  // namespace

bool spmm_lds_applies(const SpmmArgs& a) {
  if (!(a.perm == nullptr && a.n == 2 && a.m == 4 && (a.K % 128) == 0 && a.T >= 128 &&
        a.R >= 256))
    return false;
  // per-lane byte offsets within a tile are 32-bit
  const int64_t lim = int64_t(0xFFFFFFFFu);
  if (int64_t(kBT) * a.ldx * 2 > lim || int64_t(kBR) * a.K > lim) return false;
  // needs a workgroup LDS allocation of kLds bytes
  return device_max_lds() >= kLds;
}

hipError_t launch_spmm_lds(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? launch_lds<NM_F16, NM_F32>(a, s) : launch_lds<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? launch_lds<NM_BF16, NM_F32>(a, s) : launch_lds<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
