// 1:4 and 1:8 sparse GEMM for prefill shapes with every operand staged
// through LDS by direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k] on
// v_smfmac_f32_16x16x64) and the same widening of a 1:4 / 1:8 row to the 2:4
// operand: a survivor at position p takes one slot of the 4-group holding p,
// its partner slot a zero at the same position, and a 4-group without a
// survivor two zeros at position 0 (RNM-TD3's ratios run at the 2:4 rate while
// only their own packed bytes move).  The MFMA operands equal those of
// nm_spmm_pipe.hip step for step; the sums differ from it only in their order
// (even and odd K steps apart, then added).
//
// Packed rows of these patterns are short: per 64-wide K step a row holds 32
// (1:4) or 16 (1:8) bytes of values and 4 or 3 bytes of index bits.  Loaded
// step by step they would arrive as 32- or 16-byte pieces, and the number of
// outstanding requests a compute unit can keep, not their bytes, would set the
// pace; so the values come in groups of steps whose rows are whole 128-byte
// runs (4 steps for 1:4, 8 for 1:8), double-buffered.  A lane takes its share
// of a step with one small LDS read, and the widening (a few VALU operations
// per fragment) is done for the next step after the MFMAs of the current one,
// where nothing waits on it.
//
// LDS layout (a direct load puts lane l's 16 bytes at slot base + l, so the
// layout is chosen by the global address each lane reads):
//   activations    one K step per stage; slot (token, chunk c) at
//                  token*8 + (c ^ (token & 7)), as in the 2:4 kernel;
//   packed values  one group of steps per buffer (128 B per row): 16-byte
//                  chunk c of row r at slot r*8 + (c ^ ((r >> 1) & 7)), so
//                  a fragment's 16 rows read the same chunk from 16 distinct
//                  bank quads;
//   index bits     block = 16 K steps of a row.  1:4: 64 bytes, slot (row,
//                  chunk) at row*4 + (chunk ^ ((row >> 2) & 3)); 1:8: 48
//                  bytes loaded 4 at a time, rows contiguous (a 48-byte row
//                  stride puts a fragment's 16 rows on distinct banks).
//
// A workgroup computes 128 x 64 tiles (a 4096-row layer at 512 tokens then
// has one tile per compute unit, where 256 x 128 tiles would leave three
// quarters of the chip idle) with 8 waves in two groups of four: the first
// group multiplies the even K steps, the second the odd ones, each wave 32
// rows x 64 tokens (2 x 4 fragments, every row fragment widened by one wave of
// its group).  So each SIMD holds one wave of each group, and one wave's
// fragment reads, widening and waits run beside the other's MFMAs.  At the
// end of a tile the odd steps' partial sums reach the even group through LDS
// and are added once (even + odd, the same order on every run).  Activation
// stages form a ring of four step pairs (three pairs of loads in flight while
// one is read), each group loading its own step of a pair; a value group is
// loaded with the activations of its first pair, three groups buffered; counted
// vmcnt waits and one fence-free barrier per pair; every pair issues the same
// loads (past the last step a slot is refilled with that step again, and past
// the last group the last group is loaded again), so the wait counts are
// fixed.  Each tile fills its own ring.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

constexpr int kBR = 128;
constexpr int kBT = 64;
constexpr int kWaves = 8;            // two groups of four waves: even and odd K steps
constexpr int kNP = 4;               // step pairs in the ring (8 one-step stages)
constexpr int kStageB = kBT * 128;   // activations, one step
constexpr int kPerPair = 2;          // activation loads per wave per step pair (its group's step)
constexpr int kGroupLoads = 2;       // packed-value loads per wave per group
constexpr int kNG = 3;               // packed-value group buffers
constexpr int kSAG = kBR * 128;      // packed values, one group (128 B per row)

// P = 1: 1:4, P = 2: 1:8 (32 or 16 value bytes per row per K step).  GS: steps
// per 128-byte value group; IBLK: index bytes per row per 16-step block (2 or
// 3 bits per survivor); IL: index loads per wave per block.
template <int P>
struct NmPat;
template <>
struct NmPat<1> {
  static constexpr int GS = 4, IBLK = 64, IL = 1;
};
template <>
struct NmPat<2> {
  static constexpr int GS = 8, IBLK = 48, IL = 3;
};

template <int P>
constexpr int lds_bytes() {
  return 2 * kNP * kStageB + kNG * kSAG + 2 * kBR * NmPat<P>::IBLK;
}

// Tile i of the grid-stride sequence -> (row tile, token tile), token tiles
// fastest.  Within a full round of `grid` tiles each XCD gets a contiguous run
// (workgroup p runs on XCD p % 8), so an XCD's tiles share rows of W and the
// L2 holds them once.
struct TileMapNM {
  int tilesT, ntiles, grid;
  __device__ void rt(int i, int& R0, int& T0) const {
    const int round = i / grid, p = i - round * grid;
    int q = p;
    if ((grid & 7) == 0 && (round + 1) * grid <= ntiles) q = (p & 7) * (grid >> 3) + (p >> 3);
    const int b = round * grid + q;
    R0 = (b / tilesT) * kBR;
    T0 = (b % tilesT) * kBT;
  }
};

// Widening of one lane's share of a row fragment to the 2:4 operand (the
// lane covers four 4-groups of the step).
//   1:4 values: the 4 survivors (two per word) each with a zero partner.
//   1:4 index: ib2 holds the lane's index byte of row fragment 0 in bits 0..7
//     and of fragment 1 in bits 16..23 (four 2-bit positions each); every
//     position p becomes the 4-bit field p | p << 2 = 5p (both slots of its
//     4-group), so fragment 0's 16 index bits come out in the low half and
//     fragment 1's in the high half of one register.
//   1:8: v = the lane's 2 survivors, bits = their 3-bit positions in their
//     8-groups; bit 2 (bit 5) tells which 4-group of the pair holds survivor
//     0 (1); the other 4-group gets zeros at position 0.
__device__ inline void widen_1of4_values(uint32_t v0, uint32_t v1, u32x4& a) {
  a[0] = v0 & 0xFFFFu;
  a[1] = v0 >> 16;
  a[2] = v1 & 0xFFFFu;
  a[3] = v1 >> 16;
}

__device__ inline uint32_t widen_1of4_index2(uint32_t ib2) {
  uint32_t x = (ib2 | (ib2 << 4)) & 0x0F0F0F0Fu;  // fields 0,1 | 2,3 into separate bytes
  x = (x | (x << 2)) & 0x33333333u;               // one field per nibble
  return x * 5u;                                  // p -> p | p << 2 (no carries: p <= 3)
}

__device__ inline void widen_1of8(uint32_t v, uint32_t bits, u32x4& a, uint32_t& idx16) {
  const uint64_t a01 = uint64_t(v & 0xFFFFu) << ((bits << 3) & 32u);
  const uint64_t a23 = uint64_t(v >> 16) << (bits & 32u);
  a[0] = uint32_t(a01);
  a[1] = uint32_t(a01 >> 32);
  a[2] = uint32_t(a23);
  a[3] = uint32_t(a23 >> 32);
  // Each survivor's index byte depends only on its 3-bit position p:
  // 5 (p & 3) in the nibble of its 4-group, 5 (p & 3) << 4 (p >> 2).  The
  // eight possible bytes form a table that one byte permute reads at p0 and
  // p1 (selector byte 0x0C gives zero).
  constexpr uint32_t kTabLo = 0x0F0A0500u, kTabHi = 0xF0A05000u;
  const uint32_t sel = ((bits >> 3) << 8) | (bits & 7u) | 0x0C0C0000u;
  idx16 = __builtin_amdgcn_perm(kTabHi, kTabLo, sel);
}

template <int P, int DT, int OUT>
__global__ __launch_bounds__(kWaves * 64, 1) void spmm_lds_nm_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K, int irow_bytes,
    const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y, int64_t ldy,
    TileMapNM tm) {
  constexpr int FR = 2, FT = 4;
  static_assert(FR == 2, "1:4 index registers hold two row fragments");
  constexpr int GS = NmPat<P>::GS, IBLK = NmPat<P>::IBLK, IL = NmPat<P>::IL;
  constexpr int SI = kBR * IBLK;    // index bits, one block
  constexpr int HG = GS / 2;        // step pairs per value group
  constexpr int G0 = P == 1 ? 2 : 1;  // value groups loaded before the first pair
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* bbuf = smem;                     // [2 kNP][kStageB]
  unsigned char* abuf = smem + 2 * kNP * kStageB;  // [kNG][kSAG]
  unsigned char* ibuf = abuf + kNG * kSAG;         // [2][SI]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform: LDS destinations of the direct loads (M0) are then scalar sums
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int grp = wave >> 2;  // 0: K steps 0, 2, 4, ...; 1: steps 1, 3, 5, ...
  const int wr = wave & 3;    // rows wr*32 .. wr*32+31 of the tile, all 64 tokens
  const int nsteps = K >> 6;  // a multiple of 4 on this path
  const int npairs = nsteps >> 1;
  const int S = K / (P == 1 ? 4 : 8);
  const int iwords = irow_bytes >> 2;  // index words per row
  const int ngroups = (nsteps + GS - 1) / GS;
  // 1:8 with nsteps % 8 == 4: the last group holds four steps (64 B per row)
  const bool half_last = P == 2 && (nsteps % GS) != 0;

  // Per-lane index-block slots, instruction j of a wave.  1:4: 16-byte slots
  // [(wave + j)*64, +64), slot (row, chunk) at row*4 + (chunk ^ ((row >> 2) & 3));
  // 1:8: 4-byte slots [(wave*3 + j)*64, +64), slot (row, word d) at row*12 + d.
  int ipart[IL];
#pragma unroll
  for (int j = 0; j < IL; ++j) {
    const int slot = (wave * IL + j) * 64 + lane;
    ipart[j] = P == 1 ? (slot & 3) ^ ((slot >> 4) & 3) : slot % 12;
  }

  // Packed-value loads: bit j of ahi is set when load j puts this lane's
  // chunk in the second half of its row's 128-byte run.
  int ahi = 0;
#pragma unroll
  for (int j = 0; j < kGroupLoads; ++j) {
    const int slot = (wave * kGroupLoads + j) * 64 + lane;
    ahi |= (((slot & 7) ^ ((slot >> 4) & 7)) >= 4 ? 1 : 0) << j;
  }

  // A tile's load sources: buffer resources at the tile's corner and per-lane
  // 32-bit byte offsets (rows / tokens past the edge reread the last one).
  // Every load is kept inside its row by construction; the index resource
  // also ends with the array.
  __amdgpu_buffer_rsrc_t rb, ra, ri;
  uint32_t boff[kPerPair], aoff[kGroupLoads], ioff[IL];
  auto make_src = [&](int R0, int T0) {
    rb = make_rsrc(act + int64_t(T0) * ldx, 0xFFFFFFFFu);
    ra = make_rsrc(values + int64_t(R0) * S, 0xFFFFFFFFu);
    const int64_t ibytes = int64_t(R - R0) * irow_bytes;
    ri = make_rsrc(reinterpret_cast<const unsigned char*>(idx) + int64_t(R0) * irow_bytes,
                   uint32_t(ibytes < 0xFFFFFFFFll ? ibytes : 0xFFFFFFFFll));
    // activations: the four waves of a group load their group's step, part
    // (wr*2 + j) of 8 (64 tokens x 128 bytes)
#pragma unroll
    for (int j = 0; j < kPerPair; ++j) {
      const int slot = (wr * 2 + j) * 64 + lane;
      const int tok = slot >> 3;
      const int c = (slot & 7) ^ (tok & 7);
      const int t = min(T0 + tok, T - 1) - T0;
      boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(c) * 16u;
    }
    // index: the row's start (the part within the block is added per block)
#pragma unroll
    for (int j = 0; j < IL; ++j) {
      const int slot = (wave * IL + j) * 64 + lane;
      const int row = P == 1 ? slot >> 2 : slot / 12;
      const int r = min(R0 + row, R - 1) - R0;
      ioff[j] = uint32_t(r) * uint32_t(irow_bytes);
    }
    // packed values: load j of a wave fills slots [(wave*2 + j)*64, +64) of a
    // group buffer, 8 whole rows; slot (row, chunk c) at row*8 + (c ^ ((row >> 1) & 7))
#pragma unroll
    for (int j = 0; j < kGroupLoads; ++j) {
      const int slot = (wave * kGroupLoads + j) * 64 + lane;
      const int row = slot >> 3;
      const int c = (slot & 7) ^ ((row >> 1) & 7);
      const int r = min(R0 + row, R - 1) - R0;
      aoff[j] = uint32_t(r) * uint32_t(S) * 2u + uint32_t(c) * 16u;
    }
  };

  // this wave's share of the activations of step src (its group's parity)
  // into ring slot buf
  auto issue_step = [&](int src, int buf) {
#pragma unroll
    for (int j = 0; j < kPerPair; ++j)
      dma16(rb, boff[j], uint32_t(src) * 128u, bbuf + buf * kStageB + (wr * 2 + j) * 1024);
  };
  // the packed values of group g (clamped to the last group) into buffer gb.
  // Every load stays inside its row: a row is nsteps * VB bytes, whole groups
  // of 128 bytes except a four-step last 1:8 group, whose missing half
  // (chunks 4..7) rereads chunks 0..3; those slots are never read.
  auto issue_group = [&](int g, int gb) {
    g = min(g, ngroups - 1);
    const bool part = half_last && g == ngroups - 1;
#pragma unroll
    for (int j = 0; j < kGroupLoads; ++j) {
      const uint32_t back = (part && ((ahi >> j) & 1)) ? 64u : 0u;
      dma16(ra, aoff[j] - back, uint32_t(g) * 128u, abuf + gb * kSAG + (wave * kGroupLoads + j) * 1024);
    }
  };
  // index block q into buffer ib.  Every load stays inside the row: 1:4
  // chunks hold whole steps (4 bytes each, nsteps % 4 == 0) and a chunk past
  // the row's last step rereads the block's chunk 0; 1:8 words past the row
  // reread its last word.  Those slots are never used.
  auto issue_index = [&](int q, int ib) {
#pragma unroll
    for (int j = 0; j < IL; ++j) {
      if constexpr (P == 1) {
        const int o = q * IBLK + ipart[j] * 16;
        const uint32_t in_row = uint32_t(o + 16 <= irow_bytes ? o : q * IBLK);
        dma16(ri, ioff[j] + in_row, 0u, ibuf + ib * SI + (wave * IL + j) * 1024);
      } else {
        const int d = min(q * (IBLK / 4) + ipart[j], iwords - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (lds_byte*)(ibuf + ib * SI + (wave * IL + j) * 256), 4,
                                                 int(ioff[j] + uint32_t(d) * 4u), 0, 0, 0);
      }
    }
  };

  // Fragment reads.  Row fragment i of this wave: rows wr*32 + i*16 + li.
  auto read_b = [&](int sl, int j, int h, u32x8& bf) {
    const unsigned char* sb = bbuf + sl * kStageB;
    const int tok = j * 16 + li;
    const u32x4 v = *reinterpret_cast<const u32x4*>(sb + (tok * 8 + ((lq + 4 * h) ^ (tok & 7))) * 16);
    bf[4 * h + 0] = v[0];
    bf[4 * h + 1] = v[1];
    bf[4 * h + 2] = v[2];
    bf[4 * h + 3] = v[3];
  };
  // packed values of step u (t = u % GS) of row fragment i: the lane's 8
  // (1:4) or 4 (1:8) bytes, at byte t*VB + lq*(VB/4) of the row's 128-byte run
  auto read_v = [&](int u, int t, int i, uint32_t (&v)[2]) {
    const unsigned char* sa = abuf + ((u / GS) % kNG) * kSAG;
    const int row = wr * 32 + i * 16 + li;
    const int f = (row >> 1) & 7;
    if constexpr (P == 1) {
      const int c = 2 * t + (lq >> 1);
      // (a uint64_t load: read through the uint2 struct, the compiler cannot
      // tell this from the slots the direct loads are filling and waits for them)
      const uint64_t w = *reinterpret_cast<const uint64_t*>(sa + (row * 8 + (c ^ f)) * 16 + (lq & 1) * 8);
      v[0] = uint32_t(w);
      v[1] = uint32_t(w >> 32);
    } else {
      v[0] = *reinterpret_cast<const uint32_t*>(sa + (row * 8 + (t ^ f)) * 16 + lq * 4);
      v[1] = 0u;
    }
  };
  // index bits of four steps (group g of block buffer ib) of row fragment i:
  // 1:4 one 16-byte chunk (4 bytes per step), 1:8 three words (24 bits per step)
  auto read_ix = [&](int ib, int g, int i, uint32_t (&w)[4]) {
    const unsigned char* si = ibuf + ib * SI;
    const int row = wr * 32 + i * 16 + li;
    if constexpr (P == 1) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(si + row * 64 + (g ^ ((row >> 2) & 3)) * 16);
      w[0] = v[0];
      w[1] = v[1];
      w[2] = v[2];
      w[3] = v[3];
    } else {
#pragma unroll
      for (int e = 0; e < 3; ++e) w[e] = *reinterpret_cast<const uint32_t*>(si + row * 48 + (3 * g + e) * 4);
      w[3] = 0u;
    }
  };
  // Widen step t (0..3, a compile-time constant) of the current four-step
  // index group into row operands a[] and index registers k[] (1:4: one
  // register for both fragments, read through the MFMA's abid; 1:8: one each).
  // byte selector: byte lq of fragment 0's word into bits 0..7, of fragment
  // 1's into bits 16..23, zeros elsewhere
  const uint32_t sel14 = uint32_t(lq) | (0x0Cu << 8) | (uint32_t(4 + lq) << 16) | (0x0Cu << 24);
  const uint32_t off6 = uint32_t(6 * lq);  // the lane's 6 bits in a 1:8 step's 24
  auto widen = [&](auto t_c, const uint32_t (&v)[FR][2], const uint32_t (&w)[FR][4], u32x4 (&a)[FR],
                   uint32_t (&k)[FR]) {
    constexpr int t = decltype(t_c)::value;
    if constexpr (P == 1) {
#pragma unroll
      for (int i = 0; i < FR; ++i) widen_1of4_values(v[i][0], v[i][1], a[i]);
      k[0] = widen_1of4_index2(__builtin_amdgcn_perm(w[1][t], w[0][t], sel14));
      k[1] = k[0];
    } else {
#pragma unroll
      for (int i = 0; i < FR; ++i) {
        // step t's 24 bits start at bit 24t of the group's three words
        const uint32_t x = t == 0   ? w[i][0]
                           : t == 1 ? __builtin_amdgcn_alignbit(w[i][1], w[i][0], 24u)
                           : t == 2 ? __builtin_amdgcn_alignbit(w[i][2], w[i][1], 16u)
                                    : w[i][2] >> 8;
        widen_1of8(v[i][0], (x >> off6) & 63u, a[i], k[i]);
      }
    }
  };
  using std::integral_constant;
  // step t0 + grp of the four-step index group: t0 is a constant, grp uniform
  auto widen_own = [&](auto t0_c, const uint32_t (&v)[FR][2], const uint32_t (&w)[FR][4], u32x4 (&a)[FR],
                       uint32_t (&k)[FR]) {
    constexpr int t0 = decltype(t0_c)::value;
    if (grp) widen(integral_constant<int, t0 + 1>{}, v, w, a, k);
    else widen(integral_constant<int, t0>{}, v, w, a, k);
  };

  f32x4 acc[FR][FT];
  u32x4 a0[FR], a1[FR];
  uint32_t k0[FR], k1[FR];
  u32x8 b0[FT], b1[FT];
  uint32_t rv[FR][2];  // raw packed values of the step being read
  uint32_t rw[FR][4];  // raw index words of the current four-step group

  // Value group m is loaded by the body that loads the activations of its
  // first pair (pair HG*m, body HG*m - 4), into buffer m % kNG; groups below
  // G0 by the prologue.  Three buffers: the group loaded in body x replaces
  // the one whose last step was read three groups earlier.
  auto group_at = [&](int x) { return x >= 0 && ((x + 4) % HG) == 0 && (x + 4) / HG >= G0; };

  // One pair p of K steps (steps 2p and 2p+1; this wave's step s = 2p + grp,
  // the pair's parity PAR a compile-time constant): make pair p+1 visible,
  // refill this wave's slot with step s + 8, read step s + 2, multiply step s,
  // widen s + 2.  The two groups' waves share each SIMD, so one group's
  // fragment reads and widening run beside the other's MFMAs.
  auto body = [&](auto par_c, int p, u32x4 (&ca)[FR], uint32_t (&ck)[FR], u32x8 (&cb)[FT],
                  u32x4 (&na)[FR], uint32_t (&nk)[FR], u32x8 (&nb)[FT]) {
    constexpr int PAR = decltype(par_c)::value;
    // Pair p+1 has landed once at most the loads issued after this wave's
    // share of it remain: its shares of pairs p+2, p+3, and a value group if
    // body p-2 or p-1 loaded one (an index block loaded in between only
    // makes the wait stricter).
    if (group_at(p - 2) || group_at(p - 1))
      wait_vmcnt<2 * kPerPair + kGroupLoads>();
    else
      wait_vmcnt<2 * kPerPair>();
    wait_lgkm0();        // this wave's reads of step s are done
    barrier_no_fence();  // publishes pair p+1; every wave is done reading pair p
    if constexpr (PAR == 0) {
      if ((p & 7) == 0 && 2 * p + 16 < nsteps) issue_index((p >> 3) + 1, ((p >> 3) + 1) & 1);
    }
    if (group_at(p)) {
      const int m = (p + 4) / HG;
      issue_group(m, m % kNG);
    }
    const int s = 2 * p + grp;
    issue_step(min(s + 2 * kNP, nsteps - 1), s & 7);
    const int s1 = s + 2;
    const int rs = s1 & 7;
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      read_b(rs, j, 0, nb[j]);
      read_b(rs, j, 1, nb[j]);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) read_v(s1, P == 1 ? (s1 & 3) : (s1 & 7), i, rv[i]);
    if constexpr (PAR == 1) {
      // step s + 2 opens its four-step index group
#pragma unroll
      for (int i = 0; i < FR; ++i) read_ix((s1 >> 4) & 1, (s1 >> 2) & 3, i, rw[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      acc[0][j] = smfmac<DT, 0>(ca[0], cb[j], acc[0][j], ck[0]);
      acc[1][j] = smfmac<DT, P == 1 ? 1 : 0>(ca[1], cb[j], acc[1][j], ck[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // step s + 2 sits at position 2 (pair p even) or 0 (p odd), plus grp, of
    // its four-step index group
    widen_own(integral_constant<int, PAR == 0 ? 2 : 0>{}, rv, rw, na, nk);
    // keeps the widening here, behind the MFMAs it overlaps, rather than in
    // front of the next step's MFMAs, which need its results
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int tile = blockIdx.x; tile < tm.ntiles; tile += tm.grid) {
    int R0, T0;
    tm.rt(tile, R0, T0);
    make_src(R0, T0);
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: index block 0, the first value groups and pairs
    // 0 .. kNP-2, then pair kNP-1 and this wave's step of pair 0 into
    // register set 0
    issue_index(0, 0);
#pragma unroll
    for (int m = 0; m < G0; ++m) issue_group(m, m);
#pragma unroll
    for (int q = 0; q < kNP - 1; ++q) issue_step(min(2 * q + grp, nsteps - 1), (2 * q + grp) & 7);
    wait_vmcnt<2 * kPerPair>();  // index block 0, the first groups and pair 0
    barrier_no_fence();
    issue_step(min(2 * (kNP - 1) + grp, nsteps - 1), (2 * (kNP - 1) + grp) & 7);
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      read_b(grp, j, 0, b0[j]);
      read_b(grp, j, 1, b0[j]);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      read_v(grp, grp, i, rv[i]);
      read_ix(0, 0, i, rw[i]);
    }
    widen_own(integral_constant<int, 0>{}, rv, rw, a0, k0);

    for (int p = 0; p < npairs; p += 2) {
      body(integral_constant<int, 0>{}, p, a0, k0, b0, a1, k1, b1);
      body(integral_constant<int, 1>{}, p + 1, a1, k1, b1, a0, k0, b0);
    }

    // The refills past the last step are still landing and every wave may
    // still read: drain both before the ring is reused.  Stores share the
    // load counter, so this comes before the epilogue's stores, which then
    // overlap the next tile's first loads.
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier_no_fence();

    // ---- the odd steps' partial sums join the even steps' through LDS (the
    // ring is idle): sum = even + odd, the same order every run
    f32x4* red = reinterpret_cast<f32x4*>(bbuf);  // [4 waves][FR * FT][64 lanes]
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) red[(wr * (FR * FT) + i * FT + j) * 64 + lane] = acc[i][j];
    }
    wait_lgkm0();
    barrier_no_fence();
    f32x4 odd[FR][FT];
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < FR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) odd[i][j] = red[(wr * (FR * FT) + i * FT + j) * 64 + lane];
    }
    wait_lgkm0();
    barrier_no_fence();  // the next tile's prologue may refill the ring
    if (grp != 0) continue;

    // ---- epilogue (the even-step group's waves)
    const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int r = R0 + wr * 32 + i * 16 + lq * 4;
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int t = T0 + j * 16 + li;
        if (t >= T || r >= R) continue;
        const f32x4 v = acc[i][j] + odd[i][j];
        if constexpr (OUT == NM_F32) {
          float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
          if (vec_ok && r + 3 < R) {
            *reinterpret_cast<f32x4*>(y) = v;
          } else {
            for (int e = 0; e < 4 && r + e < R; ++e) y[e] = v[e];
          }
        } else {
          uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
          const uint16_t h0 = to_half_bits<DT>(v[0]), h1 = to_half_bits<DT>(v[1]);
          const uint16_t h2 = to_half_bits<DT>(v[2]), h3 = to_half_bits<DT>(v[3]);
          if (vec_ok && r + 3 < R) {
            *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(h0) | (uint32_t(h1) << 16),
                                                      uint32_t(h2) | (uint32_t(h3) << 16));
          } else {
            const uint16_t hh[4] = {h0, h1, h2, h3};
            for (int e = 0; e < 4 && r + e < R; ++e) y[e] = hh[e];
          }
        }
      }
    }
  }
}

template <int P, int DT, int OUT>
hipError_t launch_lds_nm(const SpmmArgs& a, hipStream_t s) {
  const int tilesR = int((a.R + kBR - 1) / kBR);
  const int tilesT = int((a.T + kBT - 1) / kBT);
  const int64_t ntiles = int64_t(tilesR) * tilesT;
  if (ntiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int cus = device_cu_count();
  // one workgroup (eight waves, two per SIMD) per CU; more tiles are walked
  TileMapNM tm;
  tm.tilesT = tilesT;
  tm.ntiles = int(ntiles);
  tm.grid = int(ntiles > cus ? cus : ntiles);
  auto kern = spmm_lds_nm_kernel<P, DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds_bytes<P>()); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tm.grid)), dim3(kWaves * 64), lds_bytes<P>(), s, a.values, a.idx,
                     int(a.R), int(a.K), int(a.idx_row_words * 4), a.act, int(a.T), a.ldx, a.Y, a.ldy, tm);
  return hipGetLastError();
}

template <int P, int DT>
hipError_t lds_nm_out(const SpmmArgs& a, hipStream_t s) {
  return a.out_dtype == NM_F32 ? launch_lds_nm<P, DT, NM_F32>(a, s) : launch_lds_nm<P, DT, DT>(a, s);
}

template <int P>
hipError_t lds_nm_dtype(const SpmmArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? lds_nm_out<P, NM_F16>(a, s) : lds_nm_out<P, NM_BF16>(a, s);
}

}  // namespace

bool spmm_lds_nm_applies(const SpmmArgs& a) {
  if (!(a.perm == nullptr && a.n == 1 && (a.m == 4 || a.m == 8) && (a.K % 256) == 0 && a.T >= 64 &&
        a.R >= 128))
    return false;
  // per-lane byte offsets within a tile are 32-bit
  const int64_t lim = int64_t(0xFFFFFFFFu);
  const int64_t S = a.K / a.m;
  if (int64_t(kBT) * a.ldx * 2 > lim || int64_t(kBR) * S * 2 > lim ||
      int64_t(kBR) * a.idx_row_words * 4 > lim)
    return false;
  return true;
}

hipError_t launch_spmm_lds_nm(const SpmmArgs& a, hipStream_t s) {
  if (a.n == 1 && a.m == 4) return lds_nm_dtype<1>(a, s);
  if (a.n == 1 && a.m == 8) return lds_nm_dtype<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nm
