// 1:4 and 1:8 sparse GEMM for prefill shapes with every operand staged
// through LDS by direct global->LDS loads (gfx950 global_load_lds_dwordx4).
//
// Same product as nm_spmm.hip (Y^T[t, r] = sum_k W_nm[r, k] act[t, k] on
// v_smfmac_f32_16x16x64) and the same widening of a 1:4 / 1:8 row to the 2:4
// operand: a survivor at position p takes one slot of the 4-group holding p,
// its partner slot a zero at the same position, and a 4-group without a
// survivor two zeros at position 0 (RNM-TD3's ratios run at the 2:4 rate while
// only their own packed bytes move).  The MFMA operands equal those of
// nm_spmm_pipe.hip step for step, so the results are bit-identical to it.
//
// Packed rows of these patterns are short: per 64-wide K step a row holds 32
// (1:4) or 16 (1:8) bytes of values and 4 or 3 bytes of index bits.  A lane
// takes its share with one small LDS read, and the widening (a few VALU
// operations per fragment) is done for the next step after the MFMAs of the
// current one, where nothing waits on it.
//
// LDS layout (a direct load puts lane l's 16 bytes at slot base + l, so the
// layout is chosen by the global address each lane reads):
//   activations    one K step per stage; slot (token, chunk c) at
//                  token*8 + (c ^ (token & 7)), as in the 2:4 kernel;
//   packed values  one K step per stage; rows contiguous (32 or 16 B each),
//                  so a fragment's 16 rows are one conflict-free run;
//   index bits     block = 16 K steps of a row.  1:4: 64 bytes, slot (row,
//                  chunk) at row*4 + (chunk ^ ((row >> 2) & 3)); 1:8: 48
//                  bytes loaded 4 at a time, rows contiguous (a 48-byte row
//                  stride puts a fragment's 16 rows on distinct banks).
//
// A workgroup (4 waves stacked along the rows, each 32 rows x 64 tokens = 2 x 4
// fragments, so every row fragment is widened by one wave only) computes
// 128 x 64 tiles: a 4096-row layer at 512 tokens then has one tile
// per compute unit, where 256 x 128 tiles would leave three quarters of the
// chip idle.  Stages form a 4-deep ring (three K steps of loads in flight),
// with counted vmcnt waits and one fence-free barrier per step; every step
// issues the same loads (past the last step a slot is refilled with that step
// again), so the wait counts are constants.  Each tile fills its own ring.
#include "nm_internal.h"

namespace nm {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16_t __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_byte;

// ABID selects the 16-bit half of the index register the instruction reads.
template <int DT, int ABID>
__device__ inline f32x4 smfmac(const u32x4& a, const u32x8& b, const f32x4& c, uint32_t idx) {
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(half8_t, a),
                                                    __builtin_bit_cast(half16_t, b), c, int(idx), 0, ABID);
  } else {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf8_t, a),
                                                     __builtin_bit_cast(bf16_t, b), c, int(idx), 0, ABID);
  }
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <int DT>
__device__ inline uint16_t to_half_bits(float f) {
  if constexpr (DT == NM_F16) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  } else {
    return f32_to_bf16_rne(f);
  }
}

__device__ inline void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline void wait_lgkm0() {
  // lgkmcnt(0), vmcnt/expcnt untouched (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Buffer resource over [base, base + bytes): raw 32-bit data.  A lane whose
// offset lies past `bytes` reads zeros and touches no memory.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// 16 bytes per lane from base + voff + soff into LDS slot lds_dst + lane*16.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, unsigned char* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_byte*)lds_dst, 16, int(voff), int(soff), 0, 0);
}

constexpr int kBR = 128;
constexpr int kBT = 64;
constexpr int kNS = 4;               // one-K-step stages in the ring
constexpr int kStageB = kBT * 128;   // activations, one step
constexpr int kPerStep = 3;          // direct loads per wave per step: 2 activation + 1 packed-value

// P = 1: 1:4, P = 2: 1:8.  VB: packed-value bytes per row per step; IBLK:
// index bytes per row per 16-step block (2 or 3 bits per survivor); IL:
// index loads per wave per block.
template <int P>
struct NmPat;
template <>
struct NmPat<1> {
  static constexpr int VB = 32, IBLK = 64, IL = 2;
};
template <>
struct NmPat<2> {
  static constexpr int VB = 16, IBLK = 48, IL = 6;
};

template <int P>
constexpr int lds_bytes() {
  return kNS * (kStageB + kBR * NmPat<P>::VB) + 2 * kBR * NmPat<P>::IBLK;
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
__global__ __launch_bounds__(256, 2) void spmm_lds_nm_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K, int irow_bytes,
    const uint16_t* __restrict__ act, int T, int64_t ldx, void* __restrict__ Y, int64_t ldy,
    TileMapNM tm) {
  constexpr int FR = 2, FT = 4;
  static_assert(FR == 2, "1:4 index registers hold two row fragments");
  constexpr int VB = NmPat<P>::VB, IBLK = NmPat<P>::IBLK;
  constexpr int SA = kBR * VB;      // packed values, one step
  constexpr int SI = kBR * IBLK;    // index bits, one block
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* bbuf = smem;                        // [kNS][kStageB]
  unsigned char* abuf = smem + kNS * kStageB;        // [kNS][SA]
  unsigned char* ibuf = smem + kNS * (kStageB + SA);  // [2][SI]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // uniform: LDS destinations of the direct loads (M0) are then scalar sums
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int wr = wave;  // rows wr*32 .. wr*32+31 of the tile, all 64 tokens
  const int nsteps = K >> 6;  // a multiple of 4 on this path
  const int S = K / (P == 1 ? 4 : 8);
  const int iwords = irow_bytes >> 2;  // index words per row

  // Per-lane index-block slots, instruction j of a wave.  1:4: 16-byte slots
  // [(wave*2 + j)*64, +64), slot (row, chunk) at row*4 + (chunk ^ ((row >> 2) & 3));
  // 1:8: 4-byte slots [(wave*6 + j)*64, +64), slot (row, word d) at row*12 + d.
  int ipart[NmPat<P>::IL];
#pragma unroll
  for (int j = 0; j < NmPat<P>::IL; ++j) {
    const int slot = (wave * NmPat<P>::IL + j) * 64 + lane;
    ipart[j] = P == 1 ? (slot & 3) ^ ((slot >> 4) & 3) : slot % 12;
  }

  // A tile's load sources: buffer resources at the tile's corner and per-lane
  // 32-bit byte offsets (rows / tokens past the edge reread the last one).
  // Every load is kept inside its row by construction; the index resource
  // also ends with the array.
  __amdgpu_buffer_rsrc_t rb, ra, ri;
  uint32_t boff[2], aoff, ioff[NmPat<P>::IL];
  auto make_src = [&](int R0, int T0) {
    rb = make_rsrc(act + int64_t(T0) * ldx, 0xFFFFFFFFu);
    ra = make_rsrc(values + int64_t(R0) * S, 0xFFFFFFFFu);
    const int64_t ibytes = int64_t(R - R0) * irow_bytes;
    ri = make_rsrc(reinterpret_cast<const unsigned char*>(idx) + int64_t(R0) * irow_bytes,
                   uint32_t(ibytes < 0xFFFFFFFFll ? ibytes : 0xFFFFFFFFll));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int slot = (wave * 2 + j) * 64 + lane;
      const int tok = slot >> 3;
      const int c = (slot & 7) ^ (tok & 7);
      const int t = min(T0 + tok, T - 1) - T0;
      boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(c) * 16u;
    }
    // index: the row's start (the part within the block is added per block)
#pragma unroll
    for (int j = 0; j < NmPat<P>::IL; ++j) {
      const int slot = (wave * NmPat<P>::IL + j) * 64 + lane;
      const int row = P == 1 ? slot >> 2 : slot / 12;
      const int r = min(R0 + row, R - 1) - R0;
      ioff[j] = uint32_t(r) * uint32_t(irow_bytes);
    }
    // packed values: 1:4 slot (row, half) = wave*64 + lane; 1:8 slot row =
    // wave*32 + lane, lanes 0..31 only
    const int arow = P == 1 ? (wave * 64 + lane) >> 1 : wave * 32 + (lane & 31);
    const int ac = P == 1 ? (lane & 1) : 0;
    const int r = min(R0 + arow, R - 1) - R0;
    aoff = uint32_t(r) * uint32_t(S) * 2u + uint32_t(ac) * 16u;
  };

  // the loads of step src into ring slot buf
  auto issue_step = [&](int src, int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(rb, boff[j], uint32_t(src) * 128u, bbuf + buf * kStageB + (wave * 2 + j) * 1024);
    if constexpr (P == 1) {
      dma16(ra, aoff, uint32_t(src) * uint32_t(VB), abuf + buf * SA + wave * 1024);
    } else {
      if (lane < 32) dma16(ra, aoff, uint32_t(src) * uint32_t(VB), abuf + buf * SA + wave * 512);
    }
  };
  // index block q into buffer ib.  Every load stays inside the row: 1:4
  // chunks hold whole steps (4 bytes each, nsteps % 4 == 0) and a chunk past
  // the row's last step rereads the block's chunk 0; 1:8 words past the row
  // reread its last word.  Those slots are never used.
  auto issue_index = [&](int q, int ib) {
#pragma unroll
    for (int j = 0; j < NmPat<P>::IL; ++j) {
      if constexpr (P == 1) {
        const int o = q * IBLK + ipart[j] * 16;
        const uint32_t in_row = uint32_t(o + 16 <= irow_bytes ? o : q * IBLK);
        dma16(ri, ioff[j] + in_row, 0u, ibuf + ib * SI + (wave * 2 + j) * 1024);
      } else {
        const int d = min(q * (IBLK / 4) + ipart[j], iwords - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (lds_byte*)(ibuf + ib * SI + (wave * 6 + j) * 256), 4,
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
  auto read_v = [&](int sl, int i, uint32_t (&v)[2]) {
    const unsigned char* sa = abuf + sl * SA;
    const int row = wr * 32 + i * 16 + li;
    if constexpr (P == 1) {
      // (a uint64_t load: read through the uint2 struct, the compiler cannot
      // tell this from the slots the direct loads are filling and waits for them)
      const uint64_t w = *reinterpret_cast<const uint64_t*>(sa + row * 32 + lq * 8);
      v[0] = uint32_t(w);
      v[1] = uint32_t(w >> 32);
    } else {
      v[0] = *reinterpret_cast<const uint32_t*>(sa + row * 16 + lq * 4);
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
  // Widen step t (0..3, a constant at every call) of the current four-step
  // index group into row operands a[] and index registers k[] (1:4: one
  // register for both fragments, read through the MFMA's abid; 1:8: one each).
  // byte selector: byte lq of fragment 0's word into bits 0..7, of fragment
  // 1's into bits 16..23, zeros elsewhere
  const uint32_t sel14 = uint32_t(lq) | (0x0Cu << 8) | (uint32_t(4 + lq) << 16) | (0x0Cu << 24);
  const uint32_t off6 = uint32_t(6 * lq);  // the lane's 6 bits in a 1:8 step's 24
  auto widen = [&](int t, const uint32_t (&v)[FR][2], const uint32_t (&w)[FR][4], u32x4 (&a)[FR],
                   uint32_t (&k)[FR]) {
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

  f32x4 acc[FR][FT];
  u32x4 a0[FR], a1[FR];
  uint32_t k0[FR], k1[FR];
  u32x8 b0[FT], b1[FT];
  uint32_t rv[FR][2];  // raw packed values of the step being read
  uint32_t rw[FR][4];  // raw index words of the current four-step group

  // One step s (position C = s & 3, a compile-time constant: every tile
  // starts at ring slot 0 and nsteps % 4 == 0): make step s+1 visible,
  // refill slot C with step s+4, read step s+1, multiply step s, widen s+1.
  auto body = [&](auto c_, int s, u32x4 (&ca)[FR], uint32_t (&ck)[FR], u32x8 (&cb)[FT],
                  u32x4 (&na)[FR], uint32_t (&nk)[FR], u32x8 (&nb)[FT]) {
    constexpr int C = decltype(c_)::value;
    // step s+1 has landed once at most the loads of steps s+2, s+3 remain (an
    // index block issued in between only makes the wait stricter)
    wait_vmcnt<2 * kPerStep>();
    wait_lgkm0();        // this wave's reads of step s are done
    barrier_no_fence();  // publishes step s+1; every wave is done reading step s
    if constexpr (C == 0) {
      if ((s & 15) == 0 && s + 16 < nsteps) issue_index((s >> 4) + 1, ((s >> 4) + 1) & 1);
    }
    issue_step(min(s + kNS, nsteps - 1), C);
    constexpr int RS = (C + 1) & 3;  // slot and group position of step s+1
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      read_b(RS, j, 0, nb[j]);
      read_b(RS, j, 1, nb[j]);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) read_v(RS, i, rv[i]);
    if constexpr (RS == 0) {
      const int s1 = s + 1;
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
    widen(RS, rv, rw, na, nk);
    // keeps the widening here, behind the MFMAs it overlaps, rather than in
    // front of the next step's MFMAs, which need its results
    __builtin_amdgcn_sched_barrier(0);
  };

  using std::integral_constant;
  for (int tile = blockIdx.x; tile < tm.ntiles; tile += tm.grid) {
    int R0, T0;
    tm.rt(tile, R0, T0);
    make_src(R0, T0);
#pragma unroll
    for (int i = 0; i < FR; ++i)
#pragma unroll
      for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: index block 0 and steps 0 .. kNS-2, then step kNS-1 into
    // the last slot and step 0 into register set 0
    issue_index(0, 0);
#pragma unroll
    for (int p = 0; p < kNS - 1; ++p) issue_step(min(p, nsteps - 1), p);
    wait_vmcnt<2 * kPerStep>();  // index block 0 and step 0
    barrier_no_fence();
    issue_step(min(kNS - 1, nsteps - 1), kNS - 1);
#pragma unroll
    for (int j = 0; j < FT; ++j) {
      read_b(0, j, 0, b0[j]);
      read_b(0, j, 1, b0[j]);
    }
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      read_v(0, i, rv[i]);
      read_ix(0, 0, i, rw[i]);
    }
    widen(0, rv, rw, a0, k0);

    for (int s = 0; s < nsteps; s += 4) {
      body(integral_constant<int, 0>{}, s, a0, k0, b0, a1, k1, b1);
      body(integral_constant<int, 1>{}, s + 1, a1, k1, b1, a0, k0, b0);
      body(integral_constant<int, 2>{}, s + 2, a0, k0, b0, a1, k1, b1);
      body(integral_constant<int, 3>{}, s + 3, a1, k1, b1, a0, k0, b0);
    }

    // The refills past the last step are still landing and every wave may
    // still read: drain both before the next tile's prologue reuses the ring
    // (and before the workgroup ends, so no direct load writes LDS after it).
    // Stores share the load counter, so this comes before the epilogue's
    // stores, which then overlap the next tile's first loads.
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier_no_fence();

    // ---- epilogue
    const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const int r = R0 + wr * 32 + i * 16 + lq * 4;
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const int t = T0 + j * 16 + li;
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
  // two workgroups fit a CU (LDS and registers); more tiles than that are walked
  TileMapNM tm;
  tm.tilesT = tilesT;
  tm.ntiles = int(ntiles);
  tm.grid = int(ntiles > 2 * cus ? 2 * cus : ntiles);
  auto kern = spmm_lds_nm_kernel<P, DT, OUT>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds_bytes<P>()); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(tm.grid)), dim3(256), lds_bytes<P>(), s, a.values, a.idx, int(a.R),
                     int(a.K), int(a.idx_row_words * 4), a.act, int(a.T), a.ldx, a.Y, a.ldy, tm);
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
