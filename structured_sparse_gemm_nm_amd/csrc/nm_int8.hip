// 8-bit 2:4 weights: prune + pack, decompress, and the sparse GEMM, for INT8
// (v_smfmac_i32_16x16x128_i8, exact int32 Y) and for OCP FP8 E4M3
// (v_smfmac_f32_16x16x128_fp8_fp8, fp32 Y) from one template.
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
// So every operand is a plain 16- or 4-byte load of the stored data.  E4M3
// differs only in the magnitude key (the pattern's low 7 bits, so +x and -x
// tie) and in the accumulator: the fp8 instruction was checked the same way
// and takes the same operand layout.
#include "nm_device.h"
#include "nm_internal.h"

#include <type_traits>

namespace nm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One-byte element types: F8 = false int8 (exact int32 product), true OCP FP8
// E4M3 (v_smfmac_f32_16x16x128_fp8_fp8, fp32 accumulators; the same operand
// layout, found the same way).  Magnitude key: |w| for int8, bits & 0x7F for
// E4M3 (the sign bit dropped; finite E4M3 values order by their low 7 bits).
template <bool F8>
using acc8_t = std::conditional_t<F8, f32x4, i32x4>;

template <bool F8>
__device__ inline acc8_t<F8> smfmac8(const i32x4& a, const i32x8& b, const acc8_t<F8>& c, uint32_t idx) {
  if constexpr (F8) {
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(a, b, c, int(idx), 0, 0);
  } else {
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, int(idx), 0, 0);
  }
}

// One group of four int8 weights (byte p = position p): the two kept
// positions, ascending, with their bytes.  Composite keys put |w| above the
// tie-break (the lower position wins), so they are distinct and a position is
// kept when fewer than two keys exceed its own.
template <bool F8>
__device__ inline void top2_of_4(uint32_t g, uint32_t& p0, uint32_t& p1, uint32_t& v0, uint32_t& v1) {
  uint32_t key[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t byte = (g >> (8 * p)) & 0xFFu;
    const int w = int(int8_t(uint8_t(byte)));
    const uint32_t mag = F8 ? (byte & 0x7Fu) : uint32_t(w < 0 ? -w : w);
    key[p] = (mag << 2) | uint32_t(3 - p);
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
template <bool F8>
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
    top2_of_4<F8>(g4[g], p0, p1, v0, v1);
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

template <bool F8>
__global__ __launch_bounds__(256) void spmm_i8_kernel(const uint8_t* __restrict__ values,
                                                      const uint32_t* __restrict__ idx, int R, int K,
                                                      int words, const uint8_t* __restrict__ act, int T,
                                                      int64_t ldx, acc8_t<F8>* __restrict__ Yv, int64_t ldy,
                                                      int tilesT) {
  using acc_t = acc8_t<F8>;
  using out_t = std::conditional_t<F8, float, int32_t>;
  out_t* Y = reinterpret_cast<out_t*>(Yv);
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

  acc_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  auto mma = [&](const i32x4 (&a)[4], const uint32_t (&x)[4], const i32x8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = smfmac8<F8>(a[i], b[j], acc[i][j], x[i]);
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
      out_t* y = Y + int64_t(t) * ldy + r;
      if (vec_ok && r + 3 < R) {
        *reinterpret_cast<acc_t*>(y) = acc[i][j];
      } else {
        for (int e = 0; e < 4 && r + e < R; ++e) y[e] = acc[i][j][e];
      }
    }
  }
}

// The prefill kernel for INT8: 256 x 128 tiles, 4 waves as 2 x 2 (128 rows x
// 64 tokens each, 8 x 4 fragments), both operands staged in LDS by direct
// global->LDS loads through a 4-deep ring of 128-wide K steps.  At one byte
// per element a step's packed values (64 B per row) and activations (128 B
// per token) have the byte layout of a 64-wide step of the 16-bit kernel, so
// its XOR-swizzled slots serve here unchanged:
//   packed values  slot (row, quarter q) at row*4 + (q ^ ((row >> 1) & 3));
//   activations    slot (token, chunk c) at token*8 + (c ^ (token & 7)).
// Index bits (16 bytes per row and step) are staged the same way in blocks
// of four steps (64 bytes per row, two blocks in LDS): slot (row, step c of
// the block) at row*4 + (c ^ ((row >> 2) & 3)), so a fragment's 16 rows x 4
// lanes read distinct banks; a lane's index word is one 4-byte LDS read.
// (Per-lane 4-byte global loads of the words took more than the rest of the
// step together, and one 16-byte load per row and step used an eighth of each
// line it fetched.)  Fragments go through two register
// sets: step s+1 is read while step s multiplies.  Every step issues the same loads (past the last
// step the last one again, into a slot nothing reads any more), so each wait
// is one constant count.  Shapes: R % 256 == 0, T % 128 == 0, K % 128 == 0.
constexpr int kBR8L = 256, kBT8L = 128, kNS8 = 4;
constexpr int kStage8 = 16384;                    // one operand, one step
constexpr int kBlockI8 = kBR8L * 64;              // index bits, four steps
constexpr int kLds8 = kNS8 * 2 * kStage8 + 2 * kBlockI8;  // 160 KB
constexpr int kPer8 = 8;                          // direct loads per wave per step: 4 + 4

template <bool F8>
__global__ __launch_bounds__(256, 1) void spmm_i8_lds_kernel(const uint8_t* __restrict__ values,
                                                             const uint32_t* __restrict__ idx, int K,
                                                             int words, const uint8_t* __restrict__ act,
                                                             int64_t ldx, acc8_t<F8>* __restrict__ Y,
                                                             int64_t ldy, int tilesT) {
  extern __shared__ __align__(16) unsigned char smem8[];
  unsigned char* bbuf = smem8;                  // [kNS8][kStage8] activations
  unsigned char* abuf = smem8 + kNS8 * kStage8;  // [kNS8][kStage8] packed values
  unsigned char* ibuf = smem8 + 2 * kNS8 * kStage8;  // [2][kBlockI8] index blocks
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int wr = wave >> 1, wt = wave & 1;
  // Tile order: each XCD (workgroup p runs on XCD p % 8) takes a contiguous run
  // of the tile sequence, which goes through groups of up to four row tiles
  // sharing activation columns.
  int R0, T0;
  {
    const int grid = int(gridDim.x), p = int(blockIdx.x);
    const int q = (grid & 7) == 0 ? (p & 7) * (grid >> 3) + (p >> 3) : p;
    const int tilesR = grid / tilesT;
    const int gr = tilesR < 4 ? tilesR : 4;
    const int per_group = gr * tilesT;
    const int grp = q / per_group, rem = q - grp * per_group;
    const int rows_in = min(gr, tilesR - grp * gr);
    R0 = (grp * gr + rem % rows_in) * kBR8L;
    T0 = (rem / rows_in) * kBT8L;
  }
  const int64_t S = K >> 1;
  const int nsteps = K >> 7;

  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(act + int64_t(T0) * ldx), (short)0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(values + int64_t(R0) * S), (short)0, -1, 0x00020000);
  // per-lane byte offsets of the direct loads within a step (instruction j)
  uint32_t boff[4], aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int tok = slot >> 3, c = (slot & 7) ^ (tok & 7);
    boff[j] = uint32_t(tok) * uint32_t(ldx) + uint32_t(c) * 16u;
    const int row = slot >> 2, q = (slot & 3) ^ ((row >> 1) & 3);
    aoff[j] = uint32_t(row) * uint32_t(S) + uint32_t(q) * 16u;
  }
  // index blocks: instruction j of wave w fills slots [(w*4 + j)*64, +64),
  // slot (row, position p) holding step c = p ^ ((row >> 2) & 3) of the block
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(idx + int64_t(R0) * words), (short)0, -1, 0x00020000);
  uint32_t ioff[4];
  int istep[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int slot = (wave * 4 + j) * 64 + lane;
    const int row = slot >> 2;
    istep[j] = (slot & 3) ^ ((row >> 2) & 3);
    ioff[j] = uint32_t(row) * uint32_t(words) * 4u;
  }
  // block q into buffer ib; a step past the last rereads the last step, so
  // no load leaves the row
  auto issue_block = [&](int q, int ib) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int st = min(4 * q + istep[j], nsteps - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ri, (lds_byte*)(ibuf + ib * kBlockI8 + (wave * 4 + j) * 1024),
                                               16, int(ioff[j] + uint32_t(st) * 16u), 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  // A step's loads, fenced so that no load of another step moves in between
  // (the counted waits rely on whole steps completing in order).
  auto issue = [&](int src, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_byte*)(bbuf + SL * kStage8 + (wave * 4 + j) * 1024),
                                               16, int(boff[j]), int(src * 128), 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_byte*)(abuf + SL * kStage8 + (wave * 4 + j) * 1024),
                                               16, int(aoff[j]), int(src * 64), 0, 0);
    }
    asm volatile("" ::: "memory");
  };

  using acc_t = acc8_t<F8>;
  acc_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // fragments of step t (ring slot SL = t & 3, index block t / 4)
  auto read_frags = [&](int t, auto slot_c, i32x4 (&a)[8], i32x8 (&b)[4], uint32_t (&x)[8]) {
    constexpr int SL = decltype(slot_c)::value;
    const unsigned char* sb = bbuf + SL * kStage8;
    const unsigned char* sa = abuf + SL * kStage8;
    const unsigned char* si = ibuf + ((t >> 2) & 1) * kBlockI8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = wt * 64 + j * 16 + li;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(sb + (tok * 8 + (lq ^ (tok & 7))) * 16);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(sb + (tok * 8 + ((lq + 4) ^ (tok & 7))) * 16);
      b[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wr * 128 + i * 16 + li;
      a[i] = *reinterpret_cast<const i32x4*>(sa + (row * 4 + (lq ^ ((row >> 1) & 3))) * 16);
      x[i] = *reinterpret_cast<const uint32_t*>(si + (row * 4 + (SL ^ ((row >> 2) & 3))) * 16 + lq * 4);
    }
  };

  // Load j of a step: 0..3 activations, 4..7 packed values, of step src into
  // ring slot SL.
  auto issue_one = [&](int src, auto slot_c, int j) {
    constexpr int SL = decltype(slot_c)::value;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_byte*)(bbuf + SL * kStage8 + (wave * 4 + j) * 1024),
                                               16, int(boff[j]), int(src * 128), 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_byte*)(abuf + SL * kStage8 + (wave * 4 + j - 4) * 1024),
                                               16, int(aoff[j - 4]), int(src * 64), 0, 0);
  };

  // One step s: make step s+1 visible, refill step s's slot with step s+4,
  // read step s+1's fragments, multiply step s (fragments read one step
  // earlier).  The step runs as eight chunks, each: some of step s+1's
  // fragment reads, the 4 MFMAs of row fragment k of step s, and one load.
  // The token fragments and index words come first (the next step needs
  // them from its first chunk on), the row fragments after them, and the last
  // chunk reads nothing; scheduling barriers keep this order, so no MFMA
  // waits on a read issued just before it.
  auto step = [&](int s, auto slot_c, const i32x4 (&ca)[8], const i32x8 (&cb)[4], const uint32_t (&cx)[8],
                  i32x4 (&na)[8], i32x8 (&nb)[4], uint32_t (&nx)[8]) {
    constexpr int SL = decltype(slot_c)::value;
    constexpr int RS = (SL + 1) & 3;  // slot of step s+1
    wait_vmcnt<2 * kPer8>();  // step s+1 has landed (steps s+2, s+3 may remain)
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // this wave's reads of step s are done
    __builtin_amdgcn_s_barrier();  // step s+1 visible; every wave is done reading step s
    asm volatile("" ::: "memory");
    // at a block's first step every wave is done with the block before it:
    // its buffer takes the next block (first read three steps later)
    if (SL == 0 && s + 4 < nsteps) issue_block((s >> 2) + 1, ((s >> 2) + 1) & 1);
    const int src = min(s + 4, nsteps - 1);
    const unsigned char* sb = bbuf + RS * kStage8;
    const unsigned char* sa = abuf + RS * kStage8;
    const unsigned char* si = ibuf + (((s + 1) >> 2) & 1) * kBlockI8;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < 4) {
        const int tok = wt * 64 + k * 16 + li;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(sb + (tok * 8 + (lq ^ (tok & 7))) * 16);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(sb + (tok * 8 + ((lq + 4) ^ (tok & 7))) * 16);
        nb[k] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int i = 2 * k; i < 2 * k + 2; ++i) {
          const int row = wr * 128 + i * 16 + li;
          nx[i] = *reinterpret_cast<const uint32_t*>(si + (row * 4 + (RS ^ ((row >> 2) & 3))) * 16 + lq * 4);
        }
      } else {
#pragma unroll
        for (int i = 3 * (k - 4); i < 3 * (k - 4) + 3; ++i) {
          if (i < 8) {
            const int row = wr * 128 + i * 16 + li;
            na[i] = *reinterpret_cast<const i32x4*>(sa + (row * 4 + (lq ^ ((row >> 1) & 3))) * 16);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[k][j] = smfmac8<F8>(ca[k], cb[j], acc[k][j], cx[k]);
      issue_one(src, slot_c, k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using std::integral_constant;
  i32x4 a0[8], a1[8];
  i32x8 b0[4], b1[4];
  uint32_t x0[8], x1[8];
  issue_block(0, 0);
  issue(0, integral_constant<int, 0>{});
  issue(min(1, nsteps - 1), integral_constant<int, 1>{});
  issue(min(2, nsteps - 1), integral_constant<int, 2>{});
  wait_vmcnt<2 * kPer8>();  // index block 0 and step 0 have landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  issue(min(3, nsteps - 1), integral_constant<int, 3>{});
  read_frags(0, integral_constant<int, 0>{}, a0, b0, x0);
  int s = 0;
  for (; s + 4 <= nsteps; s += 4) {
    step(s, integral_constant<int, 0>{}, a0, b0, x0, a1, b1, x1);
    step(s + 1, integral_constant<int, 1>{}, a1, b1, x1, a0, b0, x0);
    step(s + 2, integral_constant<int, 2>{}, a0, b0, x0, a1, b1, x1);
    step(s + 3, integral_constant<int, 3>{}, a1, b1, x1, a0, b0, x0);
  }
  if (s < nsteps) step(s, integral_constant<int, 0>{}, a0, b0, x0, a1, b1, x1);
  if (s + 1 < nsteps) step(s + 1, integral_constant<int, 1>{}, a1, b1, x1, a0, b0, x0);
  if (s + 2 < nsteps) step(s + 2, integral_constant<int, 2>{}, a0, b0, x0, a1, b1, x1);
  wait_vmcnt<0>();  // no direct load still writing LDS when the workgroup ends

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = R0 + wr * 128 + i * 16 + 4 * lq;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = T0 + wt * 64 + j * 16 + li;
      Y[(int64_t(t) * ldy + r) >> 2] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_prune_pack_i8(const uint8_t* W, int64_t R, int64_t K, int64_t ldw, uint8_t* values,
                                uint32_t* idx, int64_t idx_row_words, bool f8, hipStream_t s) {
  const int64_t chunks = R * (K >> 4);
  if (chunks <= 0) return hipSuccess;
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (f8)
    hipLaunchKernelGGL(prune_pack_i8_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, s, W, R, K, ldw,
                       values, idx, idx_row_words);
  else
    hipLaunchKernelGGL(prune_pack_i8_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, s, W, R, K, ldw,
                       values, idx, idx_row_words);
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

template <bool F8>
hipError_t launch_spmm_b8(const SpmmArgs& a, hipStream_t s) {
  // whole tiles only, 32-bit per-lane offsets, 16-byte output rows
  const bool lds = a.R % kBR8L == 0 && a.T % kBT8L == 0 && a.K % 128 == 0 && (a.ldy & 3) == 0 &&
                   int64_t(kBT8L) * a.ldx < 0x7FFFFFFF && int64_t(kBR8L) * (a.K >> 1) < 0x7FFFFFFF &&
                   int64_t(kBR8L) * a.idx_row_words * 4 < 0x7FFFFFFF &&
                   a.variant != NM_VARIANT_GENERIC && device_max_lds() >= kLds8;
  if (lds) {
    const int64_t tiles = (a.R / kBR8L) * (a.T / kBT8L);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    auto kfn = spmm_i8_lds_kernel<F8>;
    const void* kern = reinterpret_cast<const void*>(kfn);
    if (hipError_t e = ensure_lds_limit(kern, kLds8); e != hipSuccess) return e;
    hipLaunchKernelGGL(kfn, dim3(unsigned(tiles)), dim3(256), kLds8, s,
                       reinterpret_cast<const uint8_t*>(a.values), a.idx, int(a.K), int(a.idx_row_words),
                       reinterpret_cast<const uint8_t*>(a.act), a.ldx, static_cast<acc8_t<F8>*>(a.Y), a.ldy,
                       int(a.T / kBT8L));
    return hipGetLastError();
  }
  const int64_t tilesR = (a.R + kBR8 - 1) / kBR8;
  const int64_t tilesT = (a.T + kBT8 - 1) / kBT8;
  if (tilesR * tilesT > 0x7FFFFFFF || a.R > 0x7FFFFFFF || a.T > 0x7FFFFFFF || a.K > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(spmm_i8_kernel<F8>, dim3(unsigned(tilesR * tilesT)), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(a.values), a.idx, int(a.R), int(a.K),
                     int(a.idx_row_words), reinterpret_cast<const uint8_t*>(a.act), int(a.T), a.ldx,
                     static_cast<acc8_t<F8>*>(a.Y), a.ldy, int(tilesT));
  return hipGetLastError();
}

hipError_t launch_spmm_i8(const SpmmArgs& a, hipStream_t s) {
  return a.dtype == NM_FP8 ? launch_spmm_b8<true>(a, s) : launch_spmm_b8<false>(a, s);
}

}  // namespace nm
