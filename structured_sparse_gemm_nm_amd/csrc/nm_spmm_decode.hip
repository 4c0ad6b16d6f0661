// Sparse GEMM for few tokens (T <= 16, decode): Y^T[t, r] = sum_k W_nm[r, k] X'[t, k]
// with X' = act, or act read through the index map perm (SHUFFLESPARSE
// technical summary, inference-efficiency item of section 2: the permutation is
// applied on the input reads).
//
// With T <= 16 the product is bound by streaming the packed weight from HBM;
// the MFMA work is small (tokens are padded to the instruction's 16 columns;
// lanes of absent tokens load nothing and hold zeros).  The kernel is built to
// keep as many bytes in flight as possible:
//   * a workgroup of 8 waves owns RB x 16 rows; the K steps are split evenly
//     over the 8 waves;
//   * each wave issues every load of its share (packed values + index bits of
//     RB fragments and the activation fragment, per 64-wide K step) before its
//     first MFMA;
//   * the 8 partial tiles are summed in LDS in a fixed order (deterministic).
// Operand layouts and the 1:4 / 1:8 widening are those of nm_spmm.hip.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

constexpr int pat_n(int P) { return P == 0 ? 2 : 1; }
constexpr int pat_m(int P) { return P == 2 ? 8 : 4; }

struct AFrag {
  uint32_t v[4];
  uint32_t ib;
};

// Lane (row, lq) share of step s.  Rows past R and quarters past K load nothing.
template <int P>
__device__ inline void load_afrag(AFrag& f, const uint16_t* __restrict__ values,
                                  const uint32_t* __restrict__ idx, int64_t S, int64_t words, int row,
                                  int R, int K, int s, int lq) {
  f.v[0] = f.v[1] = f.v[2] = f.v[3] = 0u;
  f.ib = 0u;
  if (row >= R || s * 64 + lq * 16 >= K) return;
  const uint16_t* vrow = values + int64_t(row) * S;
  const unsigned char* irow = reinterpret_cast<const unsigned char*>(idx + int64_t(row) * words);
  if constexpr (P == 0) {
    const uint4 t = *reinterpret_cast<const uint4*>(vrow + s * 32 + lq * 8);
    f.v[0] = t.x; f.v[1] = t.y; f.v[2] = t.z; f.v[3] = t.w;
    f.ib = *reinterpret_cast<const uint16_t*>(irow + s * 8 + lq * 2);
  } else if constexpr (P == 1) {
    const uint2 t = *reinterpret_cast<const uint2*>(vrow + s * 16 + lq * 4);
    f.v[0] = t.x; f.v[1] = t.y;
    f.ib = irow[s * 4 + lq];
  } else {  // 1:8: 2 values (4 B), 6 index bits at bit 24 s + 6 lq of the row
    f.v[0] = *reinterpret_cast<const uint32_t*>(vrow + s * 8 + lq * 2);
    f.v[3] = 0u;
    // the aligned word holding the first bit and the next one (clamped to the
    // row's last word, whose bits then suffice): two loads from every lane,
    // kept as loaded (widen extracts the bits, so nothing here waits for them)
    const uint32_t* wrow = idx + int64_t(row) * words;
    const int bit = 24 * s + 6 * lq;
    const int w0 = bit >> 5;
    const int w1 = min(w0 + 1, int(words) - 1);
    f.v[1] = wrow[w0];
    f.v[2] = wrow[w1];
    f.ib = uint32_t(bit & 31);
  }
}

template <int P>
__device__ inline void widen(const AFrag& f, u32x4& a, uint32_t& idx16) {
  if constexpr (P == 0) {
    a[0] = f.v[0]; a[1] = f.v[1]; a[2] = f.v[2]; a[3] = f.v[3];
    idx16 = f.ib & 0xFFFFu;
  } else if constexpr (P == 1) {
    a[0] = f.v[0] & 0xFFFFu; a[1] = f.v[0] >> 16; a[2] = f.v[1] & 0xFFFFu; a[3] = f.v[1] >> 16;
    const uint32_t ib = f.ib;
    const uint32_t t = (ib & 0x3u) | ((ib & 0xCu) << 2) | ((ib & 0x30u) << 4) | ((ib & 0xC0u) << 6);
    idx16 = t | (t << 2);
  } else {
    const uint32_t v0 = f.v[0] & 0xFFFFu, v1 = f.v[0] >> 16;
    const uint32_t ib = uint32_t((uint64_t(f.v[1]) | (uint64_t(f.v[2]) << 32)) >> f.ib);
    const uint32_t p0 = ib & 7u, p1 = (ib >> 3) & 7u;
    const bool h0 = p0 >= 4, h1 = p1 >= 4;
    a[0] = h0 ? 0u : v0; a[1] = h0 ? v0 : 0u;
    a[2] = h1 ? 0u : v1; a[3] = h1 ? v1 : 0u;
    const uint32_t f0 = (p0 & 3u) * 5u, f1 = (p1 & 3u) * 5u;
    idx16 = (h0 ? (f0 << 4) : f0) | (h1 ? (f1 << 12) : (f1 << 8));
  }
}

// Activation fragment of step s for lane (token t, lq): K positions
// 8lq..8lq+7 and 32+8lq..32+8lq+7 of the step, read directly or through perm.
template <bool PERM>
__device__ inline void load_bfrag(u32x8& b, const uint16_t* __restrict__ act, int64_t ldx,
                                  const int32_t* __restrict__ perm, int t, int T, int K, int s,
                                  int lq) {
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = 0u;
  if (t >= T) return;
  const uint16_t* arow = act + int64_t(t) * ldx;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = s * 64 + h * 32 + lq * 8;
    if (k >= K) continue;
    if constexpr (PERM) {
      // entries outside [0, K) (a broken precondition) are clamped into the
      // row: a wrong value, never a wrong address
      const uint32_t kmax = uint32_t(K - 1);
      const int4 p0 = *reinterpret_cast<const int4*>(perm + k);
      const int4 p1 = *reinterpret_cast<const int4*>(perm + k + 4);
      const uint32_t q[8] = {umin(uint32_t(p0.x), kmax), umin(uint32_t(p0.y), kmax),
                             umin(uint32_t(p0.z), kmax), umin(uint32_t(p0.w), kmax),
                             umin(uint32_t(p1.x), kmax), umin(uint32_t(p1.y), kmax),
                             umin(uint32_t(p1.z), kmax), umin(uint32_t(p1.w), kmax)};
      b[4 * h + 0] = uint32_t(arow[q[0]]) | (uint32_t(arow[q[1]]) << 16);
      b[4 * h + 1] = uint32_t(arow[q[2]]) | (uint32_t(arow[q[3]]) << 16);
      b[4 * h + 2] = uint32_t(arow[q[4]]) | (uint32_t(arow[q[5]]) << 16);
      b[4 * h + 3] = uint32_t(arow[q[6]]) | (uint32_t(arow[q[7]]) << 16);
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(arow + k);
      b[4 * h + 0] = v.x; b[4 * h + 1] = v.y; b[4 * h + 2] = v.z; b[4 * h + 3] = v.w;
    }
  }
}

constexpr int kWaves = 8;

// Workgroup barrier that waits only for this wave's LDS operations.
// __syncthreads() also waits for every outstanding global load (vmcnt(0)),
// which would drain the prefetched blocks.
__device__ inline void barrier_lds() {
  // vmcnt left at its maximum (63), expcnt 7, lgkmcnt 0 (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// SPW: K steps per wave (compile time, so the loads sit in registers).
template <int P, int DT, int OUT, bool PERM, int RB, int SPW>
__global__ __launch_bounds__(kWaves * 64) void spmm_decode_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    int64_t words, const uint16_t* __restrict__ act, int T, int64_t ldx,
    const int32_t* __restrict__ perm, void* __restrict__ Y, int64_t ldy) {
  __shared__ f32x4 part[kWaves][RB][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int R0 = blockIdx.x * (RB * 16);
  const int64_t S = int64_t(K) / pat_m(P) * pat_n(P);
  const int s0 = wave * SPW;  // first K step of this wave

  AFrag af[SPW][RB];
  u32x8 bf[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
      load_afrag<P>(af[u][i], values, idx, S, words, R0 + i * 16 + li, R, K, s0 + u, lq);
    load_bfrag<PERM>(bf[u], act, ldx, perm, li, T, K, s0 + u, lq);
  }
  f32x4 acc[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      u32x4 a;
      uint32_t ix;
      widen<P>(af[u][i], a, ix);
      acc[i] = smfmac<DT>(a, bf[u], acc[i], ix);
    }
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) part[wave][i][lane] = acc[i];
  __syncthreads();
  // wave i < RB sums the 8 partials of fragment i in wave order
  if (wave < RB) {
    f32x4 sum = part[0][wave][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += part[w][wave][lane];
    const int t = li;
    const int r = R0 + wave * 16 + lq * 4;
    if (t < T && r < R) {
      const bool vec_ok = (ldy & 3) == 0 && r + 3 < R;
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok) *reinterpret_cast<f32x4*>(y) = sum;
        else for (int e = 0; e < 4 && r + e < R; ++e) y[e] = sum[e];
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint16_t h[4] = {to_half_bits<DT>(sum[0]), to_half_bits<DT>(sum[1]),
                               to_half_bits<DT>(sum[2]), to_half_bits<DT>(sum[3])};
        if (vec_ok) {
          *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                                    uint32_t(h[2]) | (uint32_t(h[3]) << 16));
        } else {
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = h[e];
        }
      }
    }
  }
}

// 2:4 variant of the same kernel whose packed operand goes through LDS: the
// wave's 16 rows x SPW steps are fetched with direct global->LDS loads that
// read each row's SPW*64 contiguous bytes (whole lines; a direct load
// deposits lane l's 16 bytes at slot base + l, so the lane addresses pick the
// layout), instead of 16 rows x 64 bytes per instruction.  Slot (row, chunk c)
// sits at row*CPR + (c ^ (row & 15)) (CPR 16-byte chunks per row) so a
// fragment read by 8 consecutive rows hits distinct banks.  Index bits take
// one more load per wave: 16 rows x SPW*8 bytes.
template <int DT, int OUT, bool PERM, int SPW>
__global__ __launch_bounds__(kWaves * 64) void spmm_decode_lds_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, const int32_t* __restrict__ perm,
    void* __restrict__ Y, int64_t ldy) {
  constexpr int CPR = SPW * 4;                 // 16-byte value chunks per row
  constexpr int VBYTES = 16 * CPR * 16;        // values region per wave
  constexpr int IBYTES = 16 * SPW * 8;         // index region per wave
  constexpr int IPR = SPW * 8 / 16;            // index chunks per row (SPW >= 2)
  __shared__ __align__(16) unsigned char stage[kWaves][VBYTES + IBYTES];
  __shared__ f32x4 part[kWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lq = lane >> 4;
  const int R0 = blockIdx.x * 16;
  const int S = K >> 1;
  const int irow_bytes = K >> 3;
  const int s0 = wave * SPW;
  const int nsteps = (K + 63) >> 6;
  unsigned char* vst = stage[wave];
  unsigned char* ist = stage[wave] + VBYTES;

  // values: instruction j covers slots [j*64, j*64 + 64) = 64/CPR rows
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int slot = j * 64 + lane;
    const int row = slot / CPR;
    const int c = (slot % CPR) ^ (row & 15 & (CPR - 1));
    const int r = min(R0 + row, R - 1);
    // chunk c of the wave's slice; past K reread the row's first chunk
    int64_t off = int64_t(s0) * 32 + c * 8;
    if (s0 * 64 + c * 16 >= K) off = 0;
    __builtin_amdgcn_global_load_lds(values + int64_t(r) * S + off,
                                     (lds_byte*)(vst + j * 1024), 16, 0, 0);
  }
  // index bits: 16 rows x IPR chunks (one instruction; lanes past 16*IPR idle)
  if (lane < 16 * IPR) {
    const int row = lane / IPR;
    const int c = lane % IPR;
    const int r = min(R0 + row, R - 1);
    int64_t off = int64_t(s0) * 8 + c * 16;
    if (s0 * 64 + c * 128 >= K) off = 0;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(idx) + int64_t(r) * irow_bytes + off,
                                     (lds_byte*)ist, 16, 0, 0);
  }
  u32x8 bf[SPW];
#pragma unroll
  for (int u = 0; u < SPW; ++u) load_bfrag<PERM>(bf[u], act, ldx, perm, li, T, K, s0 + u, lq);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int row = li;
#pragma unroll
  for (int u = 0; u < SPW; ++u) {
    const int s = s0 + u;
    u32x4 a = *reinterpret_cast<const u32x4*>(vst + (row * CPR + ((u * 4 + lq) ^ (row & 15 & (CPR - 1)))) * 16);
    uint32_t ix = *reinterpret_cast<const uint16_t*>(ist + row * (SPW * 8) + u * 8 + lq * 2);
    if (s >= nsteps || s * 64 + lq * 16 >= K) {
      a = u32x4{0u, 0u, 0u, 0u};
      ix = 0u;
    }
    acc = smfmac<DT>(a, bf[u], acc, ix);
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += part[w][lane];
    const int t = li;
    const int r = R0 + lq * 4;
    if (t < T && r < R) {
      const bool vec_ok = (ldy & 3) == 0 && r + 3 < R;
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok) *reinterpret_cast<f32x4*>(y) = sum;
        else for (int e = 0; e < 4 && r + e < R; ++e) y[e] = sum[e];
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint16_t h[4] = {to_half_bits<DT>(sum[0]), to_half_bits<DT>(sum[1]),
                               to_half_bits<DT>(sum[2]), to_half_bits<DT>(sum[3])};
        if (vec_ok) {
          *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                                    uint32_t(h[2]) | (uint32_t(h[3]) << 16));
        } else {
          for (int e = 0; e < 4 && r + e < R; ++e) y[e] = h[e];
        }
      }
    }
  }
}

// Persistent 2:4 variant: one workgroup per CU owns an equal, contiguous
// range of rows (ceil(R / grid) of them, NBLK blocks of 16; a range with fewer
// rows, at the end of R, rereads its last row and stores nothing for it), so
// every CU streams the same number of bytes.  With the block count fixed at
// compile time every load is issued unconditionally and every wait count is
// a constant.  Each wave keeps its K slice of the
// activations in registers and double buffers its wave-private LDS staging
// across blocks: block b+2's direct loads are issued as soon as block b's
// fragments are in registers.  No wave waits for another until every block
// is multiplied: each wave keeps one accumulator tile per block, and the
// partial tiles of all blocks are summed across waves once, at the end (in
// LDS reused from the staging area), in a fixed wave order.
template <int DT, int OUT, bool PERM, int SPW, int NBLK>
__global__ __launch_bounds__(kWaves * 64, 1) void spmm_decode_stream_kernel(
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ idx, int R, int K,
    const uint16_t* __restrict__ act, int T, int64_t ldx, const int32_t* __restrict__ perm,
    void* __restrict__ Y, int64_t ldy, int rows_per_wg) {
  constexpr int CPR = SPW * 4;
  constexpr int VBYTES = 16 * CPR * 16;
  constexpr int IBYTES = 16 * SPW * 8;
  constexpr int IPR = SPW * 8 / 16;
  constexpr int PER_BLOCK = SPW + 1;           // direct loads per wave per block
  static_assert(16 * IPR == 64, "the index load must use every lane");
  static_assert(NBLK * kWaves * 64 * 16 <= 2 * kWaves * (VBYTES + IBYTES), "partials fit the staging");
  // Staging [2][kWaves][VBYTES + IBYTES] in dynamic LDS; after the last block
  // it holds the partial tiles [kWaves][NBLK][64].  Explicit counted waits
  // order the direct loads and the fragment reads.
  extern __shared__ __align__(16) unsigned char dyn[];
  auto stage_at = [&](int buf, int w) { return dyn + (buf * kWaves + w) * (VBYTES + IBYTES); };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int li = lane & 15, lq = lane >> 4;
  const int row_begin = blockIdx.x * rows_per_wg;
  const int row_end = min(R, row_begin + rows_per_wg);
  if (row_begin >= row_end) return;  // uniform over the workgroup
  constexpr int nblk = NBLK;
  const int S = K >> 1;
  const int irow_bytes = K >> 3;
  const int s0 = wave * SPW;
  const int nsteps = K >> 6;

  auto issue_block = [&](int blk, int buf) {
    const int R0 = row_begin + blk * 16;
    unsigned char* vst = stage_at(buf, wave);
    unsigned char* ist = vst + VBYTES;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int slot = j * 64 + lane;
      const int row = slot / CPR;
      const int c = (slot % CPR) ^ (row & 15 & (CPR - 1));
      int64_t off = int64_t(s0) * 32 + c * 8;
      if (s0 * 64 + c * 16 >= K) off = 0;
      // Every lane issues its load so the per-block load count is fixed (the
      // counted waits below rely on it); rows past the range reread the
      // range's last row and their outputs are not stored.
      const int r = min(R0 + row, row_end - 1);
      __builtin_amdgcn_global_load_lds(values + int64_t(r) * S + off, (lds_byte*)(vst + j * 1024),
                                       16, 0, 0);
    }
    {
      const int row = lane / IPR;
      const int c = lane % IPR;
      int64_t off = int64_t(s0) * 8 + c * 16;
      if (s0 * 64 + c * 128 >= K) off = 0;
      const int r = min(R0 + row, row_end - 1);
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const unsigned char*>(idx) + int64_t(r) * irow_bytes + off,
          (lds_byte*)ist, 16, 0, 0);
    }
  };

  f32x4 acc[NBLK];
#pragma unroll
  for (int b = 0; b < NBLK; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x8 bf[SPW];
  constexpr int kOne = PER_BLOCK;
  constexpr int kTwo = 2 * PER_BLOCK;

  // Fragments of block b from its staging slot into registers; once they are
  // there, the slot takes block b+2.
  auto take_block = [&](int b, u32x4 (&a)[SPW], uint32_t (&ix)[SPW]) {
    const unsigned char* vst = stage_at(b & 1, wave);
    const unsigned char* ist = vst + VBYTES;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      a[u] = *reinterpret_cast<const u32x4*>(vst + (li * CPR + ((u * 4 + lq) ^ (li & 15 & (CPR - 1)))) * 16);
      ix[u] = *reinterpret_cast<const uint16_t*>(ist + li * (SPW * 8) + u * 8 + lq * 2);
    }
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    if (b + 2 < nblk) issue_block(b + 2, b & 1);
  };
  // steps past K (whole steps: K % 128 == 0 here) are skipped by the wave
  auto multiply = [&](int b, const u32x4 (&a)[SPW], const uint32_t (&ix)[SPW]) {
#pragma unroll
    for (int u = 0; u < SPW; ++u)
      if (s0 + u < nsteps) acc[b] = smfmac<DT>(a[u], bf[u], acc[b], ix[u]);
  };
  // block b has landed once at most block b+1's loads remain
  auto wait_block = [&](int b) {
    if (b + 1 < nblk) __builtin_amdgcn_s_waitcnt((kOne & 0xF) | (0x7 << 4) | (0xF << 8) | ((kOne >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
  };

  if constexpr (!PERM) {
    // Blocks 0 and 1 go out first (with a single block, block 1 rereads it
    // into the unused buffer, so the count is fixed), then this wave's K slice
    // of the activations: exactly 2*SPW loads, every lane issuing one (lanes
    // of absent tokens reread token T-1 into output columns that are not
    // stored; steps past K reread the row's first step and are skipped).
    // Nothing but the MFMAs reads these registers.  The activations
    // queue behind the weight streams, and loads complete in order, so block 0
    // is waited for past them: its slot is refilled before they arrive, and
    // its MFMAs wait for block 1, by which time they have.
    issue_block(0, 0);
    issue_block(nblk > 1 ? 1 : 0, 1);
    const int t = min(li, T - 1);
    const uint16_t* arow = act + int64_t(t) * ldx;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = (s0 + u < nsteps ? (s0 + u) * 64 : 0) + h * 32 + lq * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(arow + k);
        bf[u][4 * h + 0] = v.x;
        bf[u][4 * h + 1] = v.y;
        bf[u][4 * h + 2] = v.z;
        bf[u][4 * h + 3] = v.w;
      }
    }
    constexpr int kFirst = PER_BLOCK + 2 * SPW;
    __builtin_amdgcn_s_waitcnt((kFirst & 0xF) | (0x7 << 4) | (0xF << 8) | ((kFirst >> 4) << 14));
    asm volatile("" ::: "memory");
    u32x4 a0[SPW];
    uint32_t ix0[SPW];
    take_block(0, a0, ix0);
    if constexpr (nblk == 1) {
      __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));  // the activations
      asm volatile("" ::: "memory");
      multiply(0, a0, ix0);
    }
#pragma unroll
    for (int b = 1; b < NBLK; ++b) {
      wait_block(b);
      if (b == 1) multiply(0, a0, ix0);  // the activations have landed
      u32x4 a[SPW];
      uint32_t ix[SPW];
      take_block(b, a, ix);
      multiply(b, a, ix);
    }
  } else {
    // Through the index map the activation loads depend on loaded indices,
    // so they go first and are waited for before the blocks' loads are counted.
#pragma unroll
    for (int u = 0; u < SPW; ++u) load_bfrag<PERM>(bf[u], act, ldx, perm, li, T, K, s0 + u, lq);
    issue_block(0, 0);
    issue_block(nblk > 1 ? 1 : 0, 1);
    __builtin_amdgcn_s_waitcnt((kTwo & 0xF) | (0x7 << 4) | (0xF << 8) | ((kTwo >> 4) << 14));
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      wait_block(b);
      u32x4 a[SPW];
      uint32_t ix[SPW];
      take_block(b, a, ix);
      multiply(b, a, ix);
    }
  }

  // Partial tiles of every block, summed across waves in wave order.  The
  // last block's wait left no direct load in flight; the barrier makes every
  // wave's staging reads complete before the area is rewritten.
  f32x4 (*part)[NBLK][64] = reinterpret_cast<f32x4 (*)[NBLK][64]>(dyn);
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NBLK; ++b) part[wave][b][lane] = acc[b];
  __syncthreads();
  for (int b = wave; b < nblk; b += kWaves) {
    f32x4 sum = part[0][b][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += part[w][b][lane];
    const int t = li;
    const int r = row_begin + b * 16 + lq * 4;
    if (t < T && r < row_end) {
      const bool vec_ok = (ldy & 3) == 0 && r + 3 < row_end;
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(Y) + int64_t(t) * ldy + r;
        if (vec_ok) *reinterpret_cast<f32x4*>(y) = sum;
        else for (int e = 0; e < 4 && r + e < row_end; ++e) y[e] = sum[e];
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + int64_t(t) * ldy + r;
        const uint16_t h[4] = {to_half_bits<DT>(sum[0]), to_half_bits<DT>(sum[1]),
                               to_half_bits<DT>(sum[2]), to_half_bits<DT>(sum[3])};
        if (vec_ok) {
          *reinterpret_cast<uint2*>(y) = make_uint2(uint32_t(h[0]) | (uint32_t(h[1]) << 16),
                                                    uint32_t(h[2]) | (uint32_t(h[3]) << 16));
        } else {
          for (int e = 0; e < 4 && r + e < row_end; ++e) y[e] = h[e];
        }
      }
    }
  }
}

template <int DT, int OUT, bool PERM, int SPW, int NBLK>
hipError_t launch_dec_stream_n(const SpmmArgs& a, hipStream_t s, int grid, int rows_per_wg) {
  constexpr int lds = 2 * kWaves * (16 * SPW * 4 * 16 + 16 * SPW * 8);
  auto kern = spmm_decode_stream_kernel<DT, OUT, PERM, SPW, NBLK>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kWaves * 64), lds, s, a.values, a.idx, int(a.R),
                     int(a.K), a.act, int(a.T), a.ldx, a.perm, a.Y, a.ldy, rows_per_wg);
  return hipGetLastError();
}

// One workgroup per CU while that keeps a workgroup's rows within 8 blocks of
// 16; more rows than that take more workgroups.
template <int DT, int OUT, bool PERM, int SPW>
hipError_t launch_dec_stream(const SpmmArgs& a, hipStream_t s) {
  const int cus = device_cu_count();
  const int64_t blocks16 = (a.R + 15) / 16;
  int64_t grid = blocks16 < cus ? blocks16 : cus;
  if ((blocks16 + grid - 1) / grid > 8) grid = (blocks16 + 7) / 8;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  // rows per workgroup: the even split (a range's last block may be partial)
  const int64_t even = (a.R + grid - 1) / grid;
  const int nblk = int((even + 15) / 16);
  const int rows_per_wg = int(even);
  switch (nblk) {
    case 1: return launch_dec_stream_n<DT, OUT, PERM, SPW, 1>(a, s, int(grid), rows_per_wg);
    case 2: return launch_dec_stream_n<DT, OUT, PERM, SPW, 2>(a, s, int(grid), rows_per_wg);
    case 3: return launch_dec_stream_n<DT, OUT, PERM, SPW, 3>(a, s, int(grid), rows_per_wg);
    case 4: return launch_dec_stream_n<DT, OUT, PERM, SPW, 4>(a, s, int(grid), rows_per_wg);
    case 5: return launch_dec_stream_n<DT, OUT, PERM, SPW, 5>(a, s, int(grid), rows_per_wg);
    case 6: return launch_dec_stream_n<DT, OUT, PERM, SPW, 6>(a, s, int(grid), rows_per_wg);
    case 7: return launch_dec_stream_n<DT, OUT, PERM, SPW, 7>(a, s, int(grid), rows_per_wg);
    default: return launch_dec_stream_n<DT, OUT, PERM, SPW, 8>(a, s, int(grid), rows_per_wg);
  }
}

template <int DT, int OUT, bool PERM, int SPW>
hipError_t launch_dec_lds(const SpmmArgs& a, hipStream_t s) {
  const int64_t blocks = (a.R + 15) / 16;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((spmm_decode_lds_kernel<DT, OUT, PERM, SPW>), dim3(unsigned(blocks)),
                     dim3(kWaves * 64), 0, s, a.values, a.idx, int(a.R), int(a.K), a.act, int(a.T),
                     a.ldx, a.perm, a.Y, a.ldy);
  return hipGetLastError();
}

template <int P, int DT, int OUT, bool PERM, int RB, int SPW>
hipError_t launch_dec(const SpmmArgs& a, hipStream_t s) {
  const int64_t blocks = (a.R + RB * 16 - 1) / (RB * 16);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((spmm_decode_kernel<P, DT, OUT, PERM, RB, SPW>), dim3(unsigned(blocks)),
                     dim3(kWaves * 64), 0, s, a.values, a.idx, int(a.R), int(a.K), a.idx_row_words,
                     a.act, int(a.T), a.ldx, a.perm, a.Y, a.ldy);
  return hipGetLastError();
}

// K steps per wave: the smallest instantiated SPW with 8 * SPW * 64 >= K.
template <int P, int DT, int OUT, bool PERM, int RB>
hipError_t pick_spw(const SpmmArgs& a, hipStream_t s) {
  const int64_t steps = (a.K + 63) / 64;
  if (steps <= 8 * 2) return launch_dec<P, DT, OUT, PERM, RB, 2>(a, s);
  if (steps <= 8 * 4) return launch_dec<P, DT, OUT, PERM, RB, 4>(a, s);
  if (steps <= 8 * 8) return launch_dec<P, DT, OUT, PERM, RB, 8>(a, s);
  return hipErrorInvalidValue;  // caller checks decode_applies
}

template <int P, int DT, int OUT, bool PERM>
hipError_t pick_rb(const SpmmArgs& a, hipStream_t s) {
  if constexpr (P == 0) {
    const int64_t steps = (a.K + 63) / 64;
    if (a.K % 128 == 0) {
      if (steps <= 8 * 2) return launch_dec_lds<DT, OUT, PERM, 2>(a, s);
      if (steps <= 8 * 4) return launch_dec_lds<DT, OUT, PERM, 4>(a, s);
      if (a.R >= 16 * 256) return launch_dec_stream<DT, OUT, PERM, 8>(a, s);
      return launch_dec_lds<DT, OUT, PERM, 8>(a, s);
    }
  }
  // Two row blocks per workgroup halve the activation re-reads when enough
  // workgroups remain to cover the chip.
  if (a.T > 4 && a.R >= 2 * 16 * 256) return pick_spw<P, DT, OUT, PERM, 2>(a, s);
  return pick_spw<P, DT, OUT, PERM, 1>(a, s);
}

template <int P, int DT>
hipError_t pick_out(const SpmmArgs& a, hipStream_t s) {
  const bool perm = a.perm != nullptr;
  if (a.out_dtype == NM_F32)
    return perm ? pick_rb<P, DT, NM_F32, true>(a, s) : pick_rb<P, DT, NM_F32, false>(a, s);
  return perm ? pick_rb<P, DT, DT, true>(a, s) : pick_rb<P, DT, DT, false>(a, s);
}

template <int P>
hipError_t pick_dt(const SpmmArgs& a, hipStream_t s) {
  return a.dtype == NM_F16 ? pick_out<P, NM_F16>(a, s) : pick_out<P, NM_BF16>(a, s);
}

}  // namespace

bool spmm_decode_applies(const SpmmArgs& a) {
  return a.T <= 16 && a.K <= 8 * 8 * 64;
}

hipError_t launch_spmm_decode(const SpmmArgs& a, hipStream_t s) {
  if (a.n == 2 && a.m == 4) return pick_dt<0>(a, s);
  if (a.n == 1 && a.m == 4) return pick_dt<1>(a, s);
  if (a.n == 1 && a.m == 8) return pick_dt<2>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace nm
