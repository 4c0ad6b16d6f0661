// Hybrid dense / 2:4 weight tiles on gfx950.
//
// Source: thelatestinai.com "Structured Sparsity" topic cards, the PATCH
// abstract: the weight matrix is cut into tiles, each kept dense or made 2:4
// sparse, which puts the fraction of zeros anywhere from 0 to 50%.  Tiles are
// tile_rows x tile_cols blocks (both multiples of 64 here); a row stores its
// tiles in column order, a dense tile as its tile_cols values, a 2:4 tile as
// its tile_cols/2 survivors plus tile_cols/8 index bytes (2 bits per
// survivor, LSB first), and the layout tables give each tile-row's row lengths
// and starting offsets (nmsparse.h, nm_hybrid_layout).
//
// Pack: one thread per 16-byte chunk (eight weights) of a row: a dense tile's
// chunk is copied, a 2:4 tile's chunk gives its four survivors and its index
// byte with the selection nm_compress uses (same largest-magnitude rule).
//
// Product: the register-pipelined layout of the N:M kernel (nm_spmm_pipe.hip):
// a workgroup owns 256 x 64 (or 128 x 64) of Y^T, each wave 64 (32) rows and
// all tokens; activations go through an LDS ring of direct global->LDS loads,
// each wave's weight fragments straight from global memory into registers
// several K steps ahead.  A 64-wide K step of a dense tile is two
// v_mfma_f32_16x16x32 per fragment pair, of a 2:4 tile one
// v_smfmac_f32_16x16x64: the activation operand the sparse instruction takes
// (K 8q..8q+7 and 32+8q..32+8q+7 of token i in lane 16q + i) is the two dense
// instructions' operands side by side, so both read the same LDS fragments.
// Tile-rows are multiples of 64 rows, so a wave's rows share one flag per
// step and the choice is one uniform branch per step.  Every fragment issues
// two loads per step either way (dense: two 16-byte runs of the row; 2:4: 16
// bytes of survivors and the 16-byte index block holding the lane's 16 index
// bits), and without a branch: the second load's buffer and offset are
// selected, so the counted waits hold on either kind of tile.  Weight reads go through buffer descriptors bounded by
// the arrays' sizes: offsets from a wrong layout table read zeros instead of
// memory outside the arrays, and the pack's stores are bounded the same way.
#include "nm_device.h"
#include "nm_internal.h"
#include "nm_select.h"

#include <type_traits>
#include <utility>

namespace nm {
namespace {

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>): stage
// indices stay compile-time constants, so per-stage registers never need an
// indexed (memory) array.
template <typename F, int... I>
__device__ inline void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

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
  if (i0 < 0) {  // dense tile: the chunk as it is
    __builtin_amdgcn_raw_buffer_store_b128(w, rv, bounded((v0 + rr * Lv + kin) * 2, values_bytes), 0, 0);
  } else {       // 2:4 tile: four survivors and their index byte
    const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
    uint32_t kept[2];
    uint32_t bits = 0;
    select_chunk<2, 4>(ww, kept, bits);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{kept[0], kept[1]}, rv,
                                          bounded((v0 + rr * Lv + kin / 2) * 2, values_bytes), 0, 0);
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx, idx_bytes);
    __builtin_amdgcn_raw_buffer_store_b8(uint8_t(bits), ri, bounded(i0 + rr * Li + kin / 8, idx_bytes), 0, 0);
  }
}

template <int DT>
__device__ inline f32x4 mfma_dense(const u32x4& a, const u32x4& b, const f32x4& c) {
  if constexpr (DT == NM_F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b),
                                                  c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c,
                                                   0, 0, 0);
  }
}

// One lane's weight operand of one 16-row fragment for one K step: dense,
// the row's K 8q..8q+7 (lo) and 32+8q..32+8q+7 (hi); 2:4, the 8 survivors
// (lo) and the aligned 16 index bytes holding the lane's two (hi).
struct HFrag {
  u32x4 lo, hi;
};

constexpr int kMaxFlagWords = 256;  // tile-columns per row up to 32 * 256

template <int DT, int OUT, int BR, int BT, int NS>
__global__ __launch_bounds__(256) void hybrid_gemm_kernel(
    const uint16_t* __restrict__ values, uint32_t values_bytes, const uint8_t* __restrict__ idx,
    uint32_t idx_bytes, const int64_t* __restrict__ tile_meta, const int64_t* __restrict__ row_meta, int R,
    int K, int tile_rows, int tile_cols, int KB, const uint16_t* __restrict__ act, int T, int64_t ldx,
    void* __restrict__ Y, int64_t ldy, int tilesR, int tilesT, int group_r) {
  constexpr int WROWS = BR / 4;    // rows per wave
  constexpr int FR = WROWS / 16;   // 16-row fragments per wave
  constexpr int FT = BT / 16;      // 16-token fragments
  constexpr int STAGE = BT * 128;  // bytes of one activation stage (BT x 64 halves)
  constexpr int BLOADS = BT / 32;  // 16-byte direct loads per thread per stage
  constexpr int PER_STEP = BLOADS + 2 * FR;
  static_assert((NS - 2) * PER_STEP < 64, "vmcnt range");
  extern __shared__ __align__(16) unsigned char smem[];     // [NS][STAGE], then the flag words
  uint32_t* flag_words = reinterpret_cast<uint32_t*>(smem + NS * STAGE);  // [4][kMaxFlagWords]

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
  const int li = lane & 15, lq = lane >> 4;
  const int nsteps = K >> 6;
  const int spt = tile_cols >> 6;  // K steps per tile-column

  // ---- this wave's tile-row (its rows lie in one: tile_rows % WROWS == 0;
  // rows past R read row R - 1, whose tile-row is the last)
  const int wrow0 = R0 + wave * WROWS;
  const int b = __builtin_amdgcn_readfirstlane(min(wrow0, R - 1) / tile_rows);
  const int64_t Lv = row_meta[b * 4], Li = row_meta[b * 4 + 1];
  const int64_t VB = row_meta[b * 4 + 2], IB = row_meta[b * 4 + 3];
  // dense flags of the tile-row's tiles, one bit each, into this wave's words
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

  // per-fragment row parts of the weight offsets (elements / bytes)
  uint32_t vrow[FR], irow[FR];
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = min(wrow0 + i * 16 + li, R - 1);
    const int64_t rr = r - int64_t(b) * tile_rows;
    vrow[i] = uint32_t(VB + rr * Lv) + uint32_t(lq) * 8u;
    irow[i] = uint32_t(IB + rr * Li) + uint32_t(lq) * 2u;  // IB, Li: multiples of 8
  }
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(values, values_bytes);
  const __amdgpu_buffer_rsrc_t ri = make_rsrc(idx, idx_bytes);

  // activation slots this thread fills each stage: instruction j covers slots
  // [(wave*BLOADS + j)*64, +64), lane l takes slot base + l; byte offsets from
  // the tile's first token row (rows past T reread row T - 1, whose outputs
  // are dropped), through a descriptor ending with the tile's last row
  const int tlast = min(T0 + BT, T) - 1;
  const __amdgpu_buffer_rsrc_t rb =
      make_rsrc(act + int64_t(T0) * ldx, uint32_t((int64_t(tlast - T0) * ldx + K) * 2));
  uint32_t boff[BLOADS];
#pragma unroll
  for (int j = 0; j < BLOADS; ++j) {
    const int slot = (wave * BLOADS + j) * 64 + lane;
    const int tok = slot >> 3;
    const int chunk = (slot & 7) ^ (tok & 7);
    const int t = min(T0 + tok, T - 1) - T0;
    boff[j] = uint32_t(t) * uint32_t(ldx) * 2u + uint32_t(chunk) * 16u;
  }
  // the activations of step s (past the last step: zeros, from an offset the
  // descriptor refuses)
  auto issue_b = [&](int s, int stage) {
    const uint32_t so = s < nsteps ? uint32_t(s) * 128u : 0x80000000u;
#pragma unroll
    for (int j = 0; j < BLOADS; ++j) dma16(rb, boff[j], so, smem + stage * STAGE + (wave * BLOADS + j) * 1024);
  };

  // The weight stream walks the row's tiles in order: lv / li are the next
  // step's value / index-byte positions along a row of the tile-row, jt and
  // kt its tile-column and step within it.
  uint32_t lv = 0, lio = 0;
  int jt = 0, kt = 0;
  HFrag ar[NS][FR];
  uint32_t sdense = 0;  // bit u: the step held by register stage u is dense
  // Per step and fragment: the row's next 16 bytes of values, then either
  // its following 16 value bytes (dense) or the aligned index block holding
  // this lane's two index bytes (2:4): same instructions and counts for both.
  // The lane's index bytes sit at byte irow[i] + lio; the block starts at that
  // offset rounded down to 16 and (irow[i] + lio) & 15 locates them in it, so
  // each register stage keeps the lio it was loaded with.
  uint32_t sio[NS];
  // Past the last step the loads read zeros (offsets the descriptors refuse),
  // so those steps' MFMAs add exactly zero.
  auto issue_a = [&](auto stage_c, int step) {
    constexpr int stage_u = decltype(stage_c)::value;
    const int jc = min(jt, KB - 1);
    const uint32_t dense = (__builtin_amdgcn_readfirstlane(wflags[jc >> 5]) >> (jc & 31)) & 1u;
    const bool live = step < nsteps;
    const uint32_t v = lv, io = lio;
    const __amdgpu_buffer_rsrc_t r1 = dense ? rv : ri;
#pragma unroll
    for (int i = 0; i < FR; ++i) {
      const uint32_t e = vrow[i] + v;
      const uint32_t o0 = live ? e * 2u : 0xFFFFFFF0u;
      const uint32_t o1 = !live ? 0xFFFFFFF0u : dense ? (e + 32u) * 2u : (irow[i] + io) & ~15u;
      ar[stage_u][i].lo = __builtin_amdgcn_raw_buffer_load_b128(rv, o0, 0, 0);
      ar[stage_u][i].hi = __builtin_amdgcn_raw_buffer_load_b128(r1, o1, 0, 0);
    }
    sdense = (sdense & ~(1u << stage_u)) | (dense << stage_u);
    sio[stage_u] = io;
    lv = v + (dense ? 64u : 32u);
    lio = io + (dense ? 0u : 8u);
    const int nk = kt + 1;
    jt += nk == spt ? 1 : 0;
    kt = nk == spt ? 0 : nk;
  };

  f32x4 acc[FR][FT];
#pragma unroll
  for (int i = 0; i < FR; ++i)
#pragma unroll
    for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: steps 0 .. NS-2 in flight.  Every step issues the same
  // loads (zeros past the last step) and runs its MFMAs, so the waits are
  // fixed counts and the loop holds no data-dependent branch but the uniform
  // dense / 2:4 choice.
  unroll<NS - 1>([&](auto pc) {
    constexpr int p = decltype(pc)::value;
    issue_b(p, p);
    issue_a(pc, p);
  });

  for (int s0 = 0; s0 < nsteps; s0 += NS) {
    unroll<NS>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int s = s0 + u;
      {
        // step s's loads are done once at most the later steps' loads remain
        wait_vmcnt<(NS - 2) * PER_STEP>();
        barrier_no_fence();
        issue_b(s + NS - 1, (u + NS - 1) % NS);
        issue_a(std::integral_constant<int, (u + NS - 1) % NS>{}, s + NS - 1);
        const unsigned char* st = smem + u * STAGE;
        u32x8 bf[FT];
#pragma unroll
        for (int j = 0; j < FT; ++j) {
          const int tok = j * 16 + li;
          const int sw = tok & 7;
          const u32x4 lo = *reinterpret_cast<const u32x4*>(st + (tok * 8 + (lq ^ sw)) * 16);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(st + (tok * 8 + ((lq + 4) ^ sw)) * 16);
          bf[j] = u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        if ((sdense >> u) & 1u) {
#pragma unroll
          for (int j = 0; j < FT; ++j) {
            const u32x4 blo = {bf[j][0], bf[j][1], bf[j][2], bf[j][3]};
            const u32x4 bhi = {bf[j][4], bf[j][5], bf[j][6], bf[j][7]};
#pragma unroll
            for (int i = 0; i < FR; ++i) {
              acc[i][j] = mfma_dense<DT>(ar[u][i].lo, blo, acc[i][j]);
              acc[i][j] = mfma_dense<DT>(ar[u][i].hi, bhi, acc[i][j]);
            }
          }
        } else {
          // this lane's 16 index bits: bytes pos, pos + 1 of its fragment's block
          uint32_t ix[FR];
#pragma unroll
          for (int i = 0; i < FR; ++i) {
            const uint32_t pos = (irow[i] + sio[u]) & 15u;
            const u32x4& h = ar[u][i].hi;
            const uint32_t d = (pos & 8u) ? ((pos & 4u) ? h[3] : h[2]) : ((pos & 4u) ? h[1] : h[0]);
            ix[i] = (d >> ((pos & 2u) * 8u)) & 0xFFFFu;
          }
#pragma unroll
          for (int j = 0; j < FT; ++j)
#pragma unroll
            for (int i = 0; i < FR; ++i) acc[i][j] = smfmac<DT>(ar[u][i].lo, bf[j], acc[i][j], ix[i]);
        }
      }
    });
  }
  // the loads past the last step are still landing: LDS and registers are
  // done with only once they have
  wait_vmcnt<0>();

  // ---- epilogue
  const bool vec_ok = (ldy & 3) == 0;
#pragma unroll
  for (int i = 0; i < FR; ++i) {
    const int r = R0 + wave * WROWS + i * 16 + lq * 4;
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
  constexpr int lds = NS * BT * 128 + 4 * kMaxFlagWords * 4;
  auto kern = hybrid_gemm_kernel<DT, OUT, BR, BT, NS>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(unsigned(ntiles)), dim3(256), lds, s, a.values, uint32_t(a.values_bytes), a.idx,
                     uint32_t(a.idx_bytes), a.tile_meta, a.row_meta, int(a.R), int(a.K), int(a.tile_rows),
                     int(a.tile_cols), int(a.K / a.tile_cols), a.act, int(a.T), a.ldx, a.Y, a.ldy, tilesR,
                     tilesT, group_r);
  return hipGetLastError();
}

template <int DT, int OUT>
hipError_t hybrid_tile(const HybridArgs& a, hipStream_t s) {
  // 256 x 64 tiles when they cover the chip's 256 CUs, else 128 x 64 (a
  // 256 x 128 tile's eight-register weight fragments four steps deep do not
  // fit beside its accumulators without spilling)
  const int64_t big = ((a.R + 255) / 256) * ((a.T + 63) / 64);
  if (big >= 256) return launch_hybrid_cfg<DT, OUT, 256, 64, 4>(a, s);
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
