// 2:4 sparse GEMM with the activation tile resident in LDS, for layers whose
// reduction length is short enough that a tile of tokens fits whole
// (K <= 1024 for 64 tokens, K <= 2048 for 32, K <= 4096 for 16).  It also
// carries the permuted product y = (W Pi) x.
//
// SHUFFLESPARSE technical summary, section 2 and the inference-efficiency item
// of its technical components: the hardened permutation is a precomputed
// index map, and the structured GEMM reads its input at the permuted
// addresses, so no separate permutation pass runs and the FLOPs are those of
// the plain GEMM.  Here the map is applied once per token tile while the tile
// is staged: the tile's activation rows are copied unpermuted into a staging
// area of LDS, and each thread then builds 8 consecutive permuted columns of
// a row with 8 LDS reads at perm[k .. k+7] and one 16-byte LDS write into the
// resident tile.  Every weight row of the layer then streams past the
// resident tile, so the gather's cost is shared by all R rows.
//
// Work unit: TU tokens x a range of row passes (a pass = 8 waves x 64 rows).
// One workgroup per CU walks the units.  Per unit:
//   1. the first blocks of packed weights are requested (registers, below);
//   2. the resident tile is built: [K/128 blocks][TU tokens][256 bytes], the
//      16-byte chunk c (K 128p + 8c .. +7 of block p) of token t at slot
//      c ^ (t & 15), so the fragment reads of 16 consecutive tokens hit 16
//      distinct slots (all banks) and so do the gather's writes;
//   3. each wave multiplies its 64 rows (4 fragments) by all TU tokens, 128 K
//      at a time, with the packed values and index bits loaded from global
//      memory straight into registers (rows are private to a wave, so
//      nothing is shared through LDS) one block ahead of use.
//
// Loads of a 128-wide block.  A row fragment's packed values are two 64-wide
// MFMA steps; in each, lane (row li, quarter lq) takes its 16 bytes at 16 lq,
// so one load instruction reads 16 rows x 64 contiguous bytes.  The index
// bits of the block are 16 bytes per row; lane lq loads the aligned word at
// 4 lq, and two cross-quarter swaps (v_permlane16_swap, v_permlane32_swap)
// give every lane the word holding its own 16 bits of each step (quarter lq
// needs bytes 2 lq and 8 + 2 lq), which a shift by 16 (lq & 1) moves into
// the low half the MFMA reads.  The K order is that of every other prefill
// family, so the sums (and bits) are the same.
#include "nm_device.h"
#include "nm_internal.h"

namespace nm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kRW = 64;                   // rows per wave per pass
constexpr int kFR = kRW / 16;             // row fragments per wave
constexpr int kPassRows = kWaves * kRW;   // 512
constexpr int kLdsMax = 160 * 1024;

struct ResArgs {
  const uint16_t* values;
  const uint32_t* idx;
  const uint16_t* act;
  const int32_t* perm;
  void* Y;
  int64_t ldx, ldy;
  int R, K, T;
  int tilesT;          // token tiles
  int passes;          // row passes over R
  int ppu;             // passes per unit
  int nunits;          // tilesT * ceil(passes / ppu)
  int G;               // tokens per gather round (permuted product)
};

// Packed weights of one 128-wide block for a wave's 4 row fragments.
struct ABlk {
  u32x4 v0[kFR], v1[kFR];   // the lane's 8 survivors of the block's first and second 64-wide step
  uint32_t ix[kFR];         // index bytes 4 lq .. 4 lq + 3 of the row's 16
};

template <int DT, int OUT, bool PERM, bool FAST, int TU>
__global__ __launch_bounds__(kThreads, 1) void spmm_res_kernel(ResArgs a) {
  constexpr int FT = TU / 16;           // token fragments
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K, R = a.R, T = a.T;
  const int nb = K >> 7;                // 128-wide K blocks per pass
  const int S = K >> 1;                 // packed values per row
  const int ibytes = K >> 3;            // index bytes per row
  unsigned char* bres = smem;                         // [nb][TU][256]
  unsigned char* stage = smem + TU * K * 2;           // [G][K] halves (permuted product)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;

  // lane-constant parts of the resident-tile fragment addresses: step h of a
  // block reads chunks 8h + lq and 8h + 4 + lq, at slots chunk ^ li, i.e.
  // (lq ^ li) ^ 4e for e = 0 (chunk lq), 1 (lq + 4), 2 (8 + lq), 3 (12 + lq)
  uint32_t boff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) boff[e] = uint32_t(li) * 256u + (uint32_t((lq ^ li) ^ (4 * e)) << 4);
  const uint32_t ishift = 16u * uint32_t(lq & 1);

  // gather roles (permuted product): thread -> one 8-column chunk c of every
  // row it builds, rows r0, r0 + rstep, ... of a round; its 8 map entries are
  // read once, as byte offsets into a staged row
  const int C8 = K >> 3;
  const int rstep = kThreads / C8;           // >= 1 (K <= 4096)
  const int glanes = rstep * C8;
  const int gc = tid % C8;
  const int gr0 = tid / C8;
  uint32_t q[8];
  if constexpr (PERM) {
    const uint32_t kmax = uint32_t(K - 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = 0u;
    if (tid < glanes) {
      const int4 p0 = *reinterpret_cast<const int4*>(a.perm + gc * 8);
      const int4 p1 = *reinterpret_cast<const int4*>(a.perm + gc * 8 + 4);
      // entries outside [0, K) (a broken precondition) are clamped into the
      // row: a wrong value, never a wrong address
      q[0] = umin(uint32_t(p0.x), kmax) * 2u; q[1] = umin(uint32_t(p0.y), kmax) * 2u;
      q[2] = umin(uint32_t(p0.z), kmax) * 2u; q[3] = umin(uint32_t(p0.w), kmax) * 2u;
      q[4] = umin(uint32_t(p1.x), kmax) * 2u; q[5] = umin(uint32_t(p1.y), kmax) * 2u;
      q[6] = umin(uint32_t(p1.z), kmax) * 2u; q[7] = umin(uint32_t(p1.w), kmax) * 2u;
    }
  }

  ABlk A[2];
  f32x4 acc[kFR][FT];

  for (int u = blockIdx.x; u < a.nunits; u += gridDim.x) {
    const int tt = u % a.tilesT;
    const int pass0 = (u / a.tilesT) * a.ppu;
    const int npass = min(a.ppu, a.passes - pass0);
    const int T0 = tt * TU;
    const int nblk = npass * nb;     // blocks of this unit

    // Loads of unit block g (pass g / nb, block g % nb) into dst.  Blocks
    // past the unit's last reread it, so every block issues the same loads.
    // Rows past R reread row R - 1 (their outputs are not stored): the row
    // sits in the per-lane offset, the block in the scalar one.
    auto load_blk = [&](int g, ABlk& dst) {
      g = min(g, nblk - 1);
      const int p = g / nb, b = g - p * nb;
      const int64_t r0 = int64_t(pass0 + p) * kPassRows;
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.values + r0 * S);
      const __amdgpu_buffer_rsrc_t ri = make_rsrc(reinterpret_cast<const unsigned char*>(a.idx) + r0 * ibytes);
      const int rmax = int(int64_t(R) - 1 - r0);
#pragma unroll
      for (int i = 0; i < kFR; ++i) {
        const uint32_t row = uint32_t(min(wave * kRW + i * 16 + li, rmax));
        const int vo = int(row * uint32_t(S) * 2u + uint32_t(lq) * 16u);
        const int io = int(row * uint32_t(ibytes) + uint32_t(lq) * 4u);
        dst.v0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo, b * 128, 0));
        dst.v1[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 64, b * 128, 0));
        dst.ix[i] = __builtin_amdgcn_raw_buffer_load_b32(ri, io, b * 16, 0);
      }
    };

    // every wave is done reading the previous unit's resident tile
    wait_lgkm0();
    barrier_no_fence();
    load_blk(0, A[0]);

    // ---- resident tile
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + int64_t(T0) * a.ldx);
    const int tlast = T - 1 - T0;   // tokens past T reread token T - 1 (outputs dropped)
    if constexpr (!PERM) {
      // slot s (16 B) of the tile: block s / (16 TU), token (s / 16) % TU,
      // position s % 16 holding chunk (s % 16) ^ (token & 15)
      const int nslots = TU * C8;
      for (int s0 = wave * 64; s0 < nslots; s0 += kThreads) {
        const int s = s0 + lane;
        const int p = s / (16 * TU);
        const int t = (s >> 4) % TU;
        const int c = (s & 15) ^ (t & 15);
        const uint32_t off = uint32_t(min(t, tlast)) * uint32_t(a.ldx) * 2u + uint32_t(p) * 256u + uint32_t(c) * 16u;
        if (s < nslots) dma16(ra, off, 0, bres + s0 * 16);
      }
      wait_vmcnt<0>();
      barrier_no_fence();
    } else {
      const int G = a.G;
      for (int g0 = 0; g0 < TU; g0 += G) {
        const int gn = min(G, TU - g0);   // rows of this round
        const int nst = gn * C8;          // its 16-byte slots
        // stage rows g0 .. g0+G-1 unpermuted: slot s = (row s / C8, chunk s % C8)
        for (int s0 = wave * 64; s0 < nst; s0 += kThreads) {
          const int s = s0 + lane;
          const int t = g0 + s / C8;
          const int c = s % C8;
          const uint32_t off = uint32_t(min(t, tlast)) * uint32_t(a.ldx) * 2u + uint32_t(c) * 16u;
          if (s < nst) dma16(ra, off, 0, stage + s0 * 16);
        }
        wait_vmcnt<0>();
        barrier_no_fence();
        if (tid < glanes) {
          const int p = gc >> 4;
          for (int r = gr0; r < gn; r += rstep) {
            const unsigned char* row = stage + r * K * 2;
            u32x4 o;
            o[0] = uint32_t(*reinterpret_cast<const uint16_t*>(row + q[0])) |
                   (uint32_t(*reinterpret_cast<const uint16_t*>(row + q[1])) << 16);
            o[1] = uint32_t(*reinterpret_cast<const uint16_t*>(row + q[2])) |
                   (uint32_t(*reinterpret_cast<const uint16_t*>(row + q[3])) << 16);
            o[2] = uint32_t(*reinterpret_cast<const uint16_t*>(row + q[4])) |
                   (uint32_t(*reinterpret_cast<const uint16_t*>(row + q[5])) << 16);
            o[3] = uint32_t(*reinterpret_cast<const uint16_t*>(row + q[6])) |
                   (uint32_t(*reinterpret_cast<const uint16_t*>(row + q[7])) << 16);
            const int t = g0 + r;
            *reinterpret_cast<u32x4*>(bres + (p * TU + t) * 256 + (((gc & 15) ^ (t & 15)) << 4)) = o;
          }
        }
        wait_lgkm0();
        barrier_no_fence();   // the round's rows are consumed / the tile is complete
      }
    }

    // ---- stream every row pass of the unit past the resident tile
    auto zero_acc = [&]() {
#pragma unroll
      for (int i = 0; i < kFR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    zero_acc();

    // Epilogue of pass p.  FAST (R and ldy multiples of the store width):
    // every store is issued, with an offset past the buffer's records for
    // outputs outside Y (the hardware drops those), so the number of stores is
    // fixed and the compiler's wait for the next pass's first block leaves
    // them in flight.  Otherwise stores are skipped or split at the edges.
    auto epilogue = [&](int p) {
      const int rbase = (pass0 + p) * kPassRows + wave * kRW;
      const int trows = min(TU, T - T0);
      if constexpr (OUT == NM_F32) {
        if constexpr (FAST) {
          const uint32_t rec = uint32_t((int64_t(trows - 1) * a.ldy + R) * 4);
          const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<float*>(a.Y) + int64_t(T0) * a.ldy, rec);
#pragma unroll
          for (int i = 0; i < kFR; ++i) {
            const int r = rbase + i * 16 + lq * 4;
#pragma unroll
            for (int j = 0; j < FT; ++j) {
              const int tr = j * 16 + li;
              const bool ok = tr < trows && r < R;
              const uint32_t off = ok ? uint32_t((int64_t(tr) * a.ldy + r) * 4) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), ry, int(off), 0, 0);
            }
          }
        } else {
          const bool vec_ok = (a.ldy & 3) == 0;
#pragma unroll
          for (int i = 0; i < kFR; ++i) {
            const int r = rbase + i * 16 + lq * 4;
#pragma unroll
            for (int j = 0; j < FT; ++j) {
              const int t = T0 + j * 16 + li;
              if (t >= T || r >= R) continue;
              float* y = static_cast<float*>(a.Y) + int64_t(t) * a.ldy + r;
              const f32x4 v = acc[i][j];
              if (vec_ok && r + 3 < R) {
                *reinterpret_cast<f32x4*>(y) = v;
              } else {
                for (int e = 0; e < 4 && r + e < R; ++e) y[e] = v[e];
              }
            }
          }
        }
      } else {
        // Half outputs: fragments i and i+1 (32 rows) are exchanged across
        // lane quarters so that quarter q holds rows 8q .. 8q+7 of the pair,
        // and each lane stores 16 contiguous bytes (a token row gets 64-byte
        // runs instead of 32).
        const uint32_t rec = uint32_t((int64_t(trows - 1) * a.ldy + R) * 2);
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<uint16_t*>(a.Y) + int64_t(T0) * a.ldy, rec);
        const bool vec_ok = (a.ldy & 7) == 0;
#pragma unroll
        for (int i = 0; i < kFR; i += 2) {
          const int r = rbase + i * 16 + lq * 8;
#pragma unroll
          for (int j = 0; j < FT; ++j) {
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
            const u32x4 v = {t0[0], t1[0], t0[1], t1[1]};   // rows r .. r+7
            const int tr = j * 16 + li;
            if constexpr (FAST) {
              const bool ok = tr < trows && r < R;
              const uint32_t off = ok ? uint32_t((int64_t(tr) * a.ldy + r) * 2) : 0x80000000u;
              __builtin_amdgcn_raw_buffer_store_b128(v, ry, int(off), 0, 0);
            } else {
              if (tr >= trows || r >= R) continue;
              uint16_t* y = static_cast<uint16_t*>(a.Y) + int64_t(T0 + tr) * a.ldy + r;
              if (vec_ok && r + 7 < R) {
                *reinterpret_cast<u32x4*>(y) = v;
              } else {
                for (int e = 0; e < 8 && r + e < R; ++e) y[e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
              }
            }
          }
        }
      }
    };

    // multiply block g into the accumulators
    auto compute = [&](int g, const ABlk& cur) {
      const int b = g % nb;
      const unsigned char* bb = bres + b * TU * 256;
      u32x8 b0[FT], b1[FT];
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const unsigned char* pj = bb + j * 16 * 256;
        const u32x4 lo0 = *reinterpret_cast<const u32x4*>(pj + boff[0]);
        const u32x4 hi0 = *reinterpret_cast<const u32x4*>(pj + boff[1]);
        b0[j] = u32x8{lo0[0], lo0[1], lo0[2], lo0[3], hi0[0], hi0[1], hi0[2], hi0[3]};
      }
#pragma unroll
      for (int j = 0; j < FT; ++j) {
        const unsigned char* pj = bb + j * 16 * 256;
        const u32x4 lo1 = *reinterpret_cast<const u32x4*>(pj + boff[2]);
        const u32x4 hi1 = *reinterpret_cast<const u32x4*>(pj + boff[3]);
        b1[j] = u32x8{lo1[0], lo1[1], lo1[2], lo1[3], hi1[0], hi1[1], hi1[2], hi1[3]};
      }
      // index words: quarter q of the result rows holds word (q >> 1) (step 0)
      // or 2 + (q >> 1) (step 1) of the row's 16 bytes, as loaded by quarter
      // q' = that word's number
      uint32_t ix0[kFR], ix1[kFR];
#pragma unroll
      for (int i = 0; i < kFR; ++i) {
        const auto p = __builtin_amdgcn_permlane16_swap(cur.ix[i], cur.ix[i], false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(p[0], p[1], false, false);
        ix0[i] = h[0] >> ishift;
        ix1[i] = h[1] >> ishift;
      }
#pragma unroll
      for (int i = 0; i < kFR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = smfmac<DT>(cur.v0[i], b0[j], acc[i][j], ix0[i]);
#pragma unroll
      for (int i = 0; i < kFR; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = smfmac<DT>(cur.v1[i], b1[j], acc[i][j], ix1[i]);
    };

    // One pass: block g's registers were requested one block earlier; each
    // step requests the next block (the next pass's first after the last)
    // and then multiplies, so the compiler's wait before the MFMAs leaves the
    // newer loads, and after an epilogue its stores, in flight.  A pass has an
    // even number of blocks, so it starts and ends with the same registers.
    // (The scheduling barrier keeps the requests ahead of the MFMAs: left to
    // itself the scheduler sinks them below the block's MFMAs.)
    auto step = [&](int g, const ABlk& cur, ABlk& fill) {
      load_blk(g + 1, fill);
      __builtin_amdgcn_sched_barrier(0);
      compute(g, cur);
    };
    auto run_pass = [&](int p) {
      const int g0 = p * nb;
      step(g0, A[0], A[1]);
      for (int b = 1; b + 1 < nb; b += 2) {
        step(g0 + b, A[1], A[0]);
        step(g0 + b + 1, A[0], A[1]);
      }
      step(g0 + nb - 1, A[1], A[0]);
      epilogue(p);
      zero_acc();
    };
    // pass 0 apart, so the loop below is only entered after an epilogue
    run_pass(0);
    for (int p = 1; p < npass; ++p) run_pass(p);
  }
  wait_vmcnt<0>();   // no load still writing registers or LDS when the workgroup ends
}

template <int DT, int OUT, bool PERM, bool FAST, int TU>
hipError_t launch_res_t(const SpmmArgs& a, hipStream_t s) {
  ResArgs r;
  r.values = a.values;
  r.idx = a.idx;
  r.act = a.act;
  r.perm = a.perm;
  r.Y = a.Y;
  r.ldx = a.ldx;
  r.ldy = a.ldy;
  r.R = int(a.R);
  r.K = int(a.K);
  r.T = int(a.T);
  r.tilesT = int((a.T + TU - 1) / TU);
  r.passes = int((a.R + kPassRows - 1) / kPassRows);
  const int cus = device_cu_count();
  // Few token tiles: split the row passes too, so that every CU has work.
  int split = 1;
  if (r.tilesT < cus) split = min(r.passes, max(1, cus / r.tilesT));
  r.ppu = (r.passes + split - 1) / split;
  const int64_t units = int64_t(r.tilesT) * ((r.passes + r.ppu - 1) / r.ppu);
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  r.nunits = int(units);
  const int bres = TU * r.K * 2;
  int lds = bres;
  r.G = 0;
  if constexpr (PERM) {
    // staged rows per gather round: as many as fit beside the tile, at most TU
    int G = (kLdsMax - bres) / (r.K * 2);
    G = G > TU ? TU : G;
    r.G = G;
    lds += G * r.K * 2;
  }
  auto kern = spmm_res_kernel<DT, OUT, PERM, FAST, TU>;
  if (hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(kern), lds); e != hipSuccess) return e;
  const int grid = int(units < cus ? units : cus);
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), lds, s, r);
  return hipGetLastError();
}

template <int DT, int OUT, bool PERM, bool FAST>
hipError_t launch_res_tu(const SpmmArgs& a, hipStream_t s) {
  if (a.K <= 1024) return launch_res_t<DT, OUT, PERM, FAST, 64>(a, s);
  if (a.K <= 2048) return launch_res_t<DT, OUT, PERM, FAST, 32>(a, s);
  return launch_res_t<DT, OUT, PERM, FAST, 16>(a, s);
}

// FAST epilogue: every output chunk a lane stores lies wholly inside a row
// (R a multiple of the chunk) and starts aligned (ldy a multiple of it).
template <int DT, int OUT>
hipError_t launch_res_p(const SpmmArgs& a, hipStream_t s) {
  const int64_t chunk = OUT == NM_F32 ? 4 : 8;
  const bool fast = a.R % chunk == 0 && a.ldy % chunk == 0;
  if (a.perm)
    return fast ? launch_res_tu<DT, OUT, true, true>(a, s) : launch_res_tu<DT, OUT, true, false>(a, s);
  return fast ? launch_res_tu<DT, OUT, false, true>(a, s) : launch_res_tu<DT, OUT, false, false>(a, s);
}

}  // namespace

// Largest tokens-per-tile the shape allows (0: none): the resident tile plus
// at least 4 staged rows (permuted product) must fit the workgroup's LDS.
static int res_tu(int64_t K) {
  if (K <= 1024) return 64;
  if (K <= 2048) return 32;
  if (K <= 4096) return 16;
  return 0;
}

bool spmm_resident_applies(const SpmmArgs& a) {
  if (!(a.n == 2 && a.m == 4 && (a.K % 256) == 0 && a.T > 0 && a.R > 0)) return false;
  const int tu = res_tu(a.K);
  if (tu == 0) return false;
  const int64_t bres = int64_t(tu) * a.K * 2;
  const int64_t need = bres + (a.perm ? 4 * a.K * 2 : 0);
  if (need > kLdsMax || need > device_max_lds()) return false;
  // per-lane byte offsets are 32-bit: a token row block and a pass of rows
  const int64_t lim = int64_t(0xFFFFFFFFu);
  if (int64_t(tu) * a.ldx * 2 > lim || int64_t(kPassRows) * a.K > lim) return false;
  // store offsets below 2^31 (an offset of 2^31 marks a dropped store)
  if (int64_t(tu) * a.ldy * 4 >= (int64_t(1) << 31)) return false;
  return true;
}

hipError_t launch_spmm_resident(const SpmmArgs& a, hipStream_t s) {
  if (a.dtype == NM_F16)
    return a.out_dtype == NM_F32 ? launch_res_p<NM_F16, NM_F32>(a, s) : launch_res_p<NM_F16, NM_F16>(a, s);
  return a.out_dtype == NM_F32 ? launch_res_p<NM_BF16, NM_F32>(a, s) : launch_res_p<NM_BF16, NM_BF16>(a, s);
}

}  // namespace nm
