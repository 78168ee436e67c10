// GEMM kernels of the bridge projector: Linear(C*k*k -> hidden) + bias + GELU
// over the merged tokens, and Linear(hidden -> out) + bias whose epilogue
// writes each row to its destination (a row of the output, or its placeholder
// slot in the sequence).  mlxcel issue #533 "port DeepSeek-VL2", section
// "Projector (downsample_mlp_gelu)" steps 1-3.
//
// bf16 path (gfx950): 256x256 output tile per 256-thread workgroup, 4 waves in
// a 2x2 grid, each wave 128x128 from 8x8 v_mfma_f32_16x16x32_bf16 tiles with
// fp32 accumulation (the 16x16x32 form draws less power per flop than
// 32x32x16, so under the board's power cap it sustains a higher clock); the
// last, partly filled round of tiles runs as 128x128 tiles.  K advances 32 per stage through four LDS stages (A and B halves,
// 64-byte rows of 16-byte chunks XOR-swizzled by row), filled by
// direct-to-LDS buffer loads three stages ahead of the MFMAs.  Every operand
// is tile-blocked ([R/256][K/32][256][32]), so each load instruction of a
// wave moves one contiguous KiB.  Linear1 takes the merged tokens (K ordered
// position-major, k' = p*C + c, like the packed W1) and writes the hidden
// activation tile-blocked; Linear2 reads it and stores plain rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlb_common.h"
#include "vlb_internal.h"

namespace vlb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = kGemmBK, NTHREADS = 256;
constexpr int NSTAGE = kGemmStages;  // LDS stages; three are in flight
constexpr int GROUP_M = 8;

// Geometry of a BMT x BMT output tile (BMT = 256 or 128) computed by 4 waves
// in a 2x2 grid, each wave owning a (BMT/2)^2 block of 16x16 MFMA tiles.
template <int BMT>
struct Geo {
  static constexpr int TI = BMT / 32;          // MFMA tiles per wave per dimension
  static constexpr int WT = BMT / 2;           // wave tile side
  static constexpr int LPW = BMT / 64;         // 16-row loads per wave per operand per stage
  static constexpr int HALF = BMT * BK * 2;    // bytes of one operand in a stage
  static constexpr int STAGE = 2 * HALF;       // bytes of a stage
  static constexpr int ROWB = BMT * 2;         // bytes of one bf16 output row
  static constexpr int CCH = BMT / 8;          // 16-byte chunks per output row
  static constexpr int RPB = STAGE / ROWB;     // output rows staged per stage buffer (64)
  static_assert(RPB == 64, "C staging assumes 64 rows per stage buffer");
};

// Logical tile -> (tile row, tile column): groups of GROUP_M tile-rows, column
// by column, so tiles that run together share A and B panels in L2.
__device__ __forceinline__ void tile_coords(int logical, int tiles_m, int tiles_n, int &tm,
                                            int &tn) {
  const int span = GROUP_M * tiles_n;
  const int group = logical / span;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * span;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
// b % 8); this gives each XCD a contiguous range of the n logical indices.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Whole tiles: workgroups are dealt round-robin to the 8 XCDs (workgroup b
// runs on XCD b % 8) and each XCD starts its workgroups in order, so its j-th
// group of 32 (one per CU) runs at about the same time as every other XCD's
// j-th.  Group j of XCD x takes the 32 logical tiles of block 8j + x: in every
// round the eight XCDs work on 256 consecutive logical tiles, so the A panels
// of those tile rows are read by several XCDs at once and the B panels stay
// in use from round to round.  A last round that is not full keeps launch
// order.
__device__ __forceinline__ int whole_tile_order(int bid, int n) {
  const int full = n & ~255;
  if (bid >= full) return bid;
  const int xcd = bid & 7, local = bid >> 3;
  return ((((local >> 5) << 3) + xcd) << 5) + (local & 31);
}

// Byte offset of 16-byte chunk `chunk` (0..3) of row `row` inside a stage
// half: 64-byte rows, the chunk XOR-ed with (row >> 1) & 3.  A fragment read
// (16 consecutive rows from a multiple of 16, one logical chunk per group of
// 16 lanes) then takes 4 LDS cycles per ds_read_b128, the rate of a linear
// read; ((row >> 1) ^ (row >> 3)) & 3, or no swizzle, takes 8 (measured with
// the LDS bank-conflict counters on gfx950).
__device__ __forceinline__ int swz_xor(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 64 + ((chunk ^ swz_xor(row)) << 4);
}

// Barrier of the stage pipeline: this wave's loads are complete except the
// younger ones -- the next stage's and the first half of the one after
// (12 loads for 256-tiles, 6 for 128-tiles) -- its LDS reads are done, then
// the workgroup synchronises.  One asm block, so no memory access moves
// across it.
template <int BMT>
__device__ __forceinline__ void stage_barrier() {
  if constexpr (BMT == 256)
    asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// Token-major operand halves hold BMT/32 blocks of 2 KiB, one per 32 tile
// rows: 32 contraction indices k of 64 bytes, the 16-byte pieces of row k
// XOR-ed with tswz(k) (0 or 2).  With it the 16 lanes of a transposing read
// (4 rows k x 32 bytes) fall on 32 distinct 4-byte banks, and two groups of
// 16 lanes (k and k + 8) on all 64.
__device__ __forceinline__ int tswz(int k) { return (((k >> 1) ^ (k >> 3)) & 1) << 1; }

// Transposing LDS read (ds_read_b64_tr_b16): in every group of 16 lanes,
// lane 4y + x supplies the address of 4 consecutive 16-bit values (row y,
// columns 4x .. 4x + 3 of a 4 x 16 block) and lane l receives column l of
// the block, rows 0..3.
__device__ __forceinline__ bf16x4 tr16(lds_u8 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// Byte offset that lies past every buffer (buffers are < 2^31 bytes): a buffer
// load from it returns zeros, which is how padding and out-of-range rows are
// filled without branches.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes bytes [16 l, 16 l + 16) after `dst`.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst), 16, off, 0, 0, 0);
}

// Stage buffer i of four (a select, never an indexed private array).
__device__ __forceinline__ uint8_t *pick(uint8_t *const (&b)[4], int i) {
  return i == 0 ? b[0] : i == 1 ? b[1] : i == 2 ? b[2] : b[3];
}

// Epilogue of one tile.  The weight fragment is the MFMA's first operand, so
// acc[i][j] holds the transposed product: lane (fr, fq) = (lane % 16,
// lane / 16) of wave (wm, wn) owns token row wm*WT + 16 i + fr and features
// wn*WT + 16 j + 4 fq + e in element e (e < 4).  The accumulators start from
// the bias (gemm_tile), so the epilogue adds none.
//
// stage_tile: the activation (when ACT_ON) applied in fp32 to the
// accumulators (bias included), the tile rounded to bf16 and staged in the
// stage buffers (64 rows each; rows of 16-byte chunks XOR-swizzled by the
// row).  The caller has synchronised the workgroup after its last use of the
// buffers.
template <int ACT, int BMT, bool ACT_ON>
__device__ __forceinline__ void stage_tile(const f32x4 (&acc)[Geo<BMT>::TI][Geo<BMT>::TI],
                                           uint8_t *const (&bufs)[4]) {
  using G = Geo<BMT>;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 15, fq = lane >> 4;
#pragma unroll
  for (int j = 0; j < G::TI; ++j) {
    const int cl = wn * G::WT + j * 16 + 4 * fq;  // 4 consecutive features
    const int chunk = cl >> 3, half = (cl >> 2) & 1;
#pragma unroll
    for (int i = 0; i < G::TI; ++i) {
      const int r = wm * G::WT + i * 16 + fr;  // tile row
      const int row = r & 63;                  // inside buffer r / 64
      uint16_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = acc[i][j][e];
        h[e] = f2bf(ACT_ON ? act_fn<ACT>(v) : v);
      }
      uint2 v;
      v.x = h[0] | (static_cast<uint32_t>(h[1]) << 16);
      v.y = h[2] | (static_cast<uint32_t>(h[3]) << 16);
      *reinterpret_cast<uint2 *>(pick(bufs, r >> 6) + row * G::ROWB +
                                 ((chunk ^ (row & (G::CCH - 1))) << 4) + half * 8) = v;
    }
  }
}

// Tile-blocked output of a staged tile: for each 32-wide feature slice of the
// tile, rows' 64-byte segments are contiguous, so 4 lanes write one row
// segment and a wave 16 rows -- 1 KiB per store.
template <int BMT>
__device__ __forceinline__ void write_blocked(uint8_t *const (&bufs)[4], const GemmArgs &g, int m0,
                                              int n0, uint16_t *out) {
  using G = Geo<BMT>;
  const int tid = threadIdx.x;
  const uint32_t KBo = g.N / 32;
#pragma unroll 4
  for (int q = tid; q < BMT * BMT / 8; q += NTHREADS) {
    const int fs = q / (BMT * 4), rem = q % (BMT * 4);
    const int row = rem >> 2, c4 = rem & 3;  // tile row, chunk in the slice
    const int m = m0 + row, f = n0 + fs * 32 + c4 * 8;
    if (m >= g.M || f >= g.N) continue;
    const int chunk = fs * 4 + c4, rb = row & 63;
    const uint4 v = *reinterpret_cast<const uint4 *>(pick(bufs, row >> 6) + rb * G::ROWB +
                                                     ((chunk ^ (rb & (G::CCH - 1))) << 4));
    const int64_t e =
        ((static_cast<int64_t>(m >> 8) * KBo + (f >> 5)) * 256 + (m & 255)) * 32 + (f & 31);
    *reinterpret_cast<uint4 *>(out + e) = v;
  }
}

// Whole rows of a staged tile with 16-byte stores to row s_dst[r] (skipped
// when negative), non-temporal when g.stream_out is set.
template <int BMT>
__device__ __forceinline__ void write_rows(uint8_t *const (&bufs)[4], const GemmArgs &g, int n0,
                                           const int32_t *s_dst) {
  using G = Geo<BMT>;
  const int tid = threadIdx.x;
  uint16_t *out = static_cast<uint16_t *>(g.out);
  const int chunk = tid % G::CCH;
  const int col = n0 + chunk * 8;
  constexpr int RSTEP = NTHREADS / G::CCH;  // rows per pass
#pragma unroll
  for (int bi = 0; bi < BMT / 64; ++bi) {
#pragma unroll 4
    for (int s8 = 0; s8 < 64 / RSTEP; ++s8) {
      const int row = tid / G::CCH + RSTEP * s8;  // inside buffer bi
      const int dst = s_dst[bi * 64 + row];       // -1: past the last row, or not placed
      if (dst < 0 || col >= g.N) continue;
      const uint4 v = *reinterpret_cast<const uint4 *>(pick(bufs, bi) + row * G::ROWB +
                                                       ((chunk ^ (row & (G::CCH - 1))) << 4));
      uint4 *p = reinterpret_cast<uint4 *>(out + static_cast<int64_t>(dst) * g.ldo + col);
      if (g.stream_out)
        store_nt(p, v);
      else
        *p = v;
    }
  }
}

// fp32 rows straight from the accumulators: each lane stores its 4
// consecutive features of a row as one 16-byte store (a wave covers 16 rows x
// 64 bytes per store instruction).  No bias.
template <int BMT>
__device__ __forceinline__ void write_f32(const f32x4 (&acc)[Geo<BMT>::TI][Geo<BMT>::TI],
                                          const GemmArgs &g, int m0, int n0) {
  using G = Geo<BMT>;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 15, fq = lane >> 4;
  float *out = static_cast<float *>(g.out);
#pragma unroll
  for (int j = 0; j < G::TI; ++j) {
    const int n = n0 + wn * G::WT + j * 16 + 4 * fq;
#pragma unroll
    for (int i = 0; i < G::TI; ++i) {
      const int m = m0 + wm * G::WT + i * 16 + fr;
      if (m < g.M && n < g.N)
        *reinterpret_cast<f32x4 *>(out + static_cast<int64_t>(m) * g.ldo + n) = acc[i][j];
    }
  }
}

// The epilogue of each mode (see GemmMode).
template <int MODE, int ACT, int BMT>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[Geo<BMT>::TI][Geo<BMT>::TI],
                                           const GemmArgs &g, int m0, int n0,
                                           uint8_t *const (&bufs)[4], const int32_t *s_dst) {
  if constexpr (MODE == kGemmF32) {
    write_f32<BMT>(acc, g, m0, n0);
  } else if constexpr (MODE == kGemmRows) {
    stage_tile<ACT, BMT, false>(acc, bufs);
    __syncthreads();
    write_rows<BMT>(bufs, g, n0, s_dst);
  } else {
    if constexpr (MODE == kGemmBlockedSave) {  // pre-activation first
      stage_tile<ACT, BMT, false>(acc, bufs);
      __syncthreads();
      write_blocked<BMT>(bufs, g, m0, n0, static_cast<uint16_t *>(g.out2));
      __syncthreads();
    }
    stage_tile<ACT, BMT, true>(acc, bufs);
    __syncthreads();
    write_blocked<BMT>(bufs, g, m0, n0, static_cast<uint16_t *>(g.out));
  }
}

// One output tile: BMT x BMT at (tm, tn) of the BMT-grid, staged through
// smem0..3 (each at least Geo<BMT>::STAGE bytes) with s_dst (at least BMT
// entries).  Inlined into the kernels below, so the four stage arrays stay
// distinct LDS objects to the compiler.  K steps [ks0, ks0 + ksn) of the
// product are accumulated; with part set (kGemmF32 only) the whole BMT x BMT
// fp32 tile goes to part, row-major, instead of to out.
template <int MODE, int ACT, int BMT, bool GA, bool TB, int SZ>
__device__ __forceinline__ void gemm_tile(const GemmArgs &g, int tm, int tn, uint8_t (&smem0)[SZ],
                                          uint8_t (&smem1)[SZ], uint8_t (&smem2)[SZ],
                                          uint8_t (&smem3)[SZ], int32_t *s_dst, int ks0, int ksn,
                                          float *part) {
  using G = Geo<BMT>;
  static_assert(SZ >= G::STAGE, "stage buffers too small");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in an SGPR
  const int m0 = tm * BMT, n0 = tn * BMT;
  // A gradient GEMM writes nothing when the placeholder scan failed.
  if (MODE == kGemmF32 && g.status && g.status[kStatusWord] != 0) return;
  // The epilogue's destination rows are fetched now so their latency hides
  // under the K loop.
  if (tid < BMT) {
    const int m = m0 + tid;
    s_dst[tid] = m >= g.M ? -1 : (g.dst_row ? g.dst_row[m] : m);
  }
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(g.A, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(g.B, g.b_bytes);

  // Loader role: wave `wid` fills rows [wid*BMT/4, (wid+1)*BMT/4) of both
  // stage halves, 16 rows (1 KiB) per instruction.  Lane l lands on row
  // 16i + l/4 at physical chunk l%4, which holds logical chunk (l%4) ^ swz_xor(row).
  // Both operands are tile-blocked (the 256 rows of a 32-wide K slice of a
  // row block are one contiguous 16 KiB run), so step kt of row r sits at
  // ((r/256 * K/32 + kt) * 256 + r%256) * 64 bytes.
  const uint32_t KB = g.K / BK;
  auto blocked = [&](int r) {
    return (static_cast<uint32_t>(r >> 8) * KB * 256 + static_cast<uint32_t>(r & 255)) * 64;
  };
  // GA (gathered A, kGemmGatherBlocked): A is the bf16 patch grid itself,
  // NHWC, and row m's merged token is read through its gather descriptor.  K
  // runs position-major (k' = p*C + c, the packed W1's order), so the 32-wide
  // K step kt covers channels [32 c, 32 c + 32) of block position p = (dy, dx)
  // -- one 64-byte piece of pixel (y0 + dy, x0 + dx) per row.  a_off holds the
  // piece's offset at p = 0, a_gw the bytes of one grid row, a_inv the
  // complement of the row's inside-the-grid bits: a position outside the grid
  // (the high-end zero padding) or a row past M gets bit 31 set, which lies
  // past every buffer, so the load returns zeros.  Each load instruction then
  // moves 16 separate 64-byte pieces (half lines, the other half read one step
  // later) instead of one contiguous KiB, and this loop is sensitive to that:
  // Linear1 runs 8-11% slower than on the blocked operand.  The merge pass it
  // saves costs the same per token whatever the hidden width, so the gather
  // pays for narrow hidden widths only (the automatic choice in vlb_api.hip).
  // Token-major B (TB; see GemmArgs::tb_w).  Instruction i of wave wid fills
  // KiB gi = wid*LPW + i of the half: the 16 contraction indices k = 16 (gi &
  // 1) + lane/4 of tile rows n0 + 32 (gi >> 1) + [0, 32), lane slot lane%4
  // holding the logical 8-row piece (lane%4) ^ tswz(k).  t_off is the lane's
  // offset at step 0; rows past the stored width W read zeros.
  auto t_off = [&](int r0, int W, int i) -> uint32_t {
    const int gi = wid * G::LPW + i;
    const int k = (gi & 1) * 16 + (lane >> 2);
    const int lp = (lane & 3) ^ tswz(k);
    const int r = r0 + (gi >> 1) * 32 + lp * 8;
    return r < W ? (static_cast<uint32_t>((r >> 5) * 256 + k) * 64 + lp * 16) : kOOB;
  };
  uint32_t a_off[G::LPW], b_off[G::LPW];
  uint32_t a_gw[GA ? G::LPW : 1], a_inv[GA ? G::LPW : 1];
  const uint32_t c2 = static_cast<uint32_t>(g.C) * 2;  // bytes of one pixel (GA)
#pragma unroll
  for (int i = 0; i < G::LPW; ++i) {
    const int row = wid * (BMT / 4) + 16 * i + (lane >> 2);
    const uint32_t c_off = ((lane & 3) ^ swz_xor(row)) * 16;
    const int m = m0 + row, n = n0 + row;
    if constexpr (GA) {
      const RowDesc d = m < g.M ? g.desc[m] : RowDesc{0, 0};
      a_off[i] = static_cast<uint32_t>(d.pix) * c2 + c_off;
      a_gw[i] = static_cast<uint32_t>(d.geo & 0xffff) * c2;
      a_inv[i] = ~(static_cast<uint32_t>(d.geo) >> 16);
    } else {
      a_off[i] = m < g.M ? blocked(m) + c_off : kOOB;
    }
    if constexpr (TB)
      b_off[i] = t_off(n0, g.tb_w, i);
    else
      b_off[i] = n < g.N ? blocked(n) + c_off : kOOB;
  }
  // GA: step ka covers channels [32 c, 32 c + 32) of block position
  // p = (dy, dx), ka = p * cps + c.  The divisions are multiplications by
  // 2^20 / divisor rounded up, exact for dividends below 2^20 / divisor (ka <=
  // K / 32 + 3 <= 1155, cps <= 128, k <= 3), so the loop has no branches.
  const int ga_cps = g.C / BK;
  const uint32_t ga_inv_cps = ((1u << 20) + ga_cps - 1) / ga_cps;
  const uint32_t ga_inv_k = ((1u << 20) + g.k - 1) / g.k;
  // Loads of step kt of the range into `stage` (the first or second half of
  // them when half is 0 or 1, all when -1).  Steps at or past the end of the
  // range read zeros (the loop runs a multiple of NSTAGE steps and prefetches
  // beyond).
  const int KT = ksn;
  auto issue = [&](int kt, uint8_t *stage, int half) {
    const uint32_t dead = kt < KT ? 0u : kOOB;  // OR-ed in: keeps the loads branch-free
    const uint32_t step_off = (ks0 + kt) * (256 * 64);
    uint8_t *sa = stage + wid * G::LPW * 1024;
    uint8_t *sb = stage + G::HALF + wid * G::LPW * 1024;
    const int i0 = half == 1 ? G::LPW / 2 : 0, i1 = half == 0 ? G::LPW / 2 : G::LPW;
    // GA: the wave-uniform part of the offset; dead (bit 31) is added, not
    // OR-ed: the sum stays below 2^32 and keeps bit 31 set.
    const uint32_t ka = static_cast<uint32_t>(ks0 + kt);
    const uint32_t ga_p = (ka * ga_inv_cps) >> 20, ga_c = ka - ga_p * ga_cps;
    const uint32_t ga_dy = (ga_p * ga_inv_k) >> 20, ga_dx = ga_p - ga_dy * g.k;
    const uint32_t ga_s = ga_dx * c2 + ga_c * 64 + dead;
    // Token-major B: step ka is rows k of the stored [K][W] blocks (k / 256 =
    // ka / 8, 32 rows each); indices at or past k_valid read zero.
    const int lim = g.k_valid - static_cast<int>(ka) * BK;
    const uint32_t tb_s = ((ka >> 3) * static_cast<uint32_t>(g.tb_w >> 5) * 256 + (ka & 7) * 32) * 64;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const uint32_t kdead = ((i & 1) * 16 + (lane >> 2)) < lim ? 0u : kOOB;
      if constexpr (GA) {
        const uint32_t off = a_off[i] + ga_dy * a_gw[i] + ga_s;
        load_lds16(rA, sa + i * 1024, off | ((a_inv[i] >> ga_p) << 31));
      } else {
        load_lds16(rA, sa + i * 1024, (a_off[i] + step_off) | dead);
      }
      if constexpr (TB)
        load_lds16(rB, sb + i * 1024, (b_off[i] + tb_s) | dead | kdead);
      else
        load_lds16(rB, sb + i * 1024, (b_off[i] + step_off) | dead);
    }
  };

  // Accumulators start from the bias, so the epilogue adds none.  Each lane
  // needs the 4 bias values of its features in every column tile j, 8 bytes
  // per j, loaded here ahead of the prologue's operands (biases are 16-byte
  // aligned and N is a multiple of 8, so a column below N has all 4 inside)
  // and converted once the prologue's barrier has waited for them.  These
  // kernels use every register; the bias comes straight from memory and is
  // converted in place because reading it from LDS, or converting it in a
  // helper, left the allocator copying accumulators inside the gathered-
  // operand main loop (over 300 moves per four K steps).
  f32x4 acc[G::TI][G::TI];
  uint2 bias_v[G::TI];
  {
    const uint16_t *bias = static_cast<const uint16_t *>(g.bias);
    const int wn = wid & 1, fq = lane >> 4;
#pragma unroll
    for (int j = 0; j < G::TI; ++j) {
      const int c = n0 + wn * G::WT + j * 16 + 4 * fq;
      bias_v[j] = (bias && c < g.N) ? *reinterpret_cast<const uint2 *>(bias + c) : make_uint2(0, 0);
    }
  }

  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 15, fq = lane >> 4;  // fragment row / 8-wide K group of this lane
  // Fragments of one K step (32): TI tiles of 16 rows for each operand; two
  // sets, so the next step's are read while this step's multiply.
  bf16x8 fa0[G::TI], fb0[G::TI], fa1[G::TI], fb1[G::TI];
  // LDS offsets of this lane's fragment reads.  Fragment t covers tile rows
  // w0 + 16 t .. + 15 (w0 = wm*WT for A, wn*WT for B), and both stage layouts
  // place it at a lane offset that depends on t only through its parity, plus
  // (t >> 1) * 2048: so each operand needs two lane offsets and the rest are
  // immediates.
  //   row-major stage: row w0 + 16 t + fr, logical chunk fq (swz);
  //   token-major stage: two transposing reads of 4 K rows each -- lane 4c + q
  //   of a group reads K row 8 fq + c (then + 4: 256 bytes on, tswz(k + 4) ==
  //   tswz(k)) at tile rows w0 + 16 t + 4q .. + 3, so lane fr receives row
  //   w0 + 16 t + fr, K indices 8 fq .. 8 fq + 7.
  auto rd_off = [&](bool tmaj, int w0, int par) -> int {
    if (!tmaj) return swz(w0 + 16 * par + fr, fq);
    const int c = fr >> 2, q = fr & 3, k0 = 8 * fq + c;
    const int lp = 2 * par + (q >> 1);
    return (w0 >> 5) * 2048 + k0 * 64 + ((lp ^ tswz(k0)) << 4) + (q & 1) * 8;
  };
  const int ra0 = rd_off(false, wm * G::WT, 0), ra1 = rd_off(false, wm * G::WT, 1);
  const int rb0 = G::HALF + rd_off(TB, wn * G::WT, 0), rb1 = G::HALF + rd_off(TB, wn * G::WT, 1);
  auto frag = [&](const uint8_t *stage, bool tmaj, int off) -> bf16x8 {
    lds_u8 *p = (lds_u8 *)(stage) + off;
    if (!tmaj) return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(p);
    const bf16x4 lo = tr16(p), hi = tr16(p + 256);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto rd = [&](const uint8_t *stage, bf16x8 *fa, bf16x8 *fb) {
#pragma unroll
    for (int t = 0; t < G::TI; ++t) {
      fa[t] = frag(stage, false, ((t & 1) ? ra1 : ra0) + (t >> 1) * 2048);
      fb[t] = frag(stage, TB, ((t & 1) ? rb1 : rb0) + (t >> 1) * 2048);
    }
  };
  // LDS read instructions per step: one per fragment, two for a token-major one
  constexpr int NRD = G::TI + G::TI * (TB ? 2 : 1);
  // MFMAs [i0, i1) of the step, i-major (A tile i, B tile j), the j order
  // reversed on odd i, so that every MFMA shares an operand with the one
  // before it (the MFMA's power depends on its data, and this loop is bound
  // by power: interleaved A/B, ragged-3x3 step 2.055 -> 2.047 ms).
  auto mma = [&](const bf16x8 *fa, const bf16x8 *fb, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int jj = 0; jj < G::TI; ++jj) {
        const int j = (i & 1) ? G::TI - 1 - jj : jj;
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
      }
  };
  // One K step of 32 (TI x TI MFMAs): the loads of step kt+3 are issued into the
  // stage freed by step kt-1; after the first quarter of the MFMAs the barrier
  // (step kt+1 landed everywhere, step kt's fragments all read) lets the next
  // step's fragments be read under the remaining MFMAs.
  constexpr int Q = G::TI / 4;  // A tiles per quarter
  auto step = [&](const uint8_t *nxt, uint8_t *fut, int kt, const bf16x8 *fa, const bf16x8 *fb,
                  bf16x8 *na, bf16x8 *nb) {
    // Nothing moves across a step boundary: left free, the scheduler hoists
    // later steps' fragment reads and runs out of registers.
    __builtin_amdgcn_sched_barrier(0);
    // Half of the step's loads go out with the MFMAs before the barrier, half
    // with those after it, so the address unit never sees a burst; the next
    // step's fragment reads are interleaved with the MFMAs after the barrier.
    issue(kt + 3, fut, 0);
    mma(fa, fb, 0, Q);
    if constexpr (BMT == 256) {  // 16 MFMAs, 4 loads
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // global -> LDS load
      }
    } else {  // 4 MFMAs, 2 loads
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    stage_barrier<BMT>();
    rd(nxt, na, nb);
    issue(kt + 3, fut, 1);
    mma(fa, fb, Q, G::TI);
    if constexpr (BMT == 256) {  // 48 MFMAs, 16 or 24 LDS reads, 4 loads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // MFMA
        if (NRD == 24 && (i & 1))
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i % 4 == 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    } else {  // 12 MFMAs, 8 or 12 LDS reads, 2 loads
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (NRD == 12)
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (i % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
  };

  issue(0, smem0, -1);
  issue(1, smem1, -1);
  issue(2, smem2, -1);
  stage_barrier<BMT>();  // step 0 landed (12 or 6 younger loads may be in flight)
  {  // the barrier's wait covered the bias loads, which are older
#pragma unroll
    for (int j = 0; j < G::TI; ++j) {
      const f32x4 b = {bf2f(bias_v[j].x & 0xffff), bf2f(bias_v[j].x >> 16),
                       bf2f(bias_v[j].y & 0xffff), bf2f(bias_v[j].y >> 16)};
#pragma unroll
      for (int i = 0; i < G::TI; ++i) acc[i][j] = b;
    }
  }
  rd(smem0, fa0, fb0);
  for (int kt = 0; kt < KT; kt += NSTAGE) {  // KT rounds up: the extra steps are all-zero
    step(smem1, smem3, kt, fa0, fb0, fa1, fb1);
    step(smem2, smem0, kt + 1, fa1, fb1, fa0, fb0);
    step(smem3, smem1, kt + 2, fa0, fb0, fa1, fb1);
    step(smem0, smem2, kt + 3, fa1, fb1, fa0, fb0);
  }
  __syncthreads();  // every load and fragment read has finished: the stages become the C tile
  if constexpr (MODE == kGemmF32) {
    if (part) {  // one K range of a split tile: the whole tile, no bounds
      GemmArgs gp = g;
      gp.out = part;
      gp.M = gp.N = gp.ldo = BMT;
      write_f32<BMT>(acc, gp, 0, 0);
      return;
    }
  }
  uint8_t *const bufs[4] = {smem0, smem1, smem2, smem3};
  store_tile<MODE, ACT, BMT>(acc, g, m0, n0, bufs, s_dst);
}

// Tile coordinates of the quarter tiles: workgroup index q of the 128-tile
// part covers quarter q%4 of the 256-tile n_full + q/4 (the quarters of one
// 256-tile stay together), or -- when n_full == 0 -- tile q of the 128-grid.
__device__ __forceinline__ void tail_coords(const GemmArgs &g, int bid, int &tm, int &tn) {
  if (g.n_full > 0) {
    const int rem = g.tiles_m * g.tiles_n - g.n_full;
    const int q = xcd_remap(bid, 4 * rem);
    int bm, bn;
    tile_coords(g.n_full + (q >> 2), g.tiles_m, g.tiles_n, bm, bn);
    tm = 2 * bm + ((q >> 1) & 1);
    tn = 2 * bn + (q & 1);
  } else {
    const int tm128 = (g.M + 127) / 128, tn128 = (g.N + 127) / 128;
    tile_coords(xcd_remap(bid, tm128 * tn128), tm128, tn128, tm, tn);
  }
}

// One launch covers either the whole-tile part of the problem (BMT = 256:
// tiles [0, n_full) of the 256-grid), or the 128-tiles (BMT = 128: the four
// quarters of every 256-tile from n_full on, or -- when n_full == 0 -- the
// whole 128-grid).
template <int MODE, int ACT, int BMT, bool GA, bool TB>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_bf16(GemmArgs g) {
  using G = Geo<BMT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem3[G::STAGE];
  __shared__ int32_t s_dst[BMT];  // destination row per tile row
  int tm, tn;
  if (BMT == 256)
    tile_coords(whole_tile_order(blockIdx.x, g.n_full), g.tiles_m, g.tiles_n, tm, tn);
  else
    tail_coords(g, blockIdx.x, tm, tn);
  gemm_tile<MODE, ACT, BMT, GA, TB>(g, tm, tn, smem0, smem1, smem2, smem3, s_dst, 0, g.K / BK,
                                    nullptr);
}

// Both parts in one launch: workgroups [0, n_full) take the 256-tiles, the
// rest the quarter tiles.  Workgroups are dispatched in index order, so a CU
// whose last whole tile is done starts a quarter tile at once instead of
// waiting for the slowest whole tile of the launch.  n_full is a multiple of
// 256, so workgroup n_full + q still runs on XCD q % 8.
template <int MODE, int ACT, bool GA, bool TB>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_bf16_mixed(GemmArgs g) {
  using G = Geo<256>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem2[G::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t smem3[G::STAGE];
  __shared__ int32_t s_dst[256];
  int tm, tn, ks0 = 0, ksn = g.K / BK;
  float *part = nullptr;
  const int bid = static_cast<int>(blockIdx.x);
  if (bid < g.n_full) {
    tile_coords(whole_tile_order(bid, g.n_full), g.tiles_m, g.tiles_n, tm, tn);
  } else if (!GA && MODE == kGemmF32 && g.k_splits > 1) {
    // K range r of tail tile q, as a whole tile: workgroup n_full + q*S + r
    // (S = k_splits), its partial tile at split_part + (q*S + r) tiles.
    const int u = bid - g.n_full, q = u / g.k_splits, r = u - q * g.k_splits;
    tile_coords(g.n_full + q, g.tiles_m, g.tiles_n, tm, tn);
    ks0 = r * ksn / g.k_splits;
    ksn = (r + 1) * ksn / g.k_splits - ks0;
    part = g.split_part + static_cast<int64_t>(u) * (256 * 256);
  } else {
    tail_coords(g, bid - g.n_full, tm, tn);
    gemm_tile<MODE, ACT, 128, GA, TB>(g, tm, tn, smem0, smem1, smem2, smem3, s_dst, 0, ksn,
                                      nullptr);
    return;
  }
  gemm_tile<MODE, ACT, 256, GA, TB>(g, tm, tn, smem0, smem1, smem2, smem3, s_dst, ks0, ksn,
                                    part);
}

// out rows of the split tail tiles: tile q's k_splits partial tiles added in
// order (the same result every run).  Grid (64, tail tiles): a thread adds
// one float4 of the 256 x 256 tile.  Nothing is written when the placeholder
// scan failed.
__global__ __launch_bounds__(256) void k_split_sum(GemmArgs g) {
  if (g.status && g.status[kStatusWord] != 0) return;
  const int q = blockIdx.y;
  int tm, tn;
  tile_coords(g.n_full + q, g.tiles_m, g.tiles_n, tm, tn);
  const int e = blockIdx.x * 256 + threadIdx.x;  // float4 of the tile
  const int r = e >> 6, c = (e & 63) * 4;
  const int m = tm * 256 + r, n = tn * 256 + c;
  if (m >= g.M || n >= g.N) return;
  const f32x4 *p = reinterpret_cast<const f32x4 *>(g.split_part) +
                   static_cast<int64_t>(q) * g.k_splits * (256 * 64) + e;
  f32x4 acc = p[0];
  for (int k = 1; k < g.k_splits; ++k) acc += p[static_cast<int64_t>(k) * (256 * 64)];
  *reinterpret_cast<f32x4 *>(static_cast<float *>(g.out) + static_cast<int64_t>(m) * g.ldo + n) =
      acc;
}

template <int MODE, int ACT, bool GA = false, bool TB = false>
void launch_bf16(const GemmArgs &g, int blocks256, int blocks128, hipStream_t s) {
  // Whole tiles and the quarter-tile tail in one launch while the quarter
  // tiles fit one round at one per CU; beyond that the quarter-tile kernel of
  // its own (two per CU: a third of the registers and half the LDS) is faster
  // (dW1 of workload 1, 272 quarter tiles: 340 against 367 us).
  if (blocks256 > 0 && blocks128 > 0 && blocks128 <= kPlanCUs)
    hipLaunchKernelGGL((k_gemm_bf16_mixed<MODE, ACT, GA, TB>), dim3(blocks256 + blocks128),
                       dim3(NTHREADS), 0, s, g);
  else {
    if (blocks256 > 0)
      hipLaunchKernelGGL((k_gemm_bf16<MODE, ACT, 256, GA, TB>), dim3(blocks256), dim3(NTHREADS), 0,
                         s, g);
    if (blocks128 > 0)
      hipLaunchKernelGGL((k_gemm_bf16<MODE, ACT, 128, GA, TB>), dim3(blocks128), dim3(NTHREADS), 0,
                         s, g);
  }
}

template <int MODE, bool GA = false>
void launch_act(const GemmArgs &g, const TilePlan &tp, hipStream_t s) {
  if (g.act == 0)
    launch_bf16<MODE, 0, GA>(g, tp.n_full, tp.blocks128, s);
  else if (g.act == 1)
    launch_bf16<MODE, 1, GA>(g, tp.n_full, tp.blocks128, s);
  else
    launch_bf16<MODE, 2, GA>(g, tp.n_full, tp.blocks128, s);
}

}  // namespace

hipError_t launch_gemm_bf16(int mode, GemmArgs g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K % BK != 0) return hipErrorInvalidValue;
  const TilePlan tp = tile_plan(g.M, g.N);
  g.tiles_m = tp.tiles_m;
  g.tiles_n = tp.tiles_n;
  g.n_full = tp.n_full;
  // Token-major B: the saved activations in the weight-gradient products, a
  // packed weight read transposed in the products with a weight.
  if (g.b_tmaj && g.tb_w % BK) return hipErrorInvalidValue;
  switch (mode) {
    case kGemmBlocked:
      if (g.b_tmaj && g.act == 2)
        launch_bf16<kGemmBlocked, 2, false, true>(g, tp.n_full, tp.blocks128, s);
      else if (!g.b_tmaj)
        launch_act<kGemmBlocked>(g, tp, s);
      else
        return hipErrorInvalidValue;
      break;
    case kGemmGatherBlocked:  // A gathered from the grid through g.desc
      if (!g.desc || g.C % BK || g.k < 1 || g.k > 3 || g.b_tmaj) return hipErrorInvalidValue;
      launch_act<kGemmBlocked, true>(g, tp, s);
      break;
    case kGemmBlockedSave:
      if (!g.out2 || g.b_tmaj) return hipErrorInvalidValue;
      launch_act<kGemmBlockedSave>(g, tp, s);
      break;
    case kGemmRows:  // no activation
      if (g.act != 2) return hipErrorInvalidValue;
      if (g.b_tmaj)
        launch_bf16<kGemmRows, 2, false, true>(g, tp.n_full, tp.blocks128, s);
      else
        launch_bf16<kGemmRows, 2>(g, tp.n_full, tp.blocks128, s);
      break;
    case kGemmF32: {  // no bias, no activation
      if (g.act != 2 || g.N % 4 || g.ldo % 4) return hipErrorInvalidValue;
      const int S = g.split_part ? gemm_k_splits(tp, g.K) : 1;
      g.k_splits = S;
      if (S > 1) {  // whole tiles and the split tail in one launch, then the sums
        const int rem = tp.tiles_m * tp.tiles_n - tp.n_full;
        if (g.b_tmaj)
          hipLaunchKernelGGL((k_gemm_bf16_mixed<kGemmF32, 2, false, true>),
                             dim3(tp.n_full + rem * S), dim3(NTHREADS), 0, s, g);
        else
          hipLaunchKernelGGL((k_gemm_bf16_mixed<kGemmF32, 2, false, false>),
                             dim3(tp.n_full + rem * S), dim3(NTHREADS), 0, s, g);
        hipLaunchKernelGGL(k_split_sum, dim3(64, rem), dim3(256), 0, s, g);
      } else if (g.b_tmaj) {
        launch_bf16<kGemmF32, 2, false, true>(g, tp.n_full, tp.blocks128, s);
      } else {
        launch_bf16<kGemmF32, 2>(g, tp.n_full, tp.blocks128, s);
      }
      break;
    }
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {

// ---------------------------------------------------------------------------
// fp32 path: 64x64 tile, 16 K per stage, 4x4 outputs per thread, plain FMA.
// In gather mode K runs in the pages' feature order c*k*k + dy*k + dx and each
// A element is fetched from its pixel (zero in the padding).  Otherwise A and
// B are read through strides (GemmArgs::sa_m ...; zero strides mean row-major
// [M][K] and [N][K]), so the backward's products read transposed operands in
// place.  A null bias counts as zero; with out2 the pre-activation is written
// there as well (row-major, ldo); a set status word skips the output.
constexpr int FT = 64, FK = 16;

template <bool GATHER>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  if (g.status && g.status[kStatusWord] != 0) return;
  const int tid = threadIdx.x;
  const int64_t sam = g.sa_k ? g.sa_m : g.K, sak = g.sa_k ? g.sa_k : 1;
  const int64_t sbn = g.sb_k ? g.sb_n : g.K, sbk = g.sb_k ? g.sb_k : 1;
  const int tm = blockIdx.x / g.tiles_n, tn = blockIdx.x % g.tiles_n;
  const int m0 = tm * FT, n0 = tn * FT;
  const float *A = static_cast<const float *>(g.A);
  const float *B = static_cast<const float *>(g.B);
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  const int kk2 = g.k * g.k;
  for (int k0 = 0; k0 < g.K; k0 += FK) {
    for (int e = tid; e < FT * FK; e += 256) {
      const int r = e / FK, kq = e % FK;
      const int m = m0 + r, kidx = k0 + kq;
      float v = 0.f;
      if (m < g.M && kidx < g.K) {
        if (GATHER) {
          const RowDesc d = g.desc[m];
          const int c = kidx / kk2, p = kidx - c * kk2;
          const int dy = p / g.k, dx = p - dy * g.k;
          if ((d.geo >> (16 + p)) & 1)
            v = A[static_cast<int64_t>(d.pix + dy * (d.geo & 0xffff) + dx) * g.C + c];
        } else {
          v = A[m * sam + kidx * sak];
        }
      }
      As[kq][r] = v;
      const int n = n0 + r;
      Bs[kq][r] = (n < g.N && kidx < g.K) ? B[n * sbn + kidx * sbk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < FK; ++kq) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kq][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kq][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const float *bias = static_cast<const float *>(g.bias);
  float *out = static_cast<float *>(g.out);
  float *out2 = static_cast<float *>(g.out2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    const int dst = g.dst_row ? g.dst_row[m] : m;
    if (dst < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < g.N) {
        const float z = acc[i][j] + (bias ? bias[n] : 0.f);
        out[static_cast<int64_t>(dst) * g.ldo + n] = activate(z, g.act);
        if (out2) out2[static_cast<int64_t>(dst) * g.ldo + n] = z;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(bool gather, GemmArgs g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  g.tiles_m = (g.M + FT - 1) / FT;
  g.tiles_n = (g.N + FT - 1) / FT;
  const dim3 grid(g.tiles_m * g.tiles_n);
  if (gather)
    hipLaunchKernelGGL(k_gemm_f32<true>, grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(k_gemm_f32<false>, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace vlb
