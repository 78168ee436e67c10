// GEMM kernels of the bridge projector: Linear(C*k*k -> hidden) + bias + GELU
// fed by the space-to-depth gather, and Linear(hidden -> out) + bias whose
// epilogue writes each row to its destination (a row of the output, or its
// placeholder slot in the sequence).  mlxcel issue #533 "port DeepSeek-VL2",
// section "Projector (downsample_mlp_gelu)" steps 1-3.
//
// bf16 path (gfx950): 256x256 output tile per 256-thread workgroup, 4 waves in
// a 2x2 grid, each wave 128x128 from 4x4 v_mfma_f32_32x32x16_bf16 tiles with
// fp32 accumulation.  K advances 64 per stage through two LDS stages of
// 64 KiB (A and B, 128-byte rows, 16-byte chunks XOR-swizzled by row); the
// next stage's global loads are in flight while the current one is consumed.
// In gather mode the A rows come straight from the channels-last patch grid:
// with K ordered position-major (k' = p*C + c, the packed W1) every 64-wide K
// slice is 64 contiguous channels of one pixel, so each row of an A stage is
// one 128-byte load -- the merged tensor is never materialised.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlb_common.h"
#include "vlb_internal.h"

namespace vlb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int A_BYTES = BM * BK * 2;
constexpr int B_BYTES = BN * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 8;

// Workgroup -> output tile.  Workgroups are dealt round-robin to the 8 XCDs, so
// workgroup b runs on XCD b % 8; each XCD is given a contiguous range of
// logical tiles, and logical tiles are ordered in groups of GROUP_M tile-rows,
// column by column, so the tiles an XCD runs together share A and B panels in
// its L2.
__device__ __forceinline__ void map_tile(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nblk = tiles_m * tiles_n;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int span = GROUP_M * tiles_n;
  const int group = logical / span;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * span;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` inside a stage
// half: 128-byte rows, chunk XOR-swizzled with bits 1..3 of the row so that 16
// consecutive rows reading the same logical chunk hit distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

template <bool GATHER>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int tm, tn;
  map_tile(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint16_t *A = static_cast<const uint16_t *>(g.A);
  const uint16_t *B = static_cast<const uint16_t *>(g.B);

  // Loader role: chunk lc of rows lr + 32*i (i < 8) of both A and B stages.
  const int lc = tid & 7, lr = tid >> 3;
  int32_t a_base[8], a_geo[8], b_base[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + lr + 32 * i;
    if (GATHER) {
      RowDesc d = {0, 0};
      if (m < g.M) d = g.desc[m];
      a_base[i] = d.pix;
      a_geo[i] = d.geo;  // 0 for rows past M: every position reads as padding
    } else {
      a_base[i] = m < g.M ? m * g.K : -1;
      a_geo[i] = 0;
    }
    const int n = n0 + lr + 32 * i;
    b_base[i] = n < g.N ? n * g.K : -1;
  }

  uint4 ra[8], rb[8];
  auto gload = [&](int kt) {
    const int kk = kt * BK;
    if (GATHER) {
      const int p = kk / g.C, c0 = kk - p * g.C;
      const int dy = p / g.k, dx = p - dy * g.k;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gw = a_geo[i] & 0xffff;
        const bool in = (a_geo[i] >> (16 + p)) & 1;
        ra[i] = make_uint4(0, 0, 0, 0);
        if (in)
          ra[i] = *reinterpret_cast<const uint4 *>(A + (a_base[i] + dy * gw + dx) * g.C + c0 +
                                                   lc * 8);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = make_uint4(0, 0, 0, 0);
        if (a_base[i] >= 0)
          ra[i] = *reinterpret_cast<const uint4 *>(A + a_base[i] + kk + lc * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rb[i] = make_uint4(0, 0, 0, 0);
      if (b_base[i] >= 0) rb[i] = *reinterpret_cast<const uint4 *>(B + b_base[i] + kk + lc * 8);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t *sa = smem + stage * STAGE_BYTES;
    uint8_t *sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = lr + 32 * i;
      *reinterpret_cast<uint4 *>(sa + swz(row, lc)) = ra[i];
      *reinterpret_cast<uint4 *>(sb + swz(row, lc)) = rb[i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int wm = wid >> 1, wn = wid & 1;
  const int fr = lane & 31, fk = lane >> 5;  // fragment row / k-half of this lane
  const int KT = g.K / BK;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t *sa = smem + cur * STAGE_BYTES;
    const uint8_t *sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 af[4], bfg[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = *reinterpret_cast<const bf16x8 *>(sa + swz(wm * 128 + t * 32 + fr, ks * 2 + fk));
        bfg[t] = *reinterpret_cast<const bf16x8 *>(sb + swz(wn * 128 + t * 32 + fr, ks * 2 + fk));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column fr of each 32x32 tile and rows
  // 8*(q/4) + 4*fk + q%4 (q < 16).
  const uint16_t *bias = static_cast<const uint16_t *>(g.bias);
  uint16_t *out = static_cast<uint16_t *>(g.out);
  float bv[4];
  int col[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    col[j] = n0 + wn * 128 + j * 32 + fr;
    bv[j] = col[j] < g.N ? bf2f(bias[col[j]]) : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (q >> 2) + 4 * fk + (q & 3);
      if (m >= g.M) continue;
      const int dst = g.dst_row ? g.dst_row[m] : m;
      if (dst < 0) continue;
      uint16_t *orow = out + static_cast<int64_t>(dst) * g.ldo;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (col[j] < g.N) orow[col[j]] = f2bf(activate(acc[i][j][q] + bv[j], g.act));
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: 64x64 tile, 16 K per stage, 4x4 outputs per thread, plain FMA.
// In gather mode K runs in the pages' feature order c*k*k + dy*k + dx and each
// A element is fetched from its pixel (zero in the padding).
constexpr int FT = 64, FK = 16;

template <bool GATHER>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  const int tid = threadIdx.x;
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
          v = A[static_cast<int64_t>(m) * g.K + kidx];
        }
      }
      As[kq][r] = v;
      const int n = n0 + r;
      Bs[kq][r] = (n < g.N && kidx < g.K) ? B[static_cast<int64_t>(n) * g.K + kidx] : 0.f;
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    const int dst = g.dst_row ? g.dst_row[m] : m;
    if (dst < 0) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < g.N)
        out[static_cast<int64_t>(dst) * g.ldo + n] = activate(acc[i][j] + bias[n], g.act);
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(bool gather, GemmArgs g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + BN - 1) / BN;
  const dim3 grid(g.tiles_m * g.tiles_n);
  if (gather)
    hipLaunchKernelGGL(k_gemm_bf16<true>, grid, dim3(NTHREADS), 0, s, g);
  else
    hipLaunchKernelGGL(k_gemm_bf16<false>, grid, dim3(NTHREADS), 0, s, g);
  return hipGetLastError();
}

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
