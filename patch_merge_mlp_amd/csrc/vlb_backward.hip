// Kernels of the projector's backward pass (bf16), besides the GEMMs.
//
// The projector is the bridge's trained part ("DeepSeek-V4-Flash-Vision-BF16"
// model card, header: only its parameters are trained, tower and text model
// frozen; "La voie visuelle", "Pendant le pré-entraînement du squelette": the
// projector stays trainable).  Its gradients are the chain rule through the
// forward of mlxcel issue #533 "port DeepSeek-VL2", "Projector
// (downsample_mlp_gelu)" steps 1-3 and "Tile-sequence assembly":
//   dY = gradient rows gathered from the sequence's placeholder slots
//   dW2 = dY^T act(Z1), db2 = sum dY, dA1 = dY W2
//   dZ1 = dA1 * act'(Z1), db1 = sum dZ1, dW1 = dZ1^T Xm, dXm = dZ1 W1
//   dXm unmerged to pixels, then through the LayerNorm.
//
// The four products run on the MFMA GEMM, which contracts over the 32-wide K
// slices of tile-blocked operands (element (r, c) of [R][K] at
// ((r/256 * K/32 + c/32) * 256 + r%256) * 32 + c%32).  Its B operand may also
// be token-major (the saved activations, the packed weights), read through
// LDS transpose reads; the A operands of the weight gradients, dY^T and
// dZ^T, are written here by the kernels that produce dY and dZ anyway, and
// Xm^T (dW1's B, rows in the pages' feature order) by a pass of its own: a
// workgroup takes 32 consecutive rows t (one K slice of the transposed
// operand) and 256 columns, stages them in LDS, and writes each column's 32
// values as one contiguous 64-byte piece -- 256 such pieces are one 16 KiB
// run.  Rows past T are zero, so the padded part of every contraction over T
// adds nothing.  Column sums (the bias gradients) are written per 32-row
// slice and reduced in a fixed order, so every gradient is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vlb_common.h"
#include "vlb_internal.h"

namespace vlb {

namespace {

constexpr int kTR = 32;            // rows t per workgroup (one K slice)
constexpr int kTC = 256;           // columns per workgroup
constexpr int kPitch = kTC + 8;    // LDS row pitch in bf16 (16-byte aligned rows)
constexpr int kPackIters = kTR * (kTC / 8) / 256;  // 16-byte pieces per thread (256 threads)
static_assert(kPackIters * 256 == kTR * (kTC / 8), "a tile is a whole number of pieces per thread");

__device__ __forceinline__ int64_t blk(int64_t r, int64_t c, int64_t K) {
  return ((r >> 8) * (K >> 5) + (c >> 5)) * 8192 + (r & 255) * 32 + (c & 31);
}

// d/dz of act_fn<ACT>, in fp32.
//   erf form: Phi(z) + z phi(z), with Phi from the forward's tail
//   (gauss_tail: Phi(-a) = 2^(-h(a))) and phi(z) = exp(-z^2/2) / sqrt(2 pi);
//   tanh form: 0.5 (1 + th) + 0.5 z (1 - th^2) sqrt(2/pi) (1 + 3 * 0.044715 z^2).
template <int ACT>
__device__ __forceinline__ float act_slope(float z) {
  if constexpr (ACT == 0) {
    const float tail = gauss_tail(z);  // Phi(-|z|)
    const float cdf = z >= 0.f ? 1.0f - tail : tail;
    const float pdf = 0.39894228040143268f * __builtin_amdgcn_exp2f(-0.72134752044448170f * z * z);
    return fmaf(z, pdf, cdf);
  } else if constexpr (ACT == 1) {
    const float k0 = 0.79788456080286536f;
    const float u = k0 * (z + 0.044715f * z * z * z);
    const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2f(2.0f * 1.4426950408889634f * u) + 1.0f);
    return 0.5f * (1.0f + th) + 0.5f * z * (1.0f - th * th) * k0 * (1.0f + 3.0f * 0.044715f * z * z);
  } else {
    return 1.0f;
  }
}

// Column r of the staged 32 x 256 tile as one 64-byte piece of the
// transposed operand.
__device__ __forceinline__ void store_column(const uint16_t *tile, int r, uint16_t *dst) {
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    w[i] = tile[(2 * i) * kPitch + r] | (static_cast<uint32_t>(tile[(2 * i + 1) * kPitch + r]) << 16);
  uint4 *d = reinterpret_cast<uint4 *>(dst);
#pragma unroll
  for (int q = 0; q < 4; ++q) d[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// Columns [0, ncol) of the staged 32 x 256 tile when they map to consecutive
// rows of the transposed operand (the tile's first column a multiple of 256,
// its first row of 32): their pieces are one contiguous run from dst, 64
// bytes each.  Lane -> (column, 16-byte chunk), so each store instruction of a
// wave writes 16 whole pieces, one contiguous KiB.
__device__ __forceinline__ void store_columns(const uint16_t *tile, int ncol, uint16_t *dst) {
#pragma unroll
  for (int u = threadIdx.x; u < kTC * 4; u += 256) {
    const int col = u >> 2, ch = u & 3;
    if (col >= ncol) continue;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ch * 8 + 2 * i;
      w[i] = tile[r * kPitch + col] | (static_cast<uint32_t>(tile[(r + 1) * kPitch + col]) << 16);
    }
    *reinterpret_cast<uint4 *>(dst + col * 32 + ch * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ float col_sum(const uint16_t *tile, int r) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kTR; ++i) s += bf2f(tile[i * kPitch + r]);
  return s;
}

// Gradient rows of the token rows: dY[t] = G[dst_row[t]] (zero for t >= T or
// an unplaced row).  Writes dY tile-blocked [T][Op] (K = Op, zero past O),
// its transpose [O][Tk], and per-slice column sums part[t/32][o].
__global__ __launch_bounds__(256) void k_bwd_gather_dy(const uint16_t *G, const int32_t *dst_row,
                                                       int32_t T, int32_t O, int32_t Op,
                                                       int32_t Tk, uint16_t *dy, uint16_t *dyt,
                                                       float *part) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTR * kPitch];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTR, n0 = blockIdx.y * kTC;
  // Each thread moves kPackIters 16-byte pieces; all their loads go out before
  // the first is used (the destination rows first, then the gradient rows).
  int32_t d[kPackIters];
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, row = q >> 5, o = n0 + (q & 31) * 8;
    d[i] = (t0 + row < T && o < O) ? dst_row[t0 + row] : -1;
  }
  uint4 v[kPackIters];
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, o = n0 + (q & 31) * 8;
    v[i] = d[i] >= 0 ? load_nt(reinterpret_cast<const uint4 *>(G + static_cast<int64_t>(d[i]) * O + o))
                     : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i;
    *reinterpret_cast<uint4 *>(tile + (q >> 5) * kPitch + (q & 31) * 8) = v[i];
  }
  __syncthreads();
  for (int q = tid; q < kTR * (kTC / 8); q += 256) {  // dY: 8 slices of 32 rows x 64 bytes
    const int sl = q >> 7, row = (q >> 2) & 31, c4 = q & 3;
    const int o = n0 + sl * 32 + c4 * 8;
    if (o < Op)
      *reinterpret_cast<uint4 *>(dy + blk(t0 + row, o, Op)) =
          *reinterpret_cast<const uint4 *>(tile + row * kPitch + sl * 32 + c4 * 8);
  }
  store_columns(tile, min(kTC, O - n0), dyt + blk(n0, t0, Tk));
  const int o = n0 + tid;
  if (o < O) part[static_cast<int64_t>(blockIdx.x) * O + o] = col_sum(tile, tid);
}

// dZ1 = dA1 * act'(Z1) (both tile-blocked [T][H]): dZ1 tile-blocked, its
// transpose [H][Tk], and per-slice column sums of the rounded values (the
// values dW1 and dXm are computed from).
template <int ACT>
__global__ __launch_bounds__(256) void k_bwd_dact(const uint16_t *da1, const uint16_t *z1,
                                                  int32_t T, int32_t H, int32_t Tk, uint16_t *dz1,
                                                  uint16_t *dz1t, float *part) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTR * kPitch];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTR, n0 = blockIdx.y * kTC;
  uint4 a[kPackIters], z[kPackIters];  // all loads out before the first is used
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, sl = q >> 7, row = (q >> 2) & 31, c4 = q & 3;
    const int t = t0 + row, h = n0 + sl * 32 + c4 * 8;
    const bool in = t < T && h < H;
    const int64_t e = in ? blk(t, h, H) : 0;
    a[i] = in ? *reinterpret_cast<const uint4 *>(da1 + e) : make_uint4(0, 0, 0, 0);
    z[i] = in ? *reinterpret_cast<const uint4 *>(z1 + e) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, sl = q >> 7, row = (q >> 2) & 31, c4 = q & 3;
    const int t = t0 + row, h = n0 + sl * 32 + c4 * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (t < T && h < H) {
      const uint16_t *ae = reinterpret_cast<const uint16_t *>(&a[i]);
      const uint16_t *ze = reinterpret_cast<const uint16_t *>(&z[i]);
      uint16_t *ve = reinterpret_cast<uint16_t *>(&v);
#pragma unroll
      for (int j = 0; j < 8; ++j) ve[j] = f2bf(bf2f(ae[j]) * act_slope<ACT>(bf2f(ze[j])));
      *reinterpret_cast<uint4 *>(dz1 + blk(t, h, H)) = v;
    }
    *reinterpret_cast<uint4 *>(tile + row * kPitch + sl * 32 + c4 * 8) = v;
  }
  __syncthreads();
  store_columns(tile, min(kTC, H - n0), dz1t + blk(n0, t0, Tk));
  const int h = n0 + tid;
  if (h < H) part[static_cast<int64_t>(blockIdx.x) * H + h] = col_sum(tile, tid);
}

// Xm (tile-blocked [T][K1], K position-major j = p*C + c) -> its transpose
// with rows in the pages' feature order c*k*k + p: [K1][Tk].
__global__ __launch_bounds__(256) void k_bwd_xm_t(const uint16_t *xm, int32_t T, int32_t K1,
                                                  int32_t C, int32_t kk, int32_t Tk,
                                                  uint16_t *xmt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTR * kPitch];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTR, n0 = blockIdx.y * kTC;
  uint4 v[kPackIters];  // all loads out before the first is used
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, sl = q >> 7, row = (q >> 2) & 31, c4 = q & 3;
    const int t = t0 + row, j = n0 + sl * 32 + c4 * 8;
    v[i] = (t < T && j < K1) ? load_nt(reinterpret_cast<const uint4 *>(xm + blk(t, j, K1))) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < kPackIters; ++i) {
    const int q = tid + 256 * i, sl = q >> 7, row = (q >> 2) & 31, c4 = q & 3;
    *reinterpret_cast<uint4 *>(tile + row * kPitch + sl * 32 + c4 * 8) = v[i];
  }
  __syncthreads();
  const int j = n0 + tid;
  if (j < K1) store_column(tile, tid, xmt + blk(static_cast<int64_t>(j % C) * kk + j / C, t0, Tk));
}

// Feature gradient of the pixels of one chunk of views (see PlanChunk), one
// wave per (token row, block position): the pixel's slice dn = dXm[m][p*C ..
// p*C + C) (row-major, K position-major) goes back through the LayerNorm,
//   xh = (x - mean) * rstd, g = gamma * dn,
//   dx = rstd * (g - mean(g) - xh * mean(g * xh)),
// recomputing mean and rstd from the pixel as the forward did; without the
// LayerNorm dx = dn.  Positions in the padding are skipped.  Each workgroup
// adds its pixels' dn * xh and dn into one row of part_g / part_b (waves in
// order), so the parameter gradients come out the same on every run.  Nothing
// is written when the placeholder scan failed.
constexpr int kUmWaves = 4;  // waves per workgroup of the unmerge kernel

template <bool LN, int NCH>
__global__ __launch_bounds__(64 * kUmWaves) void k_bwd_unmerge(const uint16_t *dxm, const uint16_t *x,
                                                     PlanChunk c, int C, const uint16_t *gamma,
                                                     float eps, uint16_t *dx, float *part_g,
                                                     float *part_b, const int32_t *status) {
  if (status[kStatusWord] != 0) return;
  extern __shared__ float red[];  // [2][C] workgroup sums, then (LN) gamma as bf16 [C]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = c.k, kk = k * k, nch = C / 8;
  const int64_t K1 = static_cast<int64_t>(C) * kk;
  const int32_t t_begin = c.tok0[0], t_end = c.tok0[c.n];
  const int64_t items = static_cast<int64_t>(t_end - t_begin) * kk;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kUmWaves;
  // View table: every lane loads its entry (64 of them), entries past n masked.
  const bool have = lane < c.n;
  const int32_t e_tok0 = c.tok0[lane], e_pix0 = c.pix0[lane];
  const int32_t e_gh = c.gh[lane], e_gw = c.gw[lane];
  const int32_t l_tok0 = have ? e_tok0 : INT32_MAX;
  const int32_t l_pix0 = have ? e_pix0 : 0;
  const int32_t l_gh = have ? e_gh : 0, l_gw = have ? e_gw : 1;
  const uint4 *s_gamma = reinterpret_cast<const uint4 *>(red + 2 * C);
  if (LN) {  // gamma is read for every pixel: once into LDS
    for (int q = threadIdx.x; q < nch; q += 64 * kUmWaves)
      reinterpret_cast<uint4 *>(red + 2 * C)[q] = reinterpret_cast<const uint4 *>(gamma)[q];
    __syncthreads();
  }
  // Item it = (token row, k x k position): its dXm segment and its pixel, or
  // false for a padded cell (no pixel).  Wave-uniform.
  auto locate = [&](int64_t it, int64_t &drow, int64_t &pix) -> bool {
    const int m = t_begin + static_cast<int>(it / kk), p = static_cast<int>(it % kk);
    const int v = __popcll(__ballot(l_tok0 <= m)) - 1;
    const int tok0 = __shfl(l_tok0, v), pix0 = __shfl(l_pix0, v);
    const int gh = __shfl(l_gh, v), gw = __shfl(l_gw, v);
    const int wp = (gw + k - 1) / k, t = m - tok0;
    const int y = (t / wp) * k + p / k, xx = (t % wp) * k + p % k;
    if (y >= gh || xx >= gw) return false;
    pix = pix0 + static_cast<int64_t>(y) * gw + xx;
    drow = m * K1 + static_cast<int64_t>(p) * C;
    return true;
  };
  auto fetch = [&](int64_t drow, int64_t pix, uint4 (&dv)[NCH], uint4 (&xv)[NCH]) {
    const uint4 *dsrc = reinterpret_cast<const uint4 *>(dxm + drow);
    const uint4 *xs = reinterpret_cast<const uint4 *>(x + pix * C);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      dv[i] = q < nch ? load_nt(dsrc + q) : make_uint4(0, 0, 0, 0);  // both read once
      if (LN) xv[i] = q < nch ? load_nt(xs + q) : make_uint4(0, 0, 0, 0);
    }
  };
  float ag[NCH][8], ab[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[i][e] = ab[i][e] = 0.f;
  int64_t it = static_cast<int64_t>(blockIdx.x) * kUmWaves + wid;
  int64_t drow = 0, pix = 0;
  bool ok = it < items && locate(it, drow, pix);
  uint4 dv[NCH] = {}, xv[NCH] = {};
  if (ok) fetch(drow, pix, dv, xv);
  for (; it < items; it += nw) {
    // The next item's loads go out before this item's arithmetic.
    int64_t drow2 = 0, pix2 = 0;
    const bool ok2 = it + nw < items && locate(it + nw, drow2, pix2);
    uint4 dv2[NCH] = {}, xv2[NCH] = {};
    if (ok2) fetch(drow2, pix2, dv2, xv2);
    if (ok) {
      uint4 *ddst = dx ? reinterpret_cast<uint4 *>(dx + pix * C) : nullptr;
      if (!LN) {
        if (ddst) {
#pragma unroll
          for (int i = 0; i < NCH; ++i)
            if (lane + 64 * i < nch) ddst[lane + 64 * i] = dv[i];
        }
      } else {
        float xf[NCH][8];
        float sum = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const uint16_t *e = reinterpret_cast<const uint16_t *>(&xv[i]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            xf[i][j] = bf2f(e[j]);
            sum += xf[i][j];
          }
        }
        const float mean = wave_sum(sum) / C;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i)
          if (lane + 64 * i < nch)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float d = xf[i][j] - mean;
              ss += d * d;
            }
        const float rstd = 1.0f / sqrtf(wave_sum(ss) / C + eps);
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int q = lane + 64 * i;
          const uint4 gq = q < nch ? s_gamma[q] : make_uint4(0, 0, 0, 0);
          const uint16_t *ge = reinterpret_cast<const uint16_t *>(&gq);
          const uint16_t *de = reinterpret_cast<const uint16_t *>(&dv[i]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float xh = (xf[i][j] - mean) * rstd, dn = bf2f(de[j]);
            const float gv = bf2f(ge[j]) * dn;
            xf[i][j] = xh;
            ag[i][j] += dn * xh;
            ab[i][j] += dn;
            sg += gv;
            sgx += gv * xh;
          }
        }
        const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
        if (ddst) {
#pragma unroll
          for (int i = 0; i < NCH; ++i) {
            const int q = lane + 64 * i;
            if (q < nch) {
              const uint4 gq = s_gamma[q];
              const uint16_t *ge = reinterpret_cast<const uint16_t *>(&gq);
              const uint16_t *de = reinterpret_cast<const uint16_t *>(&dv[i]);
              uint4 o;
              uint16_t *oe = reinterpret_cast<uint16_t *>(&o);
#pragma unroll
              for (int j = 0; j < 8; ++j)
                oe[j] = f2bf(rstd * (bf2f(ge[j]) * bf2f(de[j]) - mg - xf[i][j] * mgx));
              ddst[q] = o;
            }
          }
        }
      }
    }
    ok = ok2;
    pix = pix2;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      dv[i] = dv2[i];
      xv[i] = xv2[i];
    }
  }
  if (!LN) return;
  // Workgroup sum of the waves' accumulators, wave 0 first, then one row each.
  for (int w = 0; w < kUmWaves; ++w) {
    if (wid == w) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = lane + 64 * i;
        if (q < nch)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int ch = q * 8 + j;
            red[ch] = (w == 0 ? 0.f : red[ch]) + ag[i][j];
            red[C + ch] = (w == 0 ? 0.f : red[C + ch]) + ab[i][j];
          }
      }
    }
    __syncthreads();
  }
  for (int ch = threadIdx.x; ch < C; ch += 64 * kUmWaves) {
    part_g[static_cast<int64_t>(blockIdx.x) * C + ch] = red[ch];
    part_b[static_cast<int64_t>(blockIdx.x) * C + ch] = red[C + ch];
  }
}

// The LayerNorm form of k_bwd_unmerge at C = 128 * ND (768, 1152, 1280):
// one dword (two channels) per lane and step, so every lane holds channels
// (16-byte chunks leave lanes idle in the last step at these C).  Same
// contract, items and order of the parameter-gradient sums.  gamma is staged
// in fp32; g = gamma * dn is kept for the output, which is written as
// rstd * g - rstd * mean(g) - rstd * mean(g * xh) * xh with two fmas.
template <int ND>
__global__ __launch_bounds__(64 * kUmWaves) void k_bwd_unmerge_dw(
    const uint16_t *dxm, const uint16_t *x, PlanChunk c, float eps, const uint16_t *gamma,
    uint16_t *dx, float *part_g, float *part_b, const int32_t *status) {
  if (status[kStatusWord] != 0) return;
  constexpr int ndw = 64 * ND;  // dwords per pixel
  constexpr int C = 2 * ndw;
  constexpr float inv_c = 1.0f / static_cast<float>(C);
  extern __shared__ float red[];  // [2][C] workgroup sums, then gamma as fp32 [C]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = c.k, kk = k * k;
  const int64_t K1 = static_cast<int64_t>(C) * kk;
  const int32_t t_begin = c.tok0[0], t_end = c.tok0[c.n];
  const int64_t items = static_cast<int64_t>(t_end - t_begin) * kk;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kUmWaves;
  const bool have = lane < c.n;
  const int32_t e_tok0 = c.tok0[lane], e_pix0 = c.pix0[lane];
  const int32_t e_gh = c.gh[lane], e_gw = c.gw[lane];
  const int32_t l_tok0 = have ? e_tok0 : INT32_MAX;
  const int32_t l_pix0 = have ? e_pix0 : 0;
  const int32_t l_gh = have ? e_gh : 0, l_gw = have ? e_gw : 1;
  float2 *s_gamma = reinterpret_cast<float2 *>(red + 2 * C);
  for (int q = threadIdx.x; q < ndw; q += 64 * kUmWaves) {
    const uint32_t g = reinterpret_cast<const uint32_t *>(gamma)[q];
    s_gamma[q] = make_float2(__uint_as_float(g << 16), __uint_as_float(g & 0xffff0000u));
  }
  __syncthreads();
  auto locate = [&](int64_t it, int64_t &drow, int64_t &pix) -> bool {
    const int m = t_begin + static_cast<int>(it / kk), p = static_cast<int>(it % kk);
    const int v = __popcll(__ballot(l_tok0 <= m)) - 1;
    const int tok0 = __shfl(l_tok0, v), pix0 = __shfl(l_pix0, v);
    const int gh = __shfl(l_gh, v), gw = __shfl(l_gw, v);
    const int wp = (gw + k - 1) / k, t = m - tok0;
    const int y = (t / wp) * k + p / k, xx = (t % wp) * k + p % k;
    if (y >= gh || xx >= gw) return false;
    pix = pix0 + static_cast<int64_t>(y) * gw + xx;
    drow = m * K1 + static_cast<int64_t>(p) * C;
    return true;
  };
  auto fetch = [&](int64_t drow, int64_t pix, uint32_t (&dv)[ND], uint32_t (&xv)[ND]) {
    const uint32_t *dsrc = reinterpret_cast<const uint32_t *>(dxm + drow);
    const uint32_t *xs = reinterpret_cast<const uint32_t *>(x + pix * C);
#pragma unroll
    for (int i = 0; i < ND; ++i) {  // both read once
      dv[i] = load_nt(dsrc + lane + 64 * i);
      xv[i] = load_nt(xs + lane + 64 * i);
    }
  };
  float ag[ND][2], ab[ND][2];
#pragma unroll
  for (int i = 0; i < ND; ++i) ag[i][0] = ag[i][1] = ab[i][0] = ab[i][1] = 0.f;
  int64_t it = static_cast<int64_t>(blockIdx.x) * kUmWaves + wid;
  int64_t drow = 0, pix = 0;
  bool ok = it < items && locate(it, drow, pix);
  uint32_t dv[ND] = {}, xv[ND] = {};
  if (ok) fetch(drow, pix, dv, xv);
  for (; it < items; it += nw) {
    // The next item's loads go out before this item's arithmetic.
    int64_t drow2 = 0, pix2 = 0;
    const bool ok2 = it + nw < items && locate(it + nw, drow2, pix2);
    uint32_t dv2[ND] = {}, xv2[ND] = {};
    if (ok2) fetch(drow2, pix2, dv2, xv2);
    if (ok) {
      float xl[ND], xh[ND];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        xl[i] = __uint_as_float(xv[i] << 16);
        xh[i] = __uint_as_float(xv[i] & 0xffff0000u);
        sum += xl[i] + xh[i];
      }
      const float mean = wave_sum(sum) * inv_c;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        xl[i] -= mean;
        xh[i] -= mean;
        ss = fmaf(xl[i], xl[i], ss);
        ss = fmaf(xh[i], xh[i], ss);
      }
      const float rstd = rsqrtf(wave_sum(ss) * inv_c + eps);
      float gl[ND], gh[ND];
      float sg = 0.f, sgx = 0.f;
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const float2 g = s_gamma[lane + 64 * i];
        const float dl = __uint_as_float(dv[i] << 16), dh = __uint_as_float(dv[i] & 0xffff0000u);
        xl[i] *= rstd;  // xh, the normalised pixel
        xh[i] *= rstd;
        ag[i][0] = fmaf(dl, xl[i], ag[i][0]);
        ag[i][1] = fmaf(dh, xh[i], ag[i][1]);
        ab[i][0] += dl;
        ab[i][1] += dh;
        gl[i] = g.x * dl;
        gh[i] = g.y * dh;
        sg += gl[i] + gh[i];
        sgx = fmaf(gl[i], xl[i], sgx);
        sgx = fmaf(gh[i], xh[i], sgx);
      }
      if (dx) {
        const float b = rstd * (wave_sum(sg) * inv_c), a = rstd * (wave_sum(sgx) * inv_c);
        uint32_t *ddst = reinterpret_cast<uint32_t *>(dx + pix * C);
#pragma unroll
        for (int i = 0; i < ND; ++i)
          ddst[lane + 64 * i] = f2bf2(fmaf(-a, xl[i], fmaf(rstd, gl[i], -b)),
                                      fmaf(-a, xh[i], fmaf(rstd, gh[i], -b)));
      }
    }
    ok = ok2;
    pix = pix2;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dv[i] = dv2[i];
      xv[i] = xv2[i];
    }
  }
  // Workgroup sum of the waves' accumulators, wave 0 first, then one row each.
  float2 *r2 = reinterpret_cast<float2 *>(red);  // channel pairs: [C/2] gamma, [C/2] beta
  for (int w = 0; w < kUmWaves; ++w) {
    if (wid == w) {
#pragma unroll
      for (int i = 0; i < ND; ++i) {
        const int q = lane + 64 * i;
        const float2 pg = w == 0 ? make_float2(0.f, 0.f) : r2[q];
        const float2 pb = w == 0 ? make_float2(0.f, 0.f) : r2[ndw + q];
        r2[q] = make_float2(pg.x + ag[i][0], pg.y + ag[i][1]);
        r2[ndw + q] = make_float2(pb.x + ab[i][0], pb.y + ab[i][1]);
      }
    }
    __syncthreads();
  }
  for (int ch = threadIdx.x; ch < C; ch += 64 * kUmWaves) {
    part_g[static_cast<int64_t>(blockIdx.x) * C + ch] = red[ch];
    part_b[static_cast<int64_t>(blockIdx.x) * C + ch] = red[C + ch];
  }
}

// out[n] = sum over r of part[r][n] (nothing when the scan failed).  A
// workgroup takes 32 columns; row group g (of 8) sums rows g, g + 8, ... in
// order, then the 8 group sums are added in order: the same result every run.
__global__ __launch_bounds__(256) void k_colsum(const float *part, int32_t R, int32_t N,
                                                float *out, const int32_t *status) {
  __shared__ float red[8][33];
  if (status[kStatusWord] != 0) return;
  const int c = threadIdx.x & 31, rg = threadIdx.x >> 5;
  const int n = blockIdx.x * 32 + c;
  float acc = 0.f;
  if (n < N) {
    // rows rg, rg + 8, ...: 16 loads in flight at a time, then added in row
    // order (the same order on every run)
    constexpr int B = 16;
    for (int r0 = rg; r0 < R; r0 += 8 * B) {
      float v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int r = r0 + 8 * i;
        v[i] = r < R ? part[static_cast<int64_t>(r) * N + n] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < B; ++i) acc += v[i];
    }
  }
  red[rg][c] = acc;
  __syncthreads();
  if (rg == 0 && n < N) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += red[i][c];
    out[n] = t;
  }
}

// part[b][o] = sum of G[pos[i]][o] over list entries i of block b (64 each;
// negative positions add nothing).
template <typename T>
__global__ __launch_bounds__(256) void k_rows_sum(const T *G, const int32_t *pos, int32_t n,
                                                  int32_t O, float *part) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= O) return;
  const int i0 = blockIdx.y * 64, i1 = min(n, i0 + 64);
  float s = 0.f;
  for (int i = i0; i < i1; ++i) {
    const int32_t p = pos[i];
    if (p >= 0) s += Elem<T>::load(G[static_cast<int64_t>(p) * O + o]);
  }
  part[static_cast<int64_t>(blockIdx.y) * O + o] = s;
}

// ---- fp32 backward (row-major operands; the products use the strided fp32 GEMM)

// dY[t] = G[dst_row[t]] (zero where the row was not placed); one wave per row.
__global__ __launch_bounds__(256) void k_gather_rows_f32(const float *G, const int32_t *dst_row,
                                                         int32_t T, int32_t O, float *dy) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  for (int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; t < T;
       t += nw) {
    const int32_t d = dst_row[t];
    for (int o = lane; o < O; o += 64)
      dy[t * O + o] = d >= 0 ? G[static_cast<int64_t>(d) * O + o] : 0.f;
  }
}

// d/dz of activate(z, act) in fp32: erf form Phi(z) + z phi(z); tanh form the
// derivative of 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3).
__device__ __forceinline__ float slope_f32(float z, int act) {
  if (act == 0)
    return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
           z * 0.39894228040143268f * expf(-0.5f * z * z);
  if (act == 1) {
    const float k0 = 0.79788456080286536f;
    const float th = tanhf(k0 * (z + 0.044715f * z * z * z));
    return 0.5f * (1.0f + th) + 0.5f * z * (1.0f - th * th) * k0 * (1.0f + 3.0f * 0.044715f * z * z);
  }
  return 1.0f;
}

// a = activate(z) (da == nullptr), or in place dz = da * act'(z).
__global__ __launch_bounds__(256) void k_act_f32(const float *z, int64_t n, int act, float *a,
                                                 float *da) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (da) da[i] *= slope_f32(z[i], act);
    else a[i] = activate(z[i], act);
  }
}

// fp32 feature gradient, one wave per (token row, block position) like
// k_bwd_unmerge, with dXm in the pages' feature order (dn[c] = dXm[m][c*k*k +
// p]); lane l holds channels l, l + 64, ... (NC of them).
template <bool LN, int NC>
__global__ __launch_bounds__(256) void k_bwd_unmerge_f32(const float *dxm, const float *x,
                                                         PlanChunk c, int C, const float *gamma,
                                                         float eps, float *dx, float *part_g,
                                                         float *part_b, const int32_t *status) {
  if (status[kStatusWord] != 0) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = c.k, kk = k * k;
  const int64_t K1 = static_cast<int64_t>(C) * kk;
  const int32_t t_begin = c.tok0[0], t_end = c.tok0[c.n];
  const int64_t items = static_cast<int64_t>(t_end - t_begin) * kk;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * 4;
  const bool have = lane < c.n;
  const int32_t l_tok0 = have ? c.tok0[lane] : INT32_MAX;
  const int32_t l_pix0 = have ? c.pix0[lane] : 0;
  const int32_t l_gh = have ? c.gh[lane] : 0, l_gw = have ? c.gw[lane] : 1;
  float ag[NC], ab[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) ag[i] = ab[i] = 0.f;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * 4 + wid; it < items; it += nw) {
    const int m = t_begin + static_cast<int>(it / kk), p = static_cast<int>(it % kk);
    const int v = __popcll(__ballot(l_tok0 <= m)) - 1;
    const int tok0 = __shfl(l_tok0, v), pix0 = __shfl(l_pix0, v);
    const int gh = __shfl(l_gh, v), gw = __shfl(l_gw, v);
    const int wp = (gw + k - 1) / k, t = m - tok0;
    const int y = (t / wp) * k + p / k, xx = (t % wp) * k + p % k;
    if (y >= gh || xx >= gw) continue;
    const int64_t pix = pix0 + static_cast<int64_t>(y) * gw + xx;
    float dn[NC], xv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int ch = lane + 64 * i;
      dn[i] = ch < C ? dxm[m * K1 + static_cast<int64_t>(ch) * kk + p] : 0.f;
      xv[i] = (LN && ch < C) ? x[pix * C + ch] : 0.f;
    }
    if (!LN) {
      if (dx)
#pragma unroll
        for (int i = 0; i < NC; ++i)
          if (lane + 64 * i < C) dx[pix * C + lane + 64 * i] = dn[i];
      continue;
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) sum += xv[i];
    const float mean = wave_sum(sum) / C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i)
      if (lane + 64 * i < C) ss += (xv[i] - mean) * (xv[i] - mean);
    const float rstd = 1.0f / sqrtf(wave_sum(ss) / C + eps);
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int ch = lane + 64 * i;
      const float gm = ch < C ? gamma[ch] : 0.f;
      const float xh = (xv[i] - mean) * rstd, gv = gm * dn[i];
      xv[i] = xh;
      ag[i] += dn[i] * xh;
      ab[i] += dn[i];
      sg += gv;
      sgx += gv * xh;
    }
    const float mg = wave_sum(sg) / C, mgx = wave_sum(sgx) / C;
    if (dx)
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int ch = lane + 64 * i;
        if (ch < C) dx[pix * C + ch] = rstd * (gamma[ch] * dn[i] - mg - xv[i] * mgx);
      }
  }
  if (!LN) return;
  extern __shared__ float red_f32[];  // [2][C]
  for (int w = 0; w < 4; ++w) {
    if (wid == w)
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const int ch = lane + 64 * i;
        if (ch < C) {
          red_f32[ch] = (w == 0 ? 0.f : red_f32[ch]) + ag[i];
          red_f32[C + ch] = (w == 0 ? 0.f : red_f32[C + ch]) + ab[i];
        }
      }
    __syncthreads();
  }
  for (int ch = threadIdx.x; ch < C; ch += 256) {
    part_g[static_cast<int64_t>(blockIdx.x) * C + ch] = red_f32[ch];
    part_b[static_cast<int64_t>(blockIdx.x) * C + ch] = red_f32[C + ch];
  }
}

template <bool LN, int NC>
hipError_t unmerge_f32_launch(const void *dxm, const void *x, const PlanChunk &c, int C,
                              const void *gamma, float eps, void *dx, float *part_g,
                              float *part_b, const int32_t *status, int grid, hipStream_t s) {
  const size_t lds = LN ? static_cast<size_t>(2) * C * sizeof(float) : 0;
  hipLaunchKernelGGL((k_bwd_unmerge_f32<LN, NC>), dim3(grid), dim3(256), lds, s,
                     static_cast<const float *>(dxm), static_cast<const float *>(x), c, C,
                     static_cast<const float *>(gamma), eps, static_cast<float *>(dx), part_g,
                     part_b, status);
  return hipGetLastError();
}

template <bool LN>
hipError_t unmerge_f32_dispatch(const void *dxm, const void *x, const PlanChunk &c, int C,
                                const void *gamma, float eps, void *dx, float *part_g,
                                float *part_b, const int32_t *status, int grid, hipStream_t s) {
  const int nc = (C + 63) / 64;
  if (nc <= 1) return unmerge_f32_launch<LN, 1>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
  if (nc <= 4) return unmerge_f32_launch<LN, 4>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
  if (nc <= 16) return unmerge_f32_launch<LN, 16>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
  if (nc <= 32) return unmerge_f32_launch<LN, 32>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
  return hipErrorInvalidValue;
}

template <bool LN, int NCH>
hipError_t unmerge_launch(const void *dxm, const void *x, const PlanChunk &c, int C,
                          const void *gamma, float eps, void *dx, float *part_g, float *part_b,
                          const int32_t *status, int grid, hipStream_t s) {
  // [2][C] fp32 sums, then gamma (bf16) staged once per workgroup
  const size_t lds = LN ? static_cast<size_t>(2) * C * sizeof(float) + C * sizeof(uint16_t) : 0;
  hipLaunchKernelGGL((k_bwd_unmerge<LN, NCH>), dim3(grid), dim3(64 * kUmWaves), lds, s,
                     static_cast<const uint16_t *>(dxm), static_cast<const uint16_t *>(x), c, C,
                     static_cast<const uint16_t *>(gamma), eps, static_cast<uint16_t *>(dx),
                     part_g, part_b, status);
  return hipGetLastError();
}

template <int ND>
hipError_t unmerge_dw_launch(const void *dxm, const void *x, const PlanChunk &c, const void *gamma,
                             float eps, void *dx, float *part_g, float *part_b,
                             const int32_t *status, int grid, hipStream_t s) {
  // [2][C] fp32 sums, then gamma (fp32) staged once per workgroup
  const size_t lds = static_cast<size_t>(3) * 128 * ND * sizeof(float);
  hipLaunchKernelGGL((k_bwd_unmerge_dw<ND>), dim3(grid), dim3(64 * kUmWaves), lds, s,
                     static_cast<const uint16_t *>(dxm), static_cast<const uint16_t *>(x), c, eps,
                     static_cast<const uint16_t *>(gamma), static_cast<uint16_t *>(dx), part_g,
                     part_b, status);
  return hipGetLastError();
}

template <bool LN>
hipError_t unmerge_dispatch(const void *dxm, const void *x, const PlanChunk &c, int C,
                            const void *gamma, float eps, void *dx, float *part_g, float *part_b,
                            const int32_t *status, int grid, hipStream_t s) {
  if constexpr (LN) {  // C = 768, 1152, 1280: one dword per lane and step
    if (C == 768) return unmerge_dw_launch<6>(dxm, x, c, gamma, eps, dx, part_g, part_b, status, grid, s);
    if (C == 1152) return unmerge_dw_launch<9>(dxm, x, c, gamma, eps, dx, part_g, part_b, status, grid, s);
    if (C == 1280) return unmerge_dw_launch<10>(dxm, x, c, gamma, eps, dx, part_g, part_b, status, grid, s);
  }
  switch ((C / 8 + 63) / 64) {  // 16-byte chunks per lane
    case 1: return unmerge_launch<LN, 1>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
    case 2: return unmerge_launch<LN, 2>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
    case 3: return unmerge_launch<LN, 3>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
    case 4: return unmerge_launch<LN, 4>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status, grid, s);
    default: return hipErrorInvalidValue;  // C > kBwdMaxChannels
  }
}

}  // namespace

int bwd_unmerge_grid(int64_t items) {
  const int64_t g = (items + 4 * kUmWaves - 1) / (4 * kUmWaves);  // about 4 items per wave
  return static_cast<int>(g < 1 ? 1 : (g > kBwdUnmergeGrid ? kBwdUnmergeGrid : g));
}

hipError_t launch_bwd_gather_dy(const void *G, const int32_t *dst_row, int32_t T, int32_t O,
                                int32_t Op, int32_t Tk, void *dy, void *dyt, float *part,
                                hipStream_t s) {
  if (Tk <= 0) return hipSuccess;
  const dim3 grid(Tk / kTR, (Op + kTC - 1) / kTC);
  hipLaunchKernelGGL(k_bwd_gather_dy, grid, dim3(256), 0, s, static_cast<const uint16_t *>(G),
                     dst_row, T, O, Op, Tk, static_cast<uint16_t *>(dy),
                     static_cast<uint16_t *>(dyt), part);
  return hipGetLastError();
}

hipError_t launch_bwd_dact(int act, const void *da1, const void *z1, int32_t T, int32_t H,
                           int32_t Tk, void *dz1, void *dz1t, float *part, hipStream_t s) {
  if (Tk <= 0) return hipSuccess;
  const dim3 grid(Tk / kTR, (H + kTC - 1) / kTC);
  const uint16_t *a = static_cast<const uint16_t *>(da1), *z = static_cast<const uint16_t *>(z1);
  uint16_t *d = static_cast<uint16_t *>(dz1), *dt = static_cast<uint16_t *>(dz1t);
  if (act == 0)
    hipLaunchKernelGGL(k_bwd_dact<0>, grid, dim3(256), 0, s, a, z, T, H, Tk, d, dt, part);
  else if (act == 1)
    hipLaunchKernelGGL(k_bwd_dact<1>, grid, dim3(256), 0, s, a, z, T, H, Tk, d, dt, part);
  else
    hipLaunchKernelGGL(k_bwd_dact<2>, grid, dim3(256), 0, s, a, z, T, H, Tk, d, dt, part);
  return hipGetLastError();
}

hipError_t launch_bwd_xm_t(const void *xm, int32_t T, int32_t C, int32_t k, int32_t Tk, void *xmt,
                           hipStream_t s) {
  if (Tk <= 0) return hipSuccess;
  const int32_t K1 = C * k * k;
  const dim3 grid(Tk / kTR, (K1 + kTC - 1) / kTC);
  hipLaunchKernelGGL(k_bwd_xm_t, grid, dim3(256), 0, s, static_cast<const uint16_t *>(xm), T, K1,
                     C, k * k, Tk, static_cast<uint16_t *>(xmt));
  return hipGetLastError();
}

hipError_t launch_bwd_unmerge(const void *dxm, const void *x, const PlanChunk &c, int C,
                              const void *gamma, float eps, void *dx, float *part_g,
                              float *part_b, const int32_t *status, int grid, hipStream_t s) {
  if (c.tok0[c.n] <= c.tok0[0]) return hipSuccess;
  return gamma ? unmerge_dispatch<true>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status,
                                        grid, s)
               : unmerge_dispatch<false>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status,
                                         grid, s);
}

hipError_t launch_colsum(const float *part, int32_t R, int32_t N, float *out,
                         const int32_t *status, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_colsum, dim3((N + 31) / 32), dim3(256), 0, s, part, R, N, out, status);
  return hipGetLastError();
}

hipError_t launch_rows_sum(int dtype, const void *G, const int32_t *pos, int32_t n, int32_t O,
                           float *part, hipStream_t s) {
  if (n <= 0 || O <= 0) return hipSuccess;
  const dim3 grid((O + 255) / 256, (n + 63) / 64);
  if (dtype == 0)
    hipLaunchKernelGGL(k_rows_sum<float>, grid, dim3(256), 0, s, static_cast<const float *>(G),
                       pos, n, O, part);
  else
    hipLaunchKernelGGL(k_rows_sum<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t *>(G), pos, n, O, part);
  return hipGetLastError();
}

hipError_t launch_gather_rows_f32(const void *G, const int32_t *dst_row, int32_t T, int32_t O,
                                  void *dy, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<int64_t>((T + 3) / 4, 4096));
  hipLaunchKernelGGL(k_gather_rows_f32, dim3(grid), dim3(256), 0, s,
                     static_cast<const float *>(G), dst_row, T, O, static_cast<float *>(dy));
  return hipGetLastError();
}

hipError_t launch_act_f32(int act, const void *z, int64_t n, void *a, void *da, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<int64_t>((n + 255) / 256, 8192));
  hipLaunchKernelGGL(k_act_f32, dim3(grid), dim3(256), 0, s, static_cast<const float *>(z), n, act,
                     static_cast<float *>(a), static_cast<float *>(da));
  return hipGetLastError();
}

hipError_t launch_bwd_unmerge_f32(const void *dxm, const void *x, const PlanChunk &c, int C,
                                  const void *gamma, float eps, void *dx, float *part_g,
                                  float *part_b, const int32_t *status, int grid, hipStream_t s) {
  if (c.tok0[c.n] <= c.tok0[0]) return hipSuccess;
  return gamma ? unmerge_f32_dispatch<true>(dxm, x, c, C, gamma, eps, dx, part_g, part_b, status,
                                            grid, s)
               : unmerge_f32_dispatch<false>(dxm, x, c, C, gamma, eps, dx, part_g, part_b,
                                             status, grid, s);
}

}  // namespace vlb
