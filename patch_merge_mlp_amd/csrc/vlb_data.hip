// Data-movement kernels of the bridge: gather descriptors, the placeholder
// prefix sum, the assembly map (with newline / separator rows), LayerNorm,
// the standalone row scatter and space-to-depth, and the W1 re-layout.
//
// Operations follow mlxcel issue #533 "port DeepSeek-VL2": section
// "Projector (downsample_mlp_gelu)" steps 1-2 (pad, space-to-depth) and
// section "Tile-sequence assembly" (newline / separator layout and the in-order
// overwrite of the placeholder positions).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vlb_common.h"
#include "vlb_internal.h"

namespace vlb {

namespace {

constexpr int kErrMaskCount = 6;  // VLB_ERR_MASK_COUNT
constexpr int kLnChunks = 8;      // LayerNorm: most 16-byte chunks a lane holds

// ---------------------------------------------------------------------------
// Placeholder prefix sum: slot_pos[j] = position of the j-th placeholder.
// The placeholders are the nonzero bytes of a mask, or (token-id form) the
// positions whose id equals the image token; in the id form every other id
// must lie in [0, vocab).  One workgroup streams the sequence in chunks of
// 16K positions with a running carry; each chunk's positions are gathered in
// LDS and written out with coalesced stores.  status[kCountWord] = number of
// placeholders; status[kStatusWord] = 0, VLB_ERR_MASK_COUNT when the count
// differs from P, else VLB_ERR_TOKEN_ID when a text id is out of range.
// Plain layout (direct): token row r goes to the r-th placeholder, so the
// positions are the rows' destinations.  When the input is invalid, the same
// workgroup then overwrites every dst_row entry (P of them) with -1, so
// nothing is placed.
constexpr int kScanThreads = 1024;
constexpr int kErrTokenId = 9;  // VLB_ERR_TOKEN_ID

struct ScanSrc {
  const uint8_t *mask;  // mask form, or
  const int32_t *ids;   // token-id form
  int32_t image_id;
  int64_t vocab;
};

// Placeholder flags of the 16 positions at off (bounded by S) into b; returns
// their count and adds the out-of-range text ids to bad.
__device__ __forceinline__ int scan_load(const ScanSrc &src, int64_t S, int64_t off,
                                         uint8_t (&b)[16], int &bad) {
  if (src.ids) {
    int32_t id[16];
    if (off + 16 <= S) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = reinterpret_cast<const uint4 *>(src.ids + off)[q];
        id[4 * q] = static_cast<int32_t>(v.x);
        id[4 * q + 1] = static_cast<int32_t>(v.y);
        id[4 * q + 2] = static_cast<int32_t>(v.z);
        id[4 * q + 3] = static_cast<int32_t>(v.w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) id[i] = (off + i < S) ? src.ids[off + i] : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool live = off + i < S;
      b[i] = live && id[i] == src.image_id;
      bad += live && !b[i] && (id[i] < 0 || id[i] >= src.vocab);
    }
  } else if (off + 16 <= S) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src.mask + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = ((w[i >> 2] >> (8 * (i & 3))) & 0xff) != 0;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) b[i] = (off + i < S) ? src.mask[off + i] != 0 : 0;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) cnt += b[i];
  return cnt;
}

constexpr int kScanChunk = kScanThreads * 16;  // positions per pass

// Kernel arguments of the scan (on == 0: no scan in this launch).
struct ScanArgs {
  ScanSrc src;
  int64_t S, P;
  int32_t *slot_pos;
  int32_t *status;
  int32_t direct;
  int32_t on;
  int2 *text;  // token-id form: (position, id) of every text position, in order (may be null)
};

ScanArgs scan_args(const ScanJob *j) {
  ScanArgs a{};
  if (j) {
    a.src = ScanSrc{j->mask, j->ids, j->image_id, j->vocab};
    a.S = j->S;
    a.P = j->P;
    a.slot_pos = j->slot_pos;
    a.status = j->status;
    a.direct = j->direct ? 1 : 0;
    a.on = 1;
    a.text = reinterpret_cast<int2 *>(j->text);
  }
  return a;
}

// The scan, run by one workgroup of kScanThreads threads; s_pos is LDS for
// kScanChunk positions.
__device__ __forceinline__ void scan_body(const ScanArgs &a, int32_t *s_pos) {
  __shared__ int32_t wsum[kScanThreads / 64];
  __shared__ int32_t s_bad;
  const ScanSrc &src = a.src;
  const int64_t S = a.S, P = a.P;
  int32_t *slot_pos = a.slot_pos;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t carry = 0;
  int bad = 0;
  for (int64_t base = 0; base < S; base += kScanChunk) {
    const int64_t off = base + static_cast<int64_t>(tid) * 16;
    uint8_t b[16];
    const int cnt = scan_load(src, S, off, b, bad);
    int x = cnt;  // inclusive scan inside the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    if (wid == 0) {
      int w = lane < kScanThreads / 64 ? wsum[lane] : 0;
#pragma unroll
      for (int d = 1; d < kScanThreads / 64; d <<= 1) {
        const int y = __shfl_up(w, d, 64);
        if (lane >= d) w += y;
      }
      if (lane < kScanThreads / 64) wsum[lane] = w;
    }
    __syncthreads();
    int pos = (x - cnt) + (wid > 0 ? wsum[wid - 1] : 0);  // inside this pass
    if (a.text) {  // text position q is the (q - placeholders before it)-th text position
      int64_t img = carry + pos;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t q = off + i;
        if (q < S) {
          if (b[i])
            ++img;
          else  // the id is read again (from the cache) rather than kept in registers
            a.text[q - img] = make_int2(static_cast<int32_t>(q), src.ids[q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (b[i]) s_pos[pos++] = static_cast<int32_t>(off + i);
    const int n = wsum[kScanThreads / 64 - 1];
    __syncthreads();
    for (int q = tid; q < n; q += kScanThreads)
      if (carry + q < P) slot_pos[carry + q] = s_pos[q];
    carry += n;
    __syncthreads();  // s_pos and wsum are reused by the next pass
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  const bool fail = carry != P || s_bad != 0;
  if (fail && a.direct)  // after the barrier: these stores land after the positions above
    for (int64_t r = tid; r < P; r += kScanThreads) slot_pos[r] = -1;
  if (tid == 0) {
    a.status[kCountWord] = static_cast<int32_t>(carry);
    a.status[kStatusWord] = carry != P ? kErrMaskCount : (s_bad ? kErrTokenId : 0);
  }
}

__global__ __launch_bounds__(kScanThreads) void k_scan(ScanArgs a) {
  __shared__ int32_t s_pos[kScanChunk];  // this pass's placeholder positions, in order
  scan_body(a, s_pos);
}

// ---------------------------------------------------------------------------
// Gather descriptor of every token row of a chunk of views, 1024 rows per
// workgroup.  With a ScanArgs job, workgroup 0 of the launch runs the
// placeholder scan instead (scan_body; dynamic LDS of kScanChunk positions),
// beside the descriptors: the two touch different data.
__global__ __launch_bounds__(kScanThreads) void k_plan(PlanChunk c, RowDesc *desc, ScanArgs scan) {
  extern __shared__ int32_t plan_lds[];
  int blk = blockIdx.x;
  if (scan.on) {
    if (blk == 0) {
      scan_body(scan, plan_lds);
      return;
    }
    --blk;
  }
  const int32_t r = c.tok0[0] + blk * kScanThreads + threadIdx.x;
  if (r >= c.tok0[c.n]) return;
  int lo = 0, hi = c.n - 1;
  while (lo < hi) {  // last view whose first token is <= r
    const int mid = (lo + hi + 1) >> 1;
    if (c.tok0[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int v = lo, k = c.k;
  const int gh = c.gh[v], gw = c.gw[v];
  const int wp = (gw + k - 1) / k;
  const int t = r - c.tok0[v];
  const int y0 = (t / wp) * k, x0 = (t % wp) * k;
  uint32_t inside = 0;
  for (int dy = 0; dy < k; ++dy)
    for (int dx = 0; dx < k; ++dx)
      if (y0 + dy < gh && x0 + dx < gw) inside |= 1u << (dy * k + dx);
  desc[r].pix = c.pix0[v] + y0 * gw + x0;
  desc[r].geo = gw | static_cast<int32_t>(inside << 16);
}

// ---------------------------------------------------------------------------
// Token-embedding rows: seq[q] = embed[id] for every text position q, from
// the (position, id) list the token-id scan writes -- nothing when the scan
// reported an error.  One wave per text row (the pair and the status word are
// loaded together, then the row), 16-byte copies.
template <typename T>
__global__ __launch_bounds__(256) void k_embed_rows(const int2 *text, int64_t n, const T *embed,
                                                    int D, const int32_t *status, T *seq) {
  constexpr int V = 8;  // 16-byte chunks per lane per pass: up to 8 KiB of a row in flight
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int32_t st = status[kStatusWord];  // read together with the first pair
  const int n16 = D * static_cast<int>(sizeof(T)) / 16;
  for (int64_t j = wave; j < n; j += nwaves) {
    const int2 e = text[j];
    if (st != 0) return;
    const uint4 *from = reinterpret_cast<const uint4 *>(embed + static_cast<int64_t>(e.y) * D);
    uint4 *to = reinterpret_cast<uint4 *>(seq + static_cast<int64_t>(e.x) * D);
    // All of a pass's loads are issued before its stores (the table and the
    // sequence may not be assumed apart, so a plain copy loop would wait on
    // every load in turn).
    for (int base = 0; base < n16; base += 64 * V) {
      uint4 v[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int q = base + lane + 64 * i;
        v[i] = q < n16 ? from[q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int q = base + lane + 64 * i;
        if (q < n16) to[q] = v[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2D tile layout: decode what every assembled slot holds -- a token row, the
// newline or the separator -- by inverting the assembly order of one image:
//   global view: h' rows of (w' tokens, newline)
//   separator
//   local mosaic: th*h' rows of (tw*w' tokens, newline), mosaic row R and
//                 column X taken from tile (R / h')*tw + X / w', token
//                 (R % h')*w' + X % w'
// ("tail" puts the mosaic first).  One wave per slot; token slots record the
// destination row, newline / separator slots are copied by the whole wave.
//
// REC (gradients): the sequence is not written; the sequence position of each
// newline slot goes to nl_pos[nl0 + ordinal] -- ordinal counting the image's
// newlines in assembly order (global rows, then mosaic rows; reversed with
// "tail") -- and that of the separator to sep_pos[img0 + image].
template <typename T, bool REC>
__global__ void k_place_tiled(PlaceChunk c, const int32_t *slot_pos, const int32_t *status,
                              int32_t *dst_row, const T *newline, const T *separator, T *seq,
                              int D, int32_t *nl_pos, int32_t *sep_pos) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const bool ok = status[kStatusWord] == 0;
  const int end = c.slot0[c.n];
  // Lane i keeps image i's table entry (vector loads); a slot's image is the
  // number of images starting at or before it, less one, found with one
  // ballot, and its entry is taken from that lane with shuffles.  The table is
  // never indexed with a wave-uniform image number: a scalar load from such a
  // computed kernel-argument address ignores the low address bits, which the
  // 16-bit entries do not keep dword-aligned.
  const bool have = lane < c.n;
  const int32_t l_slot0 = have ? c.slot0[lane] : INT32_MAX;
  const int32_t l_row0 = have ? c.row0[lane] : 0, l_nl0 = have ? c.nl0[lane] : 0;
  const int32_t l_hp = have ? c.hp[lane] : 1, l_wp = have ? c.wp[lane] : 1;
  const int32_t l_tw = have ? c.tw[lane] : 1, l_th = have ? c.th[lane] : 1;
  for (int64_t jj = c.slot0[0] + wave; jj < end; jj += nwaves) {
    const int j = static_cast<int>(jj);
    const int im = __popcll(__ballot(l_slot0 <= j)) - 1;
    const int hp = __shfl(l_hp, im), wp = __shfl(l_wp, im), tw = __shfl(l_tw, im),
              th = __shfl(l_th, im);
    const int row0 = __shfl(l_row0, im), nl0 = __shfl(l_nl0, im);
    const int G = hp * (wp + 1);             // global block
    const int L = th * hp * (tw * wp + 1);   // local mosaic block
    int q = j - __shfl(l_slot0, im);
    int row = -1;                            // token row, or -1 newline, -2 separator
    int nl_ord = 0;                          // newline ordinal inside the image
    bool global;
    if (!c.tail) {
      global = q < G;
      if (q == G) row = -2;
      else if (!global) q -= G + 1;
    } else {
      global = q > L;
      if (q == L) row = -2;
      else if (global) q -= L + 1;
    }
    if (row != -2) {
      if (global) {
        const int R = q / (wp + 1), X = q % (wp + 1);
        row = (X == wp) ? -1 : row0 + R * wp + X;
        nl_ord = (c.tail ? th * hp : 0) + R;
      } else {
        const int W = tw * wp + 1;
        const int R = q / W, X = q % W;
        nl_ord = (c.tail ? 0 : hp) + R;
        if (X == tw * wp) {
          row = -1;
        } else {
          const int tile = (R / hp) * tw + X / wp;
          row = row0 + (1 + tile) * hp * wp + (R % hp) * wp + (X % wp);
        }
      }
    }
    if (row >= 0) {
      if (lane == 0) dst_row[row] = ok ? slot_pos[j] : -1;
    } else if (REC) {
      if (lane == 0) {
        const int32_t pos = ok ? slot_pos[j] : -1;
        if (row == -1) nl_pos[nl0 + nl_ord] = pos;
        else sep_pos[c.img0 + im] = pos;
      }
    } else if (ok) {
      const uint4 *from = reinterpret_cast<const uint4 *>(row == -1 ? newline : separator);
      uint4 *to = reinterpret_cast<uint4 *>(seq + static_cast<int64_t>(slot_pos[j]) * D);
      const int n16 = D * static_cast<int>(sizeof(T)) / 16;
      for (int i = lane; i < n16; i += 64) to[i] = from[i];
    }
  }
}

// ---------------------------------------------------------------------------
// LayerNorm over C per pixel, one wave per pixel: mean, biased variance, eps
// inside the square root, affine.  The pixel stays in registers: NCH 16-byte
// chunks per lane (NCH chosen from C at launch, so a lane holds as few
// registers as the row needs and many waves stay resident).
template <typename T, int NCH>
__global__ __launch_bounds__(256) void k_layernorm(const T *x, int64_t npix, int C, const T *gamma,
                                                   const T *beta, float eps, T *out) {
  constexpr int E = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int nch = C / E;
  const uint4 *g4 = reinterpret_cast<const uint4 *>(gamma);
  const uint4 *b4 = reinterpret_cast<const uint4 *>(beta);
  for (int64_t px = wave; px < npix; px += nwaves) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + px * C);
    uint4 v[NCH];
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      v[i] = q < nch ? src[q] : make_uint4(0, 0, 0, 0);
      const T *e = reinterpret_cast<const T *>(&v[i]);
#pragma unroll
      for (int j = 0; j < E; ++j) s += Elem<T>::load(e[j]);
    }
    const float mean = wave_sum(s) / C;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (lane + 64 * i < nch) {
        const T *e = reinterpret_cast<const T *>(&v[i]);
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float d = Elem<T>::load(e[j]) - mean;
          ss += d * d;
        }
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(ss) / C + eps);
    uint4 *dst = reinterpret_cast<uint4 *>(out + px * C);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      if (q < nch) {
        const uint4 gv = g4[q], bv = b4[q];
        const T *e = reinterpret_cast<const T *>(&v[i]);
        const T *ge = reinterpret_cast<const T *>(&gv);
        const T *be = reinterpret_cast<const T *>(&bv);
        uint4 o;
        T *oe = reinterpret_cast<T *>(&o);
#pragma unroll
        for (int j = 0; j < E; ++j)
          oe[j] = Elem<T>::store((Elem<T>::load(e[j]) - mean) * rstd * Elem<T>::load(ge[j]) +
                                 Elem<T>::load(be[j]));
        dst[q] = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Space-to-depth into the first GEMM's tile-blocked operand (bf16), with the
// LayerNorm fused when LN is set.  Merged row m, position p = dy*k + dx holds
// pixel (y0 + dy, x0 + dx) of the token's k x k block (zeros where the block
// hangs over the grid's high edge), at columns p*C .. p*C + C - 1: the K axis
// is position-major, as in the packed W1.  Element (m, j) of the [T][C*k*k]
// result sits at ((m/256 * K/32 + j/32) * 256 + m%256) * 32 + j%32.
//
// One launch covers the token rows of a chunk of up to 64 views; lane v of
// every wave keeps view v's table entry, so a row's view is found with one
// ballot.  A workgroup of 16 waves takes one item: 16 consecutive rows
// (aligned to 16, so they share a 256-row block) at one position.  Wave r
// loads row r's pixel (NCH 16-byte chunks per lane, or with DW NCH dwords),
// normalises it and stages it in LDS; then, per 32-wide K slice, the 16 rows' 64-byte pieces -- one
// contiguous KiB of the output -- go out as one store instruction of a wave.
// gamma and beta are staged once per workgroup in LDS.  With a ScanArgs job,
// workgroup 0 of the launch runs the placeholder scan instead (scan_body),
// beside the merge: the two touch different data.
constexpr int kMbRows = 16;  // rows per item = waves per workgroup
// LayerNorm's gamma and beta are staged in fp32 when the LDS has room next to
// the staged rows: up to NCH = 6 16-byte chunks per lane (C <= 3072).  At
// NCH = 8 (C <= 4096) rows take 16 * 513 * 16 B, and fp32 gamma and beta
// would pass the 160 KiB of a workgroup.
constexpr bool mb_gb32(int nch_per_lane) { return nch_per_lane <= 6; }
static_assert(kPlanViews >= 64, "each lane reads one view-table entry");

template <bool LN, int NCH, bool DW>
__global__ __launch_bounds__(64 * kMbRows) void k_merge_blocked(const uint16_t *x, PlanChunk c,
                                                                int C, const uint16_t *gamma,
                                                                const uint16_t *beta, float eps,
                                                                uint16_t *out, ScanArgs scan) {
  extern __shared__ uint4 mb_lds[];
  static_assert(64 * kMbRows == kScanThreads, "the scan workgroup has the merge's shape");
  static_assert(LN || !DW, "the dword layout is for the LayerNorm path");
  int item = blockIdx.x;
  if (scan.on) {  // workgroup 0 runs the placeholder scan (LDS >= kScanChunk positions)
    if (item == 0) {
      scan_body(scan, reinterpret_cast<int32_t *>(mb_lds));
      return;
    }
    --item;
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int k = c.k, kk = k * k, nch = C / 8;
  const int rs = nch + 1;  // LDS row stride in 16-byte chunks (odd: rows hit distinct banks)
  const int64_t KB = static_cast<int64_t>(C) * kk / 32;
  const int32_t t_begin = c.tok0[0], t_end = c.tok0[c.n];
  const int g0 = t_begin / kMbRows;
  const int grp = g0 + item / kk, p = item % kk;
  const int dy = p / k, dx = p - dy * k;

  // This wave's row and its pixel (wave-uniform): the view is the number of
  // views starting at or before the row, less one.  Lane l reads view l's
  // entry with a vector load and the wave picks entry v with a shuffle; the
  // table is never indexed with the uniform v directly (a scalar load from a
  // computed kernel-argument address must be dword-aligned at its base, which
  // the 16-bit entries do not guarantee).
  const int m = grp * kMbRows + wid;
  bool inside = false;
  int64_t off = 0;
  if (m >= t_begin && m < t_end) {
    // Every lane loads (the tables hold kPlanViews = 64 entries), so the four
    // loads go out together; entries past n are then masked.
    const bool have = lane < c.n;
    const int32_t e_tok0 = c.tok0[lane], e_pix0 = c.pix0[lane];
    const int32_t e_gh = c.gh[lane], e_gw = c.gw[lane];
    const int32_t l_tok0 = have ? e_tok0 : INT32_MAX;
    const int32_t l_pix0 = have ? e_pix0 : 0;
    const int32_t l_gh = have ? e_gh : 0, l_gw = have ? e_gw : 1;
    const int v = __popcll(__ballot(l_tok0 <= m)) - 1;
    const int tok0 = __shfl(l_tok0, v), pix0 = __shfl(l_pix0, v);
    const int gh = __shfl(l_gh, v), gw = __shfl(l_gw, v);
    const int wp = (gw + k - 1) / k, t = m - tok0;
    const int y = (t / wp) * k + dy, xx = (t % wp) * k + dx;
    inside = y < gh && xx < gw;
    off = static_cast<int64_t>(pix0 + y * gw + xx) * C;
  }
  // gamma and beta (LN) are staged once per workgroup in LDS after the rows,
  // widened to fp32 (no conversion per element later) while that fits: up to
  // 6 chunks per lane (C <= 3072); for C up to 4096 they stay bf16.  Their
  // loads go out before the pixel's, so waiting for them (loads return in
  // order) never waits on the pixel.
  constexpr bool GB32 = DW || mb_gb32(NCH);
  float4 *s_gb = reinterpret_cast<float4 *>(mb_lds + kMbRows * rs);  // GB32: [2][C] fp32
  uint4 *s_gb16 = mb_lds + kMbRows * rs;                              // else [2][C] bf16
  const int tid = threadIdx.x;
  uint4 gb = make_uint4(0, 0, 0, 0);
  if (LN && tid < 2 * nch)
    gb = tid < nch ? reinterpret_cast<const uint4 *>(gamma)[tid]
                   : reinterpret_cast<const uint4 *>(beta)[tid - nch];
  // Stage gamma and beta in LDS; every thread of the workgroup reaches it.
  auto stage_gb = [&]() {
    if (tid < 2 * nch) {  // chunk tid: 8 values (GB32: two float4 entries)
      if (GB32) {
        s_gb[2 * tid] = make_float4(bf2f(gb.x & 0xffff), bf2f(gb.x >> 16), bf2f(gb.y & 0xffff),
                                    bf2f(gb.y >> 16));
        s_gb[2 * tid + 1] = make_float4(bf2f(gb.z & 0xffff), bf2f(gb.z >> 16),
                                        bf2f(gb.w & 0xffff), bf2f(gb.w >> 16));
      } else {
        s_gb16[tid] = gb;
      }
    }
    __syncthreads();
  };
  uint4 *row = mb_lds + wid * rs;
  // The features are read once: non-temporal loads keep them from displacing
  // the GEMMs' operands in the caches (interleaved A/B, workload 1: step
  // 0.5291 -> 0.5232 ms, the GEMMs faster, this kernel 0.6 us slower).
  if constexpr (DW) {
    // One dword (two channels) per lane and step: at C = 1152 a pixel is 9
    // dwords on every lane, where 16-byte chunks leave 48 lanes idle in the
    // third step.  x - mean is kept for the normalisation, the mean and
    // variance scale by 1/C, and 1/sqrt is the hardware reciprocal root.
    // The launcher takes this form only for C = 128 * NCH, so every lane of
    // every step holds a dword of the pixel.  inside is the same on all lanes
    // of the wave (one row per wave): made scalar, it branches the wave.
    constexpr int ndw = 64 * NCH;  // dwords per pixel (C / 2)
    const bool in_w = __builtin_amdgcn_readfirstlane(inside ? 1 : 0) != 0;
    uint32_t d[NCH];
    const uint32_t *src = reinterpret_cast<const uint32_t *>(x + off);
    if (in_w) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) d[i] = load_nt(src + lane + 64 * i);
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) d[i] = 0u;
    }
    stage_gb();
    if (in_w) {  // rows outside the grid stay zero (padding comes after the norm)
      float lo[NCH], hi[NCH];
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        lo[i] = __uint_as_float(d[i] << 16);
        hi[i] = __uint_as_float(d[i] & 0xffff0000u);
        sum += lo[i] + hi[i];
      }
      constexpr float inv_c = 1.0f / static_cast<float>(2 * ndw);
      const float mean = wave_sum(sum) * inv_c;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        lo[i] -= mean;
        hi[i] -= mean;
        ss = fmaf(lo[i], lo[i], ss);
        ss = fmaf(hi[i], hi[i], ss);
      }
      const float rstd = rsqrtf(wave_sum(ss) * inv_c + eps);
      const float2 *g2 = reinterpret_cast<const float2 *>(s_gb);  // [C] gamma, then [C] beta
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = lane + 64 * i;
        const float2 g = g2[q], be = g2[ndw + q];
        d[i] = f2bf2(fmaf(lo[i] * rstd, g.x, be.x), fmaf(hi[i] * rstd, g.y, be.y));
      }
    }
    uint32_t *row32 = reinterpret_cast<uint32_t *>(row);
#pragma unroll
    for (int i = 0; i < NCH; ++i) row32[lane + 64 * i] = d[i];
  } else {
    uint4 v[NCH];
    const uint4 *src = reinterpret_cast<const uint4 *>(x + off);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = lane + 64 * i;
      v[i] = (inside && q < nch) ? load_nt(src + q) : make_uint4(0, 0, 0, 0);
    }
    if (LN) stage_gb();
    if (LN && inside) {  // rows outside the grid stay zero (padding comes after the norm)
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint16_t *e = reinterpret_cast<const uint16_t *>(&v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += bf2f(e[j]);
      }
      const float mean = wave_sum(sum) / C;
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        if (lane + 64 * i < nch) {
          const uint16_t *e = reinterpret_cast<const uint16_t *>(&v[i]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float dlt = bf2f(e[j]) - mean;
            ss += dlt * dlt;
          }
        }
      }
      const float rstd = 1.0f / sqrtf(wave_sum(ss) / C + eps);
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int q = lane + 64 * i;
        if (q < nch) {
          float gf[8], bfv[8];
          if (GB32) {
            const float4 g0 = s_gb[2 * q], g1 = s_gb[2 * q + 1];
            const float4 b0 = s_gb[2 * (nch + q)], b1 = s_gb[2 * (nch + q) + 1];
            gf[0] = g0.x; gf[1] = g0.y; gf[2] = g0.z; gf[3] = g0.w;
            gf[4] = g1.x; gf[5] = g1.y; gf[6] = g1.z; gf[7] = g1.w;
            bfv[0] = b0.x; bfv[1] = b0.y; bfv[2] = b0.z; bfv[3] = b0.w;
            bfv[4] = b1.x; bfv[5] = b1.y; bfv[6] = b1.z; bfv[7] = b1.w;
          } else {
            const uint4 gq = s_gb16[q], bq = s_gb16[nch + q];
            const uint16_t *ge = reinterpret_cast<const uint16_t *>(&gq);
            const uint16_t *be = reinterpret_cast<const uint16_t *>(&bq);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              gf[j] = bf2f(ge[j]);
              bfv[j] = bf2f(be[j]);
            }
          }
          uint16_t *e = reinterpret_cast<uint16_t *>(&v[i]);
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = f2bf(fmaf((bf2f(e[j]) - mean) * rstd, gf[j], bfv[j]));
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (lane + 64 * i < nch) row[lane + 64 * i] = v[i];
  }
  __syncthreads();
  // Per K slice: lane -> (row lane/4, chunk lane%4); only this chunk's rows are written.
  const int r = lane >> 2, c4 = lane & 3;
  const int mr = grp * kMbRows + r;
  if (mr < t_begin || mr >= t_end) return;
  uint16_t *dst = out + (static_cast<int64_t>(mr >> 8) * KB * 256 + (mr & 255)) * 32 + c4 * 8;
  const int slices = C / 32, sl0 = p * slices;
  for (int sl = wid; sl < slices; sl += kMbRows)
    *reinterpret_cast<uint4 *>(dst + static_cast<int64_t>(sl0 + sl) * (256 * 32)) =
        mb_lds[r * rs + sl * 4 + c4];
}

// ---------------------------------------------------------------------------
// Rows of at least this many bytes are read by the standalone scatter with
// non-temporal loads (they no longer fit the 256 MiB Infinity Cache beside
// the sequence; see k_scatter).
constexpr int64_t kScatterStreamBytes = int64_t{96} << 20;

// Standalone scatter: row r of rows[T][D] -> seq[dst_row[r]] (skipped if < 0).
// One wave per row; the row's data (up to 8 KiB at a time) is loaded together
// with its destination, so the loads never wait on the index.  The sequence
// rows are written with non-temporal stores (74.6% of 8 TB/s against 67.5%
// with ordinary stores on workload 1).  NTL: the rows are also read with
// non-temporal loads, which pays once they no longer fit the Infinity Cache
// beside the rest (112 MB of rows: 51.4 -> 42.8 us; 197 MB: 90.5 -> 75.1 us)
// and costs while they do (67 MB: 22.5 -> 25.5 us).
template <typename T, bool NTL>
__global__ __launch_bounds__(256) void k_scatter(const T *rows, int64_t Trows, int D,
                                                 const int32_t *dst_row, T *seq) {
  constexpr int V = 8;  // 16-byte chunks per lane per pass
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int n16 = D * static_cast<int>(sizeof(T)) / 16;
  for (int64_t r = wave; r < Trows; r += nwaves) {
    const int32_t d = dst_row[r];
    const uint4 *from = reinterpret_cast<const uint4 *>(rows + r * D);
    for (int base = 0; base < n16; base += 64 * V) {
      uint4 v[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int q = base + lane + 64 * i;
        v[i] = q < n16 ? (NTL ? load_nt(from + q) : from[q]) : make_uint4(0, 0, 0, 0);
      }
      if (d >= 0) {
        uint4 *to = reinterpret_cast<uint4 *>(seq + static_cast<int64_t>(d) * D);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const int q = base + lane + 64 * i;
          if (q < n16) store_nt(to + q, v[i]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Standalone space-to-depth in the pages' feature order c*k*k + dy*k + dx.
// A thread owns one 4-byte unit of a token's channels (two bf16 channels, or
// one fp32) and all k*k cells: it reads the unit from each cell (consecutive
// threads read consecutive units of a pixel, so each read instruction is one
// coalesced run) and writes the k*k interleaved values of its channels as k*k
// consecutive dwords of the merged row (together the threads of a wave cover
// one contiguous stretch).  Padded cells read as zero.
template <typename T, int KK>
__global__ __launch_bounds__(256) void k_merge(const T *x, const RowDesc *desc, int64_t Trows,
                                               int C, int k, T *merged) {
  constexpr int U = 4 / sizeof(T);  // channels per 4-byte unit
  const int units = C / U;
  const int64_t total = Trows * units;
  const uint32_t *x32 = reinterpret_cast<const uint32_t *>(x);
  uint32_t *m32 = reinterpret_cast<uint32_t *>(merged);
  for (int64_t w = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; w < total;
       w += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = w / units;
    const int u = static_cast<int>(w - r * units);
    const RowDesc d = desc[r];
    const int gw = d.geo & 0xffff;
    const uint32_t inside = static_cast<uint32_t>(d.geo) >> 16;
    uint32_t cell[KK];
#pragma unroll
    for (int p = 0; p < KK; ++p) {
      const int dy = p / k, dx = p - dy * k;
      cell[p] = ((inside >> p) & 1)
                    ? x32[(static_cast<int64_t>(d.pix + dy * gw + dx) * C) / U + u]
                    : 0u;
    }
    // The unit's run in the merged row: elements (U*u + i) * KK + p, i.e.
    // KK*U values = KK dwords starting at dword u*KK.
    uint32_t *dst = m32 + (r * C * KK) / U + static_cast<int64_t>(u) * KK;
    uint32_t o[KK];
    if constexpr (U == 1) {
#pragma unroll
      for (int p = 0; p < KK; ++p) o[p] = cell[p];
    } else {
      // run element e = i*KK + p holds channel half i of cell p; dword j packs
      // elements 2j (low half) and 2j+1.
      auto elem = [&](int e) -> uint32_t {
        const int i = e / KK, p = e - i * KK;
        return i == 0 ? (cell[p] & 0xffffu) : (cell[p] >> 16);
      };
#pragma unroll
      for (int j = 0; j < KK; ++j) o[j] = elem(2 * j) | (elem(2 * j + 1) << 16);
    }
    // The run as one vector store where it can be (consecutive threads then
    // write one contiguous span per instruction): 16 bytes for KK = 4 (the
    // run starts on a 16-byte boundary: C*KK/U is a multiple of 4), three
    // 12-byte stores for KK = 9.
    if constexpr (KK == 4) {
      *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    } else if constexpr (KK == 9) {
#pragma unroll
      for (int q = 0; q < 3; ++q)
        *reinterpret_cast<uint3 *>(dst + 3 * q) = make_uint3(o[3 * q], o[3 * q + 1], o[3 * q + 2]);
    } else {
#pragma unroll
      for (int j = 0; j < KK; ++j) dst[j] = o[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Weight packing into the tile-blocked layout; with kk = k*k > 1 the K axis of
// W1 is reordered position-major on the way (packed column p*Cc + c takes
// source column c*kk + p, Cc = K / kk channels).  A workgroup takes 64 rows
// and 32 channels: it reads the rows' 32*kk source columns (contiguous) into
// LDS, then for each position p writes the 64 rows' 64-byte pieces of packed
// K slice (p*Cc + c0) / 32 -- one contiguous 4 KiB run.  Rows past R are zero.
__global__ __launch_bounds__(256) void k_pack(const uint16_t *w, int64_t R, int64_t K, int kk,
                                              uint16_t *out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t pk[];  // [64][32*kk + 8]
  const int Cc = static_cast<int>(K / kk);
  const int pitch = 32 * kk + 8, nch = 4 * kk;  // row pitch; 16-byte chunks per row
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int c0 = blockIdx.y * 32;
  for (int q = threadIdx.x; q < 64 * nch; q += 256) {
    const int row = q / nch, ch = q - row * nch;
    const int64_t r = r0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R) v = *reinterpret_cast<const uint4 *>(w + r * K + static_cast<int64_t>(c0) * kk + ch * 8);
    *reinterpret_cast<uint4 *>(pk + row * pitch + ch * 8) = v;
  }
  __syncthreads();
  const int row = threadIdx.x >> 2, c4 = threadIdx.x & 3;
  const int64_t r = r0 + row, KB = K / 32;
  for (int p = 0; p < kk; ++p) {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = pk[row * pitch + (c4 * 8 + 2 * i) * kk + p] |
             (static_cast<uint32_t>(pk[row * pitch + (c4 * 8 + 2 * i + 1) * kk + p]) << 16);
    const int64_t j = static_cast<int64_t>(p) * Cc + c0;  // packed K slice start
    const int64_t e = (((r >> 8) * KB + (j >> 5)) * 256 + (r & 255)) * 32 + c4 * 8;
    *reinterpret_cast<uint4 *>(out + e) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

int grid_for(int64_t waves_or_items, int per_block, int cap) {
  int64_t g = (waves_or_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_plan(const PlanChunk &c, RowDesc *desc, hipStream_t s, const ScanJob *scan) {
  const int64_t n = c.tok0[c.n] - c.tok0[0];
  if (n <= 0)  // no rows: the scan (if any) runs on its own
    return scan ? launch_scan(scan->mask, scan->ids, scan->image_id, scan->vocab, scan->S,
                              scan->P, scan->slot_pos, scan->status, scan->direct, s, scan->text)
                : hipSuccess;
  const ScanArgs sa = scan_args(scan);
  const int grid = grid_for(n, kScanThreads, 1 << 30) + (sa.on ? 1 : 0);
  const size_t lds = sa.on ? kScanChunk * sizeof(int32_t) : 0;
  hipLaunchKernelGGL(k_plan, dim3(grid), dim3(kScanThreads), lds, s, c, desc, sa);
  return hipGetLastError();
}

namespace {
__global__ void k_copy_status(const int32_t *src, int32_t *dst) {
  const int i = threadIdx.x;
  if (i < 4) dst[i] = src ? src[i] : 0;
}
}  // namespace

hipError_t launch_copy_status(const int32_t *src, int32_t *dst, hipStream_t s) {
  hipLaunchKernelGGL(k_copy_status, dim3(1), dim3(64), 0, s, src, dst);
  return hipGetLastError();
}

hipError_t launch_scan(const uint8_t *mask, const int32_t *ids, int32_t image_id, int64_t vocab,
                       int64_t S, int64_t P, int32_t *slot_pos, int32_t *status, bool direct,
                       hipStream_t s, int32_t *text) {
  const ScanJob j{mask, ids, image_id, vocab, S, P, slot_pos, status, direct, text};
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, s, scan_args(&j));
  return hipGetLastError();
}

hipError_t launch_embed_rows(int dtype, const int32_t *text, int64_t n, const void *embed, int D,
                             const int32_t *status, void *seq, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int grid = grid_for(n, 4, 16384);
  const int2 *t = reinterpret_cast<const int2 *>(text);
  if (dtype == 0)
    hipLaunchKernelGGL(k_embed_rows<float>, dim3(grid), dim3(256), 0, s, t, n,
                       static_cast<const float *>(embed), D, status, static_cast<float *>(seq));
  else
    hipLaunchKernelGGL(k_embed_rows<uint16_t>, dim3(grid), dim3(256), 0, s, t, n,
                       static_cast<const uint16_t *>(embed), D, status,
                       static_cast<uint16_t *>(seq));
  return hipGetLastError();
}

hipError_t launch_place_tiled(int dtype, const PlaceChunk &c, const int32_t *slot_pos,
                              const int32_t *status, int32_t *dst_row, const void *newline,
                              const void *separator, void *seq, int D, hipStream_t s) {
  const int64_t n = c.slot0[c.n] - c.slot0[0];
  if (n <= 0) return hipSuccess;
  const int grid = grid_for(n, 4, 4096);  // 4 waves per block, one slot per wave per pass
  if (dtype == 0)
    hipLaunchKernelGGL((k_place_tiled<float, false>), dim3(grid), dim3(256), 0, s, c, slot_pos,
                       status, dst_row, static_cast<const float *>(newline),
                       static_cast<const float *>(separator), static_cast<float *>(seq), D,
                       nullptr, nullptr);
  else
    hipLaunchKernelGGL((k_place_tiled<uint16_t, false>), dim3(grid), dim3(256), 0, s, c,
                       slot_pos, status, dst_row, static_cast<const uint16_t *>(newline),
                       static_cast<const uint16_t *>(separator), static_cast<uint16_t *>(seq), D,
                       nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_place_tiled_record(const PlaceChunk &c, const int32_t *slot_pos,
                                     const int32_t *status, int32_t *dst_row, int32_t *nl_pos,
                                     int32_t *sep_pos, hipStream_t s) {
  const int64_t n = c.slot0[c.n] - c.slot0[0];
  if (n <= 0) return hipSuccess;
  const int grid = grid_for(n, 4, 4096);
  hipLaunchKernelGGL((k_place_tiled<uint16_t, true>), dim3(grid), dim3(256), 0, s, c, slot_pos,
                     status, dst_row, nullptr, nullptr, nullptr, 0, nl_pos, sep_pos);
  return hipGetLastError();
}

template <typename T, int NCH>
static void ln_launch(const void *x, int64_t npix, int C, const void *gamma, const void *beta,
                      float eps, void *out, hipStream_t s) {
  const int grid = grid_for(npix, 4, 16384);
  hipLaunchKernelGGL((k_layernorm<T, NCH>), dim3(grid), dim3(256), 0, s,
                     static_cast<const T *>(x), npix, C, static_cast<const T *>(gamma),
                     static_cast<const T *>(beta), eps, static_cast<T *>(out));
}

template <typename T>
static hipError_t ln_dispatch(const void *x, int64_t npix, int C, const void *gamma,
                              const void *beta, float eps, void *out, hipStream_t s) {
  const int nch = (C * static_cast<int>(sizeof(T)) / 16 + 63) / 64;  // chunks per lane
  switch (nch) {
    case 1: ln_launch<T, 1>(x, npix, C, gamma, beta, eps, out, s); break;
    case 2: ln_launch<T, 2>(x, npix, C, gamma, beta, eps, out, s); break;
    case 3: ln_launch<T, 3>(x, npix, C, gamma, beta, eps, out, s); break;
    case 4: ln_launch<T, 4>(x, npix, C, gamma, beta, eps, out, s); break;
    case 5: case 6: ln_launch<T, 6>(x, npix, C, gamma, beta, eps, out, s); break;
    default: ln_launch<T, kLnChunks>(x, npix, C, gamma, beta, eps, out, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_layernorm(int dtype, const void *x, int64_t npix, int C, const void *gamma,
                            const void *beta, float eps, void *out, hipStream_t s) {
  if (npix <= 0) return hipSuccess;
  return dtype == 0 ? ln_dispatch<float>(x, npix, C, gamma, beta, eps, out, s)
                    : ln_dispatch<uint16_t>(x, npix, C, gamma, beta, eps, out, s);
}

int layernorm_max_channels(int dtype) { return kLnChunks * 64 * (dtype == 0 ? 4 : 8); }

template <bool LN, int NCH, bool DW = false>
static hipError_t mb_launch(const void *x, const PlanChunk &c, int C, const void *gamma,
                            const void *beta, float eps, void *out, hipStream_t s,
                            const ScanArgs &scan) {
  const int64_t items =
      ((c.tok0[c.n] + kMbRows - 1) / kMbRows - c.tok0[0] / kMbRows) * int64_t{c.k} * c.k +
      (scan.on ? 1 : 0);
  // staged rows, then (LN) gamma and beta (fp32 or bf16, see mb_gb32):
  // <= 160 KiB for every C the dispatch takes
  size_t lds = static_cast<size_t>(kMbRows) * (C / 8 + 1) * 16 +
               (LN ? static_cast<size_t>(2) * C * (DW || mb_gb32(NCH) ? 4 : 2) : 0);
  // The scan workgroup stages kScanChunk positions in the same LDS.  Two
  // 1024-thread workgroups per CU is the thread limit anyway, so 64 KiB each
  // costs the merge no occupancy.
  if (scan.on) lds = std::max(lds, kScanChunk * sizeof(int32_t));
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&k_merge_blocked<LN, NCH, DW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_merge_blocked<LN, NCH, DW>), dim3(static_cast<uint32_t>(items)),
                     dim3(64 * kMbRows), lds, s, static_cast<const uint16_t *>(x), c, C,
                     static_cast<const uint16_t *>(gamma), static_cast<const uint16_t *>(beta),
                     eps, static_cast<uint16_t *>(out), scan);
  return hipGetLastError();
}

template <bool LN>
static hipError_t mb_dispatch(const void *x, const PlanChunk &c, int C, const void *gamma,
                              const void *beta, float eps, void *out, hipStream_t s,
                              const ScanArgs &sa) {
  // LayerNorm at C = 768, 1152 or 1280: 16-byte chunks would leave lanes idle
  // in the last step (C / 8 not a multiple of 64); one dword per lane and
  // step fills every lane (C / 128 dwords per lane).
  if constexpr (LN) {
    switch (C) {
      case 768: return mb_launch<LN, 6, true>(x, c, C, gamma, beta, eps, out, s, sa);
      case 1152: return mb_launch<LN, 9, true>(x, c, C, gamma, beta, eps, out, s, sa);
      case 1280: return mb_launch<LN, 10, true>(x, c, C, gamma, beta, eps, out, s, sa);
      default: break;
    }
  }
  switch ((C / 8 + 63) / 64) {  // 16-byte chunks per lane per pixel
    case 1: return mb_launch<LN, 1>(x, c, C, gamma, beta, eps, out, s, sa);
    case 2: return mb_launch<LN, 2>(x, c, C, gamma, beta, eps, out, s, sa);
    case 3: return mb_launch<LN, 3>(x, c, C, gamma, beta, eps, out, s, sa);
    case 4: return mb_launch<LN, 4>(x, c, C, gamma, beta, eps, out, s, sa);
    case 5: case 6: return mb_launch<LN, 6>(x, c, C, gamma, beta, eps, out, s, sa);
    case 7: case 8: return mb_launch<LN, kLnChunks>(x, c, C, gamma, beta, eps, out, s, sa);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_merge_blocked(const void *x, const PlanChunk &c, int C, const void *gamma,
                                const void *beta, float eps, void *out, hipStream_t s,
                                const ScanJob *scan) {
  if (c.n <= 0 || c.tok0[c.n] <= c.tok0[0])  // no rows: the scan (if any) runs on its own
    return scan ? launch_scan(scan->mask, scan->ids, scan->image_id, scan->vocab, scan->S,
                              scan->P, scan->slot_pos, scan->status, scan->direct, s, scan->text)
                : hipSuccess;
  const ScanArgs sa = scan_args(scan);
  return gamma ? mb_dispatch<true>(x, c, C, gamma, beta, eps, out, s, sa)
               : mb_dispatch<false>(x, c, C, nullptr, nullptr, 0.f, out, s, sa);
}

hipError_t launch_scatter(int dtype, const void *rows, int64_t T, int D, const int32_t *dst_row,
                          void *seq, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int grid = grid_for(T, 4, 8192);
  const int64_t row_bytes = static_cast<int64_t>(D) * (dtype == 0 ? 4 : 2);
  const bool ntl = T * row_bytes >= kScatterStreamBytes;
  if (dtype == 0) {
    const float *r = static_cast<const float *>(rows);
    float *q = static_cast<float *>(seq);
    if (ntl)
      hipLaunchKernelGGL((k_scatter<float, true>), dim3(grid), dim3(256), 0, s, r, T, D, dst_row, q);
    else
      hipLaunchKernelGGL((k_scatter<float, false>), dim3(grid), dim3(256), 0, s, r, T, D, dst_row, q);
  } else {
    const uint16_t *r = static_cast<const uint16_t *>(rows);
    uint16_t *q = static_cast<uint16_t *>(seq);
    if (ntl)
      hipLaunchKernelGGL((k_scatter<uint16_t, true>), dim3(grid), dim3(256), 0, s, r, T, D, dst_row, q);
    else
      hipLaunchKernelGGL((k_scatter<uint16_t, false>), dim3(grid), dim3(256), 0, s, r, T, D, dst_row, q);
  }
  return hipGetLastError();
}

template <typename T>
static void merge_launch(const void *x, const RowDesc *desc, int64_t Trows, int C, int k,
                         void *merged, hipStream_t s) {
  const int64_t work = Trows * (C / (4 / static_cast<int>(sizeof(T))));
  const int grid = grid_for(work, 256, 16384);
  const T *xp = static_cast<const T *>(x);
  T *mp = static_cast<T *>(merged);
  switch (k) {
    case 1: hipLaunchKernelGGL((k_merge<T, 1>), dim3(grid), dim3(256), 0, s, xp, desc, Trows, C, k, mp); break;
    case 2: hipLaunchKernelGGL((k_merge<T, 4>), dim3(grid), dim3(256), 0, s, xp, desc, Trows, C, k, mp); break;
    default: hipLaunchKernelGGL((k_merge<T, 9>), dim3(grid), dim3(256), 0, s, xp, desc, Trows, C, k, mp); break;
  }
}

hipError_t launch_merge(int dtype, const void *x, const RowDesc *desc, int64_t T, int C, int k,
                        void *merged, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == 0)
    merge_launch<float>(x, desc, T, C, k, merged, s);
  else
    merge_launch<uint16_t>(x, desc, T, C, k, merged, s);
  return hipGetLastError();
}

hipError_t launch_pack(const void *w, int64_t R, int64_t K, int C, int k, void *packed,
                       hipStream_t s) {
  const int kk = k * k;
  if (R <= 0 || K <= 0) return hipSuccess;
  if (K % (32 * kk) != 0 || (kk > 1 && K != static_cast<int64_t>(C) * kk))
    return hipErrorInvalidValue;  // 32-channel tiles of whole positions
  const dim3 grid(static_cast<uint32_t>((R + 255) / 256 * 4), static_cast<uint32_t>(K / kk / 32));
  const size_t lds = static_cast<size_t>(64) * (32 * kk + 8) * 2;
  hipLaunchKernelGGL(k_pack, grid, dim3(256), lds, s, static_cast<const uint16_t *>(w), R, K, kk,
                     static_cast<uint16_t *>(packed));
  return hipGetLastError();
}

}  // namespace vlb
