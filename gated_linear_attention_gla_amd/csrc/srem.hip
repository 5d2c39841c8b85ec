// srem.hip -- SREM kernels: fused 3x3 depthwise conv + direction remap, and
// the plain scan-order remap.
//
// DiG paper notes, 关键设计 / DiG Block设计 steps (4)-(5) and 关键设计 / SREM:
// the mixer output (in scan order) is reshaped to 2D, passed through a 3x3
// DWConv2d and the scan direction is changed at the end of the block.  Here
// the reshape is of the scan-ordered sequence into its scan frame (R, Q), the
// conv is a zero-padded cross-correlation with fp32 accumulation, and the
// result is stored straight to the canonical token order (the arrange-back of
// the ZigMa notes, 关键设计 / 异构逐层扫描), so no remapped copy is written.
//
// Work split: a thread owns 4 channels of NC adjacent frame columns and a run
// of frame rows; its 9 x 4 fp32 weights sit in registers and a ring of rows
// slides down the columns with three rows of loads in flight.  A row costs
// NC + 2 loads for NC outputs, so wider walkers issue fewer loads per output
// (the kernel is bound by the texture units' address issue, not by HBM).
// Workgroups are ordered so that each XCD sweeps neighbouring columns, whose
// shared cells hit its L2.
#include "dig_internal.h"
#include <atomic>

namespace dig {
namespace {

// A walker's cell: 4 channels of one token, as NW 32-bit words of PW
// channels each (bf16: 2 words of 2, fp32: 4 words of 1).
template <int NW>
struct CellT;
template <>
struct CellT<2> { typedef uint2 type; };
template <>
struct CellT<4> { typedef uint4 type; };

__device__ __forceinline__ uint32_t word(const uint2 &u, int j) { return j == 0 ? u.x : u.y; }
__device__ __forceinline__ uint32_t word(const uint4 &u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}
__device__ __forceinline__ void unpack_word(uint32_t w, float *f, int pw) {
  if (pw == 2) { f[0] = bf16lo(w); f[1] = bf16hi(w); } else { f[0] = __uint_as_float(w); }
}

constexpr int kNT = 256;
constexpr unsigned kOOB = 0x80000000u;   // an offset past every valid span: loads return 0
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, unsigned off, uint2 &d) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  d = make_uint2(v.x, v.y);
}
__device__ __forceinline__ void bload(__amdgpu_buffer_rsrc_t r, unsigned off, uint4 &d) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  d = make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore(unsigned char *p, const uint32_t *w, uint2 *) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(w[0], w[1]);
}
__device__ __forceinline__ void gstore(unsigned char *p, const uint32_t *w, uint4 *) {
  *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

// A walker owns (batch, frame columns [c, c + NC), 4-channel group, run of
// frame rows [r0, r1)).  It keeps three frame rows x (NC + 2) columns of cells
// in registers as fp32 (rows t-1, t, t+1 feed output row t) while rows
// t+2 .. t+4 are in flight, so each step waits for a load issued three steps
// earlier.  Cells outside the frame (zero padding), columns past Q and rows
// past r1 come from out-of-range buffer offsets, which read as zero without
// touching memory.
template <int NW, int PW, int NC>
__global__ void __launch_bounds__(kNT)
srem_dwconv_kernel(const unsigned char *x, int64_t x_sb, int64_t x_st, const float *w,
                   unsigned char *y, int64_t y_sb, int64_t y_st, int B, int T, int C,
                   int gh, int gw, int dir, int rows_per_walker, int nseg, unsigned span) {
  typedef typename CellT<NW>::type cell_t;
  constexpr int CH = NW * PW;        // channels per walker (4)
  constexpr int ES = 4 / PW;         // bytes per element
  constexpr int NCC = NC + 2;        // cells per row: the columns and one neighbour each side
  const int CV = C / CH;
  int R, Q;
  scan_frame(dir, gh, gw, R, Q);
  const int QP = (Q + NC - 1) / NC;  // column groups
  // batch from the grid's y dimension: the buffer descriptor stays wave-uniform
  const int bb = blockIdx.y;
  const int id = xcd_linear_block(blockIdx.x, gridDim.x) * kNT + threadIdx.x;
  const int total = QP * CV * nseg;
  if (id >= total) return;
  const int cv = id % CV;
  const int rest = id / CV;
  const int c = (rest % QP) * NC;
  const int seg = rest / QP;
  const int r0 = seg * rows_per_walker;
  const int r1 = r0 + rows_per_walker < R ? r0 + rows_per_walker : R;
  if (r0 >= r1) return;
  const int ch0 = cv * CH;

  float wr[9][CH];
#pragma unroll
  for (int tap = 0; tap < 9; ++tap)
#pragma unroll
    for (int e = 0; e < CH; ++e) wr[tap][e] = w[(ch0 + e) * 9 + tap];

  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char *>(x + bb * x_sb * ES), (short)0, (int)span, 0x00020000);
  const unsigned colB = (unsigned)(x_st * ES), rowB = colB * (unsigned)Q, chB = (unsigned)(ch0 * ES);
  unsigned oc[NCC];                  // byte offset of each cell column in a row
#pragma unroll
  for (int j = 0; j < NCC; ++j) {
    const int cc = c - 1 + j;
    oc[j] = cc >= 0 && cc < Q ? chB + (unsigned)cc * colB : kOOB;
  }
  auto load_row = [&](int r, cell_t *dst) {
    const bool ok = r >= 0 && r <= r1 && r < R;
    const unsigned base = ok ? (unsigned)r * rowB : 0u;
#pragma unroll
    for (int j = 0; j < NCC; ++j) bload(rx, ok && oc[j] != kOOB ? base + oc[j] : kOOB, dst[j]);
  };

  // canonical token of frame cell (t, c + o) is affine in t for every direction
  int n0[NC];
#pragma unroll
  for (int o = 0; o < NC; ++o) n0[o] = scan_to_canon(dir, gh, gw, T, r0 * Q + (c + o < Q ? c + o : c));
  const int dn = dir == 0 ? Q : dir == 1 ? -Q : dir == 2 ? 1 : -1;
  unsigned char *yb = y + (bb * y_sb + (int64_t)ch0) * ES;

  // Two rings indexed by the local row u = t - r0 (mod 3): raw cells of the
  // rows in flight (u+1 .. u+3) and fp32 cells of the window rows (u-1 .. u+1).
  // Each cell is unpacked once, when its row enters the window.
  cell_t raw[3][NCC];
  float win[3][NCC][CH];
  auto unpack_row = [&](const cell_t *src, float (*dst)[CH]) {
#pragma unroll
    for (int e2 = 0; e2 < NCC; ++e2)
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        float v[2];
        unpack_word(word(src[e2], j), v, PW);
#pragma unroll
        for (int e = 0; e < PW; ++e) dst[e2][PW * j + e] = v[e];
      }
  };
  load_row(r0 - 1, raw[2]);
  load_row(r0, raw[0]);
  unpack_row(raw[2], win[2]);
  unpack_row(raw[0], win[0]);
  load_row(r0 + 1, raw[1]);
  load_row(r0 + 2, raw[2]);
  load_row(r0 + 3, raw[0]);

  // step for local row u with k = u mod 3: window slots (k+2)%3, k, (k+1)%3
  auto step = [&](int u, int k) {
    const int kd = (k + 1) % 3, ku = (k + 2) % 3;
    unpack_row(raw[kd], win[kd]);   // row u+1 enters the window
    load_row(r0 + u + 4, raw[kd]);  // its raw slot takes row u+4
#pragma unroll
    for (int o = 0; o < NC; ++o) {
      uint32_t out[NW];
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        float acc[2];
#pragma unroll
        for (int e = 0; e < PW; ++e) {
          const int ch = PW * j + e;
          float a = 0.f;
#pragma unroll
          for (int e2 = 0; e2 < 3; ++e2) {
            a = fmaf(wr[0 * 3 + e2][ch], win[ku][o + e2][ch], a);
            a = fmaf(wr[1 * 3 + e2][ch], win[k][o + e2][ch], a);
            a = fmaf(wr[2 * 3 + e2][ch], win[kd][o + e2][ch], a);
          }
          acc[e] = a;
        }
        out[j] = PW == 2 ? pack_bf16x2(acc[0], acc[PW - 1]) : __float_as_uint(acc[0]);
      }
      if (c + o < Q) {
        const int64_t n = n0[o] + (int64_t)u * dn;
        gstore(yb + n * y_st * ES, out, (cell_t *)nullptr);
      }
    }
  };

  // three steps per trip: every ring slot is fixed at compile time
  const int nrows = r1 - r0;
  for (int u = 0;; u += 3) {
    step(u, 0);
    if (u + 1 >= nrows) break;
    step(u + 1, 1);
    if (u + 2 >= nrows) break;
    step(u + 2, 2);
    if (u + 3 >= nrows) break;
  }
}

// Launch with walkers of NC columns.  The runs of rows are as short as keeps
// every workgroup resident at once (one round over the CUs, at the occupancy
// the kernel's registers allow) and at least 8 rows long: a second, partial
// round leaves most CUs idle while it drains, and shorter runs only add halo
// rows.
template <int NW, int PW, int NC>
hipError_t launch_walkers(const void *x, int B, int T, int C, int64_t x_sb, int64_t x_st,
                          const float *w, int gh, int gw, int dir, void *y, int64_t y_sb,
                          int64_t y_st, int num_cu, hipStream_t s) {
  constexpr int CH = NW * PW, ES = 4 / PW;
  // resident workgroups per CU: the same on every gfx950, so computed once
  // (concurrent first calls store the same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    int nb = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &nb, srem_dwconv_kernel<NW, PW, NC>, kNT, 0);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  int R, Q;
  scan_frame(dir, gh, gw, R, Q);
  const int64_t walkers = (int64_t)((Q + NC - 1) / NC) * (C / CH);   // per batch and run
  auto grid_x = [&](int64_t n) { return ((walkers * n + kNT - 1) / kNT + 7) / 8 * 8; };
  const int64_t cap = (int64_t)per_cu * num_cu;
  const int64_t nmax = (R + 7) / 8;
  int64_t nseg = 1;
  while (nseg < nmax && B * grid_x(nseg + 1) <= cap) ++nseg;
  const int rows = (int)((R + nseg - 1) / nseg);
  nseg = (R + rows - 1) / rows;
  const unsigned span = (unsigned)(((int64_t)(T - 1) * x_st + C) * ES);
  hipLaunchKernelGGL((srem_dwconv_kernel<NW, PW, NC>), dim3(grid_x(nseg), B), dim3(kNT), 0, s,
                     static_cast<const unsigned char *>(x), x_sb, x_st, w,
                     static_cast<unsigned char *>(y), y_sb, y_st, B, T, C, gh, gw, dir, rows,
                     (int)nseg, span);
  return hipGetLastError();
}

template <int ES>
__global__ void __launch_bounds__(kNT)
srem_remap_kernel(const unsigned char *x, unsigned char *y, int B, int T, int C, int gh, int gw,
                  int from, int to) {
  const int CV = C * ES / 16;
  const int64_t total = (int64_t)B * T * CV;
  const int64_t stride = (int64_t)gridDim.x * kNT;
  for (int64_t i = (int64_t)xcd_linear_block(blockIdx.x, gridDim.x) * kNT + threadIdx.x; i < total;
       i += stride) {
    const int cv = (int)(i % CV);
    const int64_t bt = i / CV;
    const int bb = (int)(bt / T);
    const int pt = (int)(bt - (int64_t)bb * T);
    const int n = scan_to_canon(to, gh, gw, T, pt);
    const int ps = canon_to_scan(from, gh, gw, T, n);
    const int64_t rowb = (int64_t)C * ES;
    *reinterpret_cast<uint4 *>(y + ((int64_t)bb * T + pt) * rowb + 16 * cv) =
        *reinterpret_cast<const uint4 *>(x + ((int64_t)bb * T + ps) * rowb + 16 * cv);
  }
}

// Row gather by a table: y[b, p] = x[b, index[p]] (16-byte copies); a table
// entry outside [0, T) gives a zero row.  Arranging rows into any scan order
// and back (an order's inverse as the table) is this one copy.
template <int ES>
__global__ void __launch_bounds__(kNT)
gather_rows_kernel(const unsigned char *x, unsigned char *y, int B, int T, int C, const int *index) {
  const int CV = C * ES / 16;
  const int64_t total = (int64_t)B * T * CV;
  const int64_t stride = (int64_t)gridDim.x * kNT;
  for (int64_t i = (int64_t)xcd_linear_block(blockIdx.x, gridDim.x) * kNT + threadIdx.x; i < total;
       i += stride) {
    const int cv = (int)(i % CV);
    const int64_t bt = i / CV;
    const int bb = (int)(bt / T);
    const int pt = (int)(bt - (int64_t)bb * T);
    const int ps = index[pt];
    const int64_t rowb = (int64_t)C * ES;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (ps >= 0 && ps < T) v = *reinterpret_cast<const uint4 *>(x + ((int64_t)bb * T + ps) * rowb + 16 * cv);
    *reinterpret_cast<uint4 *>(y + ((int64_t)bb * T + pt) * rowb + 16 * cv) = v;
  }
}

}  // namespace
}  // namespace dig

hipError_t dig_launch_gather_rows(const void *x, int dtype, int B, int T, int C, const int *index, void *y,
                                  int num_cu, hipStream_t s) {
  using namespace dig;
  const int ES = dtype == 1 ? 2 : 4;
  const int64_t total = (int64_t)B * T * (C * ES / 16);
  int64_t grid = (total + kNT - 1) / kNT;
  const int64_t cap = (int64_t)num_cu * 16;
  if (grid > cap) grid = cap;
  grid = (grid + 7) / 8 * 8;
  const auto *xp = static_cast<const unsigned char *>(x);
  auto *yp = static_cast<unsigned char *>(y);
  if (ES == 2)
    hipLaunchKernelGGL(gather_rows_kernel<2>, dim3(grid), dim3(kNT), 0, s, xp, yp, B, T, C, index);
  else
    hipLaunchKernelGGL(gather_rows_kernel<4>, dim3(grid), dim3(kNT), 0, s, xp, yp, B, T, C, index);
  return hipGetLastError();
}

hipError_t dig_launch_dwconv(const void *x, int dtype, int B, int T, int C, int64_t x_sb, int64_t x_st,
                             const float *w, int gh, int gw, int dir, void *y, int64_t y_sb,
                             int64_t y_st, int num_cu, hipStream_t s) {
  using namespace dig;
  int R, Q;
  scan_frame(dir, gh, gw, R, Q);
  if (dtype != 1)
    return launch_walkers<4, 1, 1>(x, B, T, C, x_sb, x_st, w, gh, gw, dir, y, y_sb, y_st, num_cu, s);
  // bf16: four columns per walker on wide frames; narrow ones keep two so
  // that there are still enough walkers to cover the CUs
  if (Q >= 32)
    return launch_walkers<2, 2, 4>(x, B, T, C, x_sb, x_st, w, gh, gw, dir, y, y_sb, y_st, num_cu, s);
  return launch_walkers<2, 2, 2>(x, B, T, C, x_sb, x_st, w, gh, gw, dir, y, y_sb, y_st, num_cu, s);
}

hipError_t dig_launch_remap(const void *x, int dtype, int B, int T, int C, int gh, int gw, int from,
                            int to, void *y, int num_cu, hipStream_t s) {
  using namespace dig;
  const int ES = dtype == 1 ? 2 : 4;
  const int64_t total = (int64_t)B * T * (C * ES / 16);
  int64_t grid = (total + kNT - 1) / kNT;
  const int64_t cap = (int64_t)num_cu * 16;
  if (grid > cap) grid = cap;
  grid = (grid + 7) / 8 * 8;
  if (ES == 2)
    hipLaunchKernelGGL(srem_remap_kernel<2>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const unsigned char *>(x), static_cast<unsigned char *>(y), B, T, C,
                       gh, gw, from, to);
  else
    hipLaunchKernelGGL(srem_remap_kernel<4>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const unsigned char *>(x), static_cast<unsigned char *>(y), B, T, C,
                       gh, gw, from, to);
  return hipGetLastError();
}
