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
// Work split: a thread owns one 16-byte channel group (8 bf16 / 4 fp32) of one
// frame column and a run of frame rows; its 9 x VEC fp32 weights sit in
// registers and a 3x3 window slides down the column, so every input row is
// fetched once per walker (three columns wide).  Workgroups are ordered so
// that each XCD sweeps neighbouring columns, whose shared cells hit its L2.
#include "dig_internal.h"

namespace dig {
namespace {

template <int VEC>
struct Vec;
template <>
struct Vec<8> {   // bf16
  static __device__ __forceinline__ void load(const void *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) { f[2 * e] = bf16lo(w[e]); f[2 * e + 1] = bf16hi(w[e]); }
  }
  static __device__ __forceinline__ void store(void *p, const float *f) {
    *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                               pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  static constexpr int esize = 2;
};
template <>
struct Vec<4> {   // fp32
  static __device__ __forceinline__ void load(const void *p, float *f) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w;
  }
  static __device__ __forceinline__ void store(void *p, const float *f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
  static constexpr int esize = 4;
};

constexpr int kNT = 256;

template <int VEC>
__global__ void __launch_bounds__(kNT)
srem_dwconv_kernel(const unsigned char *x, int64_t x_sb, int64_t x_st, const float *w,
                   unsigned char *y, int64_t y_sb, int64_t y_st, int B, int T, int C,
                   int gh, int gw, int dir, int rows_per_walker, int nseg) {
  // A walker owns (batch, frame column c, channel group, run of frame rows)
  // and slides a 3x3 register window down its column: each step loads the
  // three new cells of the next row and stores one output token.
  constexpr int ES = Vec<VEC>::esize;
  const int CV = C / VEC;
  int R, Q;
  scan_frame(dir, gh, gw, R, Q);
  const int64_t id = (int64_t)xcd_linear_block(blockIdx.x, gridDim.x) * kNT + threadIdx.x;
  const int64_t total = (int64_t)B * Q * CV * nseg;
  if (id >= total) return;
  const int cv = (int)(id % CV);
  int64_t rest = id / CV;
  const int c = (int)(rest % Q);
  rest /= Q;
  const int seg = (int)(rest % nseg);
  const int bb = (int)(rest / nseg);
  const int r0 = seg * rows_per_walker;
  const int r1 = r0 + rows_per_walker < R ? r0 + rows_per_walker : R;
  if (r0 >= r1) return;
  const int ch0 = cv * VEC;

  float wr[9][VEC];
#pragma unroll
  for (int tap = 0; tap < 9; ++tap)
#pragma unroll
    for (int e = 0; e < VEC; ++e) wr[tap][e] = w[(ch0 + e) * 9 + tap];

  const unsigned char *xb = x + (bb * x_sb + (int64_t)ch0) * ES;
  auto load_row = [&](int r, float (*dst)[VEC]) {
#pragma unroll
    for (int e2 = 0; e2 < 3; ++e2) {
      const int cc = c + e2 - 1;
      if (r >= 0 && r < R && cc >= 0 && cc < Q) {
        Vec<VEC>::load(xb + (int64_t)(r * Q + cc) * x_st * ES, dst[e2]);
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[e2][e] = 0.f;
      }
    }
  };
  float top[3][VEC], mid[3][VEC], bot[3][VEC];
  load_row(r0 - 1, top);
  load_row(r0, mid);
  for (int r = r0; r < r1; ++r) {
    load_row(r + 1, bot);
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float a = 0.f;
#pragma unroll
      for (int e2 = 0; e2 < 3; ++e2) {
        a = fmaf(wr[0 * 3 + e2][e], top[e2][e], a);
        a = fmaf(wr[1 * 3 + e2][e], mid[e2][e], a);
        a = fmaf(wr[2 * 3 + e2][e], bot[e2][e], a);
      }
      acc[e] = a;
    }
    const int n = scan_to_canon(dir, gh, gw, T, r * Q + c);
    Vec<VEC>::store(y + (bb * y_sb + (int64_t)n * y_st + ch0) * ES, acc);
#pragma unroll
    for (int e2 = 0; e2 < 3; ++e2)
#pragma unroll
      for (int e = 0; e < VEC; ++e) { top[e2][e] = mid[e2][e]; mid[e2][e] = bot[e2][e]; }
  }
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

}  // namespace
}  // namespace dig

hipError_t dig_launch_dwconv(const void *x, int dtype, int B, int T, int C, int64_t x_sb, int64_t x_st,
                             const float *w, int gh, int gw, int dir, void *y, int64_t y_sb,
                             int64_t y_st, int num_cu, hipStream_t s) {
  using namespace dig;
  const int VEC = dtype == 1 ? 8 : 4;
  const int CV = C / VEC;
  int R, Q;
  scan_frame(dir, gh, gw, R, Q);
  // rows per walker: enough walkers for ~8 workgroups per CU, at least 4 rows
  const int64_t cols = (int64_t)B * Q * CV;
  const int64_t want_threads = (int64_t)num_cu * 8 * kNT;
  int64_t nseg = (want_threads + cols - 1) / cols;
  if (nseg > (R + 3) / 4) nseg = (R + 3) / 4;
  if (nseg < 1) nseg = 1;
  const int rows = (int)((R + nseg - 1) / nseg);
  nseg = (R + rows - 1) / rows;
  const int64_t total = cols * nseg;
  const int64_t grid = ((total + kNT - 1) / kNT + 7) / 8 * 8;
  if (dtype == 1)
    hipLaunchKernelGGL(srem_dwconv_kernel<8>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const unsigned char *>(x), x_sb, x_st, w,
                       static_cast<unsigned char *>(y), y_sb, y_st, B, T, C, gh, gw, dir, rows, (int)nseg);
  else
    hipLaunchKernelGGL(srem_dwconv_kernel<4>, dim3(grid), dim3(kNT), 0, s,
                       static_cast<const unsigned char *>(x), x_sb, x_st, w,
                       static_cast<unsigned char *>(y), y_sb, y_st, B, T, C, gh, gw, dir, rows, (int)nseg);
  return hipGetLastError();
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
