// adaln.hip -- adaLN modulation in front of the token mixer.
//
// DiG paper notes, 关键设计 / DiG Block设计 step (2): the block normalises its
// input with adaLN before the GLA; DiT notes, 3.2: adaLN regresses the norm's
// scale and shift from the conditioning, and adaLN-Zero starts from the
// identity, hence the (1 + scale) form.  Per row (token) of C channels:
//   y = ((x - mean) / sqrt(var + eps) * (1 + scale) + shift) * out_scale
// with the population mean/variance, all in fp32, two passes over the row
// held in registers (no E[x^2] - E[x]^2 cancellation).
//
// One wave per two rows; 16-byte vectors (8 bf16 / 4 fp32) per lane; VPL
// vectors per lane chosen at launch from C.  The raw rows stay in registers
// and are unpacked at each use.  Workgroups of 4 waves, XCD-ordered.
#include "dig_internal.h"

namespace dig {
namespace {

constexpr int kWaves = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Rows a wave normalises side by side: each lane's 1 + scale and shift are
// loaded once for both rows (per row they are 4x the row's own bytes, read
// from cache: one row per wave ran at 4.0 TB/s, two at 5.0).
constexpr int kRows = 2;

template <bool BF16, int VPL>
__global__ void __launch_bounds__(kWaves * kWave)
adaln_kernel(const unsigned char *x, int64_t x_sn, const float *scale, const float *shift, float eps,
             float out_scale, unsigned char *y, int64_t y_sn, int64_t N, int C) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int ES = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)xcd_linear_block(blockIdx.x, gridDim.x) * kWaves + (threadIdx.x >> 6)) * kRows;
  if (row0 >= N) return;
  const int CV = C / VEC;
  // vector j of a row: channels VEC (lane + 64 j) ..; a lane past CV reads
  // vector 0 and drops it, a row past N reads row N - 1 and is not written
  uint4 raw[kRows][VPL];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int64_t row = row0 + k < N ? row0 + k : N - 1;
    const unsigned char *xr = x + row * x_sn * ES;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int cv = lane + 64 * j;
      raw[k][j] = *reinterpret_cast<const uint4 *>(xr + 16 * (cv < CV ? cv : 0));
    }
  }
  auto elem = [&](const uint4 &u, int e) {
    const uint32_t w = e < 2 * (VEC / 4) ? (e < VEC / 4 ? u.x : u.y) : (e < 3 * (VEC / 4) ? u.z : u.w);
    if (BF16) return (e & 1) ? bf16hi(w) : bf16lo(w);
    return __uint_as_float(w);
  };
  float mean[kRows], rstd[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < CV) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sum += elem(raw[k][j], e);
      }
    mean[k] = wave_sum(sum) / (float)C;
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (lane + 64 * j < CV) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) { const float d = elem(raw[k][j], e) - mean[k]; sq = fmaf(d, d, sq); }
      }
    rstd[k] = 1.0f / sqrtf(wave_sum(sq) / (float)C + eps);
  }
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int cv = lane + 64 * j;
    if (cv < CV) {
      float g1[VEC], sh[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) { g1[e] = 1.0f + scale[cv * VEC + e]; sh[e] = shift[cv * VEC + e]; }
#pragma unroll
      for (int k = 0; k < kRows; ++k) {
        if (row0 + k >= N) break;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = ((elem(raw[k][j], e) - mean[k]) * rstd[k] * g1[e] + sh[e]) * out_scale;
        unsigned char *yr = y + (row0 + k) * y_sn * ES;
        if (BF16) {
          *reinterpret_cast<uint4 *>(yr + 16 * cv) =
              make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                         pack_bf16x2(o[6], o[7]));
        } else {
          *reinterpret_cast<float4 *>(yr + 16 * cv) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  }
}

template <bool BF16>
hipError_t launch(const void *x, int64_t N, int C, int64_t x_sn, const float *scale, const float *shift,
                  float eps, float out_scale, void *y, int64_t y_sn, hipStream_t s) {
  const int VEC = BF16 ? 8 : 4;
  const int vpl = (C / VEC + 63) / 64;
  const int64_t grid = ((N + kWaves * kRows - 1) / (kWaves * kRows) + 7) / 8 * 8;
  const auto *xp = static_cast<const unsigned char *>(x);
  auto *yp = static_cast<unsigned char *>(y);
#define DIG_ADALN_CASE(V)                                                                        \
  if (vpl <= V) {                                                                                \
    hipLaunchKernelGGL((adaln_kernel<BF16, V>), dim3(grid), dim3(kWaves * kWave), 0, s, xp, x_sn, \
                       scale, shift, eps, out_scale, yp, y_sn, N, C);                            \
    return hipGetLastError();                                                                    \
  }
  DIG_ADALN_CASE(1)
  DIG_ADALN_CASE(2)
  DIG_ADALN_CASE(3)
  DIG_ADALN_CASE(4)
  DIG_ADALN_CASE(8)
  DIG_ADALN_CASE(16)
  DIG_ADALN_CASE(32)
#undef DIG_ADALN_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace dig

hipError_t dig_launch_adaln(const void *x, int dtype, int64_t N, int C, int64_t x_sn, const float *scale,
                            const float *shift, float eps, float out_scale, void *y, int64_t y_sn,
                            hipStream_t s) {
  if (dtype == 1) return dig::launch<true>(x, N, C, x_sn, scale, shift, eps, out_scale, y, y_sn, s);
  return dig::launch<false>(x, N, C, x_sn, scale, shift, eps, out_scale, y, y_sn, s);
}
