// gla_f32.hip -- fp32 chunk-wise GLA forward on the vector ALUs.
//
// Same chunk decomposition as the bf16 MFMA kernel (DiG paper notes,
// 关键设计 / 硬件友好的效率设计), evaluated entirely in fp32 for the fp32
// input path: per chunk of M tokens, with b the inclusive cumulative log2-gate
// from the chunk start,
//   P[t][s] = sum_i q_ti k_si 2^(b_ti - b_si)          (s <= t, exact exponent
//                                                       differences: no
//                                                       factorisation, so any
//                                                       finite log-gate works)
//   o_t     = sum_{s<=t} P[t][s] v_s + (q_t * 2^b_t) S
//   S'      = diag(2^b_last) S + sum_s (k_s * 2^(b_last - b_s))^T v_s
// One workgroup of 256 threads per (batch, head); q, k, gates, v, P and the
// fp32 state S live in LDS.  Any strides and any d <= 128 are accepted.
#include "dig_internal.h"

namespace dig {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNT = 256;

struct Params {
  const float *q, *k, *v, *g;
  float *o;
  const float *s0;
  float *s_final;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  int T, H, dk, dv, gh, gw, dir, M, nchunks, units;
  const int *order;   // nullable: scan position -> canonical token [T]
};

// Canonical token at scan position p (p < T), or -1 for a table entry
// outside [0, T) (that token then reads as zeros).
__device__ __forceinline__ int64_t token_at(const Params &P, int p) {
  if (P.order) {
    const int n = P.order[p];
    return (n >= 0 && n < P.T) ? n : -1;
  }
  return scan_to_canon(P.dir, P.gh, P.gw, P.T, p);
}

__global__ void __launch_bounds__(kNT) gla_fwd_f32_kernel(Params P) {
  extern __shared__ __align__(16) float sm[];
  const int M = P.M, dk = P.dk, dv = P.dv, T = P.T;
  float *sq = sm;               // [M][dk]
  float *sk = sq + M * dk;      // [M][dk]
  float *sb = sk + M * dk;      // [M][dk] gates -> cumulative (log2 units)
  float *sv = sb + M * dk;      // [M][dv]
  float *sP = sv + M * dv;      // [M][M]
  float *sS = sP + M * M;       // [dk][dv]

  const int unit = blockIdx.x;
  if (unit >= P.units) return;
  const int b = unit / P.H, h = unit - b * P.H;
  const int tid = threadIdx.x;
  const float *qb = P.q + b * P.qk_sb + h * P.qk_sh;
  const float *kb = P.k + b * P.qk_sb + h * P.qk_sh;
  const float *gb = P.g + b * P.qk_sb + h * P.qk_sh;
  const float *vb = P.v + b * P.v_sb + h * P.v_sh;
  float *ob = P.o + b * P.o_sb + h * P.o_sh;

  for (int x = tid; x < dk * dv; x += kNT) sS[x] = P.s0 ? P.s0[(int64_t)unit * dk * dv + x] : 0.f;

  for (int c = 0; c < P.nchunks; ++c) {
    __syncthreads();
    for (int x = tid; x < M * dk; x += kNT) {
      const int t = x / dk, i = x - t * dk, p = c * M + t;
      const int64_t n = p < T ? token_at(P, p) : -1;
      if (n >= 0) {
        sq[x] = qb[n * P.qk_st + i];
        sk[x] = kb[n * P.qk_st + i];
        sb[x] = gb[n * P.qk_st + i] * kLog2e;
      } else {
        sq[x] = 0.f; sk[x] = 0.f; sb[x] = 0.f;
      }
    }
    for (int x = tid; x < M * dv; x += kNT) {
      const int t = x / dv, j = x - t * dv, p = c * M + t;
      const int64_t n = p < T ? token_at(P, p) : -1;
      sv[x] = n >= 0 ? vb[n * P.v_st + j] : 0.f;
    }
    __syncthreads();
    if (tid < dk) {
      float run = 0.f;
      for (int t = 0; t < M; ++t) {
        run += sb[t * dk + tid];
        sb[t * dk + tid] = run;
      }
    }
    __syncthreads();
    for (int x = tid; x < M * M; x += kNT) {
      const int t = x / M, s = x - t * M;
      float acc = 0.f;
      if (s <= t)
        for (int i = 0; i < dk; ++i) acc += sq[t * dk + i] * sk[s * dk + i] * exp2f(sb[t * dk + i] - sb[s * dk + i]);
      sP[x] = acc;
    }
    __syncthreads();
    for (int x = tid; x < M * dv; x += kNT) {
      const int t = x / dv, j = x - t * dv, p = c * M + t;
      float acc = 0.f;
      for (int s = 0; s <= t; ++s) acc += sP[t * M + s] * sv[s * dv + j];
      for (int i = 0; i < dk; ++i) acc += sq[t * dk + i] * exp2f(sb[t * dk + i]) * sS[i * dv + j];
      if (p < T) ob[(int64_t)p * P.o_st + j] = acc;
    }
    __syncthreads();
    const float *bl = sb + (M - 1) * dk;
    for (int x = tid; x < dk * dv; x += kNT) {
      const int i = x / dv, j = x - i * dv;
      float acc = exp2f(bl[i]) * sS[x];
      for (int s = 0; s < M; ++s) acc += sk[s * dk + i] * exp2f(bl[i] - sb[s * dk + i]) * sv[s * dv + j];
      sS[x] = acc;
    }
  }
  __syncthreads();
  if (P.s_final)
    for (int x = tid; x < dk * dv; x += kNT) P.s_final[(int64_t)unit * dk * dv + x] = sS[x];
}

}  // namespace
}  // namespace dig

size_t dig_gla_f32_lds_bytes(int dk, int dv, int M) {
  return sizeof(float) * ((size_t)3 * M * dk + (size_t)M * dv + (size_t)M * M + (size_t)dk * dv);
}

hipError_t dig_launch_gla_f32(const DigGlaArgs &a, hipStream_t s) {
  using namespace dig;
  Params p;
  p.q = static_cast<const float *>(a.q);
  p.k = static_cast<const float *>(a.k);
  p.v = static_cast<const float *>(a.v);
  p.g = static_cast<const float *>(a.g);
  p.o = static_cast<float *>(a.o);
  p.s0 = a.s0;
  p.s_final = a.s_final;
  p.qk_sb = a.qk_sb; p.qk_st = a.qk_st; p.qk_sh = a.qk_sh;
  p.v_sb = a.v_sb; p.v_st = a.v_st; p.v_sh = a.v_sh;
  p.o_sb = a.o_sb; p.o_st = a.o_st; p.o_sh = a.o_sh;
  p.T = a.T; p.H = a.H; p.dk = a.dk; p.dv = a.dv;
  p.gh = a.gh; p.gw = a.gw; p.dir = a.dir;
  p.order = a.order;
  p.M = a.chunk;
  p.nchunks = (a.T + a.chunk - 1) / a.chunk;
  p.units = a.B * a.H;
  const size_t lds = dig_gla_f32_lds_bytes(a.dk, a.dv, a.chunk);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gla_fwd_f32_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gla_fwd_f32_kernel, dim3(p.units), dim3(kNT), lds, s, p);
  return hipGetLastError();
}
