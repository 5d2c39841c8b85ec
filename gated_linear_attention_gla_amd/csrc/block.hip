// block.hip -- one DiG block forward on gfx950: adaLN-Zero conditioning,
// the GLA token mixer with its projections, the FFN and the SREM conv.
//
// DiG notes, 关键设计 / DiG Block设计: (1) the summed timestep and class
// embeddings go through an MLP that regresses the adaLN parameters; (2) adaLN
// then GLA; (3) adaLN then FFN; (4) the sequence as a 2-D grid through the
// 3x3 depthwise conv; (5) the next block scans another direction; the block
// follows DiT's adaLN-Zero conditioning (DiT notes, 3.2: per-branch shift,
// scale and a gate alpha regressed from the conditioning, the gate starting
// at zero).  Per batch element b, with c[b] the conditioning:
//   [s1 | a1 | g1 | s2 | a2 | g2] = SiLU(c[b]) W_ada^T + b_ada          (6 C)
//   h  = LN(x) (1 + a1) + s1
//   q, k, v, u = h W_in^T + b_in;  q /= sqrt(d);  log_alpha = logsigmoid(u) / 16
//   o  = GLA over direction dir (scan order);  x1 = x + g1 (.) (o W_out^T + b_out)
//   h2 = LN(x1) (1 + a2) + s2;  x2 = x1 + g2 (.) (GELU(h2 W_1^T + b_1) W_2^T + b_2)
//   y  = DWConv3x3(x2 in the scan frame of dir), stored in canonical order.
// The residual stream stays in canonical token order; the mixer's scan-order
// output is gathered back inside the residual kernel.  Dense products run
// on hipBLASLt (bf16 operands, fp32 accumulation; the biases and the FFN's
// GELU in its epilogues) with its scratch in the caller's workspace; the
// other elementwise steps are the kernels below.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "dig_internal.h"

namespace dig {
namespace {

constexpr int kBT = 256;   // threads of the elementwise kernels

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(uint16_t *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ void unpack8(uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo(w[i]); f[2 * i + 1] = bf16hi(w[i]); }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ void ld8f(const float *p, float (&f)[8]) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// log sigmoid(z) = min(z, 0) - log(1 + e^{-|z|}); the log1p by its series
// below e = 0.01 (truncation < e^4 / 4), else the hardware log of 1 + e.
__device__ __forceinline__ float log_sigmoid(float z) {
  const float e = __expf(-fabsf(z));
  const float l = e < 0.01f ? e * (1.0f - e * (0.5f - e * (1.0f / 3.0f))) : __logf(1.0f + e);
  return fminf(z, 0.f) - l;
}

// SiLU(c) as the bf16 operand of the conditioning product.
__global__ void __launch_bounds__(kBT) silu_kernel(const float *c, uint16_t *cs, int n) {
  const int i = blockIdx.x * kBT + threadIdx.x;
  if (i < n) {
    const float x = c[i];
    cs[i] = (uint16_t)f2bf(x / (1.0f + expf(-x)));
  }
}

// LN statistics (mean, 1 / std with population variance) of one token row
// held as VPL 16-byte vectors per lane (vector cv = lane + 64 j, valid below CV).
template <int VPL>
__device__ __forceinline__ void row_stats(const uint4 (&raw)[VPL], int lane, int CV, int C, float eps, float &mean,
                                          float &rstd) {
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    if (lane + 64 * j < CV) {
      float f[8];
      unpack8(raw[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += f[e];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  mean = sum / (float)C;
  float sq = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    if (lane + 64 * j < CV) {
      float f[8];
      unpack8(raw[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float d = f[e] - mean; sq = fmaf(d, d, sq); }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
  rstd = 1.0f / sqrtf(sq / (float)C + eps);
}

// y[row] = (x - mean) rstd (1 + scale[b]) + shift[b] for the RPW rows of a
// wave; a lane loads its channels' scale and shift once for rows of one batch
// element (b_ada already in ada).
template <int VPL, int RPW>
__device__ __forceinline__ void modulate_out(const uint4 (&raw)[RPW][VPL], const float (&mean)[RPW],
                                             const float (&rstd)[RPW], const bool (&live)[RPW], const int (&bs)[RPW],
                                             const int64_t (&rows)[RPW], const float *ada, int C, int shift_off,
                                             int scale_off, uint16_t *__restrict__ y, int lane, int CV) {
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int cv = lane + 64 * j;
    if (cv < CV) {
      float sc[8], sh[8];
      int cur = bs[0];
      ld8f(ada + (int64_t)cur * 6 * C + scale_off + 8 * cv, sc);
      ld8f(ada + (int64_t)cur * 6 * C + shift_off + 8 * cv, sh);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (!live[r]) continue;
        if (bs[r] != cur) {
          cur = bs[r];
          ld8f(ada + (int64_t)cur * 6 * C + scale_off + 8 * cv, sc);
          ld8f(ada + (int64_t)cur * 6 * C + shift_off + 8 * cv, sh);
        }
        float f[8];
        unpack8(raw[r][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = (f[e] - mean[r]) * rstd[r] * (1.0f + sc[e]) + sh[e];
        st16(y + rows[r] * C + 8 * cv, pack8(f));
      }
    }
  }
}

// The rows of a wave: RPW consecutive token rows from row0 (past N: not live,
// clamped to row0 for loads), with their batch indices.
template <int RPW>
__device__ __forceinline__ void wave_rows(int64_t row0, int64_t N, int T, int64_t (&rows)[RPW], int (&bs)[RPW],
                                          bool (&live)[RPW]) {
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    live[r] = row0 + r < N;
    rows[r] = live[r] ? row0 + r : row0;
    bs[r] = (int)(rows[r] / T);
  }
}

// h = LN(x) (1 + scale[b]) + shift[b] per row of C channels (eps), scale/shift
// = ada[b][off..] (b_ada already added); RPW rows per wave, VPL 16-byte
// vectors per lane, the rows held in registers.
template <int VPL, int RPW>
__global__ void __launch_bounds__(kBT)
modulate_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ y, int64_t N, int T, int C,
                const float *__restrict__ ada, int shift_off, int scale_off, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * (kBT / 64) + (threadIdx.x >> 6)) * RPW;
  if (row0 >= N) return;
  const int CV = C / 8;
  int64_t rows[RPW];
  int bs[RPW];
  bool live[RPW];
  wave_rows<RPW>(row0, N, T, rows, bs, live);
  uint4 raw[RPW][VPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int cv = lane + 64 * j;
      raw[r][j] = ld16(x + rows[r] * C + 8 * (cv < CV ? cv : 0));
    }
  float mean[RPW], rstd[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) row_stats<VPL>(raw[r], lane, CV, C, eps, mean[r], rstd[r]);
  modulate_out<VPL, RPW>(raw, mean, rstd, live, bs, rows, ada, C, shift_off, scale_off, y, lane, CV);
}

// The gate quarter u (bias already added by the product) of the projected
// [N][4C] q | k | v | u rows, in place: u -> logsigmoid(u) / 16 (the log gate).
__global__ void __launch_bounds__(kBT) gate_prep_kernel(uint16_t *qkvu, uint32_t total, uint32_t V, int C) {
  for (uint32_t i = blockIdx.x * kBT + threadIdx.x; i < total; i += gridDim.x * kBT) {
    const uint32_t row = i / V;
    uint16_t *p = qkvu + (size_t)row * 4 * C + 3 * C + 8 * (i - row * V);
    float f[8];
    unpack8(ld16(p), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = log_sigmoid(f[e]) * (1.0f / 16.0f);
    st16(p, pack8(f));
  }
}

// out[b, n'] = x[b, n] + gate[b] (.) (y[b, n''] + bias), gate = ada[b][gate_off..]
// (b_ada already added).  With p the scan position of canonical token n under
// dir: gather (the mixer's scan-order output) reads y at n'' = p, scatter
// (the conv's scan-frame input) writes out at n' = p; otherwise n' = n'' = n.
__global__ void __launch_bounds__(kBT)
gated_residual_kernel(const uint16_t *x, const uint16_t *y, const float *bias, const float *ada, int gate_off,
                      uint16_t *out, uint32_t total, int T, int C, bool gather, bool scatter, int dir, int gh,
                      int gw) {
  const uint32_t V = C / 8;
  for (uint32_t i = blockIdx.x * kBT + threadIdx.x; i < total; i += gridDim.x * kBT) {
    const uint32_t row = i / V;
    const int col = 8 * (int)(i - row * V);
    const uint32_t b = row / T, n = row - b * T;
    const uint32_t p = (gather || scatter) ? (uint32_t)canon_to_scan(dir, gh, gw, T, (int)n) : n;
    const size_t base = (size_t)b * T;
    float fx[8], fy[8], g[8], bb[8];
    unpack8(ld16(x + (size_t)row * C + col), fx);
    unpack8(ld16(y + (base + (gather ? p : n)) * C + col), fy);
    ld8f(ada + (size_t)b * 6 * C + gate_off + col, g);
    ld8f(bias + col, bb);
#pragma unroll
    for (int e = 0; e < 8; ++e) fx[e] += g[e] * (fy[e] + bb[e]);
    st16(out + (base + (scatter ? p : n)) * C + col, pack8(fx));
  }
}

// The mixer's residual and the FFN's adaLN in one pass, RPW token rows per
// wave held in registers: x1 = x + g1 (.) (y[b, p] + bias) with p the scan
// position of the row's token under dir (the mixer's scan-order output),
// stored; then h = LN(x1) (1 + a2) + s2 over the stored (bf16) x1, as
// modulate_kernel.
template <int VPL, int RPW>
__global__ void __launch_bounds__(kBT)
residual_modulate_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ y,
                         const float *__restrict__ bias, const float *__restrict__ ada, int gate_off, int shift_off,
                         int scale_off, float eps, uint16_t *__restrict__ x1, uint16_t *__restrict__ h, int64_t N,
                         int T, int C, int dir, int gh, int gw) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * (kBT / 64) + (threadIdx.x >> 6)) * RPW;
  if (row0 >= N) return;
  const int CV = C / 8;
  int64_t rows[RPW], src[RPW];
  int bs[RPW];
  bool live[RPW];
  wave_rows<RPW>(row0, N, T, rows, bs, live);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = (int)(rows[r] - (int64_t)bs[r] * T);
    src[r] = (int64_t)bs[r] * T + canon_to_scan(dir, gh, gw, T, n);
  }
  uint4 raw[RPW][VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int cv = lane + 64 * j;
    const int c8 = 8 * (cv < CV ? cv : 0);
    uint4 ux[RPW], uy[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      ux[r] = ld16(x + rows[r] * C + c8);
      uy[r] = ld16(y + src[r] * C + c8);
    }
    float g[8], bb[8];
    int cur = bs[0];
    ld8f(ada + (int64_t)cur * 6 * C + gate_off + c8, g);
    ld8f(bias + c8, bb);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (bs[r] != cur) {
        cur = bs[r];
        ld8f(ada + (int64_t)cur * 6 * C + gate_off + c8, g);
      }
      float fx[8], fy[8];
      unpack8(ux[r], fx);
      unpack8(uy[r], fy);
#pragma unroll
      for (int e = 0; e < 8; ++e) fx[e] += g[e] * (fy[e] + bb[e]);
      raw[r][j] = pack8(fx);
      if (cv < CV && live[r]) st16(x1 + rows[r] * C + c8, raw[r][j]);
    }
  }
  float mean[RPW], rstd[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) row_stats<VPL>(raw[r], lane, CV, C, eps, mean[r], rstd[r]);
  modulate_out<VPL, RPW>(raw, mean, rstd, live, bs, rows, ada, C, shift_off, scale_off, h, lane, CV);
}

// Zero fill (uint4 granules) -- a kernel rather than a memset node.
__global__ void __launch_bounds__(kBT) zero_kernel(uint4 *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBT)
    p[i] = make_uint4(0, 0, 0, 0);
}

int ew_grid(int64_t items, int num_cu) {
  int64_t g = (items + kBT - 1) / kBT;
  const int64_t cap = (int64_t)num_cu * 16;
  return (int)(g < cap ? (g < 1 ? 1 : g) : cap);
}

// Dense products on hipBLASLt: one handle per device and one plan (matmul
// descriptor, layouts, algorithm) per shape, output type and epilogue,
// created on first use and kept.  The plan's algorithm is the fastest of the
// heuristic's candidates, each timed on the first call's own operands and
// stream (that first call waits for the stream).  The mutex also covers the
// per-call bias and launch, since a plan's descriptor holds the bias pointer.
enum class Epi { none, bias, gelu_bias };
struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo{};
};
std::mutex g_lt_mu;
hipblasLtHandle_t g_lt[64] = {};
std::map<std::tuple<int, int, int, int, bool, int, size_t>, Plan> g_plans;

constexpr int kCandidates = 8;
constexpr double kTimeFlops = 1e10;
constexpr int kTimedRuns = 10;   // after one untimed run; short products need several to rise above launch jitter

hipError_t make_plan(hipblasLtHandle_t h, int M, int N, int K, bool y_f32, Epi epi, const void *X, const void *W,
                     void *Y, const float *bias, float alpha, void *scratch, size_t scratch_bytes, hipStream_t s,
                     Plan &P) {
  // Row-major Y[M][N] = X[M][K] W[N][K]^T is column-major D (N x M) = op(A) B with
  // A = W seen as a K x N column-major matrix (op = transpose) and B = X as K x M;
  // the bias runs along D's rows, the output features.
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  const hipDataType yt = y_f32 ? HIP_R_32F : HIP_R_16BF, bt = HIP_R_32F;
  const uint32_t e = epi == Epi::none ? HIPBLASLT_EPILOGUE_DEFAULT
                     : epi == Epi::bias ? HIPBLASLT_EPILOGUE_BIAS
                                        : HIPBLASLT_EPILOGUE_GELU_BIAS;
  bool ok = hipblasLtMatmulDescCreate(&P.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &e, sizeof(e)) ==
                HIPBLAS_STATUS_SUCCESS;
  if (ok && epi != Epi::none)
    ok = hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof(bt)) ==
         HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&P.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&P.lb, HIP_R_16BF, K, M, K) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&P.ld, yt, N, M, N) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &scratch_bytes,
                                             sizeof(scratch_bytes)) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int got = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, P.desc, P.la, P.lb, P.ld, P.ld, pref, kCandidates, res, &got) ==
                 HIPBLAS_STATUS_SUCCESS &&
       got > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS;
  if (ok && epi != Epi::none)
    ok = hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) ==
         HIPBLAS_STATUS_SUCCESS;
  // Products under kTimeFlops run for about as long as their launch takes, so
  // event timing would measure the host, not the candidates: the heuristic's
  // first choice then.  No timing either while the stream is being captured
  // into a graph (the trial products would become graph nodes).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) cap = hipStreamCaptureStatusActive;
  int best = 0;
  if (ok && got > 1 && cap == hipStreamCaptureStatusNone && 2.0 * M * N * K >= kTimeFlops) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    float best_ms = 3.4e38f;
    const float beta = 0.f;
    if (hipEventCreate(&e0) == hipSuccess && hipEventCreate(&e1) == hipSuccess) {
      for (int c = 0; c < got; ++c) {
        if (res[c].state != HIPBLAS_STATUS_SUCCESS) continue;
        bool run = true;
        for (int r = 0; r < 1 + kTimedRuns && run; ++r) {
          if (r == 1) run = hipEventRecord(e0, s) == hipSuccess;
          run = run && hipblasLtMatmul(h, P.desc, &alpha, W, P.la, X, P.lb, &beta, Y, P.ld, Y, P.ld, &res[c].algo,
                                       scratch, scratch_bytes, s) == HIPBLAS_STATUS_SUCCESS;
        }
        float ms = 0.f;
        if (run && hipEventRecord(e1, s) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
            hipEventElapsedTime(&ms, e0, e1) == hipSuccess && ms < best_ms) {
          best_ms = ms;
          best = c;
        }
      }
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipGetLastError();
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (!ok) {
    if (P.la) hipblasLtMatrixLayoutDestroy(P.la);
    if (P.lb) hipblasLtMatrixLayoutDestroy(P.lb);
    if (P.ld) hipblasLtMatrixLayoutDestroy(P.ld);
    if (P.desc) hipblasLtMatmulDescDestroy(P.desc);
    P = Plan{};
    return hipErrorNotSupported;
  }
  P.algo = res[best].algo;
  return hipSuccess;
}

// Y[M][N] = alpha X[M][K] W[N][K]^T (+ bias[N], then GELU per epi), row-major,
// bf16 operands, fp32 accumulation, Y bf16 or fp32; scratch: the library's
// workspace (device memory of scratch_bytes).
hipError_t gemm(const void *X, const void *W, void *Y, bool y_f32, int M, int N, int K, Epi epi, const float *bias,
                float alpha, void *scratch, size_t scratch_bytes, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_lt_mu);
  if (!g_lt[dev] && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) return hipErrorUnknown;
  const auto key = std::make_tuple(dev, M, N, K, y_f32, (int)epi, scratch_bytes);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) {
    Plan P;
    if ((e = make_plan(g_lt[dev], M, N, K, y_f32, epi, X, W, Y, bias, alpha, scratch, scratch_bytes, s, P)) !=
        hipSuccess)
      return e;
    it = g_plans.emplace(key, P).first;
  }
  const Plan &P = it->second;
  if (epi != Epi::none &&
      hipblasLtMatmulDescSetAttribute(P.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias)) !=
          HIPBLAS_STATUS_SUCCESS)
    return hipErrorUnknown;
  const float beta = 0.f;
  return hipblasLtMatmul(g_lt[dev], P.desc, &alpha, W, P.la, X, P.lb, &beta, Y, P.ld, Y, P.ld, &P.algo, scratch,
                         scratch_bytes, s) == HIPBLAS_STATUS_SUCCESS
             ? hipSuccess
             : hipErrorUnknown;
}

}  // namespace
}  // namespace dig

// ------------------------------------------------------------------ host side
namespace {
constexpr size_t kGemmScratch = DIG_GEMM_SCRATCH;   // hipBLASLt scratch inside the workspace
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
// the bf16 GLA's chunk for this head size (64 while its LDS plan holds it)
int block_chunk(int d) { return d <= 96 ? 64 : 32; }

struct BlockLayout {
  size_t ada, cs, h, qkvu, o, o2, x1, x2, gla, gemm, bytes;
};
BlockLayout block_layout(int B, int T, int C, int H, int num_cu) {
  BlockLayout L{};
  const size_t tok = (size_t)B * T, e = 2;
  size_t off = 0;
  auto take = [&](size_t n) { const size_t o = off; off += up256(n); return o; };
  L.ada = take((size_t)B * 6 * C * 4);
  L.cs = take((size_t)B * C * e);
  L.h = take(tok * C * e);          // h, then h2
  L.qkvu = take(tok * 4 * C * e);   // q | k | v | log gate, then the FFN's hidden layer
  L.o = take(tok * C * e);          // GLA output (scan order), then the FFN output
  L.o2 = take(tok * C * e);         // out-projection (scan order)
  L.x1 = take(tok * C * e);
  L.x2 = take(tok * C * e);         // x2 in the scan order of dir (the conv's input)
  const int d = C / H;
  L.gla = take(dig_gla_bf16_workspace(B, T, H, d, d, block_chunk(d), num_cu));
  L.gemm = take(kGemmScratch);
  L.bytes = off;
  return L;
}
}  // namespace

size_t dig_block_workspace(int B, int T, int C, int H, int num_cu) {
  return block_layout(B, T, C, H, num_cu).bytes;
}

hipError_t dig_launch_linear(const void *x, const void *w, void *y, int M, int N, int K, void *scratch,
                             size_t scratch_bytes, hipStream_t s) {
  return dig::gemm(x, w, y, false, M, N, K, dig::Epi::none, nullptr, 1.0f, scratch, scratch_bytes, s);
}

hipError_t dig_launch_block(const DigBlockArgs &a, hipStream_t s) {
  using namespace dig;
  const int B = a.B, T = a.T, C = a.C, H = a.H, d = C / H;
  const int64_t N = (int64_t)B * T;
  const BlockLayout L = block_layout(B, T, C, H, a.num_cu);
  unsigned char *ws = static_cast<unsigned char *>(a.workspace);
  float *ada = reinterpret_cast<float *>(ws + L.ada);
  uint16_t *cs = reinterpret_cast<uint16_t *>(ws + L.cs);
  uint16_t *h = reinterpret_cast<uint16_t *>(ws + L.h), *qkvu = reinterpret_cast<uint16_t *>(ws + L.qkvu);
  uint16_t *o = reinterpret_cast<uint16_t *>(ws + L.o), *o2 = reinterpret_cast<uint16_t *>(ws + L.o2);
  uint16_t *x1 = reinterpret_cast<uint16_t *>(ws + L.x1), *x2 = reinterpret_cast<uint16_t *>(ws + L.x2);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  hipError_t e;
  auto G = [&](const void *X, const void *W, void *Y, bool f32, int M, int Nn, int K, Epi epi, const float *bias,
               float alpha = 1.0f) {
    return gemm(X, W, Y, f32, M, Nn, K, epi, bias, alpha, ws + L.gemm, kGemmScratch, s);
  };
  const int vpl = (C / 8 + 63) / 64;
  // two rows per wave while the rows fit the registers (VPL <= 4: C <= 2048)
  auto modulate = [&](const uint16_t *in, uint16_t *out, int shift_off, int scale_off) {
#define DIG_MOD_CASE(V, R)                                                                                  \
  if (vpl <= V) {                                                                                           \
    const int grid = (int)((N + 4 * R - 1) / (4 * R));                                                      \
    hipLaunchKernelGGL((modulate_kernel<V, R>), dim3(grid), dim3(kBT), 0, s, in, out, N, T, C, ada, shift_off, \
                       scale_off, 1e-6f);                                                                   \
    return hipGetLastError();                                                                               \
  }
    DIG_MOD_CASE(1, 2)
    DIG_MOD_CASE(2, 2)
    DIG_MOD_CASE(3, 2)
    DIG_MOD_CASE(4, 2)
    DIG_MOD_CASE(8, 1)
    DIG_MOD_CASE(16, 1)
    DIG_MOD_CASE(32, 1)
#undef DIG_MOD_CASE
    return hipErrorInvalidValue;
  };
  auto residual_modulate = [&]() {
#define DIG_RM_CASE(V, R)                                                                                    \
  if (vpl <= V) {                                                                                            \
    const int grid = (int)((N + 4 * R - 1) / (4 * R));                                                       \
    hipLaunchKernelGGL((residual_modulate_kernel<V, R>), dim3(grid), dim3(kBT), 0, s, x, o2, a.b_out, ada, 2 * C, \
                       3 * C, 4 * C, 1e-6f, x1, h, N, T, C, a.dir, a.gh, a.gw);                              \
    return hipGetLastError();                                                                                \
  }
    DIG_RM_CASE(1, 2)
    DIG_RM_CASE(2, 2)
    DIG_RM_CASE(3, 2)
    DIG_RM_CASE(4, 2)
    DIG_RM_CASE(8, 1)
    DIG_RM_CASE(16, 1)
    DIG_RM_CASE(32, 1)
#undef DIG_RM_CASE
    return hipErrorInvalidValue;
  };

  // The GLA's part of the workspace (its ticket counters and launch-tagged
  // flags must start at zero) sits at a shape-dependent offset, so a
  // workspace reused across shapes may hold other data there: clear it.
  {
    const int64_t n16 = (int64_t)(L.gemm - L.gla) / 16;
    hipLaunchKernelGGL(zero_kernel, dim3(ew_grid(n16, a.num_cu)), dim3(kBT), 0, s,
                       reinterpret_cast<uint4 *>(ws + L.gla), n16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // (1) conditioning -> [s1 | a1 | g1 | s2 | a2 | g2] (fp32, b_ada added by the product)
  hipLaunchKernelGGL(silu_kernel, dim3((B * C + kBT - 1) / kBT), dim3(kBT), 0, s, a.c, cs, B * C);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = G(cs, a.w_ada, ada, true, B, 6 * C, C, Epi::bias, a.b_ada)) != hipSuccess) return e;
  // (2) mixer: adaLN, projections, GLA over dir, out-projection, gated residual
  if ((e = modulate(x, h, 0, C)) != hipSuccess) return e;
  // q | k | v | u + b_in; q's 1 / sqrt(d) is taken by the out-projection's alpha
  // (the mixer's output is linear in q)
  if ((e = G(h, a.w_in, qkvu, false, (int)N, 4 * C, C, Epi::bias, a.b_in)) != hipSuccess) return e;
  hipLaunchKernelGGL(gate_prep_kernel, dim3(ew_grid(N * C / 8, a.num_cu)), dim3(kBT), 0, s, qkvu,
                     (uint32_t)(N * C / 8), (uint32_t)(C / 8), C);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  DigGlaArgs g{};
  g.q = qkvu; g.k = qkvu + C; g.v = qkvu + 2 * C; g.g = qkvu + 3 * C;
  g.qk_sb = (int64_t)T * 4 * C; g.qk_st = 4 * C; g.qk_sh = d;
  g.v_sb = g.qk_sb; g.v_st = g.qk_st; g.v_sh = d;
  g.o = o; g.o_sb = (int64_t)T * C; g.o_st = C; g.o_sh = d;
  g.s0 = nullptr; g.s_final = nullptr;
  g.B = B; g.T = T; g.H = H; g.dk = d; g.dv = d; g.gh = a.gh; g.gw = a.gw; g.dir = a.dir; g.chunk = block_chunk(d);
  g.order = nullptr;
  g.workspace = ws + L.gla; g.workspace_bytes = L.gemm - L.gla;
  g.epoch = a.epoch; g.num_cu = a.num_cu;
  if ((e = dig_launch_gla_bf16(g, s)) != hipSuccess) return e;
  if ((e = G(o, a.w_out, o2, false, (int)N, C, C, Epi::none, nullptr, 1.0f / sqrtf((float)d))) != hipSuccess)
    return e;
  // x1 = x + g1 (.) (o2 gathered to canonical order + b_out), and (3) the FFN's
  // adaLN of x1, in one pass; then C -> 4C, GELU, 4C -> C, gated residual
  if ((e = residual_modulate()) != hipSuccess) return e;
  const int egrid = ew_grid(N * C / 8, a.num_cu);
  if ((e = G(h, a.w_ff1, qkvu, false, (int)N, 4 * C, C, Epi::gelu_bias, a.b_ff1)) != hipSuccess) return e;
  if ((e = G(qkvu, a.w_ff2, o, false, (int)N, C, 4 * C, Epi::none, nullptr)) != hipSuccess) return e;
  // x2 goes out in the scan order of dir: the conv's input
  hipLaunchKernelGGL(gated_residual_kernel, dim3(egrid), dim3(kBT), 0, s, x1, o, a.b_ff2, ada, 5 * C, x2,
                     (uint32_t)(N * C / 8), T, C, false, true, a.dir, a.gh, a.gw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // (4) SREM: the 3x3 depthwise conv of the scan frame of dir, stored in
  //     canonical order
  return dig_launch_dwconv(x2, 1, B, T, C, (int64_t)T * C, C, a.w_conv, a.gh, a.gw, a.dir, a.y,
                           (int64_t)T * C, C, a.num_cu, s);
}
