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
// on rocBLAS (bf16 operands, fp32 accumulation) with its scratch in the
// caller's workspace; the elementwise steps are the kernels below.
#include <rocblas/rocblas.h>

#include <mutex>

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

// SiLU(c) as the bf16 operand of the conditioning product.
__global__ void __launch_bounds__(kBT) silu_kernel(const float *c, uint16_t *cs, int n) {
  const int i = blockIdx.x * kBT + threadIdx.x;
  if (i < n) {
    const float x = c[i];
    cs[i] = (uint16_t)f2bf(x / (1.0f + expf(-x)));
  }
}

// y = LN(x) (1 + scale[b]) + shift[b] per row of C channels (population
// variance, eps), scale/shift = ada[b][off..] + b_ada[off..]; one wave per
// row, VPL 16-byte vectors per lane, the row held in registers.
template <int VPL>
__global__ void __launch_bounds__(kBT)
modulate_kernel(const uint16_t *x, uint16_t *y, int64_t N, int T, int C, const float *ada, const float *b_ada,
                int shift_off, int scale_off, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kBT / 64) + (threadIdx.x >> 6);
  if (row >= N) return;
  const int CV = C / 8;
  const int b = (int)(row / T);
  const uint16_t *xr = x + row * C;
  uint4 raw[VPL];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int cv = lane + 64 * j;
    raw[j] = ld16(xr + 8 * (cv < CV ? cv : 0));
    if (cv < CV) {
      float f[8];
      unpack8(raw[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += f[e];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  const float mean = sum / (float)C;
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
  const float rstd = 1.0f / sqrtf(sq / (float)C + eps);
  const float *ab = ada + (int64_t)b * 6 * C;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int cv = lane + 64 * j;
    if (cv < CV) {
      float f[8];
      unpack8(raw[j], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ch = 8 * cv + e;
        const float sc = ab[scale_off + ch] + b_ada[scale_off + ch];
        const float sh = ab[shift_off + ch] + b_ada[shift_off + ch];
        f[e] = (f[e] - mean) * rstd * (1.0f + sc) + sh;
      }
      st16(y + row * C + 8 * cv, pack8(f));
    }
  }
}

// The projected q, k, v, u (one [N][4C] product) in place: + b_in, q / sqrt(d),
// u -> logsigmoid(u) / 16 (the log gate).
__global__ void __launch_bounds__(kBT)
gla_prep_kernel(uint16_t *qkvu, int64_t N, int C, const float *b_in, float q_scale) {
  const int C4 = 4 * C, V = C4 / 8;
  const int64_t total = N * V;
  for (int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBT) {
    const int64_t row = i / V;
    const int col = 8 * (int)(i - row * V);
    const int part = col / C;   // 0 q, 1 k, 2 v, 3 u (8 columns never straddle a part: C % 8 == 0)
    uint16_t *p = qkvu + row * C4 + col;
    float f[8];
    unpack8(ld16(p), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float z = f[e] + b_in[col + e];
      if (part == 0) z *= q_scale;
      if (part == 3) z = (fminf(z, 0.f) - log1pf(expf(-fabsf(z)))) * (1.0f / 16.0f);
      f[e] = z;
    }
    st16(p, pack8(f));
  }
}

// out[b, n] = x[b, n] + gate[b] (.) (y[b, src] + bias), gate = ada[b][gate_off..]
// + b_ada[gate_off..]; src = the scan position of canonical token n under
// dir when gather (the mixer's scan-order output), else n.
__global__ void __launch_bounds__(kBT)
gated_residual_kernel(const uint16_t *x, const uint16_t *y, const float *bias, const float *ada, const float *b_ada,
                      int gate_off, uint16_t *out, int B, int T, int C, bool gather, int dir, int gh, int gw) {
  const int V = C / 8;
  const int64_t total = (int64_t)B * T * V;
  for (int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBT) {
    const int64_t row = i / V;
    const int col = 8 * (int)(i - row * V);
    const int b = (int)(row / T), n = (int)(row - (int64_t)b * T);
    const int src = gather ? canon_to_scan(dir, gh, gw, T, n) : n;
    float fx[8], fy[8];
    unpack8(ld16(x + row * C + col), fx);
    unpack8(ld16(y + ((int64_t)b * T + src) * C + col), fy);
    const float *ab = ada + (int64_t)b * 6 * C + gate_off + col;
    const float *bb = b_ada + gate_off + col;
#pragma unroll
    for (int e = 0; e < 8; ++e) fx[e] += (ab[e] + bb[e]) * (fy[e] + bias[col + e]);
    st16(out + row * C + col, pack8(fx));
  }
}

// In place: f = GELU(f + b) with the tanh form DiT's MLP uses.
__global__ void __launch_bounds__(kBT)
bias_gelu_kernel(uint16_t *f, int64_t N, int F, const float *bias) {
  const int V = F / 8;
  const int64_t total = N * V;
  for (int64_t i = (int64_t)blockIdx.x * kBT + threadIdx.x; i < total; i += (int64_t)gridDim.x * kBT) {
    const int64_t row = i / V;
    const int col = 8 * (int)(i - row * V);
    uint16_t *p = f + row * F + col;
    float v[8];
    unpack8(ld16(p), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float z = v[e] + bias[col + e];
      v[e] = 0.5f * z * (1.0f + tanhf(0.7978845608028654f * (z + 0.044715f * z * z * z)));
    }
    st16(p, pack8(v));
  }
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

// one rocBLAS handle per device, created on first use and kept
std::mutex g_handle_mu;
rocblas_handle g_handle[64] = {};

hipError_t handle_for(rocblas_handle &h) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_handle_mu);
  if (!g_handle[dev] && rocblas_create_handle(&g_handle[dev]) != rocblas_status_success) return hipErrorUnknown;
  h = g_handle[dev];
  return hipSuccess;
}

// Y[M][N] = X[M][K] W[N][K]^T (row-major), bf16 operands, fp32 accumulation,
// Y bf16 or fp32.  rocBLAS is column-major: Y^T = W (K x N, transposed) X^T.
rocblas_status gemm(rocblas_handle h, const void *X, const void *W, void *Y, bool y_f32, int M, int N, int K) {
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype yt = y_f32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
  return rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, N, M, K, &one, W,
                         rocblas_datatype_bf16_r, K, X, rocblas_datatype_bf16_r, K, &zero, Y, yt, N, Y, yt, N,
                         rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
}

}  // namespace
}  // namespace dig

// ------------------------------------------------------------------ host side
namespace {
constexpr size_t kGemmScratch = DIG_GEMM_SCRATCH;   // rocBLAS scratch inside the workspace
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
// the bf16 GLA's chunk for this head size (64 while its LDS plan holds it)
int block_chunk(int d) { return d <= 96 ? 64 : 32; }

struct BlockLayout {
  size_t ada, cs, h, qkvu, o, o2, x1, x2, xs, gla, gemm, bytes;
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
  L.x2 = take(tok * C * e);
  L.xs = take(tok * C * e);         // x2 in the scan order of dir (conv input)
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
  using namespace dig;
  rocblas_handle h;
  hipError_t e = handle_for(h);
  if (e != hipSuccess) return e;
  if (rocblas_set_stream(h, s) != rocblas_status_success) return hipErrorUnknown;
  if (rocblas_set_workspace(h, scratch, scratch_bytes) != rocblas_status_success) return hipErrorUnknown;
  return gemm(h, x, w, y, false, M, N, K) == rocblas_status_success ? hipSuccess : hipErrorUnknown;
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
  uint16_t *xs = reinterpret_cast<uint16_t *>(ws + L.xs);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  rocblas_handle hb;
  hipError_t e = handle_for(hb);
  if (e != hipSuccess) return e;
  if (rocblas_set_stream(hb, s) != rocblas_status_success) return hipErrorUnknown;
  if (rocblas_set_workspace(hb, ws + L.gemm, kGemmScratch) != rocblas_status_success) return hipErrorUnknown;
  auto G = [&](const void *X, const void *W, void *Y, bool f32, int M, int Nn, int K) {
    return gemm(hb, X, W, Y, f32, M, Nn, K) == rocblas_status_success ? hipSuccess : hipErrorUnknown;
  };
  const int vpl = (C / 8 + 63) / 64;
  auto modulate = [&](const uint16_t *in, uint16_t *out, int shift_off, int scale_off) {
    const int grid = (int)((N + 3) / 4);
#define DIG_MOD_CASE(V)                                                                                   \
  if (vpl <= V) {                                                                                         \
    hipLaunchKernelGGL((modulate_kernel<V>), dim3(grid), dim3(kBT), 0, s, in, out, N, T, C, ada, a.b_ada, \
                       shift_off, scale_off, 1e-6f);                                                      \
    return hipGetLastError();                                                                             \
  }
    DIG_MOD_CASE(1)
    DIG_MOD_CASE(2)
    DIG_MOD_CASE(3)
    DIG_MOD_CASE(4)
    DIG_MOD_CASE(8)
    DIG_MOD_CASE(16)
    DIG_MOD_CASE(32)
#undef DIG_MOD_CASE
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
  // (1) conditioning -> [s1 | a1 | g1 | s2 | a2 | g2] (fp32; b_ada added where used)
  hipLaunchKernelGGL(silu_kernel, dim3((B * C + kBT - 1) / kBT), dim3(kBT), 0, s, a.c, cs, B * C);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = G(cs, a.w_ada, ada, true, B, 6 * C, C)) != hipSuccess) return e;
  // (2) mixer: adaLN, projections, GLA over dir, out-projection, gated residual
  if ((e = modulate(x, h, 0, C)) != hipSuccess) return e;
  if ((e = G(h, a.w_in, qkvu, false, (int)N, 4 * C, C)) != hipSuccess) return e;
  hipLaunchKernelGGL(gla_prep_kernel, dim3(ew_grid(N * C / 2, a.num_cu)), dim3(kBT), 0, s, qkvu, N, C, a.b_in,
                     1.0f / sqrtf((float)d));
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
  if ((e = G(o, a.w_out, o2, false, (int)N, C, C)) != hipSuccess) return e;
  const int egrid = ew_grid(N * C / 8, a.num_cu);
  hipLaunchKernelGGL(gated_residual_kernel, dim3(egrid), dim3(kBT), 0, s, x, o2, a.b_out, ada, a.b_ada, 2 * C, x1, B,
                     T, C, true, a.dir, a.gh, a.gw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // (3) FFN: adaLN, C -> 4C, GELU, 4C -> C, gated residual
  if ((e = modulate(x1, h, 3 * C, 4 * C)) != hipSuccess) return e;
  if ((e = G(h, a.w_ff1, qkvu, false, (int)N, 4 * C, C)) != hipSuccess) return e;
  hipLaunchKernelGGL(bias_gelu_kernel, dim3(ew_grid(N * C / 2, a.num_cu)), dim3(kBT), 0, s, qkvu, N, 4 * C, a.b_ff1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = G(qkvu, a.w_ff2, o, false, (int)N, C, 4 * C)) != hipSuccess) return e;
  hipLaunchKernelGGL(gated_residual_kernel, dim3(egrid), dim3(kBT), 0, s, x1, o, a.b_ff2, ada, a.b_ada, 5 * C, x2, B,
                     T, C, false, a.dir, a.gh, a.gw);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // (4) SREM: x2 in the scan order of dir, then the 3x3 depthwise conv of its
  //     scan frame, stored in canonical order
  const uint16_t *conv_in = x2;
  if (a.dir != 0) {
    if ((e = dig_launch_remap(x2, 1, B, T, C, a.gh, a.gw, 0, a.dir, xs, a.num_cu, s)) != hipSuccess) return e;
    conv_in = xs;
  }
  return dig_launch_dwconv(conv_in, 1, B, T, C, (int64_t)T * C, C, a.w_conv, a.gh, a.gw, a.dir, a.y,
                           (int64_t)T * C, C, a.num_cu, s);
}
