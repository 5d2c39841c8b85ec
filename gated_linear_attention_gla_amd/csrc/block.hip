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
// The residual stream stays in canonical token order.  The dense products run
// on the library's own MFMA GEMM (gemm.hip) with their elementwise steps in
// its epilogue: b_ada; b_in and the log gate on the u quarter; 1 / sqrt(d),
// b_out and the mixer's gated residual, gathering the scan-ordered rows back
// to canonical order; b_1 and GELU; b_2 and the FFN's gated residual, written
// straight into the scan frame of dir (the conv's input).  The adaLN
// modulations are the row kernels below.
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

}  // namespace
}  // namespace dig

// ------------------------------------------------------------------ host side
namespace {
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }
// the bf16 GLA's chunk for this head size (64 while its LDS plan holds it)
int block_chunk(int d) { return d <= 96 ? 64 : 32; }

struct BlockLayout {
  size_t ada, cs, h, qkvu, o, x1, x2, gla, bytes;
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
  L.o = take(tok * C * e);          // GLA output (scan order)
  L.x1 = take(tok * C * e);
  L.x2 = take(tok * C * e);         // x2 in the scan order of dir (the conv's input)
  const int d = C / H;
  L.gla = take(dig_gla_bf16_workspace(B, T, H, d, d, block_chunk(d), num_cu));
  L.bytes = off;
  return L;
}
}  // namespace

size_t dig_block_workspace(int B, int T, int C, int H, int num_cu) {
  return block_layout(B, T, C, H, num_cu).bytes;
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
  uint16_t *o = reinterpret_cast<uint16_t *>(ws + L.o);
  uint16_t *x1 = reinterpret_cast<uint16_t *>(ws + L.x1), *x2 = reinterpret_cast<uint16_t *>(ws + L.x2);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  hipError_t e;
  // one product of the block: Y[M][Nn] = alpha X W^T (+ bias), epilogue `kind`
  auto G = [&](const void *X, const void *W, void *Y, bool f32, int M, int Nn, int K, int kind, const float *bias,
               float alpha = 1.0f) {
    DigGemmArgs g{};
    g.X = X; g.W = W; g.Y = Y; g.y_f32 = f32; g.M = M; g.N = Nn; g.K = K; g.kind = kind; g.alpha = alpha;
    g.bias = bias; g.T = T; g.dir = a.dir; g.gh = a.gh; g.gw = a.gw; g.num_cu = a.num_cu;
    return g;
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

  // The GLA's part of the workspace (its flags and published states) sits at
  // a shape-dependent offset, so a workspace reused across shapes may hold
  // other data there: clear it.
  {
    const int64_t n16 = (int64_t)(L.bytes - L.gla) / 16;
    hipLaunchKernelGGL(zero_kernel, dim3(ew_grid(n16, a.num_cu)), dim3(kBT), 0, s,
                       reinterpret_cast<uint4 *>(ws + L.gla), n16);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // (1) conditioning -> [s1 | a1 | g1 | s2 | a2 | g2] (fp32, + b_ada)
  hipLaunchKernelGGL(silu_kernel, dim3((B * C + kBT - 1) / kBT), dim3(kBT), 0, s, a.c, cs, B * C);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = dig_launch_gemm(G(cs, a.w_ada, ada, true, B, 6 * C, C, DIG_EPI_NONE, a.b_ada), s)) != hipSuccess) return e;
  // (2) mixer: adaLN, then q | k | v | u + b_in with the log gate
  //     logsigmoid(u) / 16 formed on the u quarter in the product's epilogue
  if ((e = modulate(x, h, 0, C)) != hipSuccess) return e;
  {
    DigGemmArgs g = G(h, a.w_in, qkvu, false, (int)N, 4 * C, C, DIG_EPI_GATE, a.b_in);
    g.gate_col = 3 * C;
    if ((e = dig_launch_gemm(g, s)) != hipSuccess) return e;
  }
  DigGlaArgs g{};
  g.q = qkvu; g.k = qkvu + C; g.v = qkvu + 2 * C; g.g = qkvu + 3 * C;
  g.qk_sb = (int64_t)T * 4 * C; g.qk_st = 4 * C; g.qk_sh = d;
  g.v_sb = g.qk_sb; g.v_st = g.qk_st; g.v_sh = d;
  g.o = o; g.o_sb = (int64_t)T * C; g.o_st = C; g.o_sh = d;
  g.s0 = nullptr; g.s_final = nullptr;
  g.B = B; g.T = T; g.H = H; g.dk = d; g.dv = d; g.gh = a.gh; g.gw = a.gw; g.dir = a.dir; g.chunk = block_chunk(d);
  g.order = nullptr;
  g.workspace = ws + L.gla; g.workspace_bytes = L.bytes - L.gla;
  g.epoch = a.epoch; g.num_cu = a.num_cu;
  if ((e = dig_launch_gla_bf16(g, s)) != hipSuccess) return e;
  // out-projection with the mixer's gated residual in its epilogue:
  // x1[b, n] = x[b, n] + g1 (.) (o[b, p] W_out^T / sqrt(d) + b_out), the row of
  // scan position p stored at its canonical token n (q's 1 / sqrt(d) is taken
  // here: the mixer's output is linear in q)
  {
    DigGemmArgs r = G(o, a.w_out, x1, false, (int)N, C, C, DIG_EPI_RESIDUAL, a.b_out, 1.0f / sqrtf((float)d));
    r.res = x; r.gate = ada; r.gate_stride = 6 * C; r.gate_off = 2 * C; r.rowmap = 1;
    if ((e = dig_launch_gemm(r, s)) != hipSuccess) return e;
  }
  // (3) FFN: adaLN of x1, C -> 4C with b_1 and GELU, 4C -> C with b_2 and the
  //     gated residual x2 = x1 + g2 (.) (.), each row written at its scan
  //     position under dir: the conv's input
  if ((e = modulate(x1, h, 3 * C, 4 * C)) != hipSuccess) return e;
  if ((e = dig_launch_gemm(G(h, a.w_ff1, qkvu, false, (int)N, 4 * C, C, DIG_EPI_GELU, a.b_ff1), s)) != hipSuccess)
    return e;
  {
    DigGemmArgs r = G(qkvu, a.w_ff2, x2, false, (int)N, C, 4 * C, DIG_EPI_RESIDUAL, a.b_ff2);
    r.res = x1; r.gate = ada; r.gate_stride = 6 * C; r.gate_off = 5 * C; r.rowmap = 2;
    if ((e = dig_launch_gemm(r, s)) != hipSuccess) return e;
  }
  // (4) SREM: the 3x3 depthwise conv of the scan frame of dir, stored in
  //     canonical order
  return dig_launch_dwconv(x2, 1, B, T, C, (int64_t)T * C, C, a.w_conv, a.gh, a.gw, a.dir, a.y,
                           (int64_t)T * C, C, a.num_cu, s);
}
