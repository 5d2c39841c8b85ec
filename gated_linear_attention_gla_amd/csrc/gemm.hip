// gemm.hip -- the dense products of the DiG block on gfx950 bf16 MFMA.
//
// Y[M][N] = alpha * X[M][K] W[N][K]^T with an elementwise epilogue, row-major,
// bf16 operands, fp32 accumulation (DiG notes, 关键设计 / DiG Block设计: the
// q/k/v/gate, output and FFN projections around the mixer; DiT notes, 3.2:
// the adaLN-Zero regression of the conditioning).  Both operands are
// K-contiguous, so a tile of either is a set of K-rows.
//
// Block tile: 256 tokens (M) x BN features (N, 256 or 128), K in steps of
// 64; sixteen waves, 4 along tokens x 4 along features, each owning 64
// tokens x BN/4 features as 32 x 32 tiles on v_mfma_f32_32x32x16_bf16 (four
// waves per SIMD keep a product ready to issue while others wait on LDS:
// 3-10 % faster than eight waves of 64 x BN/2; the 16 x 16 shape reads as
// many operand registers per instruction for half the products: 6-17 %
// slower at the block's shapes).  Tiles go through LDS double-buffered with
// one barrier per K step: the rows of step k+1 are loaded into registers
// halfway through step k-1 and written to the other buffer halfway through
// step k, so a load has a whole step to arrive and the LDS writes overlap
// products.  LDS rows are 36 dwords (64 + 8 bf16): a fragment is one 16-byte
// read per lane from 32 rows, conflict free at a stride of 4 * odd dwords.
//
// W is the A operand and X the B operand: accumulator register 4 q + e of
// lane l holds feature 8 q + 4 (l / 32) + e of token l % 32 -- four
// consecutive features of one row of Y.  The epilogue finishes those values
// per lane (alpha, bias, GELU, the log gate), stages the tile in LDS, and
// writes it as 16-byte pieces of whole rows, applying the row permutation
// and the gated residual on the way out.
#include "dig_internal.h"
#include "dig_mfma.h"

namespace dig {
namespace {

constexpr int GBM = 256;        // tokens per block tile
constexpr int GBK = 64;         // K per step
constexpr int GLD = GBK + 8;    // LDS row stride (elements)
constexpr int GGM = 8;          // M tiles per group in the block order (L2 reuse)

// v_mfma_f32_32x32x16_bf16: lane l supplies row (A) / column (B) l % 32 and
// the 8-element K slice l / 32; the accumulator register 4 q + e of lane l
// holds row 8 q + 4 (l / 32) + e, column l % 32.
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
__device__ __forceinline__ f32x16_t mfma32x32(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

struct Epi {
  int kind;            // DIG_EPI_*
  float alpha;
  const float *bias;   // [N] fp32 or null
  int gate_col;        // kind GATE: columns >= gate_col take logsigmoid(.) / 16
  // kind RESIDUAL: out[r'][n] = res[c][n] + gate[b][gate_off + n] * (alpha acc + bias[n]),
  // r' the mapped output row, c the canonical row of the token
  const uint16_t *res;
  const float *gate;
  int gate_stride, gate_off;
  int rowmap;          // 0 identity; 1 rows in scan order -> canonical; 2 canonical -> scan order
  int T, dir, gh, gw;
};

// log sigmoid(z) = min(z, 0) - log(1 + e^{-|z|}); log1p by its series below
// e = 0.01 (truncation < e^4 / 4), else the hardware log of 1 + e.
__device__ __forceinline__ float log_sigmoid_f(float z) {
  const float e = __expf(-fabsf(z));
  const float l = e < 0.01f ? e * (1.0f - e * (0.5f - e * (1.0f / 3.0f))) : __logf(1.0f + e);
  return fminf(z, 0.f) - l;
}
// tanh-form GELU: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))), with
// tanh(u) = 1 - 2 / (e^{2u} + 1) (exact at both saturations).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float u = 0.7978845608028654f * (z + 0.044715f * z * z * z);
  const float t = 1.0f - 2.0f / (__expf(2.0f * u) + 1.0f);
  return 0.5f * z * (1.0f + t);
}

template <int BN, int WV, bool F32OUT>
__global__ void __launch_bounds__(64 * WV, 1)
gemm_bf16_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, void *__restrict__ Y, int M, int N,
                 int K, int ntm, int ntn, Epi ep) {
  constexpr int GT = 64 * WV;              // threads
  constexpr int WVN = WV / 4;              // waves along features (4 along tokens)
  constexpr int WM = GBM / 4;              // tokens per wave
  constexpr int WN = BN / WVN;             // features per wave
  constexpr int TN = WN / 32;              // 32-feature tiles per wave (A operand)
  constexpr int TM = WM / 32;              // 32-token tiles per wave (B operand)
  constexpr int XR = GBM * GBK / 8 / GT;   // 16-byte X chunks per thread per K step
  constexpr int WR = BN * GBK / 8 / GT;    // and W chunks
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                  // [2][GBM][GLD]
  uint16_t *wsh = xs + 2 * GBM * GLD;                                  // [2][BN][GLD]

  // ---- block -> tile (tm, tn): blocks of one XCD (i % 8) take a contiguous
  // range of the tile order, which walks groups of GGM token tiles across
  // every feature tile, so concurrently running blocks share X and W rows in L2
  const int ntiles = ntm * ntn;
  const int lb = xcd_linear_block(blockIdx.x, gridDim.x);
  if (lb >= ntiles) return;
  const int grp = lb / (GGM * ntn), within = lb - grp * GGM * ntn;
  const int gm = min(GGM, ntm - grp * GGM);
  const int tm = grp * GGM + within % gm, tn = within / gm;
  const int m0 = tm * GBM, n0 = tn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WVN, wn = wave % WVN;   // token rows [WM wm, +WM), features [WN wn, +WN)
  const int l32 = lane & 31, h32 = lane >> 5;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (unsigned)((int64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (unsigned)((int64_t)N * K * 2));

  // global -> registers: chunk idx = tid + GT r -> row idx / 8, 8-element K
  // column 8 (idx % 8).  Per chunk, computed once: its byte offset at k0 = 0
  // and its K column (a row past M / N gets column K, i.e. never loads: the
  // offset past the buffer reads zeros); a step adds 2 k0.
  struct Rows { uint4 x[XR], w[WR]; };
  Rows ra;
  unsigned xo[XR], wo[WR];
  int xk[XR], wk[WR];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int idx = tid + GT * r, row = idx >> 3, c = idx & 7;
    const bool ok = m0 + row < M;
    xo[r] = ok ? (unsigned)(((int64_t)(m0 + row) * K + 8 * c) * 2) : 0u;
    xk[r] = ok ? 8 * c : K;
  }
#pragma unroll
  for (int r = 0; r < WR; ++r) {
    const int idx = tid + GT * r, row = idx >> 3, c = idx & 7;
    const bool ok = n0 + row < N;
    wo[r] = ok ? (unsigned)(((int64_t)(n0 + row) * K + 8 * c) * 2) : 0u;
    wk[r] = ok ? 8 * c : K;
  }
  auto load = [&](Rows &rr, int k0) {
#pragma unroll
    for (int r = 0; r < XR; ++r) rr.x[r] = bload16(rx, xk[r] + k0 < K ? xo[r] + 2u * k0 : kOOB);
#pragma unroll
    for (int r = 0; r < WR; ++r) rr.w[r] = bload16(rw, wk[r] + k0 < K ? wo[r] + 2u * k0 : kOOB);
  };
  auto store = [&](const Rows &rr, int buf) {
    uint16_t *xb = xs + buf * GBM * GLD, *wb = wsh + buf * BN * GLD;
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const int idx = tid + GT * r;
      *reinterpret_cast<uint4 *>(xb + (idx >> 3) * GLD + 8 * (idx & 7)) = rr.x[r];
    }
#pragma unroll
    for (int r = 0; r < WR; ++r) {
      const int idx = tid + GT * r;
      *reinterpret_cast<uint4 *>(wb + (idx >> 3) * GLD + 8 * (idx & 7)) = rr.w[r];
    }
  };

  f32x16_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // One 32-wide K block (kh) of the step in LDS buffer buf, as two 16-wide
  // K slices; lane l reads row l % 32 of each 32-row tile at K offset
  // 8 (l / 32).  (Issuing the reads ahead of the products by hand, one to
  // three W fragments deep, measured the same as the compiler's order.)
  auto compute_half = [&](int buf, int kh) {
    const uint16_t *xb = xs + buf * GBM * GLD + (WM * wm + l32) * GLD + 8 * h32 + 32 * kh;
    const uint16_t *wb = wsh + buf * BN * GLD + (WN * wn + l32) * GLD + 8 * h32 + 32 * kh;
    uint4 a[2][TN], b[2][TM];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
#pragma unroll
      for (int j = 0; j < TM; ++j) b[sl][j] = lds4(xb + 32 * j * GLD + 16 * sl);
#pragma unroll
      for (int i = 0; i < TN; ++i) a[sl][i] = lds4(wb + 32 * i * GLD + 16 * sl);
    }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = mfma32x32(a[sl][i], b[sl][j], acc[i][j]);
  };

  const int KT = (K + GBK - 1) / GBK;
  load(ra, 0);
  store(ra, 0);
  if (KT > 1) load(ra, GBK);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    compute_half(kt & 1, 0);
    // the rows of step kt+1 (loaded halfway through the previous step) go to
    // the buffer step kt-1 read, which every wave left at the barrier that
    // ended it; then the rows of step kt+2 are loaded
    if (kt + 1 < KT) {
      store(ra, (kt + 1) & 1);
      if (kt + 2 < KT) load(ra, (kt + 2) * GBK);
    }
    compute_half(kt & 1, 1);
    __syncthreads();
  }

  // ---- epilogue, in two passes through LDS (free once the last step's
  // barrier has passed): (1) each lane finishes its values -- alpha, bias,
  // GELU or the log gate -- and writes them into an LDS copy of the tile,
  // bf16, or fp32 where the output is fp32 or the residual is still to be
  // added (so the final value is rounded once); (2) the tile leaves as whole
  // 16-byte pieces of rows, consecutive threads along a row, with the row
  // permutation and the gated residual applied there.  (Stored straight from
  // the accumulators, every 128-byte line of Y arrived as eight 16-byte
  // pieces from as many instructions: 7.8 us of a 46 us tile.)
  const bool resid = ep.kind == DIG_EPI_RESIDUAL;
  const bool stage32 = F32OUT || resid;                  // fp32 staging
  constexpr int RB = BN * 4 + 16;                        // staged row stride, bytes (fp32 rows; bf16 rows use half)
  const int rb = stage32 ? RB : BN * 2 + 16;
  unsigned char *stg = smem;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int ml = WM * wm + 32 * j + l32;
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = WN * wn + 32 * i + 8 * q + 4 * h32;
        const int nf = n0 + nl;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * ep.alpha;
        if (ep.bias && nf < N) {
          const float4 bb = *reinterpret_cast<const float4 *>(ep.bias + nf);
          v[0] += bb.x; v[1] += bb.y; v[2] += bb.z; v[3] += bb.w;
        }
        if (ep.kind == DIG_EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(v[e]);
        } else if (ep.kind == DIG_EPI_GATE && nf >= ep.gate_col) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = log_sigmoid_f(v[e]) * (1.0f / 16.0f);
        }
        if (stage32)
          *reinterpret_cast<float4 *>(stg + ml * rb + nl * 4) = make_float4(v[0], v[1], v[2], v[3]);
        else
          *reinterpret_cast<uint2 *>(stg + ml * rb + nl * 2) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
  }
  __syncthreads();
  // pass 2: OE output elements (16 bytes) per piece, BN / OE pieces per row
  constexpr int OE = F32OUT ? 4 : 8, CPR = BN / OE;
  for (int c = tid; c < GBM * CPR; c += GT) {
    const int row = c / CPR, nl = (c - row * CPR) * OE;
    const int m = m0 + row, nf = n0 + nl;
    if (m >= M || nf >= N) continue;   // N is a multiple of 8: a piece is all in or all out
    int64_t orow = m, rrow = m;
    int bidx = 0;
    if (resid) {
      // rowmap 1 reads X in scan order and writes canonical rows; rowmap 2
      // the reverse; the residual is read at the token's canonical row
      bidx = m / ep.T;
      const int t = m - bidx * ep.T;
      const int t2 = ep.rowmap == 1 ? scan_to_canon(ep.dir, ep.gh, ep.gw, ep.T, t)
                     : ep.rowmap == 2 ? canon_to_scan(ep.dir, ep.gh, ep.gw, ep.T, t)
                                      : t;
      orow = (int64_t)bidx * ep.T + t2;
      rrow = ep.rowmap == 2 ? m : orow;
    }
    const unsigned char *sp = stg + row * rb + nl * (stage32 ? 4 : 2);
    if constexpr (F32OUT) {
      *reinterpret_cast<uint4 *>(static_cast<float *>(Y) + orow * N + nf) = *reinterpret_cast<const uint4 *>(sp);
    } else if (!resid) {
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(Y) + orow * N + nf) = *reinterpret_cast<const uint4 *>(sp);
    } else {
      const float4 v0 = *reinterpret_cast<const float4 *>(sp), v1 = *reinterpret_cast<const float4 *>(sp + 16);
      const uint4 rr = *reinterpret_cast<const uint4 *>(ep.res + rrow * N + nf);
      const float *gp = ep.gate + (int64_t)bidx * ep.gate_stride + ep.gate_off + nf;
      const float4 g0 = *reinterpret_cast<const float4 *>(gp), g1 = *reinterpret_cast<const float4 *>(gp + 4);
      uint4 o;
      o.x = pack_bf16x2(bf16lo(rr.x) + g0.x * v0.x, bf16hi(rr.x) + g0.y * v0.y);
      o.y = pack_bf16x2(bf16lo(rr.y) + g0.z * v0.z, bf16hi(rr.y) + g0.w * v0.w);
      o.z = pack_bf16x2(bf16lo(rr.z) + g1.x * v1.x, bf16hi(rr.z) + g1.y * v1.y);
      o.w = pack_bf16x2(bf16lo(rr.w) + g1.z * v1.z, bf16hi(rr.w) + g1.w * v1.w);
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(Y) + orow * N + nf) = o;
    }
  }
}

template <int BN, int WV, bool F32OUT>
hipError_t launch_gemm(const void *X, const void *W, void *Y, int M, int N, int K, const Epi &ep, hipStream_t s) {
  const int ntm = (M + GBM - 1) / GBM, ntn = (N + BN - 1) / BN;
  const int grid = ((ntm * ntn + 7) / 8) * 8;
  // operand buffers, or the staged output tile (fp32 rows) if larger
  const size_t lds_ops = (size_t)2 * (GBM + BN) * GLD * 2, lds_out = (size_t)GBM * (BN * 4 + 16);
  const size_t lds = BN == 256 ? lds_ops : (lds_ops > lds_out ? lds_ops : lds_out);
  auto *fn = gemm_bf16_kernel<BN, WV, F32OUT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * WV), lds, s, static_cast<const uint16_t *>(X),
                     static_cast<const uint16_t *>(W), Y, M, N, K, ntm, ntn, ep);
  return hipGetLastError();
}

// Few rows (M <= 16, e.g. the conditioning product over the batch): the MFMA
// tile would be almost all padding, and the product is one pass over W, so
// the kernel is built for memory-level parallelism: one row of W per wave,
// eight waves per block, the 16-byte pieces of the row that a lane needs (up
// to 4 x 512 elements of K ahead) requested before X (M x K) is staged in
// LDS per block.  A lane's M dot products are summed across the wave by a
// reduce-scatter (each step exchanges half of the remaining values: 17
// shuffles for 16 rows rather than 6 per row), after which lanes 4 m ..
// 4 m + 3 hold row m's sum.  alpha, bias, fp32 or bf16 output.  (8 x 6912 x
// 1152: 57 us for eight rows per wave walked one after another, 26 us now.)
constexpr int SK_MAXM = 16, SK_T = 512, SK_KU = 4;
constexpr int SK_XMAX = 64 * 1024 / 16 / SK_T;   // X pieces per thread at most (64 KiB of LDS)
template <bool F32OUT>
__global__ void __launch_bounds__(SK_T)
gemm_skinny_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ W, void *__restrict__ Y, int M, int N,
                   int K, float alpha, const float *__restrict__ bias) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *xs = reinterpret_cast<uint16_t *>(smem);   // [M][K]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * (SK_T / 64) + wave;
  const uint16_t *wrow = W + (int64_t)(n < N ? n : N - 1) * K;   // past N: row N-1, never stored
  // the first SK_KU pieces of the row are requested before X is staged
  uint4 wv[SK_KU];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int u = 0; u < SK_KU; ++u)
      if (k0 + 512 * u < K) wv[u] = *reinterpret_cast<const uint4 *>(wrow + k0 + 512 * u);
  };
  load_w(8 * lane);
  {
    const int nx = M * K / 8;
    uint4 t[SK_XMAX];
#pragma unroll
    for (int r = 0; r < SK_XMAX; ++r) {
      const int i = threadIdx.x + SK_T * r;
      if (i < nx) t[r] = reinterpret_cast<const uint4 *>(X)[i];
    }
#pragma unroll
    for (int r = 0; r < SK_XMAX; ++r) {
      const int i = threadIdx.x + SK_T * r;
      if (i < nx) reinterpret_cast<uint4 *>(xs)[i] = t[r];
    }
  }
  __syncthreads();
  float acc[SK_MAXM];
#pragma unroll
  for (int m = 0; m < SK_MAXM; ++m) acc[m] = 0.f;
  for (int k0 = 8 * lane; k0 < K; k0 += 512 * SK_KU) {
    if (k0 != 8 * lane) load_w(k0);
#pragma unroll
    for (int u = 0; u < SK_KU; ++u) {
      const int k = k0 + 512 * u;
      if (k >= K) break;
      const uint32_t ww[4] = {wv[u].x, wv[u].y, wv[u].z, wv[u].w};
#pragma unroll
      for (int m = 0; m < SK_MAXM; ++m) {
        if (m < M) {
          const uint4 xv = *reinterpret_cast<const uint4 *>(xs + m * K + k);
          const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[m] += bf16lo(ww[e]) * bf16lo(xw[e]) + bf16hi(ww[e]) * bf16hi(xw[e]);
        }
      }
    }
  }
  // reduce-scatter over the 64 lanes: at the step across lane bit b, a lane
  // keeps the half of its values selected by its bit b and adds its
  // partner's copy of that half
#pragma unroll
  for (int h = SK_MAXM / 2, b = 32; h >= 1; h >>= 1, b >>= 1) {
    const bool up = (lane & b) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? acc[i] : acc[i + h];
      const float keep = up ? acc[i + h] : acc[i];
      acc[i] = keep + __shfl_xor(send, b, 64);
    }
  }
  acc[0] += __shfl_xor(acc[0], 2, 64);
  acc[0] += __shfl_xor(acc[0], 1, 64);
  const int m = lane >> 2;   // lanes 4 m .. 4 m + 3 hold the sum of row m
  if ((lane & 3) == 0 && m < M && n < N) {
    const float v = acc[0] * alpha + (bias ? bias[n] : 0.f);
    if constexpr (F32OUT) static_cast<float *>(Y)[(int64_t)m * N + n] = v;
    else static_cast<uint16_t *>(Y)[(int64_t)m * N + n] = (uint16_t)f2bf(v);
  }
}

}  // namespace
}  // namespace dig

hipError_t dig_launch_gemm(const DigGemmArgs &a, hipStream_t s) {
  dig::Epi ep{};
  ep.kind = a.kind;
  ep.alpha = a.alpha;
  ep.bias = a.bias;
  ep.gate_col = a.gate_col;
  ep.res = static_cast<const uint16_t *>(a.res);
  ep.gate = a.gate;
  ep.gate_stride = a.gate_stride;
  ep.gate_off = a.gate_off;
  ep.rowmap = a.rowmap;
  ep.T = a.T > 0 ? a.T : 1;
  ep.dir = a.dir;
  ep.gh = a.gh;
  ep.gw = a.gw;
  if (a.M <= dig::SK_MAXM && a.kind == DIG_EPI_NONE && (size_t)a.M * a.K * 2 <= 64 * 1024) {
    const int rows_per_block = dig::SK_T / 64;
    const size_t lds = (size_t)a.M * a.K * 2;
    auto *fn = a.y_f32 ? dig::gemm_skinny_kernel<true> : dig::gemm_skinny_kernel<false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((a.N + rows_per_block - 1) / rows_per_block), dim3(dig::SK_T), lds, s,
                       static_cast<const uint16_t *>(a.X), static_cast<const uint16_t *>(a.W), a.Y, a.M, a.N, a.K,
                       a.alpha, a.bias);
    return hipGetLastError();
  }
  // 128-wide feature tiles when 256-wide ones would leave the chip's CUs
  // short of tiles or waste a half-empty last tile (256-wide tiles at
  // N = 1152 measured no faster than 128-wide ones)
  const int ntm = (a.M + dig::GBM - 1) / dig::GBM;
  const bool wide = a.N % 256 == 0 && (int64_t)ntm * (a.N / 256) >= 2 * a.num_cu;
  if (a.y_f32) return dig::launch_gemm<128, 16, true>(a.X, a.W, a.Y, a.M, a.N, a.K, ep, s);
  // (256-wide tiles stage bf16 only: the residual epilogue, staged in fp32,
  // runs on 128-wide tiles)
  if (wide && a.kind != DIG_EPI_RESIDUAL)
    return dig::launch_gemm<256, 16, false>(a.X, a.W, a.Y, a.M, a.N, a.K, ep, s);
  return dig::launch_gemm<128, 16, false>(a.X, a.W, a.Y, a.M, a.N, a.K, ep, s);
}
