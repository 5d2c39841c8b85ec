// gla_bf16.hip -- chunk-wise Gated Linear Attention forward on gfx950 MFMA.
//
// Method (DiG paper notes, 关键设计 / 硬件友好的效率设计: chunk-wise parallel
// GLA computed on chip; diffusers issue #20 for the recurrence itself):
// the scan-ordered sequence of one (batch, head) is cut into chunks of M
// tokens.  Inside chunk c, with b_t the inclusive cumulative log-gate from the
// chunk start (per key channel) and S the state entering the chunk,
//   o_t = sum_{s<=t, s in chunk} [ sum_i q_ti k_si e^{b_ti - b_si} ] v_s      (intra)
//       + (q_t * e^{b_t}) S                                                  (inter)
//   S'  = diag(e^{b_last}) S + sum_s (k_s * e^{b_last - b_s})^T v_s          (state)
// which is the token recurrence S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,
// o_t = q_t S_t regrouped.  The intra term uses the factorised operands
// q~ = q e^{b}, k~ = k e^{-b} (one bf16 MFMA product per tile); when a chunk's
// cumulative gate leaves [-2^6, 2^6] in log2 units that factorisation could
// overflow, so such a chunk computes the intra weights pairwise on the VALU
// instead (exact exponent differences), which keeps any finite log-gate <= 0
// accurate.  Every other product is already bounded (e^{b} <= 1 and
// e^{b_last - b_s} <= 1 for non-positive gates).
//
// gfx950 mapping
//   * one workgroup per (batch, head); NW = max(DP/16, 4) waves; wave w owns
//     the value columns [16w, 16w+16) of the state and of the output, so the
//     fp32 state lives in that wave's MFMA accumulators for the whole scan;
//   * the scan permutation is applied in the loads: scan position p reads
//     canonical token scan_to_canon(p), whole 16-byte channel groups per lane,
//     so no transposed or flipped copy of the inputs is ever written;
//   * v_mfma_f32_16x16x32_bf16 with fp32 accumulation, the only MFMA shape
//     used: key channels are zero-padded to a multiple of 32 and an odd
//     16-token tile count pads its last token block with zeros;
//     operands staged in LDS in the two orders the products need
//     (token-major q~, k~; channel-major k^, v);
//   * the next chunk's loads are issued before this chunk's MFMA work.
//
// Operand layout facts used (CDNA3/CDNA4 MFMA 16x16xK): lane l supplies row
// (A) / column (B) l % 16 and the K slice of group l / 16; the accumulator
// holds rows 4*(l/16) + e, column l % 16.  The K order inside one MFMA is
// free as long as A and B agree, which lets accumulators be reused directly
// as the next product's operands (P^T -> B of the P V product, S -> A of the
// S^T q~^T product) without a trip through LDS.
#include "dig_internal.h"

namespace dig {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kFastRange = 64.0f;   // |cumulative log2 gate| bound of the factorised path

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint2 pack4(f32x4_t x) {
  return make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ uint4 cat(uint2 lo, uint2 hi) { return make_uint4(lo.x, lo.y, hi.x, hi.y); }
__device__ __forceinline__ uint2 lds2(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
__device__ __forceinline__ uint4 lds4(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

struct Params {
  const uint16_t *q, *k, *v, *g;
  uint16_t *o;
  const float *s0;
  float *s_final;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  int B, T, H, dk, dv, gh, gw, dir, nchunks, units;
};

template <int DP>
struct Shape {
  static constexpr int NW = DP / 16 > 4 ? DP / 16 : 4;   // waves per workgroup
  static constexpr int NT = NW * kWave;
};

template <int DP, int M>
struct Lds {
  static constexpr int QS = DP + 8;   // token-major row stride (elements)
  static constexpr int TS = M + 8;    // channel-major row stride (elements)
  static constexpr int oQt = 0;                       // q~  [M][QS] bf16
  static constexpr int oKt = oQt + M * QS * 2;        // k~  [M][QS] bf16 (raw k on the pairwise path)
  static constexpr int oKh = oKt + M * QS * 2;        // k^  [DP][TS] bf16 (channel-major)
  static constexpr int oVT = oKh + DP * TS * 2;       // v   [DP][TS] bf16 (channel-major)
  static constexpr int oP = oVT + DP * TS * 2;        // P   [M][TS] bf16 (pairwise path)
  static constexpr int oB = oP + M * TS * 2;          // b   [M][DP] fp32 (log2 units)
  static constexpr int oGam = oB + M * DP * 4;        // e^{b_last} [DP] fp32
  static constexpr int oFlag = oGam + DP * 4;
  static constexpr int bytes = oFlag + 16;
};

template <int DP, int M>
__global__ void __launch_bounds__(Shape<DP>::NT)
gla_fwd_bf16_kernel(Params P) {
  constexpr int NT = Shape<DP>::NT;
  constexpr int CG = DP / 8;                 // 16-byte channel groups per token row
  constexpr int ITEMS = M * CG;
  constexpr int R = (ITEMS + NT - 1) / NT;   // 16-byte items per thread per tensor
  constexpr int MT = M / 16;                 // token tiles per chunk
  constexpr int DT = DP / 16;                // channel tiles
  constexpr int K32 = DP / 32;               // 32-wide channel blocks (DP is a multiple of 32)
  static_assert(DP % 32 == 0, "key channels are padded to a multiple of 32");
  constexpr int QS = Lds<DP, M>::QS, TS = Lds<DP, M>::TS;

  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *sQt = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oQt);
  uint16_t *sKt = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oKt);
  uint16_t *sKh = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oKh);
  uint16_t *sVT = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oVT);
  uint16_t *sP = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oP);
  float *sB = reinterpret_cast<float *>(smem + Lds<DP, M>::oB);
  float *sGam = reinterpret_cast<float *>(smem + Lds<DP, M>::oGam);
  int *sFlag = reinterpret_cast<int *>(smem + Lds<DP, M>::oFlag);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;

  const int unit = xcd_linear_block(blockIdx.x, gridDim.x);
  if (unit >= P.units) return;
  const int b = unit / P.H, h = unit - b * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv;

  const uint16_t *qb = P.q + b * P.qk_sb + h * P.qk_sh;
  const uint16_t *kb = P.k + b * P.qk_sb + h * P.qk_sh;
  const uint16_t *gb = P.g + b * P.qk_sb + h * P.qk_sh;
  const uint16_t *vb = P.v + b * P.v_sb + h * P.v_sh;
  uint16_t *ob = P.o + b * P.o_sb + h * P.o_sh;

  const int n0 = 16 * wave;                 // this wave's value columns
  const bool has_cols = (n0 < dv);

  // fp32 state, accumulator layout: S[r][e] = S[16r + 4*g4 + e][n0 + l16]
  f32x4_t S[DT];
#pragma unroll
  for (int r = 0; r < DT; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = 16 * r + 4 * g4 + e, n = n0 + l16;
      S[r][e] = (P.s0 && ch < dk && n < dv) ? P.s0[((int64_t)unit * dk + ch) * dv + n] : 0.f;
    }
  }

  uint4 rq[R], rk[R], rg[R], rv[R];
  auto load_chunk = [&](int c) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      const int p = c * M + tl;
      const bool tok = (idx < ITEMS) && (p < T);
      const int64_t n = tok ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : 0;
      const uint4 z = make_uint4(0, 0, 0, 0);
      const bool kin = tok && (8 * cg < dk), vin = tok && (8 * cg < dv);
      rq[r] = kin ? *reinterpret_cast<const uint4 *>(qb + n * P.qk_st + 8 * cg) : z;
      rk[r] = kin ? *reinterpret_cast<const uint4 *>(kb + n * P.qk_st + 8 * cg) : z;
      rg[r] = kin ? *reinterpret_cast<const uint4 *>(gb + n * P.qk_st + 8 * cg) : z;
      rv[r] = vin ? *reinterpret_cast<const uint4 *>(vb + n * P.v_st + 8 * cg) : z;
    }
  };

  load_chunk(0);

  for (int c = 0; c < P.nchunks; ++c) {
    // ---- stage 1: gates (log2 units, fp32) token-major; v channel-major
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NT;
      if (idx < ITEMS) {
        const int tl = idx / CG, cg = idx - tl * CG;
        const uint32_t gw4[4] = {rg[r].x, rg[r].y, rg[r].z, rg[r].w};
        float4 lo, hi;
        lo.x = bf16lo(gw4[0]) * kLog2e; lo.y = bf16hi(gw4[0]) * kLog2e;
        lo.z = bf16lo(gw4[1]) * kLog2e; lo.w = bf16hi(gw4[1]) * kLog2e;
        hi.x = bf16lo(gw4[2]) * kLog2e; hi.y = bf16hi(gw4[2]) * kLog2e;
        hi.z = bf16lo(gw4[3]) * kLog2e; hi.w = bf16hi(gw4[3]) * kLog2e;
        float4 *dst = reinterpret_cast<float4 *>(sB + tl * DP + 8 * cg);
        dst[0] = lo;
        dst[1] = hi;
        const uint32_t vw[4] = {rv[r].x, rv[r].y, rv[r].z, rv[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sVT[(8 * cg + 2 * e) * TS + tl] = (uint16_t)(vw[e] & 0xffffu);
          sVT[(8 * cg + 2 * e + 1) * TS + tl] = (uint16_t)(vw[e] >> 16);
        }
      }
    }
    if (tid == 0) *sFlag = 0;
    __syncthreads();

    // ---- stage 2: inclusive cumulative gate per key channel
    if (tid < DP) {
      float run = 0.f, amax = 0.f;
#pragma unroll 8
      for (int t = 0; t < M; ++t) {
        run += sB[t * DP + tid];
        sB[t * DP + tid] = run;
        amax = fmaxf(amax, fabsf(run));
      }
      sGam[tid] = exp2f(run);
      if (!(amax <= kFastRange)) *sFlag = 1;   // also catches NaN
    }
    __syncthreads();
    const bool pairwise = (*sFlag != 0);

    // ---- stage 3: scaled operands
    if (pairwise) {
      // raw q, k for the exact pairwise intra weights
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = tid + r * NT;
        if (idx < ITEMS) {
          const int tl = idx / CG, cg = idx - tl * CG;
          *reinterpret_cast<uint4 *>(sQt + tl * QS + 8 * cg) = rq[r];
          *reinterpret_cast<uint4 *>(sKt + tl * QS + 8 * cg) = rk[r];
        }
      }
      __syncthreads();
      for (int pr = tid; pr < M * M; pr += NT) {
        const int t = pr / M, s = pr - t * M;
        float acc = 0.f;
        if (s <= t) {
          for (int i = 0; i < dk; i += 2) {
            const uint32_t qw = *reinterpret_cast<const uint32_t *>(sQt + t * QS + i);
            const uint32_t kw = *reinterpret_cast<const uint32_t *>(sKt + s * QS + i);
            acc += bf16lo(qw) * bf16lo(kw) * exp2f(sB[t * DP + i] - sB[s * DP + i]);
            acc += bf16hi(qw) * bf16hi(kw) * exp2f(sB[t * DP + i + 1] - sB[s * DP + i + 1]);
          }
        }
        sP[t * TS + s] = (uint16_t)f2bf(acc);
      }
      __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NT;
      if (idx < ITEMS) {
        const int tl = idx / CG, cg = idx - tl * CG;
        const float *bt = sB + tl * DP + 8 * cg;
        const float *bl = sB + (M - 1) * DP + 8 * cg;
        const uint32_t qw[4] = {rq[r].x, rq[r].y, rq[r].z, rq[r].w};
        const uint32_t kw[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
        uint32_t oq[4], ok[4];
        float kh[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float b0 = bt[2 * e], b1 = bt[2 * e + 1];
          const float q0 = bf16lo(qw[e]), q1 = bf16hi(qw[e]);
          const float k0 = bf16lo(kw[e]), k1 = bf16hi(kw[e]);
          oq[e] = pack_bf16x2(q0 * exp2f(b0), q1 * exp2f(b1));
          ok[e] = pack_bf16x2(k0 * exp2f(-b0), k1 * exp2f(-b1));
          kh[2 * e] = k0 * exp2f(bl[2 * e] - b0);
          kh[2 * e + 1] = k1 * exp2f(bl[2 * e + 1] - b1);
        }
        *reinterpret_cast<uint4 *>(sQt + tl * QS + 8 * cg) = make_uint4(oq[0], oq[1], oq[2], oq[3]);
        if (!pairwise)
          *reinterpret_cast<uint4 *>(sKt + tl * QS + 8 * cg) = make_uint4(ok[0], ok[1], ok[2], ok[3]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sKh[(8 * cg + e) * TS + tl] = (uint16_t)f2bf(kh[e]);
      }
    }
    if (c + 1 < P.nchunks) load_chunk(c + 1);
    __syncthreads();

    // ---- stage 4: MFMA products of this wave's 16 value columns
    if (has_cols) {
      // v fragments, k = token pairs (16j0 + 4g4 + e, 16j1 + 4g4 + e)
      uint4 vf[(MT + 1) / 2];
#pragma unroll
      for (int jp = 0; jp < MT / 2; ++jp)
        vf[jp] = cat(lds2(sVT + (n0 + l16) * TS + 32 * jp + 4 * g4),
                     lds2(sVT + (n0 + l16) * TS + 32 * jp + 16 + 4 * g4));
      if (MT & 1)   // odd tile count (16-token chunks): zero upper half of the last K block
        vf[MT / 2] = cat(lds2(sVT + (n0 + l16) * TS + 16 * (MT - 1) + 4 * g4), make_uint2(0, 0));

      // S^T as the A operand of the inter-chunk product (bf16)
      uint4 sa[K32];
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) sa[kb] = cat(pack4(S[2 * kb]), pack4(S[2 * kb + 1]));

#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint16_t *qrow = sQt + (16 * i + l16) * QS;
        f32x4_t O = {0.f, 0.f, 0.f, 0.f};
        // intra-chunk weights P^T[s][t] for the s-tiles j <= i
        uint2 pt[MT];
        if (!pairwise) {
          uint4 qn[K32];
#pragma unroll
          for (int kb = 0; kb < K32; ++kb) qn[kb] = lds4(qrow + 32 * kb + 8 * g4);
#pragma unroll
          for (int j = 0; j <= i; ++j) {
            const uint16_t *krow = sKt + (16 * j + l16) * QS;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < K32; ++kb) acc = mfma32(lds4(krow + 32 * kb + 8 * g4), qn[kb], acc);
            if (j == i) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (4 * g4 + e > l16) acc[e] = 0.f;   // causal: s > t
            }
            pt[j] = pack4(acc);
          }
        } else {
#pragma unroll
          for (int j = 0; j <= i; ++j) pt[j] = lds2(sP + (16 * i + l16) * TS + 16 * j + 4 * g4);
        }
        // O^T += V^T P^T over the s-tiles j <= i
#pragma unroll
        for (int jp = 0; jp < MT / 2; ++jp) {
          const int j0 = 2 * jp, j1 = 2 * jp + 1;
          if (j0 <= i) {
            const uint2 hi = (j1 <= i) ? pt[j1] : make_uint2(0, 0);
            O = mfma32(vf[jp], cat(pt[j0], hi), O);
          }
        }
        if ((MT & 1) && i == MT - 1) O = mfma32(vf[MT / 2], cat(pt[MT - 1], make_uint2(0, 0)), O);
        // O^T += S^T q~^T
#pragma unroll
        for (int kb = 0; kb < K32; ++kb)
          O = mfma32(sa[kb], cat(lds2(qrow + 32 * kb + 4 * g4), lds2(qrow + 32 * kb + 16 + 4 * g4)), O);
        // store o[t][n0 + 4g4 .. +4], t = c*M + 16i + l16 (scan position)
        const int p = c * M + 16 * i + l16;
        const int n = n0 + 4 * g4;
        if (p < T && n < dv)
          *reinterpret_cast<uint2 *>(ob + (int64_t)p * P.o_st + n) = pack4(O);
      }

      // S = diag(e^{b_last}) S + k^T v
#pragma unroll
      for (int r = 0; r < DT; ++r) {
        const float4 gm = *reinterpret_cast<const float4 *>(sGam + 16 * r + 4 * g4);
        S[r][0] *= gm.x; S[r][1] *= gm.y; S[r][2] *= gm.z; S[r][3] *= gm.w;
        const uint16_t *krow = sKh + (16 * r + l16) * TS;
#pragma unroll
        for (int jp = 0; jp < MT / 2; ++jp)
          S[r] = mfma32(cat(lds2(krow + 32 * jp + 4 * g4), lds2(krow + 32 * jp + 16 + 4 * g4)), vf[jp], S[r]);
        if (MT & 1)
          S[r] = mfma32(cat(lds2(krow + 16 * (MT - 1) + 4 * g4), make_uint2(0, 0)), vf[MT / 2], S[r]);
      }
    }
    __syncthreads();
  }

  if (P.s_final && has_cols) {
#pragma unroll
    for (int r = 0; r < DT; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * r + 4 * g4 + e, n = n0 + l16;
        if (ch < dk && n < dv) P.s_final[((int64_t)unit * dk + ch) * dv + n] = S[r][e];
      }
    }
  }
}

template <int DP, int M>
hipError_t launch(const Params &p, hipStream_t s) {
  const int grid = ((p.units + 7) / 8) * 8;
  const size_t lds = Lds<DP, M>::bytes;
  auto *fn = gla_fwd_bf16_kernel<DP, M>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(Shape<DP>::NT), lds, s, p);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_m(const Params &p, int M, hipStream_t s) {
  switch (M) {
    case 16: return launch<DP, 16>(p, s);
    case 32: return launch<DP, 32>(p, s);
    case 64: return launch<DP, 64>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace dig

size_t dig_gla_bf16_workspace(int, int, int, int, int, int, int) { return 0; }

hipError_t dig_launch_gla_bf16(const DigGlaArgs &a, hipStream_t s) {
  using namespace dig;
  Params p;
  p.q = static_cast<const uint16_t *>(a.q);
  p.k = static_cast<const uint16_t *>(a.k);
  p.v = static_cast<const uint16_t *>(a.v);
  p.g = static_cast<const uint16_t *>(a.g);
  p.o = static_cast<uint16_t *>(a.o);
  p.s0 = a.s0;
  p.s_final = a.s_final;
  p.qk_sb = a.qk_sb; p.qk_st = a.qk_st; p.qk_sh = a.qk_sh;
  p.v_sb = a.v_sb; p.v_st = a.v_st; p.v_sh = a.v_sh;
  p.o_sb = a.o_sb; p.o_st = a.o_st; p.o_sh = a.o_sh;
  p.B = a.B; p.T = a.T; p.H = a.H; p.dk = a.dk; p.dv = a.dv;
  p.gh = a.gh; p.gw = a.gw; p.dir = a.dir;
  const int M = a.chunk;
  p.nchunks = (a.T + M - 1) / M;
  p.units = a.B * a.H;
  const int d = a.dk > a.dv ? a.dk : a.dv;
  const int DP = ((d + 31) / 32) * 32;
  switch (DP) {
    case 32: return launch_m<32>(p, M, s);
    case 64: return launch_m<64>(p, M, s);
    case 96: return launch_m<96>(p, M, s);
    case 128: return launch_m<128>(p, M, s);
    default: return hipErrorInvalidValue;
  }
}
