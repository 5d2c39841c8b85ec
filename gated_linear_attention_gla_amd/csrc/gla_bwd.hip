// gla_bwd.hip -- backward of the chunk-wise Gated Linear Attention on gfx950.
//
// The forward (gla_bf16.hip) computes, per (batch, head) in scan order,
//   S_p = diag(a_p) S_{p-1} + k_p^T v_p,   o_p = q_p S_p,   a_p = exp(log_alpha_p);
// the DiG paper notes (关键设计 / 硬件友好的效率设计) train the model with this
// operator, so its gradients are the reverse-mode derivative of the same
// recurrence.  With G_p = dL/dS_p,
//   G_p = q_p^T do_p + diag(a_{p+1}) G_{p+1}   (G after the last token: dS_final)
//   dq_p = S_p do_p^T,  dk_p = G_p v_p^T,  dv_p = k_p G_p,
//   dlog_alpha_p = a_p * rowsum(G_p (.) S_{p-1}),  ds0 = diag(a_0) G_0.
//
// Chunk form (chunks of M tokens; b the inclusive cumulative log-gate from
// the chunk start, per key channel, B its last value; S_in the state entering
// the chunk, D the gradient of the state leaving it):
//   A  = dO V^T and P = [q_t . (k_s e^{b_t - b_s})] on s <= t, zero above
//   dq = e^{b} (.) (dO S_in^T + A (k e^{-b}))
//   dk = e^{-b} (.) (A^T (q e^{b})) + e^{B - b} (.) (V D^T)
//   dv = P^T dO + (k e^{B - b}) D
//   D for the chunk before = diag(e^{B}) D + (q e^{b})^T dO
//   dlog_alpha_t = sum_{t' >= t in the chunk} (q (.) dq - k (.) dk)_{t'} + rowsum(S_out (.) D)
// The last line follows from the explicit form of o: log_alpha_t enters
// through the cumulative gates of t and of every later token, and the shift
// of all gates after a point by a constant only rescales the state at that
// point (so the later tokens' total is rowsum(S (.) dL/dS) there).
//
// Three launches:
//   gla_bwd_scan<.., false>  S_in of every chunk (forward over chunks);
//   gla_bwd_scan<.., true>   D of every chunk (reverse over chunks), and ds0;
//   gla_bwd_chunk            every chunk independently: dq, dk, dv, dlog_alpha.
// The scans use only factors e^{B - b} and e^{b} (<= 1 for gates <= 0).  The
// chunk kernel factorises e^{b_t - b_s} as e^{b_t} e^{-b_s} when every |b| of
// the chunk is within 2^64 in log2 units (the forward's bound); other chunks
// evaluate the decayed intra-chunk sums with exact exponent differences on
// the vector ALUs.
#include "dig_mfma.h"

namespace dig {
namespace {

// Largest |cumulative log2 gate| of a chunk for the factorised products.
constexpr float kBwdFastRange = 64.0f;

struct BwdParams {
  const uint16_t *q, *k, *v, *g, *dout;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, do_sb, do_st, do_sh;
  const float *s0, *ds_final;
  uint16_t *gq, *gk, *gv;   // dq, dk, dv: [B, T, H, dk | dv] contiguous, canonical order
  float *dg;                // [B, T, H, dk] contiguous, canonical order
  float *ds0;               // nullable [B, H, dk, dv]
  uint16_t *st_s;           // [units][N][DP][DP] bf16: state entering chunk c
  uint16_t *st_d;           // [units][N][DP][DP] bf16: gradient of the state leaving chunk c
  uint16_t *st_dt;          // the same, transposed ([j][i])
  int B, T, H, dk, dv, gh, gw, dir, nchunks;
  unsigned qk_span, v_span, do_span;   // bytes addressable in one (batch, head) slice
};

template <int DP>
struct BwdRow {
  // token-major bf16 row stride: conflict-free row and transposing reads (as
  // in the forward)
  static constexpr int QS = (DP == 64 || DP == 96) ? DP + 8 : DP + 24;
};

__device__ __forceinline__ float bf_at(const uint16_t *p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ uint16_t to_bf(float x) { return (uint16_t)f2bf(x); }
__device__ __forceinline__ uint2 gload8(const uint16_t *p) {
  const u32x2_t v = *(__attribute__((address_space(1))) const u32x2_t *)(size_t)p;
  return make_uint2(v.x, v.y);
}

// Inclusive sum over the chunk's tokens of a token-major bf16 tile (rows =
// tokens, columns = channels) for token tile I and channel tile r, on MFMA
// with a lower-triangular matrix of ones (bf16 values times 1.0 are exact,
// the sum is fp32).  Result in accumulator layout: rows t = 16 I + 4 (l/16)
// + e, channel 16 r + l%16.
template <int MT, int QS>
__device__ __forceinline__ f32x4_t tile_cumsum(const uint16_t *tg, int I, int r, int l16, int g4) {
  constexpr int JP = (MT + 1) / 2;
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);
  const int t = 16 * I + l16;   // this lane's row of the ones matrix
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jp = 0; jp < JP; ++jp) {
    if (32 * jp > 16 * I + 15) break;
    const bool hi_ok = 2 * jp + 1 < MT;
    uint32_t w[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s0 = 32 * jp + 16 * h + 4 * g4;   // K slots 4h .. 4h+3: tokens s0 .. s0+3
      const uint32_t o0 = (s0 + 0 <= t) ? 0x3f80u : 0u, o1 = (s0 + 1 <= t) ? 0x3f80u : 0u;
      const uint32_t o2 = (s0 + 2 <= t) ? 0x3f80u : 0u, o3 = (s0 + 3 <= t) ? 0x3f80u : 0u;
      w[2 * h] = o0 | (o1 << 16);
      w[2 * h + 1] = o2 | (o3 << 16);
    }
    const uint2 lo = lds_tr(tg + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
    const uint2 hi = hi_ok ? lds_tr(tg + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff) : make_uint2(0, 0);
    acc = mfma32(make_uint4(w[0], w[1], hi_ok ? w[2] : 0u, hi_ok ? w[3] : 0u), cat(lo, hi), acc);
  }
  return acc;
}

// ============================== state scans ==================================
// One workgroup per (batch, head); wave w holds value columns 16w .. 16w+15 of
// the dk x dv state in its accumulators (rows 16 r + 4 (l/16) + e, column
// 16 w + l%16).  Forward: X = k, Y = v, Z from s0, stores the state entering
// each chunk.  Reverse: X = q, Y = do (scan order), Z from ds_final, stores
// the gradient leaving each chunk (and its transpose), then ds0.
template <int DP, int M, bool REV>
__global__ void __launch_bounds__(DP / 16 * kWave)
gla_bwd_scan(BwdParams P) {
  constexpr int DT = DP / 16, NT = DT * kWave, MT = M / 16, JP = (MT + 1) / 2;
  constexpr int QS = BwdRow<DP>::QS, CG = DP / 8;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *tX = reinterpret_cast<uint16_t *>(smem);
  uint16_t *tG = tX + M * QS;
  uint16_t *tY = tG + M * QS;
  float *gam = reinterpret_cast<float *>(tY + M * QS);   // [DP] e^{B}

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);
  const int n0 = 16 * wave;
  const int unit = blockIdx.x, bb = unit / P.H, hh = unit - bb * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv, N = P.nchunks;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc((REV ? P.q : P.k) + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(P.g + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t ry = REV ? make_rsrc(P.dout + bb * P.do_sb + hh * P.do_sh, P.do_span)
                                        : make_rsrc(P.v + bb * P.v_sb + hh * P.v_sh, P.v_span);
  const int64_t y_st = REV ? P.do_st : P.v_st;

  f32x4_t Z[DT];
  const float *z0 = REV ? P.ds_final : P.s0;
#pragma unroll
  for (int r = 0; r < DT; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * r + 4 * g4 + e, j = n0 + l16;
      Z[r][e] = (z0 && i < dk && j < dv) ? z0[((int64_t)unit * dk + i) * dv + j] : 0.f;
    }

  // chunk rows go global -> registers (one chunk ahead) -> LDS
  constexpr int IT = (M * CG + NT - 1) / NT;
  uint4 px[IT], pg[IT], py[IT];
  auto fetch = [&](int c) {
#pragma unroll
    for (int kq = 0; kq < IT; ++kq) {
      const int idx = tid + kq * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      const int p = c * M + tl;
      const bool ok = idx < M * CG && p < T;
      const int n = ok ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : 0;
      const int64_t yrow = REV ? (int64_t)p : n;
      const unsigned oxg = (ok && 8 * cg < dk) ? (unsigned)(((int64_t)n * P.qk_st + 8 * cg) * 2) : kOOB;
      const unsigned oy = (ok && 8 * cg < dv) ? (unsigned)((yrow * y_st + 8 * cg) * 2) : kOOB;
      px[kq] = bload16(rx, oxg);
      pg[kq] = bload16(rg, oxg);
      py[kq] = bload16(ry, oy);
    }
  };
  fetch(REV ? N - 1 : 0);

  for (int it = 0; it < N; ++it) {
    const int c = REV ? N - 1 - it : it;
    // the state for chunk c, bf16, padding included (it is zero)
    const int64_t blk = ((int64_t)unit * N + c) * DP * DP;
    uint16_t *zs = (REV ? P.st_d : P.st_s) + blk;
#pragma unroll
    for (int r = 0; r < DT; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) zs[(16 * r + 4 * g4 + e) * DP + n0 + l16] = to_bf(Z[r][e]);
      if (REV) *reinterpret_cast<uint2 *>(P.st_dt + blk + (n0 + l16) * DP + 16 * r + 4 * g4) = pack4(Z[r]);
    }
    // chunk c's rows into LDS (zeros past T and in the channel padding)
#pragma unroll
    for (int kq = 0; kq < IT; ++kq) {
      const int idx = tid + kq * NT;
      if (idx < M * CG) {
        const int tl = idx / CG, cg = idx - tl * CG;
        *reinterpret_cast<uint4 *>(tX + tl * QS + 8 * cg) = px[kq];
        *reinterpret_cast<uint4 *>(tG + tl * QS + 8 * cg) = pg[kq];
        *reinterpret_cast<uint4 *>(tY + tl * QS + 8 * cg) = py[kq];
      }
    }
    __syncthreads();
    if (it + 1 < N) fetch(REV ? c - 1 : c + 1);
    // cumulative gates of key-channel tile `wave`; X scaled in place by
    // e^{B - b} (forward) or e^{b} (reverse), both <= 1
    {
      f32x4_t cum[MT];
#pragma unroll
      for (int I = 0; I < MT; ++I) cum[I] = tile_cumsum<MT, QS>(tG, I, wave, l16, g4);
      const float tot = __shfl(cum[MT - 1][3], 48 + l16, 64);   // token M-1: lane group 3, e = 3
      const int i = n0 + l16;
#pragma unroll
      for (int I = 0; I < MT; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * I + 4 * g4 + e;
          const float f = fexp2((REV ? cum[I][e] : tot - cum[I][e]) * kLog2e);
          tX[t * QS + i] = to_bf(bf_at(tX + t * QS + i) * f);
        }
      if (g4 == 0) gam[i] = fexp2(tot * kLog2e);
    }
    __syncthreads();
    // Z = diag(e^{B}) Z + X^T Y, K = the chunk's tokens (transposing reads)
    uint4 yf[JP];
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const uint2 lo = lds_tr(tY + (32 * jp + 4 * g4 + rowoff) * QS + n0 + coloff);
      const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(tY + (32 * jp + 16 + 4 * g4 + rowoff) * QS + n0 + coloff)
                                         : make_uint2(0, 0);
      yf[jp] = cat(lo, hi);
    }
#pragma unroll
    for (int r = 0; r < DT; ++r) {
      const float4 gm = *reinterpret_cast<const float4 *>(gam + 16 * r + 4 * g4);
      Z[r][0] *= gm.x; Z[r][1] *= gm.y; Z[r][2] *= gm.z; Z[r][3] *= gm.w;
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const uint2 lo = lds_tr(tX + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
        const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(tX + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff)
                                           : make_uint2(0, 0);
        Z[r] = mfma32(cat(lo, hi), yf[jp], Z[r]);
      }
    }
    __syncthreads();
  }
  if (REV && P.ds0) {
#pragma unroll
    for (int r = 0; r < DT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r + 4 * g4 + e, j = n0 + l16;
        if (i < dk && j < dv) P.ds0[((int64_t)unit * dk + i) * dv + j] = Z[r][e];
      }
  }
}

// ============================ chunk gradients ================================
template <int DP, int M>
struct BwdLds {
  static constexpr int QS = BwdRow<DP>::QS;
  static constexpr int SA = M + 8;                     // row stride of the M x M tiles
  static constexpr int TILE = M * QS * 2;
  static constexpr int oQ = 0, oK = TILE, oV = 2 * TILE, oO = 3 * TILE;   // raw q, k, v, do
  static constexpr int oQt = 4 * TILE, oKt = 5 * TILE;  // q e^{b}, k e^{-b}; extreme chunks: fp32 dq sums
  static constexpr int oKh = 6 * TILE;                  // gates, then k e^{B - b}
  static constexpr int oB = 7 * TILE;                   // [M][DP] fp32 b (log2 units)
  static constexpr int oA = oB + M * DP * 4;            // [M][SA] bf16 A = dO V^T (causal)
  static constexpr int oP = oA + M * SA * 2;            // [M][SA] bf16 P (causal)
  static constexpr int oR = oP + M * SA * 2;            // [M][DP] fp32 q dq - k dk (extreme: dk sums first)
  static constexpr int oBt = oR + M * DP * 4;           // [DP] B (log2 units)
  static constexpr int oGam = oBt + DP * 4;             // [DP] e^{B}
  static constexpr int oSuf = oGam + DP * 4;            // [DP/16][DP] rowsum(S_out (.) D), per column tile
  static constexpr int oTok = oSuf + (DP / 16) * DP * 4;   // [M] canonical token, -1 past T
  static constexpr int oFlag = oTok + M * 4;            // bit pattern of max |b|
  static constexpr int bytes = oFlag + 16;
  static_assert(2 * TILE >= M * DP * 4, "the fp32 dq sums of extreme chunks overlay the q~, k~ tiles");
};

constexpr int kChunkWaves = 8;

template <int DP, int M>
__global__ void __launch_bounds__(kChunkWaves * kWave)
gla_bwd_chunk(BwdParams P) {
  using L = BwdLds<DP, M>;
  constexpr int NT = kChunkWaves * kWave, MT = M / 16, JP = (MT + 1) / 2, DT = DP / 16;
  constexpr int K32 = DP / 32;
  constexpr bool KH = (DP % 32) != 0;
  constexpr int QS = L::QS, SA = L::SA, CG = DP / 8;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *tQ = reinterpret_cast<uint16_t *>(smem + L::oQ), *tK = reinterpret_cast<uint16_t *>(smem + L::oK);
  uint16_t *tV = reinterpret_cast<uint16_t *>(smem + L::oV), *tO = reinterpret_cast<uint16_t *>(smem + L::oO);
  uint16_t *tQt = reinterpret_cast<uint16_t *>(smem + L::oQt), *tKt = reinterpret_cast<uint16_t *>(smem + L::oKt);
  uint16_t *tKh = reinterpret_cast<uint16_t *>(smem + L::oKh);
  float *bL = reinterpret_cast<float *>(smem + L::oB);
  uint16_t *tA = reinterpret_cast<uint16_t *>(smem + L::oA), *tP = reinterpret_cast<uint16_t *>(smem + L::oP);
  float *E1 = reinterpret_cast<float *>(smem + L::oQt);   // extreme chunks only
  float *R = reinterpret_cast<float *>(smem + L::oR);
  float *gam = reinterpret_cast<float *>(smem + L::oGam), *suf = reinterpret_cast<float *>(smem + L::oSuf);
  float *Bt = reinterpret_cast<float *>(smem + L::oBt);
  int *tok = reinterpret_cast<int *>(smem + L::oTok);
  unsigned *flag = reinterpret_cast<unsigned *>(smem + L::oFlag);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);
  const int N = P.nchunks;
  const int unit = blockIdx.x / N, c = blockIdx.x - unit * N;
  const int bb = unit / P.H, hh = unit - bb * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv, H = P.H;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(P.q + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(P.k + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(P.g + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(P.v + bb * P.v_sb + hh * P.v_sh, P.v_span);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(P.dout + bb * P.do_sb + hh * P.do_sh, P.do_span);
  const int64_t blk = ((int64_t)unit * N + c) * DP * DP;
  const uint16_t *Sin = P.st_s + blk, *Dm = P.st_d + blk, *Dt = P.st_dt + blk;

  // ---- 1. the chunk's rows (q, k, gates, v canonical; do in scan order)
  if (tid < M) {
    const int p = c * M + tid;
    tok[tid] = p < T ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : -1;
  }
  if (tid == 0) *flag = 0u;
  __syncthreads();
  for (int idx = tid; idx < M * CG; idx += NT) {
    const int tl = idx / CG, cg = idx - tl * CG;
    const int n = tok[tl];
    const unsigned oqk = (n >= 0 && 8 * cg < dk) ? (unsigned)(((int64_t)n * P.qk_st + 8 * cg) * 2) : kOOB;
    const unsigned ov = (n >= 0 && 8 * cg < dv) ? (unsigned)(((int64_t)n * P.v_st + 8 * cg) * 2) : kOOB;
    const unsigned oo = (n >= 0 && 8 * cg < dv) ? (unsigned)((((int64_t)c * M + tl) * P.do_st + 8 * cg) * 2) : kOOB;
    const int at = tl * QS + 8 * cg;
    *reinterpret_cast<uint4 *>(tQ + at) = bload16(rq, oqk);
    *reinterpret_cast<uint4 *>(tK + at) = bload16(rk, oqk);
    *reinterpret_cast<uint4 *>(tKh + at) = bload16(rg, oqk);
    *reinterpret_cast<uint4 *>(tV + at) = bload16(rv, ov);
    *reinterpret_cast<uint4 *>(tO + at) = bload16(ro, oo);
  }
  __syncthreads();

  // ---- 2. cumulative gates (log2 units; ones-triangle MFMA over the gate
  //         tile) and the scaled rows
  for (int tt = wave; tt < MT * DT; tt += kChunkWaves) {
    const int I = tt / DT, r = tt - I * DT;
    const f32x4_t cum = tile_cumsum<MT, QS>(tKh, I, r, l16, g4);
    const int i = 16 * r + l16;
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float b = cum[e] * kLog2e;
      bL[(16 * I + 4 * g4 + e) * DP + i] = b;
      mx = fmaxf(mx, fabsf(b));
    }
    if (I == MT - 1 && g4 == 3) Bt[i] = cum[3] * kLog2e;   // token M-1
    if (!(mx <= kBwdFastRange)) atomicOr(flag, 1u);          // NaN / inf too
  }
  __syncthreads();
  for (int x = tid; x < M * DP; x += NT) {
    const int t = x / DP, i = x - t * DP;
    const float b = bL[x], B = Bt[i];
    const float q = bf_at(tQ + t * QS + i), k = bf_at(tK + t * QS + i);
    tQt[t * QS + i] = to_bf(q * fexp2(b));
    tKt[t * QS + i] = to_bf(k * fexp2(-b));
    tKh[t * QS + i] = to_bf(k * fexp2(B - b));
  }
  if (tid < DP) gam[tid] = fexp2(Bt[tid]);
  __syncthreads();
  const bool fast = *flag == 0u;

  // ---- 3. A = dO V^T and (factorised chunks) P = Q~ K~^T on s <= t, zero above
  for (int tt = wave; tt < MT * MT; tt += kChunkWaves) {
    const int I = tt / MT, J = tt - I * MT;   // rows t (tile I), columns s (tile J)
    f32x4_t a = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
    if (J <= I) {
      const uint16_t *orow = tO + (16 * I + l16) * QS, *vrow = tV + (16 * J + l16) * QS;
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) a = mfma32(lds4(orow + 32 * kb + 8 * g4), lds4(vrow + 32 * kb + 8 * g4), a);
      if (KH) a = mfma16(lds2(orow + 32 * K32 + 4 * g4), lds2(vrow + 32 * K32 + 4 * g4), a);
      if (fast) {
        const uint16_t *qrow = tQt + (16 * I + l16) * QS, *krow = tKt + (16 * J + l16) * QS;
#pragma unroll
        for (int kb = 0; kb < K32; ++kb)
          pp = mfma32(lds4(qrow + 32 * kb + 8 * g4), lds4(krow + 32 * kb + 8 * g4), pp);
        if (KH) pp = mfma16(lds2(qrow + 32 * K32 + 4 * g4), lds2(krow + 32 * K32 + 4 * g4), pp);
      }
      if (J == I) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (l16 > 4 * g4 + e) { a[e] = 0.f; pp[e] = 0.f; }   // causal: s > t
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int at = (16 * I + 4 * g4 + e) * SA + 16 * J + l16;
      tA[at] = to_bf(a[e]);
      if (fast) tP[at] = to_bf(pp[e]);
    }
  }
  __syncthreads();

  // ---- 3b. chunks beyond the factorised range: exact exponent differences
  if (!fast) {
    for (int x = tid; x < M * M; x += NT) {
      const int t = x / M, s = x - t * M;
      float acc = 0.f;
      if (s <= t)
        for (int i = 0; i < dk; ++i)
          acc += bf_at(tQ + t * QS + i) * bf_at(tK + s * QS + i) * fexp2(bL[t * DP + i] - bL[s * DP + i]);
      tP[t * SA + s] = to_bf(acc);
    }
    for (int x = tid; x < M * DP; x += NT) {
      const int t = x / DP, i = x - t * DP;
      float aq = 0.f, ak = 0.f;
      if (i < dk) {
        for (int s = 0; s <= t; ++s)   // dq sums: keys s <= t
          aq += bf_at(tA + t * SA + s) * bf_at(tK + s * QS + i) * fexp2(bL[t * DP + i] - bL[s * DP + i]);
        for (int u = t; u < M; ++u)    // dk sums: queries u >= t (t as the key)
          ak += bf_at(tA + u * SA + t) * bf_at(tQ + u * QS + i) * fexp2(bL[u * DP + i] - bL[t * DP + i]);
      }
      E1[t * DP + i] = aq;
      R[t * DP + i] = ak;
    }
    __syncthreads();
  }

  // ---- 4. dq, dk (unit (I, r): tokens of tile I, key channels of tile r) and
  //         dv (unit (I, cc): tokens of tile I, value channels of tile cc)
  for (int u = wave; u < 2 * MT * DT; u += kChunkWaves) {
    const bool is_v = u >= MT * DT;
    const int uu = is_v ? u - MT * DT : u;
    const int I = uu / DT, r = uu - I * DT;
    const uint16_t *orow = tO + (16 * I + l16) * QS;
    if (!is_v) {
      // dO S_in^T and V D^T: K = value channels; B operands straight from the
      // state blocks (rows i of S_in and D)
      f32x4_t x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *vrow = tV + (16 * I + l16) * QS;
      const uint16_t *srow = Sin + (16 * r + l16) * DP, *drow = Dm + (16 * r + l16) * DP;
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) {
        x1 = mfma32(lds4(orow + 32 * kb + 8 * g4), gload16(srow + 32 * kb + 8 * g4), x1);
        x2 = mfma32(lds4(vrow + 32 * kb + 8 * g4), gload16(drow + 32 * kb + 8 * g4), x2);
      }
      if (KH) {
        x1 = mfma16(lds2(orow + 32 * K32 + 4 * g4), gload8(srow + 32 * K32 + 4 * g4), x1);
        x2 = mfma16(lds2(vrow + 32 * K32 + 4 * g4), gload8(drow + 32 * K32 + 4 * g4), x2);
      }
      // A K~ and A^T Q~ (K = tokens): only the blocks on the causal side
      f32x4_t y1 = {0.f, 0.f, 0.f, 0.f}, y2 = {0.f, 0.f, 0.f, 0.f};
      if (fast) {
        const uint16_t *arow = tA + (16 * I + l16) * SA;
#pragma unroll
        for (int jp = 0; jp < JP; ++jp) {
          const bool hi_ok = 2 * jp + 1 < MT;
          if (32 * jp <= 16 * I + 15) {   // keys s <= t
            const uint4 af = cat(lds2(arow + 32 * jp + 4 * g4), hi_ok ? lds2(arow + 32 * jp + 16 + 4 * g4) : make_uint2(0, 0));
            const uint2 lo = lds_tr(tKt + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
            const uint2 hi = hi_ok ? lds_tr(tKt + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff) : make_uint2(0, 0);
            y1 = mfma32(af, cat(lo, hi), y1);
          }
          if (32 * jp + 31 >= 16 * I) {   // queries u >= t
            const uint2 alo = lds_tr(tA + (32 * jp + 4 * g4 + rowoff) * SA + 16 * I + coloff);
            const uint2 ahi = hi_ok ? lds_tr(tA + (32 * jp + 16 + 4 * g4 + rowoff) * SA + 16 * I + coloff) : make_uint2(0, 0);
            const uint2 qlo = lds_tr(tQt + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
            const uint2 qhi = hi_ok ? lds_tr(tQt + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff) : make_uint2(0, 0);
            y2 = mfma32(cat(alo, ahi), cat(qlo, qhi), y2);
          }
        }
      }
      // combine, store, and keep q dq - k dk for the gate gradient
      const int i = 16 * r + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * I + 4 * g4 + e;
        const float b = bL[t * DP + i], B = bL[(M - 1) * DP + i];
        float dqv, dkv;
        if (fast) {
          dqv = fexp2(b) * (x1[e] + y1[e]);
          dkv = fexp2(-b) * y2[e] + fexp2(B - b) * x2[e];
        } else {
          dqv = fexp2(b) * x1[e] + E1[t * DP + i];
          dkv = R[t * DP + i] + fexp2(B - b) * x2[e];
        }
        R[t * DP + i] = bf_at(tQ + t * QS + i) * dqv - bf_at(tK + t * QS + i) * dkv;
        const int n = tok[t];
        if (n >= 0 && i < dk) {
          const int64_t o = (((int64_t)bb * T + n) * H + hh) * dk + i;
          P.gq[o] = to_bf(dqv);
          P.gk[o] = to_bf(dkv);
        }
      }
    } else {
      // dv = P^T dO + K^ D: K = tokens for the first (transposing reads), key
      // channels for the second (rows of D^T)
      const int cc = r;
      f32x4_t y3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const bool hi_ok = 2 * jp + 1 < MT;
        if (32 * jp + 31 >= 16 * I) {   // queries t >= s
          const uint2 plo = lds_tr(tP + (32 * jp + 4 * g4 + rowoff) * SA + 16 * I + coloff);
          const uint2 phi = hi_ok ? lds_tr(tP + (32 * jp + 16 + 4 * g4 + rowoff) * SA + 16 * I + coloff) : make_uint2(0, 0);
          const uint2 olo = lds_tr(tO + (32 * jp + 4 * g4 + rowoff) * QS + 16 * cc + coloff);
          const uint2 ohi = hi_ok ? lds_tr(tO + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * cc + coloff) : make_uint2(0, 0);
          y3 = mfma32(cat(plo, phi), cat(olo, ohi), y3);
        }
      }
      const uint16_t *hrow = tKh + (16 * I + l16) * QS, *dtrow = Dt + (16 * cc + l16) * DP;
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) y3 = mfma32(lds4(hrow + 32 * kb + 8 * g4), gload16(dtrow + 32 * kb + 8 * g4), y3);
      if (KH) y3 = mfma16(lds2(hrow + 32 * K32 + 4 * g4), gload8(dtrow + 32 * K32 + 4 * g4), y3);
      const int j = 16 * cc + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = tok[16 * I + 4 * g4 + e];
        if (n >= 0 && j < dv) P.gv[(((int64_t)bb * T + n) * H + hh) * dv + j] = to_bf(y3[e]);
      }
    }
  }

  // ---- 5. rowsum(S_out (.) D): S_out = diag(e^{B}) S_in + K^^T V
  for (int u = wave; u < DT * DT; u += kChunkWaves) {
    const int r = u / DT, cc = u - r * DT;
    f32x4_t so = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const bool hi_ok = 2 * jp + 1 < MT;
      const uint2 klo = lds_tr(tKh + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
      const uint2 khi = hi_ok ? lds_tr(tKh + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff) : make_uint2(0, 0);
      const uint2 vlo = lds_tr(tV + (32 * jp + 4 * g4 + rowoff) * QS + 16 * cc + coloff);
      const uint2 vhi = hi_ok ? lds_tr(tV + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * cc + coloff) : make_uint2(0, 0);
      so = mfma32(cat(klo, khi), cat(vlo, vhi), so);
    }
    const int j = 16 * cc + l16;
    const uint2 dd = gload8(Dt + j * DP + 16 * r + 4 * g4);   // D[i][j], i = 16 r + 4 g + e
    const float dval[4] = {bf16lo(dd.x), bf16hi(dd.x), bf16lo(dd.y), bf16hi(dd.y)};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * r + 4 * g4 + e;
      float x = (gam[i] * bf_at(Sin + i * DP + j) + so[e]) * dval[e];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);   // over the 16 columns
      if (l16 == 0) suf[cc * DP + i] = x;   // summed over the column tiles in a fixed order below
    }
  }
  __syncthreads();

  // ---- 6. dlog_alpha: reverse sum over the chunk plus the later chunks' total
  if (tid < dk) {
    const int i = tid;
    float run = 0.f;
#pragma unroll
    for (int cc = 0; cc < DT; ++cc) run += suf[cc * DP + i];
    for (int t = M - 1; t >= 0; --t) {
      run += R[t * DP + i];
      const int n = tok[t];
      if (n >= 0) P.dg[(((int64_t)bb * T + n) * H + hh) * dk + i] = run;
    }
  }
}

// ------------------------------ host side -----------------------------------
int bwd_pad(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 80 ? 80 : d <= 96 ? 96 : 128; }

template <int DP, int M>
hipError_t launch_bwd(const BwdParams &p, hipStream_t s) {
  constexpr int QS = BwdRow<DP>::QS;
  const size_t scan_lds = (size_t)3 * M * QS * 2 + DP * 4 + M * 4;
  const size_t chunk_lds = BwdLds<DP, M>::bytes;
  hipError_t e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(gla_bwd_scan<DP, M, false>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_lds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(gla_bwd_scan<DP, M, true>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)scan_lds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(gla_bwd_chunk<DP, M>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)chunk_lds);
  if (e != hipSuccess) return e;
  const int units = p.B * p.H;
  hipLaunchKernelGGL((gla_bwd_scan<DP, M, false>), dim3(units), dim3(DP / 16 * kWave), scan_lds, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((gla_bwd_scan<DP, M, true>), dim3(units), dim3(DP / 16 * kWave), scan_lds, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((gla_bwd_chunk<DP, M>), dim3((int64_t)units * p.nchunks), dim3(kChunkWaves * kWave),
                     chunk_lds, s, p);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_bwd_m(const BwdParams &p, int M, hipStream_t s) {
  switch (M) {
    case 16: return launch_bwd<DP, 16>(p, s);
    case 32: return launch_bwd<DP, 32>(p, s);
    case 64:
      if constexpr (DP <= 80) return launch_bwd<DP, 64>(p, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace dig

int dig_gla_bwd_chunk(int dk, int dv, int chunk) {
  if (chunk != 0) return chunk;
  return dig::bwd_pad(dk > dv ? dk : dv) <= 80 ? 64 : 32;
}

size_t dig_gla_bwd_workspace(int B, int T, int H, int dk, int dv, int chunk) {
  const int DP = dig::bwd_pad(dk > dv ? dk : dv);
  const int M = dig_gla_bwd_chunk(dk, dv, chunk);
  const size_t N = ((size_t)T + M - 1) / M;
  return 3 * (size_t)B * H * N * DP * DP * 2;
}

hipError_t dig_launch_gla_bwd(const DigGlaBwdArgs &a, hipStream_t s) {
  using namespace dig;
  const int DP = bwd_pad(a.dk > a.dv ? a.dk : a.dv);
  const int M = dig_gla_bwd_chunk(a.dk, a.dv, a.chunk);
  BwdParams p;
  p.q = static_cast<const uint16_t *>(a.q);
  p.k = static_cast<const uint16_t *>(a.k);
  p.v = static_cast<const uint16_t *>(a.v);
  p.g = static_cast<const uint16_t *>(a.g);
  p.dout = static_cast<const uint16_t *>(a.dout);
  p.qk_sb = a.qk_sb; p.qk_st = a.qk_st; p.qk_sh = a.qk_sh;
  p.v_sb = a.v_sb; p.v_st = a.v_st; p.v_sh = a.v_sh;
  p.do_sb = a.do_sb; p.do_st = a.do_st; p.do_sh = a.do_sh;
  p.s0 = a.s0; p.ds_final = a.ds_final;
  p.gq = static_cast<uint16_t *>(a.dq);
  p.gk = static_cast<uint16_t *>(a.dk_out);
  p.gv = static_cast<uint16_t *>(a.dv_out);
  p.dg = a.dlog_alpha;
  p.ds0 = a.ds0;
  p.B = a.B; p.T = a.T; p.H = a.H; p.dk = a.dk; p.dv = a.dv;
  p.gh = a.gh; p.gw = a.gw; p.dir = a.dir;
  p.nchunks = (a.T + M - 1) / M;
  const size_t blkb = (size_t)a.B * a.H * p.nchunks * DP * DP * 2;
  unsigned char *ws = static_cast<unsigned char *>(a.workspace);
  p.st_s = reinterpret_cast<uint16_t *>(ws);
  p.st_d = reinterpret_cast<uint16_t *>(ws + blkb);
  p.st_dt = reinterpret_cast<uint16_t *>(ws + 2 * blkb);
  auto span = [](int64_t st, int d, int T_) {
    return (unsigned)(((int64_t)(T_ - 1) * st + d) * 2);
  };
  p.qk_span = span(a.qk_st, a.dk, a.T);
  p.v_span = span(a.v_st, a.dv, a.T);
  p.do_span = span(a.do_st, a.dv, a.T);
  switch (DP) {
    case 32: return launch_bwd_m<32>(p, M, s);
    case 64: return launch_bwd_m<64>(p, M, s);
    case 80: return launch_bwd_m<80>(p, M, s);
    case 96: return launch_bwd_m<96>(p, M, s);
    default: return launch_bwd_m<128>(p, M, s);
  }
}
