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
// Two launches:
//   gla_bwd_scan   S_in of every chunk (forward over chunks) and, side by
//                  side, D of every chunk (reverse over chunks), and ds0;
//   gla_bwd_chunk  the chunks, independently: dq, dk, dv, dlog_alpha.
// Both state sets are kept transposed ([value channel j][key channel i],
// bf16).  The scans use only factors e^{B - b} and e^{b} (<= 1 for gates <=
// 0).  The chunk kernel factorises e^{b_t - b_s} as e^{b_t} e^{-b_s} when
// every |b| of the chunk is within 2^64 in log2 units (the forward's bound);
// other chunks evaluate the decayed intra-chunk sums with exact exponent
// differences on the vector ALUs.
#include "dig_mfma.h"
#include <atomic>

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
  uint16_t *st_s;           // [units][N] blocks of DP x DP bf16: state entering chunk c, transposed,
                            // in 16 x 16 tiles (see gla_bwd_scan)
  uint16_t *st_d;           // the same layout: gradient of the state leaving chunk c
  int B, T, H, dk, dv, gh, gw, dir, nchunks;
  const int *order;         // scan position -> canonical token [T] (the kernels' ORD path)
  unsigned qk_span, v_span, do_span;   // bytes addressable in one (batch, head) slice
};

// ORD path: table entry p (0 for p outside the table), loaded through a
// buffer descriptor so that the load is issued by every lane.
__device__ __forceinline__ int ord_entry(__amdgpu_buffer_rsrc_t r, bool ok, int p) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, ok ? p * 4 : (int)kOOB, 0, 0);
}

template <int DP>
struct BwdRow {
  // token-major bf16 row stride: conflict-free row and transposing reads (as
  // in the forward)
  static constexpr int QS = (DP == 64 || DP == 96) ? DP + 8 : DP + 24;
};

__device__ __forceinline__ float bf_at(const uint16_t *p) { return __uint_as_float((uint32_t)(*p) << 16); }
__device__ __forceinline__ uint16_t to_bf(float x) { return (uint16_t)f2bf(x); }
__device__ __forceinline__ float4 unpack4(uint2 u) {
  return make_float4(bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y));
}
__device__ __forceinline__ float elt(const float4 &v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

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

// Token tiles I = 2 jp and 2 jp + 1 of a channel column held in accumulator
// layout (4 bf16 per lane per tile) as the 32 token K slots of one MFMA
// operand: slots 8 (l/16) .. +3 are tokens 32 jp + 4 (l/16) + e, slots +4 ..
// +7 tokens 32 jp + 16 + 4 (l/16) + e -- the order of an lds_tr pair.
template <int MT>
__device__ __forceinline__ uint4 kslots(const uint2 (&x)[MT], int jp) {
  return cat(x[2 * jp], (2 * jp + 1 < MT) ? x[(2 * jp + 1 < MT) ? 2 * jp + 1 : 0] : make_uint2(0, 0));
}
// The matching operand read from a token-major tile (rows = tokens), for
// channels col .. col+15.
template <int MT>
__device__ __forceinline__ uint4 tr_pair(const uint16_t *tile, int stride, int jp, int col, int g4, int rowoff,
                                         int coloff) {
  const uint2 lo = lds_tr(tile + (32 * jp + 4 * g4 + rowoff) * stride + col + coloff);
  const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(tile + (32 * jp + 16 + 4 * g4 + rowoff) * stride + col + coloff)
                                     : make_uint2(0, 0);
  return cat(lo, hi);
}

// ============================== state scans ==================================
// One workgroup of DT waves per (batch, head) unit; wave r holds rows i =
// 16 r .. 16 r + 15 of the dk x dv state in DT accumulators (rows 16 r +
// 4 (l/16) + e, columns 16 cc + l%16).  The waves load each chunk's rows
// together (two chunks ahead, in registers) and share them through LDS;
// otherwise each works on its own rows: the cumsum of its key channels'
// gates, X scaled in registers and used directly as the MFMA's A operand.
// Forward: X = k, Y = v, Z from s0, stores the state entering each chunk.
// Reverse: X = q, Y = do (scan order), Z from ds_final, stores the gradient
// of the state leaving each chunk, then ds0.  States are stored tile-major:
// 16 x 16 tile (cc, r) of the transposed state ([j][i]) at (cc DT + r) 256,
// so each wave's store is 512 contiguous bytes.
template <int DP, int M>
struct ScanLds {
  static constexpr int QS = BwdRow<DP>::QS;
  static constexpr int bytes = 3 * M * QS * 2;   // X, gates, Y: token-major [M][QS]
};

template <int DP, int M, bool REV, bool ORD>
__device__ __forceinline__ void scan_unit(const BwdParams &P, int unit) {
  constexpr int DT = DP / 16, MT = M / 16, JP = (MT + 1) / 2, NT = DT * kWave;
  constexpr int QS = ScanLds<DP, M>::QS, CG = DP / 8;
  constexpr int IT = (M * CG + NT - 1) / NT;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *tX = reinterpret_cast<uint16_t *>(smem);
  uint16_t *tG = tX + M * QS;
  uint16_t *tY = tG + M * QS;

  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);   // key-channel tile of this wave
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);
  const int bb = unit / P.H, hh = unit - bb * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv, N = P.nchunks;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc((REV ? P.q : P.k) + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(P.g + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t ry = REV ? make_rsrc(P.dout + bb * P.do_sb + hh * P.do_sh, P.do_span)
                                        : make_rsrc(P.v + bb * P.v_sb + hh * P.v_sh, P.v_span);
  const int64_t y_st = REV ? P.do_st : P.v_st;

  f32x4_t Z[DT];
  const float *z0 = REV ? P.ds_final : P.s0;
#pragma unroll
  for (int cc = 0; cc < DT; ++cc)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * r + 4 * g4 + e, j = 16 * cc + l16;
      Z[cc][e] = (z0 && i < dk && j < dv) ? z0[((int64_t)unit * dk + i) * dv + j] : 0.f;
    }

  // ORD: a set's table entries for the chunk it fetches next, loaded by the
  // fetch before
  const __amdgpu_buffer_rsrc_t rord = make_rsrc(ORD ? P.order : nullptr, ORD ? (unsigned)T * 4u : 0u);
  struct Rows {
    uint4 x[IT], g[IT], y[IT];
    int ord[IT];
  };
  auto ord_rows = [&](Rows &f, int c) {
    if constexpr (ORD) {
#pragma unroll
      for (int kq = 0; kq < IT; ++kq) {
        const int idx = tid + kq * NT, tl = idx / CG;
        f.ord[kq] = ord_entry(rord, idx < M * CG && c * M + tl < T, c * M + tl);
      }
    }
  };
  auto fetch = [&](Rows &f, int c, int c_next) {
#pragma unroll
    for (int kq = 0; kq < IT; ++kq) {
      const int idx = tid + kq * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      const int p = c * M + tl;
      bool ok = idx < M * CG && p < T;
      int n;
      if constexpr (ORD) {
        n = f.ord[kq];
        ok = ok && n >= 0 && n < T;
      } else {
        n = ok ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : 0;
      }
      const int64_t yrow = REV ? (int64_t)p : (int64_t)n;
      const unsigned oxg = (ok && 8 * cg < dk) ? (unsigned)(((int64_t)n * P.qk_st + 8 * cg) * 2) : kOOB;
      const unsigned oy = (ok && 8 * cg < dv) ? (unsigned)((yrow * y_st + 8 * cg) * 2) : kOOB;
      f.x[kq] = bload16(rx, oxg);
      f.g[kq] = bload16(rg, oxg);
      f.y[kq] = bload16(ry, oy);
    }
    ord_rows(f, c_next);
  };
  auto stash = [&](const Rows &f) {
#pragma unroll
    for (int kq = 0; kq < IT; ++kq) {
      const int idx = tid + kq * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      if ((M * CG) % NT == 0 || idx < M * CG) {
        *reinterpret_cast<uint4 *>(tX + tl * QS + 8 * cg) = f.x[kq];
        *reinterpret_cast<uint4 *>(tG + tl * QS + 8 * cg) = f.g[kq];
        *reinterpret_cast<uint4 *>(tY + tl * QS + 8 * cg) = f.y[kq];
      }
    }
  };

  uint16_t *zbase = (REV ? P.st_d : P.st_s) + (int64_t)unit * N * DP * DP;
  auto step = [&](Rows &f, int it) {
    const int c = REV ? N - 1 - it : it;
    // the state for chunk c (transposed, tile-major; padding included, zero)
    uint16_t *zt = zbase + (int64_t)c * DP * DP + r * 256 + l16 * 16 + 4 * g4;
#pragma unroll
    for (int cc = 0; cc < DT; ++cc) *reinterpret_cast<uint2 *>(zt + cc * DT * 256) = pack4(Z[cc]);
    stash(f);
    lds_barrier();
    // issued on every step (past the ends: the last chunk again, unused) so
    // the wait before each stash covers exactly the rows it needs
    {
      const int cf = REV ? max(c - 2, 0) : min(c + 2, N - 1);
      fetch(f, cf, REV ? max(cf - 2, 0) : min(cf + 2, N - 1));
    }
    // cumulative gates of key-channel tile r (accumulator layout: token
    // 16 I + 4 (l/16) + e, channel 16 r + l%16) and X scaled by e^{B - b}
    // (forward) or e^{b} (reverse), both <= 1
    uint2 xh[MT];
    float tot;
    {
      f32x4_t cum[MT];
#pragma unroll
      for (int I = 0; I < MT; ++I) cum[I] = tile_cumsum<MT, QS>(tG, I, r, l16, g4);
      tot = __shfl(cum[MT - 1][3], 48 + l16, kWave);   // token M-1: lane group 3, e = 3
#pragma unroll
      for (int I = 0; I < MT; ++I) {
        const float4 xv = unpack4(lds_tr(tX + (16 * I + 4 * g4 + rowoff) * QS + 16 * r + coloff));
        f32x4_t sx;
#pragma unroll
        for (int e = 0; e < 4; ++e) sx[e] = elt(xv, e) * fexp2((REV ? cum[I][e] : tot - cum[I][e]) * kLog2e);
        xh[I] = pack4(sx);
      }
    }
    float gm[4];   // e^{B} of rows 16 r + 4 (l/16) + e
#pragma unroll
    for (int e = 0; e < 4; ++e) gm[e] = fexp2(__shfl(tot, 4 * g4 + e, kWave) * kLog2e);
    // Z = diag(e^{B}) Z + X^T Y, K = the chunk's tokens
#pragma unroll
    for (int cc = 0; cc < DT; ++cc) {
#pragma unroll
      for (int e = 0; e < 4; ++e) Z[cc][e] *= gm[e];
#pragma unroll
      for (int jp = 0; jp < JP; ++jp)
        Z[cc] = mfma32(kslots<MT>(xh, jp), tr_pair<MT>(tY, QS, jp, 16 * cc, g4, rowoff, coloff), Z[cc]);
    }
    lds_barrier();
  };

  Rows fa, fb;
  {
    const int ca = REV ? N - 1 : 0, cb = REV ? max(N - 2, 0) : min(1, N - 1);
    ord_rows(fa, ca);
    ord_rows(fb, cb);
    fetch(fa, ca, REV ? max(ca - 2, 0) : min(ca + 2, N - 1));
    fetch(fb, cb, REV ? max(cb - 2, 0) : min(cb + 2, N - 1));
  }
  // whole pairs in the loop (no conditional step, so each stash waits for
  // exactly its own rows), an odd last chunk after it
  int it = 0;
  for (; it + 1 < N; it += 2) {
    step(fa, it);
    step(fb, it + 1);
  }
  if (it < N) step(fa, it);
  if (REV && P.ds0) {
#pragma unroll
    for (int cc = 0; cc < DT; ++cc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r + 4 * g4 + e, j = 16 * cc + l16;
        if (i < dk && j < dv) P.ds0[((int64_t)unit * dk + i) * dv + j] = Z[cc][e];
      }
  }
}

// Both scans in one launch (they are independent): work items [0, units)
// are the forward scans, [units, 2 units) the reverse ones.  Workgroup i
// runs on XCD i % 8; with a grid of whole XCD rounds each XCD takes a
// contiguous range of items, so the heads of a batch element, whose
// 144-byte rows share 128-byte lines, are read through one L2.
template <int DP, int M, bool ORD>
__global__ void __launch_bounds__(DP / 16 * kWave)
gla_bwd_scan(BwdParams P) {
  const int units = P.B * P.H;
  const int item = (gridDim.x & 7) == 0 ? xcd_linear_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  if (item < units) scan_unit<DP, M, false, ORD>(P, item);
  else scan_unit<DP, M, true, ORD>(P, item - units);
}

// ============================ chunk gradients ================================
template <int DP, int M>
struct BwdLds {
  static constexpr int QS = BwdRow<DP>::QS;
  static constexpr int SA = M + 8;                     // row stride of the M x M tiles
  static constexpr int TILE = M * QS * 2;              // token-major [M][QS] bf16
  static constexpr int STB = DP * QS * 2;              // transposed state [DP (j)][QS] bf16
  static constexpr int oQ = 0, oK = TILE;              // q, k; then q e^{b}, k e^{-b}
  static constexpr int oG = 2 * TILE;                  // gates, then k e^{B - b}
  static constexpr int oV = 3 * TILE, oO = 4 * TILE;   // v, do
  static constexpr int oS = 5 * TILE, oD = oS + STB;   // S_in^T, D^T
  static constexpr int oA = oD + STB;                  // [M][SA] bf16 A = dO V^T (causal)
  static constexpr int oP = oA + M * SA * 2;           // [M][SA] bf16 P (causal)
  static constexpr int oB = oP + M * SA * 2;           // [M][DP] fp32: b (log2 units) of extreme chunks, then d log alpha
  static constexpr int oTok = oB + M * DP * 4;         // [2][M] canonical token, -1 past T (this chunk, the one before)
  static constexpr int oFlag = oTok + 2 * M * 4;       // any |b| beyond the factorised range
  static constexpr int oEB = oFlag + 16;               // [DP] fp32 e^{B} per key channel
  static constexpr int oSuf = oEB + DP * 4;            // [DP] fp32 rowsum(S_out (.) D) per key channel
  static constexpr int bytes = oSuf + DP * 4;
};

constexpr int kChunkWaves = 8;

// Persistent: each workgroup takes a run of consecutive chunks; the next chunk's
// rows and both state blocks are loaded into registers while the current one
// is computed.  Wave r < DT owns key-channel tile r from the gate cumsum to
// its dq, dk and dlog_alpha (b, raw and scaled q, k and the rowsum of
// S_out (.) D stay in its registers); the other waves compute A and P, and
// all share dv.
//   phase 1: cumsum, range check, raw q, k (channel waves) | A tiles
//   phase 2: scaled rows into LDS, rowsum(S_out (.) D) (channel waves)
//   phase 3: dq, dk, dlog_alpha (channel waves, token tiles last to first) | P tiles
//   phase 4: dq, dk staged in LDS; dv
//   phase 5: the staged outputs into registers
// The outputs leave as 16-byte rows at the end of the next chunk's phase 2,
// after that chunk's first prefetch and its own arithmetic of phases 1 and
// 2; both are long complete when the rows after it are needed.
template <int DP, int M, bool ORD>
__global__ void __launch_bounds__(kChunkWaves * kWave)
gla_bwd_chunk(BwdParams P) {
  using L = BwdLds<DP, M>;
  constexpr int NT = kChunkWaves * kWave, MT = M / 16, JP = (MT + 1) / 2, DT = DP / 16;
  constexpr int K32 = DP / 32;
  constexpr bool KH = (DP % 32) != 0;
  constexpr int QS = L::QS, SA = L::SA, CG = DP / 8;
  constexpr int ITT = (M * CG + NT - 1) / NT, ITS = (DP * CG + NT - 1) / NT;
  constexpr int NTRI = MT * (MT + 1) / 2;   // token tile pairs (I, J), J <= I
  static_assert(DT <= kChunkWaves, "one wave per key-channel tile");
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *tQ = reinterpret_cast<uint16_t *>(smem + L::oQ), *tK = reinterpret_cast<uint16_t *>(smem + L::oK);
  uint16_t *tG = reinterpret_cast<uint16_t *>(smem + L::oG);
  uint16_t *tV = reinterpret_cast<uint16_t *>(smem + L::oV), *tO = reinterpret_cast<uint16_t *>(smem + L::oO);
  uint16_t *tS = reinterpret_cast<uint16_t *>(smem + L::oS), *tD = reinterpret_cast<uint16_t *>(smem + L::oD);
  uint16_t *tA = reinterpret_cast<uint16_t *>(smem + L::oA), *tP = reinterpret_cast<uint16_t *>(smem + L::oP);
  float *bL = reinterpret_cast<float *>(smem + L::oB);
  int *tok = reinterpret_cast<int *>(smem + L::oTok);
  unsigned *flag = reinterpret_cast<unsigned *>(smem + L::oFlag);
  float *tEB = reinterpret_cast<float *>(smem + L::oEB), *tSuf = reinterpret_cast<float *>(smem + L::oSuf);
  // With waves to spare beyond the channel waves (DT < 8), the rowsum of
  // S_out (.) D -- a constant of each key channel over the chunk, added to
  // every d log alpha of it -- is formed by those spare waves in phase 3 and
  // added to d log alpha in phase 5, off the channel waves' path.
  constexpr int NH = kChunkWaves - DT;   // spare (non-channel) waves
  constexpr bool kSpareSuf = NH > 0;

  const int tid0 = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int N = P.nchunks, total = P.B * P.H * N;
  const int T = P.T, dk = P.dk, dv = P.dv, H = P.H;
  const bool chan = wave < DT;
  const int r = wave;                                          // key-channel tile of a channel wave
  const int wslot = (wave + kChunkWaves - DT) % kChunkWaves;   // A, P, dv: the other waves first

  // tiles above the diagonal of A and P stay zero
  for (int x = tid0; x < 2 * M * SA / 8; x += NT) reinterpret_cast<uint4 *>(tA)[x] = make_uint4(0, 0, 0, 0);

  // prefetch registers, filled in three groups spread over the chunk before
  // (the rows' canonical tokens are kept from the first group for the second)
  uint4 fq[ITT], fk[ITT], fg[ITT], fv[ITT], fo[ITT], fs[ITS], fd[ITS];
  int pn[ITT];
  // ORD: table entries of the rows the next fetch_qkg loads (ordq) and of
  // the tokens of the chunk just fetched (ordt, threads < M), one fetch ahead
  const __amdgpu_buffer_rsrc_t rord = make_rsrc(ORD ? P.order : nullptr, ORD ? (unsigned)T * 4u : 0u);
  int ordq[ITT], ordt = -1;
  auto ord_rows = [&](int w) {
    if constexpr (ORD) {
      const int c = w - (w / N) * N;
#pragma unroll
      for (int kq = 0; kq < ITT; ++kq) {
        const int idx = tid0 + kq * NT, tl = idx / CG;
        ordq[kq] = ord_entry(rord, idx < M * CG && c * M + tl < T, c * M + tl);
      }
    }
  };
  auto fetch_qkg = [&](int w, int w_next) {
    const int unit = w / N, c = w - unit * N, bb = unit / H, hh = unit - bb * H;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(P.q + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(P.k + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(P.g + bb * P.qk_sb + hh * P.qk_sh, P.qk_span);
    if constexpr (ORD) ordt = ord_entry(rord, tid0 < M && c * M + tid0 < T, c * M + tid0);
#pragma unroll
    for (int kq = 0; kq < ITT; ++kq) {
      const int idx = tid0 + kq * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      const int p = c * M + tl;
      int n;
      if constexpr (ORD) {
        n = (idx < M * CG && p < T && ordq[kq] >= 0 && ordq[kq] < T) ? ordq[kq] : -1;
      } else {
        n = (idx < M * CG && p < T) ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : -1;
      }
      pn[kq] = n;
      const unsigned oqk = (n >= 0 && 8 * cg < dk) ? (unsigned)(((int64_t)n * P.qk_st + 8 * cg) * 2) : kOOB;
      fq[kq] = bload16(rq, oqk);
      fk[kq] = bload16(rk, oqk);
      fg[kq] = bload16(rg, oqk);
    }
    ord_rows(w_next);
  };
  auto fetch_vo = [&](int w) {
    const int unit = w / N, c = w - unit * N, bb = unit / H, hh = unit - bb * H;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(P.v + bb * P.v_sb + hh * P.v_sh, P.v_span);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(P.dout + bb * P.do_sb + hh * P.do_sh, P.do_span);
#pragma unroll
    for (int kq = 0; kq < ITT; ++kq) {
      const int idx = tid0 + kq * NT;
      const int tl = idx / CG, cg = idx - tl * CG;
      const int n = pn[kq];
      const bool ok = n >= 0 && 8 * cg < dv;
      fv[kq] = bload16(rv, ok ? (unsigned)(((int64_t)n * P.v_st + 8 * cg) * 2) : kOOB);
      fo[kq] = bload16(ro, ok ? (unsigned)((((int64_t)c * M + tl) * P.do_st + 8 * cg) * 2) : kOOB);
    }
  };
  auto fetch_states = [&](int w) {
    const int64_t blk = (int64_t)w * DP * DP;   // chunk w of unit w / N
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(P.st_s + blk, DP * DP * 2);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(P.st_d + blk, DP * DP * 2);
#pragma unroll
    for (int kq = 0; kq < ITS; ++kq) {
      const int idx = tid0 + kq * NT;
      const unsigned off = idx < DP * CG ? (unsigned)idx * 16u : kOOB;
      fs[kq] = bload16(rs, off);
      fd[kq] = bload16(rd, off);
    }
  };

  // one chunk's outputs, read back from the LDS staging (phase 5) and stored
  // to memory at the end of the next chunk's phase 2
  constexpr int ITO = (M * CG + NT - 1) / NT, ITG = (M * (DP / 4) + NT - 1) / NT;
  uint4 oq[ITO], ok[ITO], ov[ITO], og[ITG];
  auto store_outputs = [&](int wp, const int *tk, bool valid) {
    const int unit = wp / N, bb = unit / H, hh = unit - bb * H;
    const int64_t row0 = (int64_t)bb * T * H + hh;   // token 0 of this (batch, head), in rows of H
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(P.gq + row0 * dk, (unsigned)(((int64_t)(T - 1) * H * dk + dk) * 2));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(P.gk + row0 * dk, (unsigned)(((int64_t)(T - 1) * H * dk + dk) * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(P.gv + row0 * dv, (unsigned)(((int64_t)(T - 1) * H * dv + dv) * 2));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(P.dg + row0 * dk, (unsigned)(((int64_t)(T - 1) * H * dk + dk) * 4));
#pragma unroll
    for (int kq = 0; kq < ITO; ++kq) {
      const int idx = tid0 + kq * NT;
      const int t = idx / CG, cg = idx - t * CG;
      const int n = (valid && idx < M * CG) ? tk[t] : -1;
      const unsigned oqk = (n >= 0 && 8 * cg < dk) ? (unsigned)(((int64_t)n * H * dk + 8 * cg) * 2) : kOOB;
      const unsigned ovv = (n >= 0 && 8 * cg < dv) ? (unsigned)(((int64_t)n * H * dv + 8 * cg) * 2) : kOOB;
      bstore16(rq, oqk, oq[kq]);
      bstore16(rk, oqk, ok[kq]);
      bstore16(rv, ovv, ov[kq]);
    }
#pragma unroll
    for (int kq = 0; kq < ITG; ++kq) {
      const int idx = tid0 + kq * NT;
      const int t = idx / (DP / 4), cg = idx - t * (DP / 4);
      const int n = (valid && idx < M * (DP / 4)) ? tk[t] : -1;
      const unsigned og4 = (n >= 0 && 4 * cg < dk) ? (unsigned)(((int64_t)n * H * dk + 4 * cg) * 4) : kOOB;
      bstore16(rg, og4, og[kq]);
    }
  };

  // a contiguous run of chunks per workgroup: consecutive chunks of one
  // (batch, head) share memory pages.  With a grid of whole XCD rounds
  // (workgroup i runs on XCD i % 8) each XCD takes a contiguous range of
  // runs, so the workgroups of the heads of one batch element, which walk
  // the same token range side by side and whose 144-byte rows share
  // 128-byte lines, meet in one L2.
  const int lb = (gridDim.x & 7) == 0 ? xcd_linear_block(blockIdx.x, gridDim.x) : (int)blockIdx.x;
  const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
  const int wend = min(total, (lb + 1) * per);
  int w = lb * per, wprev = -1, par = 0;
  if (w < wend) {
    ord_rows(w);
    fetch_qkg(w, min(w + 1, wend - 1));
    fetch_vo(w);
    fetch_states(w);
  }
  for (; w < wend; wprev = w, ++w, par ^= 1) {
    const int c = w - (w / N) * N;
    // The lane index is hidden from the optimiser here, so the per-lane LDS
    // addresses are formed inside each chunk's code rather than hoisted out
    // of the loop (hundreds of them, which would not fit in registers).
    int lane = tid0 & 63;
    asm volatile("" : "+v"(lane));
    const int tid = wave * kWave + lane, l16 = lane & 15, g4 = lane >> 4;
    const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);
    // ---- 0. this chunk's rows (q, k, gates, v canonical; do in scan order)
    //         and state blocks into LDS; the next chunk's loads go out
#pragma unroll
    for (int kq = 0; kq < ITT; ++kq) {
      const int idx = tid + kq * NT;
      if (idx < M * CG) {
        const int tl = idx / CG, cg = idx - tl * CG;
        const int at = tl * QS + 8 * cg;
        *reinterpret_cast<uint4 *>(tQ + at) = fq[kq];
        *reinterpret_cast<uint4 *>(tK + at) = fk[kq];
        *reinterpret_cast<uint4 *>(tG + at) = fg[kq];
        *reinterpret_cast<uint4 *>(tV + at) = fv[kq];
        *reinterpret_cast<uint4 *>(tO + at) = fo[kq];
      }
    }
#pragma unroll
    for (int kq = 0; kq < ITS; ++kq) {
      const int idx = tid + kq * NT;
      if (idx < DP * CG) {
        // tile-major blocks: 16-byte group idx is row jj, columns ii .. ii+7
        // of tile (cc, r) = (tile / DT, tile % DT)
        const int tile = idx >> 5, cc = tile / DT, rr = tile - cc * DT;
        const int at = (16 * cc + ((idx & 31) >> 1)) * QS + 16 * rr + 8 * (idx & 1);
        *reinterpret_cast<uint4 *>(tS + at) = fs[kq];
        *reinterpret_cast<uint4 *>(tD + at) = fd[kq];
      }
    }
    int *tk = tok + par * M;   // this chunk's canonical tokens; the other half: the chunk before
    if (tid < M) {
      const int p = c * M + tid;
      if constexpr (ORD) tk[tid] = (p < T && ordt >= 0 && ordt < T) ? ordt : -1;
      else tk[tid] = p < T ? scan_to_canon(P.dir, P.gh, P.gw, T, p) : -1;
    }
    if (tid == 0) *flag = 0u;
    lds_barrier();
    // every memory operation below is issued on every chunk (the last chunk
    // refetches itself; the first stores nothing), so the compiler's waits
    // before the next chunk's rows are exact
    const int wn = min(w + 1, wend - 1);
    fetch_qkg(wn, min(wn + 1, wend - 1));

    // ---- 1. cumulative gates (log2 units) and raw q, k of tile r, in
    //         accumulator layout (token 16 I + 4 (l/16) + e, channel 16 r + l%16)
    float bl[MT][4];
    float Bt = 0.f;
    uint2 qa[MT], ka[MT];
    if (chan) {
      float mx = 0.f;
#pragma unroll
      for (int I = 0; I < MT; ++I) {
        const f32x4_t cum = tile_cumsum<MT, QS>(tG, I, r, l16, g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bl[I][e] = cum[e] * kLog2e;
          mx = fmaxf(mx, fabsf(bl[I][e]));
        }
        qa[I] = lds_tr(tQ + (16 * I + 4 * g4 + rowoff) * QS + 16 * r + coloff);
        ka[I] = lds_tr(tK + (16 * I + 4 * g4 + rowoff) * QS + 16 * r + coloff);
      }
      Bt = __shfl(bl[MT - 1][3], 48 + l16, kWave);   // token M-1: lane group 3, e = 3
      if (!(mx <= kBwdFastRange)) atomicOr(flag, 1u);   // NaN / inf too
    }
    //         A = dO V^T on tiles J <= I, the diagonal masked to s <= t
    for (int a = wslot; a < NTRI; a += kChunkWaves) {
      int I = 0;
      while ((I + 1) * (I + 2) / 2 <= a) ++I;
      const int J = a - I * (I + 1) / 2;
      const uint16_t *orow = tO + (16 * I + l16) * QS, *vrow = tV + (16 * J + l16) * QS;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) acc = mfma32(lds4(orow + 32 * kb + 8 * g4), lds4(vrow + 32 * kb + 8 * g4), acc);
      if (KH) acc = mfma16(lds2(orow + 32 * K32 + 4 * g4), lds2(vrow + 32 * K32 + 4 * g4), acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = J < I || l16 <= 4 * g4 + e;
        tA[(16 * I + 4 * g4 + e) * SA + 16 * J + l16] = to_bf(keep ? acc[e] : 0.f);
      }
    }
    lds_barrier();

    // ---- 2. scaled rows of tile r into LDS (k e^{B - b} always; q e^{b},
    //         k e^{-b} where factorised, else b itself), and rowsum(S_out (.) D)
    //         with S_out = diag(e^{B}) S_in + K^^T V
    fetch_vo(wn);
    const bool fast = __builtin_amdgcn_readfirstlane(*flag) == 0u;   // uniform: a scalar branch
    uint2 qt[MT], kt[MT];
    float sufS = 0.f;   // rowsum(S_out (.) D) of channel 16 r + l%16
    float eB = 1.f;     // e^{B} of channel 16 r + l%16
    if (chan) {
      uint2 kh[MT];
      const int i = 16 * r + l16;
      eB = fexp2(Bt);
#pragma unroll
      for (int I = 0; I < MT; ++I) {
        const float4 q4 = unpack4(qa[I]), k4 = unpack4(ka[I]);
        f32x4_t a1, a2, a3;
        if (fast) {
          // |b| <= 64: e^{B - b} = e^{B} e^{-b} in fp32 (two exponentials
          // per element instead of three)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float b = bl[I][e];
            a1[e] = elt(q4, e) * fexp2(b);
            a2[e] = elt(k4, e) * fexp2(-b);
            a3[e] = a2[e] * eB;
          }
        } else {
          // only k^ is used (with exact exponent differences)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a1[e] = a2[e] = 0.f;
            a3[e] = elt(k4, e) * fexp2(Bt - bl[I][e]);
          }
        }
        qt[I] = pack4(a1);
        kt[I] = pack4(a2);
        kh[I] = pack4(a3);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int at = (16 * I + 4 * g4 + e) * QS + i;
          const int sh = (e & 1) * 16;
          tG[at] = (uint16_t)((e < 2 ? kh[I].x : kh[I].y) >> sh);
          if (fast) {
            tQ[at] = (uint16_t)((e < 2 ? qt[I].x : qt[I].y) >> sh);
            tK[at] = (uint16_t)((e < 2 ? kt[I].x : kt[I].y) >> sh);
          } else {
            bL[(16 * I + 4 * g4 + e) * DP + i] = bl[I][e];
          }
        }
      }
      if constexpr (kSpareSuf) {
        if (g4 == 0) tEB[i] = eB;
      } else {
        float gm[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) gm[e] = fexp2(__shfl(Bt, 4 * g4 + e, kWave));
#pragma unroll
        for (int cc = 0; cc < DT; ++cc) {
          f32x4_t so = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jp = 0; jp < JP; ++jp)
            so = mfma32(kslots<MT>(kh, jp), tr_pair<MT>(tV, QS, jp, 16 * cc, g4, rowoff, coloff), so);
          // rows 16 r + 4 (l/16) + e, column 16 cc + l%16 of S_in and D
          const float4 s4 = unpack4(lds2(tS + (16 * cc + l16) * QS + 16 * r + 4 * g4));
          const float4 d4 = unpack4(lds2(tD + (16 * cc + l16) * QS + 16 * r + 4 * g4));
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(fmaf(gm[e], elt(s4, e), so[e]), elt(d4, e), acc[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) acc[e] += __shfl_xor(acc[e], off, kWave);
        // row 16 r + m sits in lane group m / 4, element m % 4
        const int src = 16 * (l16 >> 2);
        const float v0 = __shfl(acc[0], src, kWave), v1 = __shfl(acc[1], src, kWave);
        const float v2 = __shfl(acc[2], src, kWave), v3 = __shfl(acc[3], src, kWave);
        const int m4 = l16 & 3;
        sufS = m4 == 0 ? v0 : m4 == 1 ? v1 : m4 == 2 ? v2 : v3;
      }
    }
    // the chunk before's outputs leave here, after this chunk's arithmetic of
    // phases 1 and 2 rather than before it: a wave whose stores wait for
    // room in the memory pipeline then waits at the barrier, not in front of
    // its own work (C2 526 -> 497 us against issuing them at the top of
    // phase 1)
    store_outputs(wprev >= 0 ? wprev : w, tok + (par ^ 1) * M, wprev >= 0);
    lds_barrier();

    fetch_states(wn);
    // ---- 3. (chunks beyond the factorised range) P with exact exponent differences
    if (!fast) {
      for (int x = tid; x < M * M; x += NT) {
        const int t = x / M, s = x - t * M;
        float acc = 0.f;
        if (s <= t)
          for (int i = 0; i < dk; ++i)
            acc += bf_at(tQ + t * QS + i) * bf_at(tK + s * QS + i) * fexp2(bL[t * DP + i] - bL[s * DP + i]);
        tP[t * SA + s] = to_bf(acc);
      }
      lds_barrier();   // every b read for P before d log alpha replaces it
    }
    //         dq, dk, dlog_alpha of tile r, token tiles last to first (the
    //         reverse sum over the chunk runs in registers)
    if (chan) {
      const int i = 16 * r + l16;
      // S_in^T and D^T columns i as B operands (K = value channels, lds_tr order)
      uint4 sB[K32 > 0 ? K32 : 1], dB[K32 > 0 ? K32 : 1];
      uint2 sBh = make_uint2(0, 0), dBh = make_uint2(0, 0);
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) {
        sB[kb] = tr_pair<2>(tS + 32 * kb * QS, QS, 0, 16 * r, g4, rowoff, coloff);
        dB[kb] = tr_pair<2>(tD + 32 * kb * QS, QS, 0, 16 * r, g4, rowoff, coloff);
      }
      if (KH) {
        sBh = lds_tr(tS + (32 * K32 + 4 * g4 + rowoff) * QS + 16 * r + coloff);
        dBh = lds_tr(tD + (32 * K32 + 4 * g4 + rowoff) * QS + 16 * r + coloff);
      }
      float run = sufS;
      f32x4_t dgx[MT];   // extreme chunks: d log alpha held until the exact sums are done
#pragma unroll
      for (int I = MT - 1; I >= 0; --I) {
        const uint16_t *orow = tO + (16 * I + l16) * QS, *vrow = tV + (16 * I + l16) * QS;
        f32x4_t x1 = {0.f, 0.f, 0.f, 0.f}, x2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < K32; ++kb) {
          x1 = mfma32(cat(lds2(orow + 32 * kb + 4 * g4), lds2(orow + 32 * kb + 16 + 4 * g4)), sB[kb], x1);
          x2 = mfma32(cat(lds2(vrow + 32 * kb + 4 * g4), lds2(vrow + 32 * kb + 16 + 4 * g4)), dB[kb], x2);
        }
        if (KH) {
          x1 = mfma16(lds2(orow + 32 * K32 + 4 * g4), sBh, x1);
          x2 = mfma16(lds2(vrow + 32 * K32 + 4 * g4), dBh, x2);
        }
        f32x4_t y1 = {0.f, 0.f, 0.f, 0.f}, y2 = {0.f, 0.f, 0.f, 0.f};
        if (fast) {
          const uint16_t *arow = tA + (16 * I + l16) * SA;
#pragma unroll
          for (int jp = 0; jp < JP; ++jp) {
            const bool hi_ok = 2 * jp + 1 < MT;
            if (32 * jp <= 16 * I + 15) {   // keys s <= t: A K~
              const uint4 af = cat(lds2(arow + 32 * jp + 4 * g4), hi_ok ? lds2(arow + 32 * jp + 16 + 4 * g4) : make_uint2(0, 0));
              y1 = mfma32(af, kslots<MT>(kt, jp), y1);
            }
            if (32 * jp + 31 >= 16 * I)     // queries u >= t: A^T Q~
              y2 = mfma32(tr_pair<MT>(tA, SA, jp, 16 * I, g4, rowoff, coloff), kslots<MT>(qt, jp), y2);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * I + 4 * g4 + e;
            const float bt = bl[I][e];
            float a1 = 0.f, a2 = 0.f;
            for (int s = 0; s <= t; ++s)
              a1 += bf_at(tA + t * SA + s) * bf_at(tK + s * QS + i) * fexp2(bt - bL[s * DP + i]);
            for (int u = t; u < M; ++u)
              a2 += bf_at(tA + u * SA + t) * bf_at(tQ + u * QS + i) * fexp2(bL[u * DP + i] - bt);
            y1[e] = a1;
            y2[e] = a2;
          }
        }
        const float4 q4 = unpack4(qa[I]), k4 = unpack4(ka[I]);
        float R[4];
        f32x4_t dq4, dk4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float b = bl[I][e];
          if (fast) {
            dq4[e] = fexp2(b) * (x1[e] + y1[e]);
            dk4[e] = fexp2(-b) * fmaf(eB, x2[e], y2[e]);   // e^{-b} y2 + e^{B - b} x2
          } else {
            dq4[e] = fexp2(b) * x1[e] + y1[e];
            dk4[e] = y2[e] + fexp2(Bt - b) * x2[e];
          }
          R[e] = elt(q4, e) * dq4[e] - elt(k4, e) * dk4[e];
        }
        qa[I] = pack4(dq4);   // the raw q, k of tile I are no longer needed
        ka[I] = pack4(dk4);
        // reverse sum: inside the lane's 4 tokens, then over the later lane groups
        const float s3 = R[3], s2 = R[2] + s3, s1 = R[1] + s2, s0 = R[0] + s1;
        const float L0 = __shfl(s0, l16, kWave), L1 = __shfl(s0, 16 + l16, kWave);
        const float L2 = __shfl(s0, 32 + l16, kWave), L3 = __shfl(s0, 48 + l16, kWave);
        const float after = run + (g4 < 1 ? L1 : 0.f) + (g4 < 2 ? L2 : 0.f) + (g4 < 3 ? L3 : 0.f);
        const float sv[4] = {s0, s1, s2, s3};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (fast) bL[(16 * I + 4 * g4 + e) * DP + i] = after + sv[e];
          else dgx[I][e] = after + sv[e];
        }
        run += ((L0 + L1) + L2) + L3;
      }
      if (!fast) {
#pragma unroll
        for (int I = 0; I < MT; ++I)
#pragma unroll
          for (int e = 0; e < 4; ++e) bL[(16 * I + 4 * g4 + e) * DP + i] = dgx[I][e];
      }
    }
    //         rowsum(S_out (.) D) of key-channel tile rr, on the spare waves:
    //         the same products and sums as the channel wave's own form
    //         (k^ from LDS as the A operand, tokens along K)
    if constexpr (kSpareSuf) {
      if (!chan) {
        for (int rr = wslot; rr < DT; rr += NH) {
          const int i0 = 16 * rr;
          float gm[4], acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) gm[e] = tEB[i0 + 4 * g4 + e];
#pragma unroll
          for (int cc = 0; cc < DT; ++cc) {
            f32x4_t so = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jp = 0; jp < JP; ++jp)
              so = mfma32(tr_pair<MT>(tG, QS, jp, i0, g4, rowoff, coloff),
                          tr_pair<MT>(tV, QS, jp, 16 * cc, g4, rowoff, coloff), so);
            const float4 s4 = unpack4(lds2(tS + (16 * cc + l16) * QS + i0 + 4 * g4));
            const float4 d4 = unpack4(lds2(tD + (16 * cc + l16) * QS + i0 + 4 * g4));
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(fmaf(gm[e], elt(s4, e), so[e]), elt(d4, e), acc[e]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) acc[e] += __shfl_xor(acc[e], off, kWave);
          if (l16 == 0)
            *reinterpret_cast<float4 *>(tSuf + i0 + 4 * g4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    //         P = Q~ K~^T on tiles J <= I (factorised chunks)
    if (fast) {
      for (int a = wslot; a < NTRI; a += kChunkWaves) {
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= a) ++I;
        const int J = a - I * (I + 1) / 2;
        const uint16_t *qrow = tQ + (16 * I + l16) * QS, *krow = tK + (16 * J + l16) * QS;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < K32; ++kb) acc = mfma32(lds4(qrow + 32 * kb + 8 * g4), lds4(krow + 32 * kb + 8 * g4), acc);
        if (KH) acc = mfma16(lds2(qrow + 32 * K32 + 4 * g4), lds2(krow + 32 * K32 + 4 * g4), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool keep = J < I || l16 <= 4 * g4 + e;
          tP[(16 * I + 4 * g4 + e) * SA + 16 * J + l16] = to_bf(keep ? acc[e] : 0.f);
        }
      }
    }
    lds_barrier();

    // ---- 4. dq, dk into the q, k tiles (free once P is formed), and
    //         dv = P^T dO + K^ D into the v tile (unit (I, cc): tokens of tile I,
    //         value channels of tile cc; K = tokens by transposing reads, then
    //         key channels along rows of D^T)
    if (chan) {
      const int i = 16 * r + l16;
#pragma unroll
      for (int I = 0; I < MT; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int at = (16 * I + 4 * g4 + e) * QS + i;
          const int sh = (e & 1) * 16;
          tQ[at] = (uint16_t)((e < 2 ? qa[I].x : qa[I].y) >> sh);
          tK[at] = (uint16_t)((e < 2 ? ka[I].x : ka[I].y) >> sh);
        }
    }
    for (int u = wslot; u < MT * DT; u += kChunkWaves) {
      const int I = u / DT, cc = u - I * DT;
      f32x4_t y3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp < JP; ++jp)
        if (32 * jp + 31 >= 16 * I)   // queries t >= s
          y3 = mfma32(tr_pair<MT>(tP, SA, jp, 16 * I, g4, rowoff, coloff),
                      tr_pair<MT>(tO, QS, jp, 16 * cc, g4, rowoff, coloff), y3);
      const uint16_t *hrow = tG + (16 * I + l16) * QS, *drow = tD + (16 * cc + l16) * QS;
#pragma unroll
      for (int kb = 0; kb < K32; ++kb) y3 = mfma32(lds4(hrow + 32 * kb + 8 * g4), lds4(drow + 32 * kb + 8 * g4), y3);
      if (KH) y3 = mfma16(lds2(hrow + 32 * K32 + 4 * g4), lds2(drow + 32 * K32 + 4 * g4), y3);
      const int j = 16 * cc + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) tV[(16 * I + 4 * g4 + e) * QS + j] = to_bf(y3[e]);
    }
    lds_barrier();

    // ---- 5. the staged outputs into registers; they are stored at the end
    //         of the next chunk's phase 2
#pragma unroll
    for (int kq = 0; kq < ITO; ++kq) {
      const int idx = tid + kq * NT;
      const int t = idx / CG, cg = idx - t * CG;
      const int at = (idx < M * CG ? t : 0) * QS + 8 * cg;
      oq[kq] = *reinterpret_cast<const uint4 *>(tQ + at);
      ok[kq] = *reinterpret_cast<const uint4 *>(tK + at);
      ov[kq] = *reinterpret_cast<const uint4 *>(tV + at);
    }
#pragma unroll
    for (int kq = 0; kq < ITG; ++kq) {
      const int idx = tid + kq * NT;
      const int t = idx / (DP / 4), cg = idx - t * (DP / 4);
      float4 gv4 = *reinterpret_cast<const float4 *>(bL + (idx < M * (DP / 4) ? t : 0) * DP + 4 * cg);
      if constexpr (kSpareSuf) {
        const float4 sf = *reinterpret_cast<const float4 *>(tSuf + 4 * cg);
        gv4.x += sf.x; gv4.y += sf.y; gv4.z += sf.z; gv4.w += sf.w;
      }
      og[kq] = __builtin_bit_cast(uint4, gv4);
    }
    lds_barrier();
  }
  if (wprev >= 0) store_outputs(wprev, tok + (par ^ 1) * M, true);
}

// ------------------------------ host side -----------------------------------
int bwd_pad(int d) { return d <= 32 ? 32 : d <= 64 ? 64 : d <= 80 ? 80 : d <= 96 ? 96 : 128; }

template <int DP, int M>
hipError_t launch_bwd(const BwdParams &p, int num_cu, hipStream_t s) {
  constexpr int scan_lds = ScanLds<DP, M>::bytes;
  constexpr int chunk_lds = BwdLds<DP, M>::bytes;
  // resident chunk workgroups per CU: the same on every gfx950, so computed
  // once (concurrent first calls store the same value)
  static std::atomic<int> per_cu_cache{0};
  int per_cu = per_cu_cache.load(std::memory_order_relaxed);
  hipError_t e;
  const bool ord = p.order != nullptr;
  auto *scan = ord ? gla_bwd_scan<DP, M, true> : gla_bwd_scan<DP, M, false>;
  auto *chunk = ord ? gla_bwd_chunk<DP, M, true> : gla_bwd_chunk<DP, M, false>;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(scan), hipFuncAttributeMaxDynamicSharedMemorySize, scan_lds);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(chunk), hipFuncAttributeMaxDynamicSharedMemorySize, chunk_lds);
  if (e != hipSuccess) return e;
  if (per_cu == 0) {   // the same for both variants (same LDS, same block)
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(gla_bwd_chunk<DP, M, false>),
                                                     kChunkWaves * kWave, chunk_lds);
    if (e != hipSuccess) return e;
    per_cu = nb > 0 ? nb : 1;
    per_cu_cache.store(per_cu, std::memory_order_relaxed);
  }
  const int units = p.B * p.H;
  hipLaunchKernelGGL(scan, dim3(2 * units), dim3(DP / 16 * kWave), scan_lds, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t chunks = (int64_t)units * p.nchunks;
  const int64_t resident = (int64_t)(num_cu > 0 ? num_cu : 1) * per_cu;
  const int grid = (int)(chunks < resident ? chunks : resident);
  hipLaunchKernelGGL(chunk, dim3(grid), dim3(kChunkWaves * kWave), chunk_lds, s, p);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_bwd_m(const BwdParams &p, int M, int num_cu, hipStream_t s) {
  switch (M) {
    case 16: return launch_bwd<DP, 16>(p, num_cu, s);
    case 32: return launch_bwd<DP, 32>(p, num_cu, s);
    case 64:
      if constexpr (DP <= 80) return launch_bwd<DP, 64>(p, num_cu, s);
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
  return 2 * (size_t)B * H * N * DP * DP * 2;
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
  p.order = a.order;
  p.nchunks = (a.T + M - 1) / M;
  const size_t blkb = (size_t)a.B * a.H * p.nchunks * DP * DP * 2;
  unsigned char *ws = static_cast<unsigned char *>(a.workspace);
  p.st_s = reinterpret_cast<uint16_t *>(ws);
  p.st_d = reinterpret_cast<uint16_t *>(ws + blkb);
  auto span = [](int64_t st, int d, int T_) {
    return (unsigned)(((int64_t)(T_ - 1) * st + d) * 2);
  };
  p.qk_span = span(a.qk_st, a.dk, a.T);
  p.v_span = span(a.v_st, a.dv, a.T);
  p.do_span = span(a.do_st, a.dv, a.T);
  switch (DP) {
    case 32: return launch_bwd_m<32>(p, M, a.num_cu, s);
    case 64: return launch_bwd_m<64>(p, M, a.num_cu, s);
    case 80: return launch_bwd_m<80>(p, M, a.num_cu, s);
    case 96: return launch_bwd_m<96>(p, M, a.num_cu, s);
    default: return launch_bwd_m<128>(p, M, a.num_cu, s);
  }
}
