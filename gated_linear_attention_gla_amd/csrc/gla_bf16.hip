// gla_bf16.hip -- chunk-wise Gated Linear Attention forward on gfx950 MFMA.
//
// Method (DiG paper notes, 关键设计 / 硬件友好的效率设计: chunk-wise parallel
// GLA computed on chip; diffusers issue #20 for the recurrence itself):
// the scan-ordered sequence of one (batch, head) is cut into chunks of M
// tokens.  Inside a chunk, with b_t the inclusive cumulative log-gate from the
// chunk start (per key channel) and S the state entering the chunk,
//   o_t = sum_{s<=t in chunk} [ sum_i q_ti k_si e^{b_ti - b_si} ] v_s        (intra)
//       + (q_t * e^{b_t}) S                                                  (inter)
//   S'  = diag(e^{b_last}) S + sum_s (k_s * e^{b_last - b_s})^T v_s          (state)
// which regroups the token recurrence S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,
// o_t = q_t S_t.  The intra weights use the factorised operands q~ = q e^{b},
// k~ = k e^{-b} (one bf16 MFMA product per tile).  When a chunk's gates are
// large enough for that factorisation to overflow, the chunk computes the
// intra weights pairwise on the VALU instead (exact exponent differences), so
// any finite log-gate <= 0 stays accurate.  Every other factor is bounded by 1
// for non-positive gates.
//
// Sequence segments.  To give the GPU enough independent work, each
// (batch, head) scan is split into G segments of whole chunks, one workgroup
// each.  A non-final segment first streams its k, v and gates once to form its
// state aggregate A_g (its own contribution, from a zero state) and the
// product of its gates Gam_g, and publishes them.  It then obtains the state
// entering it by a decoupled look-back: walk back to the nearest segment j
// that has published its inclusive state P_j (or to the start, s0), then fold
// forward S = fma(Gam_m, S, A_m) for m = j+1 .. g-1.  The fold always replays
// the serial recurrence P_m = Gam_m * P_{m-1} + A_m element by element, so the
// result is bitwise independent of which segments had finished: the output is
// deterministic.  The segment publishes P_g and then runs the full chunk loop
// from that state, writing o.  The second read of k, v and the gates mostly
// hits the L2 / Infinity Cache.
//
// gfx950 mapping
//   * NW = DP/16 waves; wave w owns value columns [16w, 16w+16): the fp32
//     state of those columns stays in the wave's MFMA accumulators;
//   * the scan permutation is applied in the loads (scan position p reads
//     canonical token scan_to_canon(p)); no permuted copy is ever written;
//   * all LDS tiles are token-major rows written with 16-byte stores; the
//     products that contract over tokens (V^T P^T and k^T v) fetch their
//     operands with ds_read_b64_tr_b16, whose transpose puts tokens along K;
//   * v_mfma_f32_16x16x32_bf16 with fp32 accumulation is the only MFMA shape:
//     channels are zero-padded to a multiple of 32, an odd 16-token tile count
//     pads its last token block with zeros;
//   * barriers fence LDS only, so the next chunk's global loads stay in flight
//     across the whole chunk;
//   * workgroups take tickets in launch order and are laid out XCD-major, so
//     the segments of one scan run on one XCD and share its L2.
//
// MFMA 16x16xK operand layout used: lane l supplies row (A) / column (B)
// l % 16 and K slice l / 16; the accumulator holds rows 4*(l/16) + e, column
// l % 16.  The K order inside one MFMA is free as long as A and B agree, which
// lets accumulators feed the next product directly (P^T -> B of V^T P^T,
// S -> A of S^T q~^T) without a trip through LDS.
#include "dig_internal.h"

namespace dig {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

constexpr float kLog2e = 1.4426950408889634f;
// Largest |cumulative log2 gate| inside a chunk for the factorised path; a
// chunk beyond it takes the pairwise path.  2^64 keeps q~, k~ and their
// products far inside the fp32/bf16 range.
constexpr float kFastRange = 64.0f;

__device__ __forceinline__ f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint2 pack4(f32x4_t x) {
  return make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ uint4 cat(uint2 lo, uint2 hi) { return make_uint4(lo.x, lo.y, hi.x, hi.y); }
__device__ __forceinline__ uint2 lds2(const uint16_t *p) { return *reinterpret_cast<const uint2 *>(p); }
// Global memory accesses through address-space-1 pointers, so they compile to
// global_load/global_store (vmcnt only) rather than FLAT instructions, which
// would also count in lgkmcnt and be waited on by every LDS barrier.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(const uint16_t *p) {
  const u32x4_t v = *(__attribute__((address_space(1))) const u32x4_t *)(size_t)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void gstore8(uint16_t *p, uint2 v) {
  *(__attribute__((address_space(1))) u32x2_t *)(size_t)p = u32x2_t{v.x, v.y};
}
// Raw buffer loads: 48-bit base (one (batch, head) slice, wave-uniform) plus
// a 32-bit byte offset per lane.  Offsets at or beyond num_records return
// zeros, which serves both the ragged tail and the channel padding without
// predication.  Word 3 = untyped 32-bit data format (CDNA).
constexpr unsigned kOOB = 0x80000000u;   // an offset past every valid span
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 lds4(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane j
// receives element (j % 4) of the 8-byte read addressed by lane 4e + j/4,
// e = 0..3.  If lane s of the group addresses row t0 + s/4, column
// c0 + 4*(s%4) of a token-major tile, lane j receives column c0 + j of rows
// t0 .. t0+3.
__device__ __forceinline__ uint2 lds_tr(const uint16_t *p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16_t *)(__attribute__((address_space(3))) char *)(size_t)(p));
  return __builtin_bit_cast(uint2, r);
}

// 2^x on the transcendental unit (v_exp_f32); results below 2^-126 flush to 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-coherent (agent-scope, sc1) accesses for the state hand-off between
// workgroups: written through to the coherence point and read from it, so no
// L2 writeback/invalidate fence is needed.
__device__ __forceinline__ void st_coherent(float *p, float4 v) {
  __hip_atomic_store(p + 0, v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 1, v.y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 2, v.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(p + 3, v.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ld_coherent(const float *p) {
  float4 v;
  v.x = __hip_atomic_load(p + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.y = __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.z = __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.w = __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
// Wait until all of this wave's vector-memory operations (loads and stores)
// have completed.
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS-only workgroup barrier: waits for this wave's LDS traffic, not for its
// global loads, so prefetches stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct Params {
  const uint16_t *q, *k, *v, *g;
  uint16_t *o;
  const float *s0;
  float *s_final;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  int B, T, H, dk, dv, gh, gw, dir, nchunks, units;
  int seg_chunks, nseg, per_xcd;   // chunks per segment, segments per scan, scans per XCD
  int cgr;                         // 16-byte channel groups holding data: ceil(max(dk, dv) / 8)
  unsigned cg_magic;               // ceil(2^31 / cgr): idx / cgr == umulhi(2 idx, cg_magic) for idx < 2^20
  unsigned qk_span, v_span;        // bytes addressable in one (batch, head) slice of q/k/g and of v
  int blk_floats;                  // floats of one published state block
  int *ticket;                     // launch-order ticket counter (reset by the last taker)
  unsigned *flags;                 // [units][nseg]: epoch*4 + {1 aggregate, 2 inclusive}
  float *gam;                      // [units][nseg][DP] product of the segment's gates
  float *agg;                      // [units][nseg][blk_floats] aggregate state
  float *inc;                      // [units][nseg][blk_floats] inclusive state
  unsigned epoch;
};

template <int DP>
struct Shape {
  static constexpr int NW = DP / 16 > 2 ? DP / 16 : 2;   // waves per workgroup
  static constexpr int NT = NW * kWave;
};

template <int DP, int M>
struct Lds {
  static constexpr int QS = DP + 16;    // token-major bf16 row stride (elements): conflict-free transpose reads
  static constexpr int HS = DP / 2 + 4; // fp32 row stride of one plane of the cumulative gates
  static constexpr int MT = M / 16;
  static constexpr int JP = (MT + 1) / 2;
  static constexpr int NPT = MT * (MT + 1) / 2;        // causal 16x16 tiles of P^T
  static constexpr int TILE = M * QS * 2;
  static constexpr int oQ = 0;                         // q~ (raw q on the pairwise path)
  static constexpr int oK = oQ + TILE;                 // k~ (raw k on the pairwise path)
  static constexpr int oKh = oK + TILE;                // raw gates, then k^ = k e^{b_last - b}
  static constexpr int oV = oKh + TILE;                // v
  static constexpr int oB = oV + TILE;                 // cumulative gates, 2 planes [2][M][HS] fp32 (log2)
  static constexpr int oPT = oB;                       // P^T tiles (MFMA fragment order, 512 B each),
                                                       // in the gate buffer once it is dead
  static constexpr int oBl = oB + 2 * M * HS * 4;      // chunk total b_last [DP] fp32 (log2)
  static constexpr int oGam = oBl + DP * 4;            // e^{b_last} [DP]
  static constexpr int oL = oGam + DP * 4;             // lower-triangular ones, MFMA fragments [MT][JP][64] x 16 B
  static constexpr int oTok = oL + MT * JP * 1024;     // byte offsets of the next chunk's tokens [2][M]
  static constexpr int oMisc = oTok + 2 * M * 4;       // flag, ticket, look-back result
  static constexpr int bytes = oMisc + 64;
  static_assert(NPT * 512 <= 2 * M * HS * 4, "P^T tiles fit in the gate buffer");
};

// Occupancy target (waves per SIMD): chunks of <= 32 tokens fit three waves
// per SIMD; 64-token chunks need the larger register budget of two.
template <int M>
struct Occ {
  static constexpr int waves_per_simd = M <= 32 ? 3 : 2;
};

template <int DP, int M>
__global__ void __launch_bounds__(Shape<DP>::NT) __attribute__((amdgpu_waves_per_eu(Occ<M>::waves_per_simd)))
gla_fwd_bf16_kernel(Params P) {
  constexpr int NT = Shape<DP>::NT;
  constexpr int NW = Shape<DP>::NW;
  constexpr int MT = M / 16;                 // token tiles per chunk
  constexpr int DT = DP / 16;                // channel tiles
  constexpr int K32 = DP / 32;               // 32-wide channel blocks
  constexpr int JP = (MT + 1) / 2;           // 32-token K blocks
  constexpr int R = (M * (DP / 8) + NT - 1) / NT;   // max 16-byte items per thread per tensor
  constexpr int QS = Lds<DP, M>::QS, HS = Lds<DP, M>::HS, NPT = Lds<DP, M>::NPT;
  static_assert(DP % 32 == 0 && NW == DT, "one wave per 16-channel tile");
  const int CG = P.cgr;                      // 16-byte channel groups carrying data (the rest stay 0)
  const int ITEMS = M * CG;

  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *sQ = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oQ);
  uint16_t *sK = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oK);
  uint16_t *sKh = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oKh);
  uint16_t *sG = sKh;   // raw gates live in the k^ tile until the scan has read them
  uint16_t *sV = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oV);
  float *sB = reinterpret_cast<float *>(smem + Lds<DP, M>::oB);
  float *sBl = reinterpret_cast<float *>(smem + Lds<DP, M>::oBl);
  float *sGam = reinterpret_cast<float *>(smem + Lds<DP, M>::oGam);
  uint16_t *sPT = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oPT);
  uint4 *sL = reinterpret_cast<uint4 *>(smem + Lds<DP, M>::oL);
  unsigned *sTok = reinterpret_cast<unsigned *>(smem + Lds<DP, M>::oTok);   // [0..M) q/k/g, [M..2M) v
  int *sMisc = reinterpret_cast<int *>(smem + Lds<DP, M>::oMisc);   // [0] pairwise [1] ticket [2] look-back

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);   // transpose-read addressing

  // ---- work assignment: tickets in launch order, XCD-major layout; segment
  // g of a scan always holds a larger ticket than segment g-1 of it.
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(P.ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == (int)gridDim.x - 1) __hip_atomic_store(P.ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sMisc[1] = t;
  }
  __syncthreads();
  const int lid = sMisc[1];
  const int xcd = lid & 7, kslot = lid >> 3;
  const int unit = xcd * P.per_xcd + kslot / P.nseg;
  const int seg = kslot % P.nseg;
  if (unit >= P.units) return;
  const int c_begin = seg * P.seg_chunks;
  if (c_begin >= P.nchunks) return;
  const int c_end = min(c_begin + P.seg_chunks, P.nchunks);
  const bool last_seg = (c_end == P.nchunks);

  const int b = unit / P.H, h = unit - b * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv;
  const __amdgpu_buffer_rsrc_t rq_ = make_rsrc(P.q + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(P.k + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rg_ = make_rsrc(P.g + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(P.v + b * P.v_sb + h * P.v_sh, P.v_span);
  uint16_t *ob = P.o + b * P.o_sb + h * P.o_sh;

  const int n0 = 16 * wave;                 // this wave's value columns / gate channels
  const bool has_cols = (n0 < dv);
  const int DTr = (dk + 15) / 16, NWv = (dv + 15) / 16;   // tiles present in a state block
  const int64_t slot0 = (int64_t)unit * P.nseg;

  // ---- one-time set-up: zero channel padding, lower-triangular fragments
  if (CG < DP / 8) {
    const int PADG = DP / 8 - CG;
    for (int x = tid; x < M * PADG; x += NT) {
      const int tl = x / PADG, cg = CG + (x - tl * PADG);
      const uint4 z = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(sQ + tl * QS + 8 * cg) = z;
      *reinterpret_cast<uint4 *>(sK + tl * QS + 8 * cg) = z;
      *reinterpret_cast<uint4 *>(sKh + tl * QS + 8 * cg) = z;
      *reinterpret_cast<uint4 *>(sV + tl * QS + 8 * cg) = z;
    }
  }
  // L^T fragment (B operand) of the scan: column t = 16i + l16, K slots =
  // tokens 32jp + 4g4 + {0..3} and 32jp + 16 + 4g4 + {0..3}; 1.0 where s <= t.
  for (int f = wave; f < MT * JP; f += NW) {
    const int i = f / JP, jp = f - i * JP;
    const int t = 16 * i + l16, s0_ = 32 * jp + 4 * g4;
    uint4 w;
    w.x = (s0_ + 0 <= t ? 0x3F80u : 0u) | (s0_ + 1 <= t ? 0x3F800000u : 0u);
    w.y = (s0_ + 2 <= t ? 0x3F80u : 0u) | (s0_ + 3 <= t ? 0x3F800000u : 0u);
    w.z = (s0_ + 16 <= t ? 0x3F80u : 0u) | (s0_ + 17 <= t ? 0x3F800000u : 0u);
    w.w = (s0_ + 18 <= t ? 0x3F80u : 0u) | (s0_ + 19 <= t ? 0x3F800000u : 0u);
    sL[f * 64 + lane] = w;
  }

  // ---- token offsets of chunk c (scan order -> canonical token), kOOB past the
  // end of the sequence and for the chunk after the segment (its loads then
  // return zeros without touching memory)
  auto fill_tok = [&](int c) {
    if (tid < M) {
      const int p = c * M + tid;
      unsigned oqk = kOOB, ov = kOOB;
      if (c < c_end && p < T) {
        const unsigned n = (unsigned)scan_to_canon(P.dir, P.gh, P.gw, T, p);
        oqk = n * (unsigned)P.qk_st * 2u;
        ov = n * (unsigned)P.v_st * 2u;
      }
      sTok[tid] = oqk;
      sTok[M + tid] = ov;
    }
  };

  // ---- loads: item idx -> (token tl, 16-byte channel group cg), from the token table
  uint4 rq[R], rk[R], rg[R], rv[R];
  auto load_chunk = [&](bool with_q) {
    // Unconditional: a load under a branch would make the loop-carried
    // registers merge with their old values, which forces the prefetch to be
    // waited for right away.
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NT;
      const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
      const bool ok = idx < ITEMS;
      const unsigned tq = sTok[ok ? tl : 0], tv = sTok[M + (ok ? tl : 0)];
      const unsigned ok_qk = ok && (8 * cg < dk) ? tq + 16u * cg : kOOB;
      const unsigned ok_v = ok && (8 * cg < dv) ? tv + 16u * cg : kOOB;
      if (with_q) rq[r] = bload16(rq_, ok_qk);
      rk[r] = bload16(rk_, ok_qk);
      rg[r] = bload16(rg_, ok_qk);
      rv[r] = bload16(rv_, ok_v);
    }
  };

  // Stage 1: raw gates and v to LDS; token table of the next chunk.
  auto stage1 = [&](int c_next) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NT;
      if (idx < ITEMS) {
        const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
        *reinterpret_cast<uint4 *>(sG + tl * QS + 8 * cg) = rg[r];
        *reinterpret_cast<uint4 *>(sV + tl * QS + 8 * cg) = rv[r];
      }
    }
    fill_tok(c_next);
    if (tid == 0) sMisc[0] = 0;
  };

  // Stage 2: inclusive cumulative gates as an MFMA product, b^T = G^T L^T
  // (bf16 gates and 1.0 are exact; fp32 sums), scaled to log2 units.  Wave w
  // owns gate channels [16w, 16w+16); lane (l16, g4) receives token 16i + l16,
  // channels 16w + 4g4 .. +3, stored as one float4 in plane (g4 & 1) of sB.
  // Also writes b_last and e^{b_last}, and flags the chunk for the pairwise
  // path when any |b| exceeds the factorisable range.
  auto stage2 = [&]() {
    uint4 gf[JP];
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const uint2 lo = lds_tr(sG + (32 * jp + 4 * g4 + rowoff) * QS + n0 + coloff);
      const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(sG + (32 * jp + 16 + 4 * g4 + rowoff) * QS + n0 + coloff)
                                         : make_uint2(0, 0);
      gf[jp] = cat(lo, hi);
    }
    float mag = 0.f;
    const int ch0 = n0 + 4 * g4;
    float *plane = sB + (g4 & 1) * (M * HS) + (ch0 >> 3) * 4;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp < JP; ++jp)
        if (32 * jp <= 16 * i + 15) acc = mfma32(gf[jp], sL[(i * JP + jp) * 64 + lane], acc);
      const float4 bv = make_float4(acc[0] * kLog2e, acc[1] * kLog2e, acc[2] * kLog2e, acc[3] * kLog2e);
      *reinterpret_cast<float4 *>(plane + (16 * i + l16) * HS) = bv;
      mag = fmaxf(mag, fmaxf(fmaxf(fabsf(bv.x), fabsf(bv.y)), fmaxf(fabsf(bv.z), fabsf(bv.w))));
      if (i == MT - 1 && l16 == 15) {
        *reinterpret_cast<float4 *>(sBl + ch0) = bv;
        *reinterpret_cast<float4 *>(sGam + ch0) = make_float4(fexp2(bv.x), fexp2(bv.y), fexp2(bv.z), fexp2(bv.w));
      }
    }
    if (!(mag <= kFastRange)) sMisc[0] = 1;   // also catches NaN
  };

  // cumulative gates of token tl, channels 8cg .. 8cg+7
  auto item_b = [&](int tl, int cg, float *bt) {
    const float4 a = *reinterpret_cast<const float4 *>(sB + tl * HS + 4 * cg);
    const float4 c2 = *reinterpret_cast<const float4 *>(sB + M * HS + tl * HS + 4 * cg);
    bt[0] = a.x; bt[1] = a.y; bt[2] = a.z; bt[3] = a.w;
    bt[4] = c2.x; bt[5] = c2.y; bt[6] = c2.z; bt[7] = c2.w;
  };
  auto b_at = [&](int t, int ch) { return sB[((ch >> 2) & 1) * (M * HS) + t * HS + (ch >> 3) * 4 + (ch & 3)]; };
  // 8 consecutive fp32 values from LDS.
  auto lds8f = [&](const float *p, float *out) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b2 = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b2.x; out[5] = b2.y; out[6] = b2.z; out[7] = b2.w;
  };

  // k^ = k e^{b_last - b} for item r (exact exponent difference)
  auto khat_direct = [&](int r, const float *bt, const float *bl) {
    const uint32_t kw[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
    uint4 oh;
    oh.x = pack_bf16x2(bf16lo(kw[0]) * fexp2(bl[0] - bt[0]), bf16hi(kw[0]) * fexp2(bl[1] - bt[1]));
    oh.y = pack_bf16x2(bf16lo(kw[1]) * fexp2(bl[2] - bt[2]), bf16hi(kw[1]) * fexp2(bl[3] - bt[3]));
    oh.z = pack_bf16x2(bf16lo(kw[2]) * fexp2(bl[4] - bt[4]), bf16hi(kw[2]) * fexp2(bl[5] - bt[5]));
    oh.w = pack_bf16x2(bf16lo(kw[3]) * fexp2(bl[6] - bt[6]), bf16hi(kw[3]) * fexp2(bl[7] - bt[7]));
    return oh;
  };

  // v fragments with tokens along K: K block jp holds tokens 32jp + 4*g4 + e
  // (slots 0..3) and 32jp + 16 + 4*g4 + e (slots 4..7); this wave's columns.
  auto v_frags = [&](uint4 *vf) {
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const uint2 lo = lds_tr(sV + (32 * jp + 4 * g4 + rowoff) * QS + n0 + coloff);
      const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(sV + (32 * jp + 16 + 4 * g4 + rowoff) * QS + n0 + coloff)
                                         : make_uint2(0, 0);
      vf[jp] = cat(lo, hi);
    }
  };

  // S = diag(e^{b_last}) S + k^^T v for this wave's columns; optionally
  // accumulates the product of the gates in gprod (same row layout as S).
  auto state_update = [&](f32x4_t *S, const uint4 *vf, f32x4_t *gprod) {
#pragma unroll
    for (int r = 0; r < DT; ++r) {
      const float4 gm = *reinterpret_cast<const float4 *>(sGam + 16 * r + 4 * g4);
      S[r][0] *= gm.x; S[r][1] *= gm.y; S[r][2] *= gm.z; S[r][3] *= gm.w;
      if (gprod) { gprod[r][0] *= gm.x; gprod[r][1] *= gm.y; gprod[r][2] *= gm.z; gprod[r][3] *= gm.w; }
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const uint2 lo = lds_tr(sKh + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
        const uint2 hi = (2 * jp + 1 < MT)
                             ? lds_tr(sKh + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff)
                             : make_uint2(0, 0);
        S[r] = mfma32(cat(lo, hi), vf[jp], S[r]);
      }
    }
  };

  // Initial state s0 for this wave's tiles (0 when absent).
  auto load_s0 = [&](f32x4_t *S) {
#pragma unroll
    for (int r = 0; r < DT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * r + 4 * g4 + e, n = n0 + l16;
        S[r][e] = (P.s0 && ch < dk && n < dv) ? P.s0[((int64_t)unit * dk + ch) * dv + n] : 0.f;
      }
  };
  auto blk_at = [&](int r) { return ((r * NWv + wave) * 64 + lane) * 4; };

  f32x4_t S[DT];
#pragma unroll
  for (int r = 0; r < DT; ++r) S[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t gp[DT];   // product of this segment's gates (rows of S)
#pragma unroll
  for (int r = 0; r < DT; ++r) gp[r] = f32x4_t{1.f, 1.f, 1.f, 1.f};

  // ======================= pass 1: segment aggregate =========================
  if (!last_seg) {
    fill_tok(c_begin);
    __syncthreads();
    load_chunk(false);
    for (int c = c_begin; c < c_end; ++c) {
      stage1(c + 1);
      lds_barrier();
      stage2();
      lds_barrier();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = tid + r * NT;
        if (idx < ITEMS) {
          const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
          float bt[8], bl[8];
          item_b(tl, cg, bt);
          lds8f(sBl + 8 * cg, bl);
          *reinterpret_cast<uint4 *>(sKh + tl * QS + 8 * cg) = khat_direct(r, bt, bl);
        }
      }
      load_chunk(false);
      lds_barrier();
      if (has_cols) {
        uint4 vf[JP];
        v_frags(vf);
        state_update(S, vf, gp);
      }
      lds_barrier();
    }
    if (has_cols) {
      float *blk = P.agg + (slot0 + seg) * P.blk_floats;
#pragma unroll
      for (int r = 0; r < DT; ++r)
        if (r < DTr) st_coherent(blk + blk_at(r), make_float4(S[r][0], S[r][1], S[r][2], S[r][3]));
      if (wave == 0 && l16 == 0) {
#pragma unroll
        for (int r = 0; r < DT; ++r)
          st_coherent(P.gam + (slot0 + seg) * DP + 16 * r + 4 * g4, make_float4(gp[r][0], gp[r][1], gp[r][2], gp[r][3]));
      }
    }
    drain_vmem();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(P.flags + slot0 + seg, P.epoch * 4u + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ================== look-back: state entering the segment ==================
  f32x4_t Sin[DT];
  if (seg == 0) {
    load_s0(Sin);
  } else {
    if (tid == 0) {
      int j = seg - 1;
      while (j >= 0) {
        unsigned f;
        while (((f = __hip_atomic_load(P.flags + slot0 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 2) !=
               P.epoch)
          __builtin_amdgcn_s_sleep(2);
        if ((f & 3u) == 2u) break;
        --j;
      }
      sMisc[2] = j;
    }
    __syncthreads();
    const int jstar = sMisc[2];
    if (jstar >= 0) {
      const float *blk = P.inc + (slot0 + jstar) * P.blk_floats;
#pragma unroll
      for (int r = 0; r < DT; ++r) {
        const float4 x = (has_cols && r < DTr) ? ld_coherent(blk + blk_at(r)) : make_float4(0.f, 0.f, 0.f, 0.f);
        Sin[r] = f32x4_t{x.x, x.y, x.z, x.w};
      }
    } else {
      load_s0(Sin);
    }
    if (has_cols) {
      for (int m = jstar + 1; m < seg; ++m) {
        const float *blk = P.agg + (slot0 + m) * P.blk_floats;
        const float *gm_ = P.gam + (slot0 + m) * DP;
#pragma unroll
        for (int r = 0; r < DT; ++r) {
          if (r < DTr) {
            const float4 a = ld_coherent(blk + blk_at(r));
            const float4 gm = ld_coherent(gm_ + 16 * r + 4 * g4);
            Sin[r][0] = fmaf(gm.x, Sin[r][0], a.x);
            Sin[r][1] = fmaf(gm.y, Sin[r][1], a.y);
            Sin[r][2] = fmaf(gm.z, Sin[r][2], a.z);
            Sin[r][3] = fmaf(gm.w, Sin[r][3], a.w);
          }
        }
      }
    }
  }
  if (!last_seg) {
    // inclusive state P_g = Gam_g * S_in + A_g
    if (has_cols) {
      float *blk = P.inc + (slot0 + seg) * P.blk_floats;
#pragma unroll
      for (int r = 0; r < DT; ++r)
        if (r < DTr)
          st_coherent(blk + blk_at(r),
                      make_float4(fmaf(gp[r][0], Sin[r][0], S[r][0]), fmaf(gp[r][1], Sin[r][1], S[r][1]),
                                  fmaf(gp[r][2], Sin[r][2], S[r][2]), fmaf(gp[r][3], Sin[r][3], S[r][3])));
    }
    drain_vmem();
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(P.flags + slot0 + seg, P.epoch * 4u + 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int r = 0; r < DT; ++r) S[r] = Sin[r];

  // ========================= pass 2: outputs ==================================
  // Drain this wave's outstanding global loads (the state loads above) so the
  // loop below never waits on anything but its own prefetches.
  drain_vmem();
  fill_tok(c_begin);
  __syncthreads();
  load_chunk(true);
  for (int c = c_begin; c < c_end; ++c) {
    stage1(c + 1);
    lds_barrier();
    stage2();
    lds_barrier();
    const bool pairwise = (sMisc[0] != 0);
    if (!pairwise) {
      // q~ = q e^{b}, k~ = k e^{-b}, k^ = k~ e^{b_last}   (|b| <= 64: no overflow)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = tid + r * NT;
        if (idx < ITEMS) {
          const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
          float bt[8], gm[8];
          item_b(tl, cg, bt);
          lds8f(sGam + 8 * cg, gm);
          const uint32_t qw[4] = {rq[r].x, rq[r].y, rq[r].z, rq[r].w};
          const uint32_t kw[4] = {rk[r].x, rk[r].y, rk[r].z, rk[r].w};
          uint32_t oq[4], ok[4], oh[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            oq[e] = pack_bf16x2(bf16lo(qw[e]) * fexp2(bt[2 * e]), bf16hi(qw[e]) * fexp2(bt[2 * e + 1]));
            const float k0 = bf16lo(kw[e]) * fexp2(-bt[2 * e]), k1 = bf16hi(kw[e]) * fexp2(-bt[2 * e + 1]);
            ok[e] = pack_bf16x2(k0, k1);
            oh[e] = pack_bf16x2(k0 * gm[2 * e], k1 * gm[2 * e + 1]);
          }
          *reinterpret_cast<uint4 *>(sQ + tl * QS + 8 * cg) = make_uint4(oq[0], oq[1], oq[2], oq[3]);
          *reinterpret_cast<uint4 *>(sK + tl * QS + 8 * cg) = make_uint4(ok[0], ok[1], ok[2], ok[3]);
          *reinterpret_cast<uint4 *>(sKh + tl * QS + 8 * cg) = make_uint4(oh[0], oh[1], oh[2], oh[3]);
        }
      }
      load_chunk(true);
      lds_barrier();
      // P^T tiles (j, i), j <= i, each computed once, spread over the waves
#pragma unroll
      for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j <= i; ++j) {
          const int ti = i * (i + 1) / 2 + j;
          if (ti % NW == wave) {
            const uint16_t *krow = sK + (16 * j + l16) * QS;
            const uint16_t *qrow = sQ + (16 * i + l16) * QS;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb2 = 0; kb2 < K32; ++kb2)
              acc = mfma32(lds4(krow + 32 * kb2 + 8 * g4), lds4(qrow + 32 * kb2 + 8 * g4), acc);
            if (j == i) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (4 * g4 + e > l16) acc[e] = 0.f;   // causal: s > t
            }
            *reinterpret_cast<uint2 *>(sPT + ti * 256 + lane * 4) = pack4(acc);
          }
        }
      }
    } else {
      // exact pairwise intra weights: raw q, k to LDS, k^ directly
      uint4 qsave[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = tid + r * NT;
        if (idx < ITEMS) {
          const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
          float bt[8], bl[8];
          item_b(tl, cg, bt);
          lds8f(sBl + 8 * cg, bl);
          const uint32_t qw[4] = {rq[r].x, rq[r].y, rq[r].z, rq[r].w};
          qsave[r].x = pack_bf16x2(bf16lo(qw[0]) * fexp2(bt[0]), bf16hi(qw[0]) * fexp2(bt[1]));
          qsave[r].y = pack_bf16x2(bf16lo(qw[1]) * fexp2(bt[2]), bf16hi(qw[1]) * fexp2(bt[3]));
          qsave[r].z = pack_bf16x2(bf16lo(qw[2]) * fexp2(bt[4]), bf16hi(qw[2]) * fexp2(bt[5]));
          qsave[r].w = pack_bf16x2(bf16lo(qw[3]) * fexp2(bt[6]), bf16hi(qw[3]) * fexp2(bt[7]));
          *reinterpret_cast<uint4 *>(sQ + tl * QS + 8 * cg) = rq[r];
          *reinterpret_cast<uint4 *>(sK + tl * QS + 8 * cg) = rk[r];
          *reinterpret_cast<uint4 *>(sKh + tl * QS + 8 * cg) = khat_direct(r, bt, bl);
        }
      }
      lds_barrier();
      // P^T fragment slots: tile ti = (j, i), lane l, element e  <->  t = 16i + l%16,
      // s = 16j + 4(l/16) + e;  value sum_c q_tc k_sc 2^(b_tc - b_sc) for s <= t, else 0
      constexpr int NSLOT = NPT * 256;
      constexpr int NS = (NSLOT + NT - 1) / NT;
      float pw[NS];
#pragma unroll
      for (int x = 0; x < NS; ++x) {
        const int sl = tid + x * NT;
        float acc = 0.f;
        if (sl < NSLOT) {
          const int ti = sl >> 8, ln = (sl >> 2) & 63, e = sl & 3;
          int i = 0;
          while ((i + 1) * (i + 2) / 2 <= ti) ++i;
          const int j = ti - i * (i + 1) / 2;
          const int t = 16 * i + (ln & 15), s_ = 16 * j + 4 * (ln >> 4) + e;
          if (s_ <= t) {
            for (int ch = 0; ch < dk; ++ch) {
              const float qv = __uint_as_float((uint32_t)sQ[t * QS + ch] << 16);
              const float kv = __uint_as_float((uint32_t)sK[s_ * QS + ch] << 16);
              acc += qv * kv * fexp2(b_at(t, ch) - b_at(s_, ch));
            }
          }
        }
        pw[x] = acc;
      }
      load_chunk(true);
      lds_barrier();
#pragma unroll
      for (int x = 0; x < NS; ++x) {
        const int sl = tid + x * NT;
        if (sl < NSLOT) sPT[sl] = (uint16_t)f2bf(pw[x]);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = tid + r * NT;
        if (idx < ITEMS) {
          const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
          *reinterpret_cast<uint4 *>(sQ + tl * QS + 8 * cg) = qsave[r];
        }
      }
    }
    lds_barrier();

    if (has_cols) {
      uint4 vf[JP];
      v_frags(vf);
      uint4 sa[K32];   // S^T (bf16) as the A operand, K = channels
#pragma unroll
      for (int kb2 = 0; kb2 < K32; ++kb2) sa[kb2] = cat(pack4(S[2 * kb2]), pack4(S[2 * kb2 + 1]));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const uint16_t *qrow = sQ + (16 * i + l16) * QS;
        f32x4_t O = {0.f, 0.f, 0.f, 0.f};
        // O^T += S^T q~^T
#pragma unroll
        for (int kb2 = 0; kb2 < K32; ++kb2)
          O = mfma32(sa[kb2], cat(lds2(qrow + 32 * kb2 + 4 * g4), lds2(qrow + 32 * kb2 + 16 + 4 * g4)), O);
        // O^T += V^T P^T over the s-tiles j <= i
#pragma unroll
        for (int jp = 0; jp < JP; ++jp) {
          const int j0 = 2 * jp, j1 = 2 * jp + 1;
          if (j0 <= i) {
            const uint2 pt0 = lds2(sPT + (i * (i + 1) / 2 + j0) * 256 + lane * 4);
            const uint2 pt1 = (j1 <= i) ? lds2(sPT + (i * (i + 1) / 2 + j1) * 256 + lane * 4) : make_uint2(0, 0);
            O = mfma32(vf[jp], cat(pt0, pt1), O);
          }
        }
        const int p = c * M + 16 * i + l16;
        const int n = n0 + 4 * g4;
        if (p < T && n < dv) gstore8(ob + (int64_t)p * P.o_st + n, pack4(O));
      }
      state_update(S, vf, nullptr);
    }
    lds_barrier();
  }

  if (last_seg && P.s_final && has_cols) {
#pragma unroll
    for (int r = 0; r < DT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * r + 4 * g4 + e, n = n0 + l16;
        if (ch < dk && n < dv) P.s_final[((int64_t)unit * dk + ch) * dv + n] = S[r][e];
      }
  }
}

// ------------------------------ host side -----------------------------------

int pad32(int d) { return ((d + 31) / 32) * 32; }

int lds_bytes(int DP, int M) {
  switch (DP * 1000 + M) {
#define DIG_LDS_CASE(D, MM) \
  case D * 1000 + MM:       \
    return Lds<D, MM>::bytes;
    DIG_LDS_CASE(32, 16) DIG_LDS_CASE(32, 32) DIG_LDS_CASE(32, 64)
    DIG_LDS_CASE(64, 16) DIG_LDS_CASE(64, 32) DIG_LDS_CASE(64, 64)
    DIG_LDS_CASE(96, 16) DIG_LDS_CASE(96, 32) DIG_LDS_CASE(96, 64)
    DIG_LDS_CASE(128, 16) DIG_LDS_CASE(128, 32) DIG_LDS_CASE(128, 64)
#undef DIG_LDS_CASE
    default: return 160 * 1024;
  }
}

struct Plan {
  int DP, M, nchunks, units, nseg, seg_chunks, per_xcd, grid, blk_floats;
  size_t off_flags, off_gam, off_agg, off_inc, bytes;
};

// Segmentation: enough workgroups for about two rounds of the workgroups that
// fit on the chip at once (LDS-limited), but segments of at least 512 tokens
// so that the published states stay small next to the streamed inputs.
Plan make_plan(int B, int T, int H, int dk, int dv, int M, int num_cu) {
  Plan pl;
  pl.DP = pad32(dk > dv ? dk : dv);
  pl.M = M;
  pl.nchunks = (T + M - 1) / M;
  pl.units = B * H;
  // workgroups resident per CU: LDS (160 KiB) and the register budget
  // (waves per SIMD, 4 SIMDs) both bound it
  int per_cu = (160 * 1024) / lds_bytes(pl.DP, M);
  const int nw = pl.DP / 16 > 2 ? pl.DP / 16 : 2;
  const int reg_cap = 4 * (M <= 32 ? Occ<32>::waves_per_simd : Occ<64>::waves_per_simd) / nw;
  if (per_cu > reg_cap) per_cu = reg_cap;
  if (per_cu < 1) per_cu = 1;
  // one wave of resident workgroups: every segment but the last of a scan
  // reads its chunks twice, so more segments than that cost more than they hide
  const long want = (long)num_cu * per_cu;
  long nseg = (want + pl.units - 1) / pl.units;
  const int min_chunks = (512 + M - 1) / M;
  long max_seg = pl.nchunks / min_chunks;
  if (max_seg < 1) max_seg = 1;
  if (nseg > max_seg) nseg = max_seg;
  if (nseg < 1) nseg = 1;
  pl.seg_chunks = (int)((pl.nchunks + nseg - 1) / nseg);
  pl.nseg = (pl.nchunks + pl.seg_chunks - 1) / pl.seg_chunks;
  pl.per_xcd = (pl.units + 7) / 8;
  pl.grid = 8 * pl.per_xcd * pl.nseg;
  const int DTr = (dk + 15) / 16, NWv = (dv + 15) / 16;
  pl.blk_floats = DTr * NWv * 64 * 4;
  const size_t slots = (size_t)pl.units * pl.nseg;
  auto up = [](size_t x) { return ((x + 255) / 256) * 256; };
  size_t off = 256;   // the ticket counter lives at offset 0
  pl.off_flags = off;
  off += up(slots * 4);
  pl.off_gam = off;
  off += up(slots * pl.DP * 4);
  pl.off_agg = off;
  off += up(slots * pl.blk_floats * 4);
  pl.off_inc = off;
  off += up(slots * pl.blk_floats * 4);
  pl.bytes = off;
  return pl;
}

template <int DP, int M>
hipError_t launch(const Params &p, int grid, hipStream_t s) {
  const size_t lds = Lds<DP, M>::bytes;
  auto *fn = gla_fwd_bf16_kernel<DP, M>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(Shape<DP>::NT), lds, s, p);
  return hipGetLastError();
}

template <int DP>
hipError_t launch_m(const Params &p, int M, int grid, hipStream_t s) {
  switch (M) {
    case 16: return launch<DP, 16>(p, grid, s);
    case 32: return launch<DP, 32>(p, grid, s);
    case 64: return launch<DP, 64>(p, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace dig

size_t dig_gla_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk, int num_cu) {
  return dig::make_plan(B, T, H, dk, dv, chunk, num_cu).bytes;
}

hipError_t dig_launch_gla_bf16(const DigGlaArgs &a, hipStream_t s) {
  using namespace dig;
  const Plan pl = make_plan(a.B, a.T, a.H, a.dk, a.dv, a.chunk, a.num_cu);
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
  p.nchunks = pl.nchunks;
  p.units = pl.units;
  p.seg_chunks = pl.seg_chunks;
  p.nseg = pl.nseg;
  p.per_xcd = pl.per_xcd;
  p.blk_floats = pl.blk_floats;
  p.cgr = ((a.dk > a.dv ? a.dk : a.dv) + 7) / 8;
  p.cg_magic = (unsigned)((0x80000000ull + p.cgr - 1) / p.cgr);
  p.qk_span = (unsigned)(((int64_t)(a.T - 1) * a.qk_st + a.dk) * 2);
  p.v_span = (unsigned)(((int64_t)(a.T - 1) * a.v_st + a.dv) * 2);
  char *ws = static_cast<char *>(a.workspace);
  p.ticket = reinterpret_cast<int *>(ws);
  p.flags = reinterpret_cast<unsigned *>(ws + pl.off_flags);
  p.gam = reinterpret_cast<float *>(ws + pl.off_gam);
  p.agg = reinterpret_cast<float *>(ws + pl.off_agg);
  p.inc = reinterpret_cast<float *>(ws + pl.off_inc);
  p.epoch = a.epoch;
  switch (pl.DP) {
    case 32: return launch_m<32>(p, a.chunk, pl.grid, s);
    case 64: return launch_m<64>(p, a.chunk, pl.grid, s);
    case 96: return launch_m<96>(p, a.chunk, pl.grid, s);
    case 128: return launch_m<128>(p, a.chunk, pl.grid, s);
    default: return hipErrorInvalidValue;
  }
}
