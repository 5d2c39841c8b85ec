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
// for non-positive gates.  The choice is made per chunk from M * max|log-gate|,
// a bound on every |b| in the chunk.
//
// Sequence segments.  To give the GPU enough independent work, each
// (batch, head) scan is split into G segments of whole chunks, one workgroup
// each.  A non-final segment first streams its k, v and gates once to form its
// state aggregate A_g (its own contribution, from a zero state) and the
// product of its gates Gam_g, and publishes them.  It then waits for the
// aggregates of all earlier segments (they are computed concurrently, so
// they arrive together) and folds them forward from s0:
// S = fma(Gam_m, S, A_m) for m = 0 .. g-1, the serial recurrence
// P_m = Gam_m * P_{m-1} + A_m element by element in a fixed order, so the
// output does not depend on timing.  The loads of several aggregates are
// issued before they are folded, so the fold costs a few memory round trips
// rather than one per segment.  The segment then runs the full chunk loop
// from that state, writing o.  With two segments the scan is split in a
// pipelined way instead (see the kernel): segment 1 aggregates a stretch that
// segment 0 is still writing and starts from the state segment 0 publishes
// at its start.
//
// gfx950 mapping
//   * a workgroup has DT = DP/16 consumer waves and DT producer waves, each
//     role running its own copy of the schedule with the same barriers.  A
//     consumer owns 16 value columns: the fp32 state of those columns stays in
//     its MFMA accumulators; it writes o (staged in LDS, stored as whole
//     rows) and updates the state.  A producer owns 16 key channels: it
//     stages a chunk loaded two chunks earlier, scans its gates and forms q~,
//     k~ (k^ for pairwise chunks); all waves build the causal P^T tiles.  The
//     producers work one chunk ahead on the other half of double-buffered LDS
//     tiles, so the two roles overlap (two barriers per chunk);
//   * the scan permutation is applied in the loads (scan position p reads
//     canonical token scan_to_canon(p)); no permuted copy is ever written;
//   * all LDS tiles are token-major rows written with 16-byte stores; the
//     products that contract over tokens (V^T P^T, k^T v and the gate scan)
//     fetch their operands with ds_read_b64_tr_b16, whose transpose puts
//     tokens along K;
//   * v_mfma_f32_16x16x32_bf16 with fp32 accumulation is the only MFMA shape:
//     channels are zero-padded to 32, 64, 80, 96 or 128 (a 16-channel tail
//     block and an odd 16-token tile count run with a zero upper half);
//   * barriers fence LDS only, so the next chunk's global loads stay in flight
//     across the whole chunk;
//   * workgroups take tickets per XCD in start order; an XCD holds a
//     contiguous range of scans (the heads of a batch element, whose rows
//     share cache lines, and all segments of each), so they share its L2.
//
// MFMA 16x16xK operand layout used: lane l supplies row (A) / column (B)
// l % 16 and K slice l / 16; the accumulator holds rows 4*(l/16) + e, column
// l % 16.  The K order inside one MFMA is free as long as A and B agree, which
// lets accumulators feed the next product directly (P^T -> B of V^T P^T,
// S -> A of S^T q~^T) without a trip through LDS.
#include <type_traits>

#include "dig_mfma.h"

namespace dig {
namespace {

// Largest |cumulative log2 gate| inside a chunk for the factorised path; a
// chunk beyond it takes the pairwise path.  2^64 keeps q~, k~ and their
// products far inside the fp32/bf16 range.
constexpr float kFastRange = 64.0f;

// Waits between workgroups are bounded: a flag that has not arrived after
// kWaitTicks of the 100 MHz real-time clock (4 s, far beyond any legitimate
// wait: a whole segment of the longest sequence the 32-bit slice offsets
// allow streams in well under a second) sets kErrWait in the workspace's
// error word and the wait gives up, so the workgroup still finishes.
constexpr long long kWaitTicks = 400000000ll;
constexpr unsigned kErrWait = 1u;

__device__ __forceinline__ void wait_flag(const unsigned *flag, unsigned epoch, unsigned *err) {
  const long long t0 = wall_clock64();
  while ((__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 2) != epoch) {
    if (wall_clock64() - t0 > kWaitTicks) {
      __hip_atomic_fetch_or(err, kErrWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

struct Params {
  const uint16_t *q, *k, *v, *g;
  uint16_t *o;
  const float *s0;
  float *s_final;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  int B, T, H, dk, dv, gh, gw, dir, nchunks, units;
  const int *order;                // scan position -> canonical token table [T] (the kernel's ORD path)
  int seg_chunks, nseg, per_xcd;   // chunks per segment, segments per scan, scans per XCD
  int split_L, split_K;            // two-segment split (split_K > 0): see the kernel
  int cgr;                         // 16-byte channel groups holding data: ceil(max(dk, dv) / 8)
  unsigned cg_magic;               // ceil(2^31 / cgr): idx / cgr == umulhi(2 idx, cg_magic) for idx < 2^20
  unsigned gh_magic;               // ceil(2^31 / gh): scan-order decode by a scalar multiply (fill_tok)
  unsigned qk_span, v_span, o_span;   // bytes addressable in one (batch, head) slice of q/k/g, v, o
  int blk_floats;                  // floats of one published state block
  unsigned *ticket;                // [8] launch-order ticket counters, one per XCD (cyclic, see the kernel)
  unsigned *err;                   // error word: kErrWait when a wait gave up
  unsigned *flags;                 // [units][nseg]: epoch*4 + {1 aggregate, 2 split hand-off}
  float *gam;                      // [units][nseg][DP] product of the segment's gates (look-back only)
  float *agg;                      // [units][nseg][blk_floats] aggregate state (look-back only)
  float *inc;                      // [units][blk_floats]: the state a two-segment split hands
                                   // over at chunk L (split only)
  unsigned epoch;
};

// Workgroup: DT = DP/16 consumer waves, one per 16 value columns (they hold
// the fp32 state of those columns and write o), and DT producer waves, one per
// 16 key channels (they stage the next chunk: loads, gate scan, q~/k~/k^,
// P^T tiles).  Producers run one chunk ahead of the consumers on the other
// half of double-buffered LDS tiles, so the two halves of the work overlap.
template <int DP>
struct Shape {
  static constexpr int DT = DP / 16;
  static constexpr int NW = 2 * DT;        // waves per workgroup
  static constexpr int NT = NW * kWave;
  static constexpr int NTP = DT * kWave;   // producer threads
};

template <int DP, int M>
struct Lds {
  // Token-major bf16 row stride (elements).  Row-parallel reads (16 lanes on
  // 16 rows, 8 or 16 bytes each) are bank-conflict free when the stride is
  // 4 * odd dwords; the transposing reads (4 rows x 32 bytes) need the four
  // rows on disjoint 8-bank groups.  DP + 8 satisfies both for 64 and 96
  // channels, DP + 24 for 32, 80 and 128.
  // 128-token chunks (32 channels only) take DP + 8 so that the plan fits
  // in 160 KiB; their transposing reads then take 1.5x their conflict-free
  // time.
  static constexpr int QS = (DP == 64 || DP == 96 || M == 128) ? DP + 8 : DP + 24;
  static constexpr int MT = M / 16;
  static constexpr int NPT = MT * (MT + 1) / 2;        // causal 16x16 tiles of P^T
  static constexpr int TILE = M * QS * 2;
  // per buffer (chunk parity): q -> q~, k -> k~, gates -> k^, v
  static constexpr int BUF = 4 * TILE;
  static constexpr int oBuf = 0;                       // [2][4][M][QS] bf16
  static constexpr int oPT = 2 * BUF;                  // [2][NPT][256] bf16 P^T tiles (MFMA fragment order)
  static constexpr int oB32 = oPT + 2 * NPT * 512;     // [M][DP] fp32 cumulative gates (pairwise chunks only)
  static constexpr int oGam = oB32 + M * DP * 4;       // [2][DP] e^{b_last}
  static constexpr int oTok = oGam + 2 * DP * 4;       // [4][2][M] token byte offsets (chunk mod 4; q/k/g, v)
  static constexpr int oVote = oTok + 8 * M * 4;       // [2][16] per producer wave: chunk needs the pairwise path
  static constexpr int oStg = oVote + 2 * 16 * 4;      // [M][QS] bf16 o of the chunk being written
  static constexpr int oMisc = oStg + TILE;            // ticket, look-back result
  static constexpr int bytes = oMisc + 64;
};

// Register budget: the whole workgroup on one CU, 2*DT waves over 4 SIMDs.
template <int DP>
struct Occ {
  static constexpr int waves_per_simd = (2 * (DP / 16) + 3) / 4 < 2 ? 2 : (2 * (DP / 16) + 3) / 4;
};

// ORD: the scan order comes from the caller's table P.order instead of one of
// the four grid orders.
template <int DP, int M, bool ORD>
__global__ void __launch_bounds__(Shape<DP>::NT) __attribute__((amdgpu_waves_per_eu(Occ<DP>::waves_per_simd)))
gla_fwd_bf16_kernel(Params P) {
  constexpr int NT = Shape<DP>::NT, NTP = Shape<DP>::NTP;
  constexpr int DT = DP / 16;                // channel tiles = consumer waves = producer waves
  constexpr int MT = M / 16;                 // token tiles per chunk
  constexpr int K32 = DP / 32;               // 32-wide channel blocks
  constexpr bool KH = (DP % 32) != 0;        // and a 16-wide one after them (80 channels)
  constexpr int JP = (MT + 1) / 2;           // 32-token K blocks
  constexpr int R = (M * (DP / 8) + NTP - 1) / NTP;
  // load split points (see mid_loads): with 64-token chunks half after the
  // staging stores, half after the transform (measured best of the three-way
  // splits at C2); shorter chunks issue them all at once
  constexpr int JA = M >= 64 ? 2 * R : 4 * R, JB = 4 * R;   // max 16-byte items per producer thread per tensor
  constexpr int QS = Lds<DP, M>::QS, NPT = Lds<DP, M>::NPT, TILE = Lds<DP, M>::TILE;
  static_assert(DP % 16 == 0 && DT <= 16, "channel tiling");
  static_assert(Lds<DP, M>::bytes <= 160 * 1024, "LDS plan exceeds 160 KiB");
  const int CG = P.cgr;                      // 16-byte channel groups carrying data (the rest stay 0)
  const int ITEMS = M * CG;

  extern __shared__ __align__(16) unsigned char smem[];
  auto tile = [&](int par, int which) {      // which: 0 q, 1 k, 2 gates / k^, 3 v
    return reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oBuf + par * Lds<DP, M>::BUF + which * TILE);
  };
  auto ptile = [&](int par) { return reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oPT + par * NPT * 512); };
  float *sB32 = reinterpret_cast<float *>(smem + Lds<DP, M>::oB32);
  auto gam = [&](int par) { return reinterpret_cast<float *>(smem + Lds<DP, M>::oGam) + par * DP; };
  unsigned *sTok = reinterpret_cast<unsigned *>(smem + Lds<DP, M>::oTok);
  int *sVote = reinterpret_cast<int *>(smem + Lds<DP, M>::oVote);
  int *sMisc = reinterpret_cast<int *>(smem + Lds<DP, M>::oMisc);   // [1] ticket [2] look-back

  // the wave index is uniform: from a scalar register, role branches are scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g4 = lane >> 4;
  const int rowoff = l16 >> 2, coloff = 4 * (l16 & 3);   // transpose-read addressing
  const bool producer = wave >= DT;
  const int pw = wave - DT;                  // producer wave index (channel tile)
  const int ptid = tid - NTP;                // producer thread index

  // ---- work assignment.  Workgroups are dealt round-robin to the 8 XCDs
  // (workgroup i runs on XCD i % 8), and all segments of the scans of one
  // XCD's slot range stay on that XCD: the heads of a batch element, whose
  // 144-byte rows share 128-byte lines, then meet in one L2.  Within an XCD,
  // tickets taken in start order assign the work, so segment g of a scan
  // always holds a larger ticket than segment g-1 of it and only ever waits
  // for a workgroup that started before it.  The counter is cyclic (atomic
  // increment wrapping at gsize - 1): a launch takes exactly gsize tickets,
  // so it leaves the counter where it found it, and whatever the counter
  // holds, the gsize tickets of a launch are a permutation of [0, gsize) --
  // from r < gsize they run r .. gsize-1, 0 .. r-1; from a value >= gsize the
  // first taker gets that value (read as gsize - 1) and the rest 0 .. gsize-2.
  // Every piece of work is therefore taken exactly once even on a workspace
  // that was never zero-filled; only the start order can then be rotated,
  // which the bounded waits turn into an error rather than a hang.
  // With one segment per scan no workgroup ever waits for another, so the
  // launch index assigns the work and no ticket is taken.
  int lid = (int)blockIdx.x;
  if (P.nseg > 1) {
    if (tid == 0) {
      const unsigned g = blockIdx.x & 7, gsize = gridDim.x >> 3;
      unsigned t = __builtin_amdgcn_atomic_inc32(P.ticket + g, gsize - 1, __ATOMIC_RELAXED, "agent");
      if (t >= gsize) t = gsize - 1;
      sMisc[1] = (int)((t << 3) | g);
    }
    __syncthreads();
    lid = sMisc[1];
  }
  const int xcd = lid & 7, kslot = lid >> 3;
  const int unit = xcd * P.per_xcd + kslot / P.nseg;
  const int seg = kslot % P.nseg;
  if (unit >= P.units) return;   // the padding slots of the last XCD range
  // Chunk ranges.  Uniform segments: segment g aggregates and then outputs
  // its own chunks.  Two-segment split (split_K > 0): segment 0 outputs
  // chunks [0, L+K) straight from s0 and publishes the state entering chunk L
  // on the way; segment 1 meanwhile aggregates chunks [L, L+K), folds that
  // onto the published state and outputs [L+K, N), so neither waits idle.
  int out_begin, out_end, agg_begin = 0, agg_end = 0, publish_at = -1;
  bool do_pass1;
  if (P.split_K > 0) {
    if (seg == 0) {
      out_begin = 0; out_end = P.split_L + P.split_K; do_pass1 = false; publish_at = P.split_L;
    } else {
      agg_begin = P.split_L; agg_end = P.split_L + P.split_K;
      out_begin = agg_end; out_end = P.nchunks; do_pass1 = true;
    }
  } else {
    out_begin = seg * P.seg_chunks;
    if (out_begin >= P.nchunks) return;
    out_end = min(out_begin + P.seg_chunks, P.nchunks);
    do_pass1 = out_end < P.nchunks;
    agg_begin = out_begin; agg_end = out_end;
  }
  const bool last_seg = (out_end == P.nchunks);
  int c_begin = agg_begin, c_end = agg_end;   // the range of the pass being run

  const int b = unit / P.H, h = unit - b * P.H;
  const int T = P.T, dk = P.dk, dv = P.dv;
  const __amdgpu_buffer_rsrc_t rq_ = make_rsrc(P.q + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rk_ = make_rsrc(P.k + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rg_ = make_rsrc(P.g + b * P.qk_sb + h * P.qk_sh, P.qk_span);
  const __amdgpu_buffer_rsrc_t rv_ = make_rsrc(P.v + b * P.v_sb + h * P.v_sh, P.v_span);
  const __amdgpu_buffer_rsrc_t ro_ = make_rsrc(P.o + b * P.o_sb + h * P.o_sh, P.o_span);

  const int n0 = 16 * (producer ? pw : wave);   // consumer: value columns; producer: key channels
  const bool has_cols = !producer && (n0 < dv), has_rows = producer && (n0 < dk);
  const int DTr = (dk + 15) / 16, NWv = (dv + 15) / 16;   // tiles present in a state block
  const int64_t slot0 = (int64_t)unit * P.nseg;
  // this scan's published segment aggregates and gate products
  // (regions a segmentation mode does not use are absent: null, zero-sized)
  const __amdgpu_buffer_rsrc_t ragg_ = make_rsrc(P.agg ? P.agg + slot0 * P.blk_floats : nullptr,
                                                 P.agg ? (unsigned)(P.nseg * P.blk_floats * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rgam_ = make_rsrc(P.gam ? P.gam + slot0 * DP : nullptr,
                                                 P.gam ? (unsigned)(P.nseg * DP * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rinc_ = make_rsrc(P.inc ? P.inc + (int64_t)unit * P.blk_floats : nullptr,
                                                 P.inc ? (unsigned)(P.blk_floats * 4) : 0u);
  const int acol = n0 + 4 * g4;             // accumulator-layout channel of this lane (4 channels)

  // ---- one-time set-up: e^{b_last} = 1 for channel tiles no wave scans
  // (beyond dk), zero the channel padding of every tile of both buffers
  for (int x = tid; x < 2 * DP; x += NT) gam(0)[x] = 1.f;
  if (CG < DP / 8) {
    const int PADG = DP / 8 - CG;
    for (int x = tid; x < 8 * M * PADG; x += NT) {
      const int tb = x / (M * PADG), r2 = x - tb * (M * PADG);
      const int tl = r2 / PADG, cg = CG + (r2 - tl * PADG);
      *reinterpret_cast<uint4 *>(tile(tb >> 2, tb & 3) + tl * QS + 8 * cg) = make_uint4(0, 0, 0, 0);
    }
  }
  // Lower-triangular ones as the B operand of the gate scan, b^T = G^T L^T:
  // column t = d + l16, K slots s = 4*g4 + {0..3} and 16 + 4*g4 + {0..3}
  // (relative to the K block); 1.0 where s <= t.  Only d = 0 and d = 16
  // occur partially, every other (tile, K block) is all ones or skipped.
  auto lfrag = [&](int d) {
    const int t = d + l16, s0_ = 4 * g4;
    uint4 w;
    w.x = (s0_ + 0 <= t ? 0x3F80u : 0u) | (s0_ + 1 <= t ? 0x3F800000u : 0u);
    w.y = (s0_ + 2 <= t ? 0x3F80u : 0u) | (s0_ + 3 <= t ? 0x3F800000u : 0u);
    w.z = (s0_ + 16 <= t ? 0x3F80u : 0u) | (s0_ + 17 <= t ? 0x3F800000u : 0u);
    w.w = (s0_ + 18 <= t ? 0x3F80u : 0u) | (s0_ + 19 <= t ? 0x3F800000u : 0u);
    return w;
  };
  const uint4 ONES = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);

  // ================================ producers =================================
  // token offsets of chunk x (scan order -> canonical token) into parity
  // buffer x & 1; kOOB past the end of the sequence and for chunks after the
  // segment (their loads then return zeros without touching memory)
  // ORD: this producer thread's table entry for the next token table, loaded
  // one table ahead (by every producer lane, out-of-range entries reading 0,
  // so the count of memory operations does not depend on the lane)
  const __amdgpu_buffer_rsrc_t rord = make_rsrc(ORD ? P.order : nullptr, ORD ? (unsigned)T * 4u : 0u);
  unsigned ord_next = 0;
  auto ord_load = [&](int x) {
    if constexpr (ORD) {
      const int p = x * M + ptid;
      const bool ok = ptid >= 0 && ptid < M && p < T;
      ord_next = (unsigned)__builtin_amdgcn_raw_buffer_load_b32(rord, ok ? (int)(p * 4) : (int)kOOB, 0, 0);
    }
  };
  auto fill_tok = [&](int x) {
    const unsigned ord_cur = ord_next;
    ord_load(x + 1);
    if (ptid >= 0 && ptid < M) {
      const int p = x * M + ptid;
      unsigned oqk = kOOB, ov = kOOB;
      if (x < c_end && p < T) {
        unsigned n;
        if constexpr (ORD) {
          n = ord_cur;   // entries outside [0, T) address past the slice and read zeros
        } else {
          // scan position -> canonical token (the four orders of scan_to_canon),
          // the quotient by gh from a magic multiplier held in scalar registers
          const unsigned s_ = (P.dir & 1) ? (unsigned)(T - 1 - p) : (unsigned)p;
          n = s_;
          if (P.dir >= 2) {
            unsigned col = __umulhi(2u * s_, P.gh_magic);   // floor(s/gh) or one more
            int row = (int)(s_ - col * (unsigned)P.gh);
            if (row < 0) { --col; row += P.gh; }
            n = (unsigned)row * (unsigned)P.gw + col;
          }
        }
        oqk = n * (unsigned)P.qk_st * 2u;
        ov = n * (unsigned)P.v_st * 2u;
        if constexpr (ORD) {
          if (n >= (unsigned)T) oqk = ov = kOOB;
        }
      }
      unsigned *tb = sTok + (x & 3) * 2 * M;
      tb[ptid] = oqk;
      tb[M + ptid] = ov;
    }
  };
  // Loads of chunk x: item idx -> (token tl, 16-byte channel group cg).
  // Unconditional: a load under a branch would make the loop-carried
  // registers merge with their old values and force an early wait.  Two
  // register sets alternate by chunk, so a chunk's loads are issued two
  // chunks before its data is stored to LDS.
  struct LoadSet { uint4 q[R], k[R], g[R], v[R]; };
  LoadSet lsA, lsB;
  // Load j of a chunk (j = 4 r + tensor, tensors q, k, g, v; q skipped
  // without with_q), for j in [j_lo, j_hi).
  auto load_chunk = [&](int x, bool with_q, LoadSet &ls, int j_lo, int j_hi) {
    const unsigned *tb = sTok + (x & 3) * 2 * M;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (4 * r + 4 <= j_lo || 4 * r >= j_hi) continue;
      const int idx = ptid + r * NTP;
      const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
      const bool ok = idx < ITEMS;
      const unsigned tq = tb[ok ? tl : 0], tv = tb[M + (ok ? tl : 0)];
      const unsigned ok_qk = ok && (8 * cg < dk) ? tq + 16u * cg : kOOB;
      const unsigned ok_v = ok && (8 * cg < dv) ? tv + 16u * cg : kOOB;
      auto in = [&](int t) { return 4 * r + t >= j_lo && 4 * r + t < j_hi; };
      if (with_q && in(0)) ls.q[r] = bload16(rq_, ok_qk);
      if (in(1)) ls.k[r] = bload16(rk_, ok_qk);
      if (in(2)) ls.g[r] = bload16(rg_, ok_qk);
      if (in(3)) ls.v[r] = bload16(rv_, ok_v);
    }
  };
  // P1(x): the loaded chunk x (register set ls) to its tiles, then the loads
  // of chunk x+2 into the same set and the token table of chunk x+3.
  // with_q: also a vote per wave on whether M * max|log-gate| * log2(e) can
  // exceed kFastRange (then the chunk takes the pairwise path; the bound
  // covers every |b| in the chunk).
  const float bound_scale = (float)M * kLog2e;
  auto produce1 = [&](int x, bool with_q, LoadSet &ls) {
    const int par = x & 1;
    uint16_t *tq = tile(par, 0), *tk = tile(par, 1), *tg = tile(par, 2), *tv = tile(par, 3);
    unsigned gmax = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = ptid + r * NTP;
      if (idx < ITEMS) {
        const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
        const unsigned off = (unsigned)(tl * QS + 8 * cg) * 2u;   // bytes, 32-bit LDS offset
        if (with_q) *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(tq) + off) = ls.q[r];
        *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(tk) + off) = ls.k[r];
        *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(tg) + off) = ls.g[r];
        *reinterpret_cast<uint4 *>(reinterpret_cast<unsigned char *>(tv) + off) = ls.v[r];
        if (with_q) {
          const uint32_t gw_[4] = {ls.g[r].x, ls.g[r].y, ls.g[r].z, ls.g[r].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            gmax = max(gmax, max(gw_[e] & 0x7fffu, (gw_[e] >> 16) & 0x7fffu));   // |bf16| bits
        }
      }
    }
    if (with_q) {
      const bool bad = !(__uint_as_float(gmax << 16) * bound_scale <= kFastRange);   // NaN / inf too
      const bool any_bad = __any(bad);
      if (lane == 0) sVote[par * 16 + pw] = any_bad ? 1 : 0;
    }
    load_chunk(x + 2, with_q, ls, 0, JA);   // the rest in later intervals
  };
  // The loads of chunk x+2 are spread over the intervals of the step (the
  // producers' vector-memory issue otherwise stalls the interval it falls
  // in): loads [0, JA) after the staging stores of chunk x, the rest and
  // the token table of chunk x+3 after the transform of chunk x, one
  // interval later.
  auto mid_loads = [&](int x, bool with_q, LoadSet &ls) { load_chunk(x + 2, with_q, ls, JA, JB); };
  auto late_loads = [&](int x, bool with_q, LoadSet &ls) {
    load_chunk(x + 2, with_q, ls, JB, 4 * R);
    fill_tok(x + 3);
  };
  auto chunk_pairwise = [&](int x) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < DT; ++w) v |= sVote[(x & 1) * 16 + w];
    return v != 0;
  };
  // Inclusive cumulative gates of this producer wave's 16 channels as an MFMA
  // product, b^T = G^T L^T (bf16 gates and 1.0 are exact; fp32 sums), log2
  // units.  bt[i] of lane (l16, g4): token 16i + l16, channels acol .. acol+3.
  auto scan = [&](const uint16_t *tg, f32x4_t *bt) {
    const uint4 L0 = lfrag(0), L1 = lfrag(16);
    uint4 gf[JP];
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const uint2 lo = lds_tr(tg + (32 * jp + 4 * g4 + rowoff) * QS + n0 + coloff);
      const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(tg + (32 * jp + 16 + 4 * g4 + rowoff) * QS + n0 + coloff)
                                         : make_uint2(0, 0);
      gf[jp] = cat(lo, hi);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const int d = 16 * i - 32 * jp;
        if (d >= 0) acc = mfma32(gf[jp], d >= 32 ? ONES : (d == 16 ? L1 : L0), acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) bt[i][e] = acc[e] * kLog2e;
    }
  };
  // b_last of this lane's 4 channels (held by lane l16 = 15 of the last tile);
  // e^{b_last} goes to LDS for the consumers' state update.
  auto chunk_total = [&](const f32x4_t *bt, float *gmo, float *bl, int par) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bl[e] = __shfl(bt[MT - 1][e], 15 + 16 * g4);
      gmo[e] = fexp2(bl[e]);
    }
    if (l16 == 0) *reinterpret_cast<float4 *>(gam(par) + acol) = make_float4(gmo[0], gmo[1], gmo[2], gmo[3]);
  };
  // k^ = k e^{b_last - b} (exact exponent difference) into the gate tile
  auto khat_direct = [&](const uint16_t *tk, uint16_t *tg, const f32x4_t *bt, const float *bl) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int off = (16 * i + l16) * QS + acol;
      const uint2 kw = lds2(tk + off);
      *reinterpret_cast<uint2 *>(tg + off) =
          make_uint2(pack_bf16x2(bf16lo(kw.x) * fexp2(bl[0] - bt[i][0]), bf16hi(kw.x) * fexp2(bl[1] - bt[i][1])),
                     pack_bf16x2(bf16lo(kw.y) * fexp2(bl[2] - bt[i][2]), bf16hi(kw.y) * fexp2(bl[3] - bt[i][3])));
    }
  };
  // q~ = q e^{b} in place
  auto qtilde = [&](uint16_t *tq, const f32x4_t *bt) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int off = (16 * i + l16) * QS + acol;
      const uint2 qw = lds2(tq + off);
      *reinterpret_cast<uint2 *>(tq + off) =
          make_uint2(pack_bf16x2(bf16lo(qw.x) * fexp2(bt[i][0]), bf16hi(qw.x) * fexp2(bt[i][1])),
                     pack_bf16x2(bf16lo(qw.y) * fexp2(bt[i][2]), bf16hi(qw.y) * fexp2(bt[i][3])));
    }
  };
  // P2(x): per producer wave, its 16 channels: b, e^{b_last}; fast chunks:
  // q~ = q e^{b}, k~ = k e^{-b} in place (|b| <= 64: no overflow; the state
  // update applies e^{b_last} after its product); pairwise chunks: b to LDS
  // (fp32) and k^ = k e^{b_last - b} directly.  bt stays in
  // registers for P3 of a pairwise chunk.
  f32x4_t bt[MT];
  // (produce2 and produce3_fast are forced inline: left to the compiler, the
  // 128-token instantiations called them as functions, with their captures
  // in a stack frame)
  auto produce2 = [&](int x, bool pairwise) __attribute__((always_inline)) {
    const int par = x & 1;
    uint16_t *tq = tile(par, 0), *tk = tile(par, 1), *tg = tile(par, 2);
    float gmo[4], bl[4];
    scan(tg, bt);
    chunk_total(bt, gmo, bl, par);
    if (!pairwise) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int off = (16 * i + l16) * QS + acol;
        const uint2 qw = lds2(tq + off), kw = lds2(tk + off);
        const uint32_t qa[2] = {qw.x, qw.y}, ka[2] = {kw.x, kw.y};
        uint32_t oq[2], ok[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          oq[e] = pack_bf16x2(bf16lo(qa[e]) * fexp2(bt[i][2 * e]), bf16hi(qa[e]) * fexp2(bt[i][2 * e + 1]));
          ok[e] = pack_bf16x2(bf16lo(ka[e]) * fexp2(-bt[i][2 * e]), bf16hi(ka[e]) * fexp2(-bt[i][2 * e + 1]));
        }
        *reinterpret_cast<uint2 *>(tq + off) = make_uint2(oq[0], oq[1]);
        *reinterpret_cast<uint2 *>(tk + off) = make_uint2(ok[0], ok[1]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        *reinterpret_cast<float4 *>(sB32 + (16 * i + l16) * DP + acol) =
            make_float4(bt[i][0], bt[i][1], bt[i][2], bt[i][3]);
      khat_direct(tk, tg, bt, bl);
    }
  };
  // P3(x), fast chunks: causal P^T tiles (j, i), j <= i, from q~ and k~,
  // spread over all waves (the consumers have nothing else to do then).
  auto produce3_fast = [&](int x) __attribute__((always_inline)) {
    const int par = x & 1;
    const uint16_t *tq = tile(par, 0), *tk = tile(par, 1);
    uint16_t *pt = ptile(par);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        const int ti = i * (i + 1) / 2 + j;
        if (ti % (2 * DT) == wave) {
          const uint16_t *krow = tk + (16 * j + l16) * QS;
          const uint16_t *qrow = tq + (16 * i + l16) * QS;
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb2 = 0; kb2 < K32; ++kb2)
            acc = mfma32(lds4(krow + 32 * kb2 + 8 * g4), lds4(qrow + 32 * kb2 + 8 * g4), acc);
          if (KH) acc = mfma16(lds2(krow + 32 * K32 + 4 * g4), lds2(qrow + 32 * K32 + 4 * g4), acc);
          if (j == i) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * g4 + e > l16) acc[e] = 0.f;   // causal: s > t
          }
          *reinterpret_cast<uint2 *>(pt + ti * 256 + lane * 4) = pack4(acc);
        }
      }
    }
  };
  // P3(x), pairwise chunks: P^T slot (tile ti = (j, i), lane l, element e) is
  // t = 16i + l%16, s = 16j + 4(l/16) + e; value sum_c q_tc k_sc 2^(b_tc - b_sc)
  // over all key channels for s <= t, else 0.  Slots spread over all threads.
  auto produce3_pairwise = [&](int x) {
    const int par = x & 1;
    const uint16_t *tq = tile(par, 0), *tk = tile(par, 1);
    uint16_t *pt = ptile(par);
    for (int sl = tid; sl < NPT * 256; sl += NT) {
      const int ti = sl >> 8, ln = (sl >> 2) & 63, e = sl & 3;
      int i = 0;
      while ((i + 1) * (i + 2) / 2 <= ti) ++i;
      const int j = ti - i * (i + 1) / 2;
      const int t = 16 * i + (ln & 15), s_ = 16 * j + 4 * (ln >> 4) + e;
      float acc = 0.f;
      if (s_ <= t) {
        for (int ch = 0; ch < dk; ++ch) {
          const float qv = __uint_as_float((uint32_t)tq[t * QS + ch] << 16);
          const float kv = __uint_as_float((uint32_t)tk[s_ * QS + ch] << 16);
          acc += qv * kv * fexp2(sB32[t * DP + ch] - sB32[s_ * DP + ch]);
        }
      }
      pt[sl] = (uint16_t)f2bf(acc);
    }
  };

  // ================================ consumers =================================
  // v fragments with tokens along K: K block jp holds tokens 32jp + 4*g4 + e
  // (slots 0..3) and 32jp + 16 + 4*g4 + e (slots 4..7); this wave's columns.
  auto v_frags = [&](const uint16_t *tv, uint4 *vf) {
#pragma unroll
    for (int jp = 0; jp < JP; ++jp) {
      const uint2 lo = lds_tr(tv + (32 * jp + 4 * g4 + rowoff) * QS + n0 + coloff);
      const uint2 hi = (2 * jp + 1 < MT) ? lds_tr(tv + (32 * jp + 16 + 4 * g4 + rowoff) * QS + n0 + coloff)
                                         : make_uint2(0, 0);
      vf[jp] = cat(lo, hi);
    }
  };
  // The state after a chunk for this wave's columns: fast chunks
  // S = diag(e^{b_last}) (S + k~^T v) (k~ = k e^{-b} in tile 1: the same
  // product as k^^T v, scaled once per row afterwards); pairwise chunks and
  // segment aggregates S = diag(e^{b_last}) S + k^^T v (k^ in tile 2), which
  // optionally also accumulates the product of the gates in gprod.  The form
  // is a template argument (std::true_type: fast), so each copy scales its
  // rows once instead of selecting a factor per element.
  auto state_update = [&](int par, f32x4_t *S, f32x4_t *gprod, auto fast_c, const uint4 *vf_in) {
    constexpr bool fast = decltype(fast_c)::value;
    const uint16_t *th = tile(par, fast ? 1 : 2);
    uint4 vf[JP];
    if (vf_in) {
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) vf[jp] = vf_in[jp];
    } else {
      v_frags(tile(par, 3), vf);
    }
    const float *gm_ = gam(par);
#pragma unroll
    for (int r = 0; r < DT; ++r) {
      const float4 gm = *reinterpret_cast<const float4 *>(gm_ + 16 * r + 4 * g4);
      const float gv[4] = {gm.x, gm.y, gm.z, gm.w};
      if constexpr (!fast) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][e] *= gv[e];
      }
      if (gprod) { gprod[r][0] *= gm.x; gprod[r][1] *= gm.y; gprod[r][2] *= gm.z; gprod[r][3] *= gm.w; }
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const uint2 lo = lds_tr(th + (32 * jp + 4 * g4 + rowoff) * QS + 16 * r + coloff);
        const uint2 hi = (2 * jp + 1 < MT)
                             ? lds_tr(th + (32 * jp + 16 + 4 * g4 + rowoff) * QS + 16 * r + coloff)
                             : make_uint2(0, 0);
        S[r] = mfma32(cat(lo, hi), vf[jp], S[r]);
      }
      if constexpr (fast) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][e] *= gv[e];
      }
    }
  };
  // o of chunk c for this wave's columns: O^T = S^T q~^T + V^T P^T (S: the
  // state entering the chunk), stored 8 bytes per lane into the staging
  // tile; the v fragments are left in vf for the state update.  Every token tile is
  // computed before the first staging store: a store between two tiles would
  // keep the compiler from issuing the next tile's LDS reads ahead of this
  // tile's products (it cannot tell the staging tile from the operand tiles),
  // and the tiles' reads then run one round trip at a time.
  uint16_t *stg = reinterpret_cast<uint16_t *>(smem + Lds<DP, M>::oStg);
  auto outputs = [&](int c, const f32x4_t *S, uint4 *vf) {
    const int par = c & 1;
    const uint16_t *tq = tile(par, 0), *pt = ptile(par);
    v_frags(tile(par, 3), vf);
    uint4 sa[K32];   // S^T (bf16) as the A operand, K = channels
#pragma unroll
    for (int kb2 = 0; kb2 < K32; ++kb2) sa[kb2] = cat(pack4(S[2 * kb2]), pack4(S[2 * kb2 + 1]));
    // every operand fragment of the chunk first (q~ rows, P^T tiles), then the products
    uint4 qf[MT][K32], pf[MT][JP];
    [[maybe_unused]] uint2 qh[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const uint16_t *qrow = tq + (16 * i + l16) * QS;
#pragma unroll
      for (int kb2 = 0; kb2 < K32; ++kb2)
        qf[i][kb2] = cat(lds2(qrow + 32 * kb2 + 4 * g4), lds2(qrow + 32 * kb2 + 16 + 4 * g4));
      if (KH) qh[i] = lds2(qrow + 32 * K32 + 4 * g4);
#pragma unroll
      for (int jp = 0; jp < JP; ++jp) {
        const int j0 = 2 * jp, j1 = 2 * jp + 1;
        if (j0 <= i) {
          const uint2 pt0 = lds2(pt + (i * (i + 1) / 2 + j0) * 256 + lane * 4);
          const uint2 pt1 = (j1 <= i) ? lds2(pt + (i * (i + 1) / 2 + j1) * 256 + lane * 4) : make_uint2(0, 0);
          pf[i][jp] = cat(pt0, pt1);
        }
      }
    }
    // (keep the scheduler from sinking the reads back between the products,
    // where the registers allow it: 128-channel tiles and the 64-channel
    // table-order kernel would spill)
    if constexpr (DP <= 96 && !(ORD && DP == 64)) __builtin_amdgcn_sched_barrier(0);
    f32x4_t O[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      O[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < K32; ++kb2) O[i] = mfma32(sa[kb2], qf[i][kb2], O[i]);
      if (KH) O[i] = mfma16(pack4(S[2 * K32]), qh[i], O[i]);
#pragma unroll
      for (int jp = 0; jp < JP; ++jp)
        if (2 * jp <= i) O[i] = mfma32(vf[jp], pf[i][jp], O[i]);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
      *reinterpret_cast<uint2 *>(stg + (16 * i + l16) * QS + n0 + 4 * g4) = pack4(O[i]);
  };
  // o of chunk c from the staging tile to memory: whole token rows, 16 bytes
  // per lane (a 64-lane store covers a few complete rows instead of 16-column
  // slices of many)
  auto store_stage = [&](int c) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = tid + r * NTP;
      const int tl = (int)__umulhi(2u * (unsigned)idx, P.cg_magic), cg = idx - tl * CG;
      const int p = c * M + tl;
      const bool ok = idx < ITEMS && 8 * cg < dv && p < T;
      const uint4 w = *reinterpret_cast<const uint4 *>(stg + (ok ? tl * QS + 8 * cg : 0));
      bstore16(ro_, ok ? ((unsigned)p * (unsigned)P.o_st + 8u * cg) * 2u : kOOB, w);
    }
  };
  // Initial state s0 for this wave's tiles (0 when absent).
  auto load_s0 = [&](f32x4_t *S) {
#pragma unroll
    for (int r = 0; r < DT; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * r + 4 * g4 + e, n = n0 + l16;
        S[r][e] = (has_cols && P.s0 && ch < dk && n < dv) ? P.s0[((int64_t)unit * dk + ch) * dv + n] : 0.f;
      }
  };
  auto blk_at = [&](int r) { return ((r * NWv + wave) * 64 + lane) * 4; };

  // The two roles run separate copies of the whole schedule with the same
  // sequence of barriers (marked B in the comments: both sides must pass
  // the same ones in the same order), so the registers one role carries (the
  // producers' in-flight loads and gate sums, the consumers' state) are never
  // allocated in the other role's code.
  if (producer) {
    // ===================== pass 1: segment aggregate ==========================
    // transform chunk c+1 (gates -> k^, e^{b_last}) while the consumers fold
    // chunk c into the aggregate, then stage chunk c+2
    if (do_pass1) {
      ord_load(c_begin);
      fill_tok(c_begin);
      fill_tok(c_begin + 1);
      fill_tok(c_begin + 2);
      __syncthreads();                                          // B a
      load_chunk(c_begin, false, lsA, 0, 4 * R);
      load_chunk(c_begin + 1, false, lsB, 0, 4 * R);
      lds_barrier();                                            // B 1
      produce1(c_begin, false, lsA);
      mid_loads(c_begin, false, lsA);
      late_loads(c_begin, false, lsA);
      lds_barrier();                                            // B 2
      // the gates of chunk x -> b, e^{b_last}, k^ = k e^{b_last - b}
      auto agg_transform = [&](int x) {
        float gmo[4], bl[4];
        scan(tile(x & 1, 2), bt);
        chunk_total(bt, gmo, bl, x & 1);
        khat_direct(tile(x & 1, 1), tile(x & 1, 2), bt, bl);
      };
      if (has_rows) agg_transform(c_begin);
      produce1(c_begin + 1, false, lsB);
      lds_barrier();                                            // B 3
      // Step c (the consumers fold chunk c into the aggregate): transform
      // chunk x = c+1 and issue the rest of chunk x+2's loads (register set
      // ls_tail), then stage chunk x+1 (set ls_stage), which goes to the
      // buffer chunk c was read from.  The staging is unconditional (past
      // the segment the token table reads zeros and the stores land in a
      // buffer nobody reads): a skipped load would make the compiler's count
      // of outstanding loads, and its waits, conservative for every chunk.
      auto agg_step = [&](int c, LoadSet &ls_tail, LoadSet &ls_stage) {
        const int x = c + 1;
        if (has_rows && x < c_end) agg_transform(x);
        mid_loads(x, false, ls_tail);
        late_loads(x, false, ls_tail);
        lds_barrier();                                          // B loop 1
        produce1(x + 1, false, ls_stage);
        lds_barrier();                                          // B loop 2
      };
      // Steps in pairs (register sets B, A); an odd count ends with a step
      // past the segment, matched by the consumers.  (A conditional second
      // step would leave the compiler unsure which set was loaded last, and
      // it would wait for both.)
      for (int c = c_begin; c < c_end; c += 2) {
        agg_step(c, lsB, lsA);
        agg_step(c + 1, lsA, lsB);
      }
      drain_vmem();
      __syncthreads();                                          // B e
    }
    // ================ look-back (the consumers' work) ========================
    // the first two output chunks' loads are issued before it
    c_begin = out_begin;
    c_end = out_end;
    ord_load(c_begin);
    fill_tok(c_begin);
    fill_tok(c_begin + 1);
    fill_tok(c_begin + 2);
    __syncthreads();                                            // B r
    load_chunk(c_begin, true, lsA, 0, 4 * R);
    load_chunk(c_begin + 1, true, lsB, 0, 4 * R);
    if (seg != 0) __syncthreads();                              // B l
    // ======================= pass 2: outputs ==================================
    __syncthreads();                                            // B s
    lds_barrier();                                              // B t
    produce1(c_begin, true, lsA);
    mid_loads(c_begin, true, lsA);
    late_loads(c_begin, true, lsA);
    lds_barrier();                                              // B u
    bool pw_next = chunk_pairwise(c_begin);
    if (has_rows) produce2(c_begin, pw_next);
    lds_barrier();                                              // B v
    if (!pw_next) produce3_fast(c_begin); else produce3_pairwise(c_begin);
    produce1(c_begin + 1, true, lsB);
    lds_barrier();                                              // B w
    if (pw_next) {
      if (has_rows) qtilde(tile(c_begin & 1, 0), bt);
      lds_barrier();                                            // B x
    }
    // Step c (the consumers write o of chunk c): the producers transform
    // chunk x = c+1 and issue the rest of chunk x+2's loads (register set
    // ls_tail), then stage chunk x+1 (set ls_stage) while all waves build the
    // P^T tiles of chunk x.
    auto out_step = [&](int c, LoadSet &ls_tail, LoadSet &ls_stage) {
      const int x = c + 1;
      const bool live = x < c_end;
      const bool pwx = live && chunk_pairwise(x);
      // interval 1: transform chunk x (the consumers write o of chunk c and
      // update the state)
      if (has_rows && live) produce2(x, pwx);
      mid_loads(x, true, ls_tail);
      late_loads(x, true, ls_tail);
      lds_barrier();                                            // B loop 1
      // interval 2: P^T tiles of chunk x; stage chunk x+1 (unconditional, as
      // in the aggregate pass)
      if (live) {
        if (!pwx) produce3_fast(x); else produce3_pairwise(x);
      }
      produce1(x + 1, true, ls_stage);
      lds_barrier();                                            // B loop 2
      if (pwx) {
        if (has_rows) qtilde(tile(x & 1, 0), bt);
        lds_barrier();                                          // B loop 3
      }
    };
    for (int c = c_begin; c < c_end; c += 2) {   // in pairs, as in the aggregate pass
      out_step(c, lsB, lsA);
      out_step(c + 1, lsA, lsB);
    }
    return;
  }

  // ================================ consumers =================================
  f32x4_t S[DT];
#pragma unroll
  for (int r = 0; r < DT; ++r) S[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t gp[DT];   // product of this segment's gates (rows of S)
#pragma unroll
  for (int r = 0; r < DT; ++r) gp[r] = f32x4_t{1.f, 1.f, 1.f, 1.f};

  // ======================= pass 1: segment aggregate =========================
  if (do_pass1) {
    __syncthreads();                                            // B a
    lds_barrier();                                              // B 1
    lds_barrier();                                              // B 2
    lds_barrier();                                              // B 3
    for (int c = c_begin; c < c_end; ++c) {
      if (has_cols) state_update(c & 1, S, gp, std::false_type{}, nullptr);
      lds_barrier();                                            // B loop 1
      lds_barrier();                                            // B loop 2
    }
    if ((c_end - c_begin) & 1) {   // the producers' step past the segment
      lds_barrier();                                            // B loop 1
      lds_barrier();                                            // B loop 2
    }
    if (has_cols && P.split_K == 0) {
      const unsigned mb = (unsigned)(seg * P.blk_floats) * 4u;
#pragma unroll
      for (int r = 0; r < DT; ++r)
        if (r < DTr) bstore_coh(ragg_, mb + (unsigned)blk_at(r) * 4u, make_float4(S[r][0], S[r][1], S[r][2], S[r][3]));
      if (wave == 0 && l16 == 0) {
#pragma unroll
        for (int r = 0; r < DT; ++r)
          bstore_coh(rgam_, (unsigned)(seg * DP + 16 * r + 4 * g4) * 4u, make_float4(gp[r][0], gp[r][1], gp[r][2], gp[r][3]));
      }
    }
    drain_vmem();
    __syncthreads();                                            // B e
    if (tid == 0 && P.split_K == 0)
      __hip_atomic_store(P.flags + slot0 + seg, P.epoch * 4u + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ================== look-back: state entering the segment ==================
  // (the producers meanwhile issue the loads of the first two output chunks)
  // Each branch leaves the state entering the segment's outputs in S.
  __syncthreads();                                              // B r
  if (seg == 0) {
    load_s0(S);
  } else if (P.split_K > 0) {
    // split segment 1: the state segment 0 publishes on its way past chunk L
    if (tid == 0) wait_flag(P.flags + slot0, P.epoch, P.err);
    __syncthreads();                                            // B l
    // S(L) folded with this segment's aggregate of chunks [L, L+K)
#pragma unroll
    for (int r = 0; r < DT; ++r) {
      const float4 xx = bload_coh(rinc_, has_cols && r < DTr ? (unsigned)blk_at(r) * 4u : kOOB);
      S[r][0] = fmaf(gp[r][0], xx.x, S[r][0]);
      S[r][1] = fmaf(gp[r][1], xx.y, S[r][1]);
      S[r][2] = fmaf(gp[r][2], xx.z, S[r][2]);
      S[r][3] = fmaf(gp[r][3], xx.w, S[r][3]);
    }
  } else {
    // Every earlier segment's aggregate: the lanes of wave 0 watch one flag
    // each.  Then S_in = P_{g-1} of the serial recurrence
    // P_m = Gam_m * P_{m-1} + A_m from P_{-1} = s0, element by element in
    // segment order, so the result does not depend on timing.  The loads of
    // kFoldBatch segments are issued before their folds.
    if (wave == 0)
      for (int j = lane; j < seg; j += 64) wait_flag(P.flags + slot0 + j, P.epoch, P.err);
    __syncthreads();                                            // B l
    load_s0(S);
    if (has_cols) {
      // segments whose aggregates are loaded before they are folded: 8 DT
      // registers each, as many as fit beside the rest (measured: no spills)
      constexpr int kFoldBatch = DT <= 4 ? 4 : DT == 5 ? 3 : 1;
      if constexpr (DT >= 8) {
        // 128 channels: sixteen waves of 128 registers; one segment at a time
        for (int m = 0; m < seg; ++m) {
#pragma unroll
          for (int r = 0; r < DT; ++r) {
            if (r < DTr) {
              const float4 av = bload_coh(ragg_, (unsigned)(m * P.blk_floats + blk_at(r)) * 4u);
              const float4 gv = bload_coh(rgam_, (unsigned)(m * DP + 16 * r + 4 * g4) * 4u);
              S[r][0] = fmaf(gv.x, S[r][0], av.x);
              S[r][1] = fmaf(gv.y, S[r][1], av.y);
              S[r][2] = fmaf(gv.z, S[r][2], av.z);
              S[r][3] = fmaf(gv.w, S[r][3], av.w);
            }
          }
        }
      } else {
        for (int m0 = 0; m0 < seg; m0 += kFoldBatch) {
          float4 av[kFoldBatch][DT], gv[kFoldBatch][DT];
#pragma unroll
          for (int i = 0; i < kFoldBatch; ++i) {
            const int m = m0 + i < seg ? m0 + i : seg - 1;
#pragma unroll
            for (int r = 0; r < DT; ++r) {
              av[i][r] = bload_coh(ragg_, r < DTr ? (unsigned)(m * P.blk_floats + blk_at(r)) * 4u : kOOB);
              gv[i][r] = bload_coh(rgam_, r < DTr ? (unsigned)(m * DP + 16 * r + 4 * g4) * 4u : kOOB);
            }
          }
          // (a select, not a branch, past the last segment: a branch would
          // let the compiler sink each segment's loads behind the previous fold)
#pragma unroll
          for (int i = 0; i < kFoldBatch; ++i) {
            const bool live = m0 + i < seg;
#pragma unroll
            for (int r = 0; r < DT; ++r) {
              if (r < DTr) {
                const float x0 = fmaf(gv[i][r].x, S[r][0], av[i][r].x);
                const float x1 = fmaf(gv[i][r].y, S[r][1], av[i][r].y);
                const float x2 = fmaf(gv[i][r].z, S[r][2], av[i][r].z);
                const float x3 = fmaf(gv[i][r].w, S[r][3], av[i][r].w);
                S[r][0] = live ? x0 : S[r][0];
                S[r][1] = live ? x1 : S[r][1];
                S[r][2] = live ? x2 : S[r][2];
                S[r][3] = live ? x3 : S[r][3];
              }
            }
          }
        }
      }
    }
  }
  // ========================= pass 2: outputs ==================================
  // Two barrier intervals per chunk c: the consumers write o of chunk c and
  // update the state while the producers transform chunk c+1; then all waves
  // build the P^T tiles of chunk c+1 while the producers stage chunk c+2 and
  // the consumers store o of chunk c.  A pairwise chunk c+1 adds one interval
  // (its q~ may be written only after every thread has read its raw q).
  drain_vmem();
  c_begin = out_begin;
  c_end = out_end;
  __syncthreads();                                              // B s
  lds_barrier();                                                // B t
  lds_barrier();                                                // B u
  bool pw_next = chunk_pairwise(c_begin);
  lds_barrier();                                                // B v
  if (!pw_next) produce3_fast(c_begin); else produce3_pairwise(c_begin);
  lds_barrier();                                                // B w
  if (pw_next) lds_barrier();                                   // B x
  bool pw_c = pw_next;   // chunk c took the pairwise path
  for (int c = c_begin; c < c_end; ++c) {
    const int x = c + 1;
    const bool live = x < c_end;
    const bool pwx = live && chunk_pairwise(x);
    // interval 1: o of chunk c into the staging tile, then the state after
    // chunk c.  Split segment 0 publishes the state entering chunk L; the
    // flag goes up right after the barrier.
    const bool pub = c + 1 == publish_at;
    if (has_cols) {
      uint4 vf[JP];
      outputs(c, S, vf);
      if (pw_c) state_update(c & 1, S, nullptr, std::false_type{}, vf);
      else state_update(c & 1, S, nullptr, std::true_type{}, vf);
      if (pub) {
#pragma unroll
        for (int r = 0; r < DT; ++r)
          if (r < DTr) bstore_coh(rinc_, (unsigned)blk_at(r) * 4u, make_float4(S[r][0], S[r][1], S[r][2], S[r][3]));
        drain_vmem();
      }
    }
    lds_barrier();                                              // B loop 1
    if (pub && tid == 0)
      __hip_atomic_store(P.flags + slot0, P.epoch * 4u + 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // interval 2: P^T tiles of chunk x; o of chunk c to memory
    if (live) {
      if (!pwx) produce3_fast(x); else produce3_pairwise(x);
    }
    store_stage(c);
    lds_barrier();                                              // B loop 2
    if (pwx) lds_barrier();                                     // B loop 3
    pw_c = pwx;
  }
  if ((c_end - c_begin) & 1) {   // the producers' step past the segment
    lds_barrier();                                              // B loop 1
    lds_barrier();                                              // B loop 2
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

// channel padding of a tile: 32, 64, 80, 96 or 128
int pad_dp(int d) { return d <= 64 ? ((d + 31) / 32) * 32 : d <= 80 ? 80 : d <= 96 ? 96 : 128; }

int lds_bytes(int DP, int M) {
  switch (DP * 1000 + M) {
#define DIG_LDS_CASE(D, MM) \
  case D * 1000 + MM:       \
    return Lds<D, MM>::bytes;
    DIG_LDS_CASE(32, 16) DIG_LDS_CASE(32, 32) DIG_LDS_CASE(32, 64) DIG_LDS_CASE(32, 128)
    DIG_LDS_CASE(64, 16) DIG_LDS_CASE(64, 32) DIG_LDS_CASE(64, 64)
    DIG_LDS_CASE(80, 16) DIG_LDS_CASE(80, 32) DIG_LDS_CASE(80, 64)
    DIG_LDS_CASE(96, 16) DIG_LDS_CASE(96, 32) DIG_LDS_CASE(96, 64)
    DIG_LDS_CASE(128, 16) DIG_LDS_CASE(128, 32) DIG_LDS_CASE(128, 64)
#undef DIG_LDS_CASE
    default: return 160 * 1024;
  }
}

// aggregate chunks of segment 1 in the two-segment split, as a fraction of
// the scan (measured best at 64-token chunks: an aggregate chunk costs about
// half an output chunk, and the hand-off of the state at chunk L takes about
// one output chunk)
constexpr float kSplitFrac = 0.38f;

struct Plan {
  int DP, M, nchunks, units, nseg, seg_chunks, per_xcd, grid, blk_floats, split_L, split_K;
  size_t off_flags, off_gam, off_agg, off_inc, bytes;
};

// Segmentation: as many workgroups as fit on the chip at once (LDS and
// registers), but segments of at least 512 tokens so that the published
// states stay small next to the streamed inputs.
Plan make_plan(int B, int T, int H, int dk, int dv, int M, int num_cu) {
  Plan pl;
  pl.DP = pad_dp(dk > dv ? dk : dv);
  pl.M = M;
  pl.nchunks = (T + M - 1) / M;
  pl.units = B * H;
  // workgroups resident per CU: LDS (160 KiB) and the register budget
  // (waves per SIMD, 4 SIMDs) both bound it
  int per_cu = (160 * 1024) / lds_bytes(pl.DP, M);
  const int nw = 2 * (pl.DP / 16);
  const int wps = (nw + 3) / 4 < 2 ? 2 : (nw + 3) / 4;   // as Occ<DP>
  const int reg_cap = 4 * wps / nw;
  if (per_cu > reg_cap) per_cu = reg_cap;
  if (per_cu < 1) per_cu = 1;
  // at most one wave of resident workgroups: a workgroup beyond it waits for
  // a whole one to finish, and every segment but the last of a scan reads
  // its chunks twice, so more segments cost more than they hide
  const long want = (long)num_cu * per_cu;
  long nseg = want / pl.units;
  const int min_chunks = (512 + M - 1) / M;
  long max_seg = pl.nchunks / min_chunks;
  if (max_seg < 1) max_seg = 1;
  if (nseg > max_seg) nseg = max_seg;
  if (nseg < 1) nseg = 1;
  pl.seg_chunks = (int)((pl.nchunks + nseg - 1) / nseg);
  pl.nseg = (pl.nchunks + pl.seg_chunks - 1) / pl.seg_chunks;
  // Two segments: pipelined split.  With p1, p2 the times of an aggregate and
  // an output chunk, segment 1 aggregates K chunks while segment 0 outputs L,
  // then each outputs N - L - K: balanced at K = N p2 / (2 p2 + p1), L = N - 2K.
  pl.split_L = pl.split_K = 0;
  if (pl.nseg == 2) {
    const int K = (int)(pl.nchunks * kSplitFrac + 0.5f), L = pl.nchunks - 2 * K;
    if (K >= 1 && L >= 1) { pl.split_K = K; pl.split_L = L; }
  }
  pl.per_xcd = (pl.units + 7) / 8;
  pl.grid = 8 * pl.per_xcd * pl.nseg;
  const int DTr = (dk + 15) / 16, NWv = (dv + 15) / 16;
  pl.blk_floats = DTr * NWv * 64 * 4;
  // Workspace: each region only where the segmentation uses it (one segment
  // per scan needs the header alone).
  const size_t slots = (size_t)pl.units * pl.nseg;
  const bool split = pl.split_K > 0, lookback = pl.nseg > 1 && !split;
  auto up = [](size_t x) { return ((x + 255) / 256) * 256; };
  size_t off = 256;   // header: the 8 ticket counters at byte 0, the error word at DIG_GLA_ERR_WORD_OFFSET
  pl.off_flags = off;
  off += pl.nseg > 1 ? up(slots * 4) : 0;
  pl.off_gam = off;
  off += lookback ? up(slots * pl.DP * 4) : 0;
  pl.off_agg = off;
  off += lookback ? up(slots * pl.blk_floats * 4) : 0;
  pl.off_inc = off;
  off += split ? up((size_t)pl.units * pl.blk_floats * 4) : 0;
  pl.bytes = off;
  return pl;
}

// Clears n 32-bit words (the segment flags of a launch that will be replayed
// from a graph, where every replay carries the same epoch).
__global__ void __launch_bounds__(256) clear_words_kernel(unsigned *w, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) w[i] = 0u;
}

template <int DP, int M>
hipError_t launch(const Params &p, int grid, hipStream_t s) {
  const size_t lds = Lds<DP, M>::bytes;
  auto *fn = p.order ? gla_fwd_bf16_kernel<DP, M, true> : gla_fwd_bf16_kernel<DP, M, false>;
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
    case 64:
      if constexpr (DP <= 96) return launch<DP, 64>(p, grid, s);   // 128 channels: LDS holds 32-token chunks
      return hipErrorInvalidValue;
    case 128:
      if constexpr (DP == 32) return launch<DP, 128>(p, grid, s);  // LDS holds 128-token chunks at 32 channels
      return hipErrorInvalidValue;
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
  p.order = a.order;
  p.nchunks = pl.nchunks;
  p.units = pl.units;
  p.seg_chunks = pl.seg_chunks;
  p.split_L = pl.split_L;
  p.split_K = pl.split_K;
  p.nseg = pl.nseg;
  p.per_xcd = pl.per_xcd;
  p.blk_floats = pl.blk_floats;
  p.cgr = ((a.dk > a.dv ? a.dk : a.dv) + 7) / 8;
  p.cg_magic = (unsigned)((0x80000000ull + p.cgr - 1) / p.cgr);
  // umulhi(2s, ceil(2^31/gh)) = floor(s/gh + s*e/(gh*2^31)) with e < gh, so it
  // exceeds floor(s/gh) by at most one for every s < 2^31: one correction
  p.gh_magic = (unsigned)((0x80000000ull + (unsigned)a.gh - 1) / (unsigned)a.gh);
  p.qk_span = (unsigned)(((int64_t)(a.T - 1) * a.qk_st + a.dk) * 2);
  p.v_span = (unsigned)(((int64_t)(a.T - 1) * a.v_st + a.dv) * 2);
  p.o_span = (unsigned)(((int64_t)(a.T - 1) * a.o_st + a.dv) * 2);
  char *ws = static_cast<char *>(a.workspace);
  p.ticket = reinterpret_cast<unsigned *>(ws);
  p.err = reinterpret_cast<unsigned *>(ws + DIG_GLA_ERR_WORD_OFFSET);
  const bool split = pl.split_K > 0, lookback = pl.nseg > 1 && !split;
  p.flags = pl.nseg > 1 ? reinterpret_cast<unsigned *>(ws + pl.off_flags) : nullptr;
  p.gam = lookback ? reinterpret_cast<float *>(ws + pl.off_gam) : nullptr;
  p.agg = lookback ? reinterpret_cast<float *>(ws + pl.off_agg) : nullptr;
  p.inc = split ? reinterpret_cast<float *>(ws + pl.off_inc) : nullptr;
  p.epoch = a.epoch;
  // Flags carry the launch's epoch, so between ordinary calls they need no
  // clearing.  A launch captured into a graph replays with one epoch, and
  // the flags of the previous replay would read as published: the flag
  // words are cleared by a fill kernel queued before the GLA kernel.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return e;
  if (cap == hipStreamCaptureStatusActive && pl.nseg > 1) {
    const int n = pl.units * pl.nseg;
    hipLaunchKernelGGL(clear_words_kernel, dim3((n + 255) / 256 < 64 ? (n + 255) / 256 : 64), dim3(256), 0, s,
                       p.flags, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (pl.DP) {
    case 32: return launch_m<32>(p, a.chunk, pl.grid, s);
    case 64: return launch_m<64>(p, a.chunk, pl.grid, s);
    case 80: return launch_m<80>(p, a.chunk, pl.grid, s);
    case 96: return launch_m<96>(p, a.chunk, pl.grid, s);
    case 128: return launch_m<128>(p, a.chunk, pl.grid, s);
    default: return hipErrorInvalidValue;
  }
}
