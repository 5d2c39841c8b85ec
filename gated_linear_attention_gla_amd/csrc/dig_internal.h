// dig_internal.h -- internal declarations shared by the HIP sources of
// libdig_gla.so (kernels, launchers and the C ABI layer).  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dig {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Scan order over a (gh x gw) grid, canonical order row-major (n = r*gw + c).
// DiG paper notes, 关键设计 / SREM: left->right, right->left, top->bottom and
// bottom->top scans made by transposing the 2D token matrix and flipping the
// sequence (flip = reversal of the whole sequence).
//   0 L2R: n = p            1 R2L: n = T-1-p
//   2 T2B: n = (p % gh) * gw + p / gh
//   3 B2T: T2B index of T-1-p
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int scan_to_canon(int dir, int gh, int gw, int T, int p) {
  const int s = (dir & 1) ? (T - 1 - p) : p;   // R2L and B2T walk backwards
  if (dir < 2) return s;
  const int col = (int)((unsigned)s / (unsigned)gh);
  const int row = s - col * gh;
  return row * gw + col;
}

// Inverse: the scan position at which canonical index n is visited.
__host__ __device__ __forceinline__ int canon_to_scan(int dir, int gh, int gw, int T, int n) {
  int s = n;
  if (dir >= 2) {
    const int row = (int)((unsigned)n / (unsigned)gw);
    const int col = n - row * gw;
    s = col * gh + row;
  }
  return (dir & 1) ? (T - 1 - s) : s;
}

// Frame of the scan-ordered sequence: (R, Q) = (gh, gw) for the row scans,
// (gw, gh) for the column scans.
__host__ __device__ __forceinline__ void scan_frame(int dir, int gh, int gw, int &R, int &Q) {
  if (dir < 2) { R = gh; Q = gw; } else { R = gw; Q = gh; }
}

// XCD-aware workgroup order: MI355X deals workgroups round-robin over its 8
// XCDs (each with its own L2), so workgroup i runs on XCD i % 8.  This maps
// blockIdx.x to a logical index such that each XCD receives a contiguous
// range of logical indices (neighbouring heads / tokens share cache lines and
// L2 on one XCD).  grid must be a multiple of 8.
__device__ __forceinline__ int xcd_linear_block(int bid, int grid) {
  const int per = grid >> 3;
  return (bid & 7) * per + (bid >> 3);
}

// ------------------------------- bf16 bits ---------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even, NaN kept quiet: gfx950's
// v_cvt_pk_bf16_f32 (two values per instruction).
typedef __bf16 dig_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const dig_bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

}  // namespace dig

// ----------------------------- launchers -----------------------------------
// Each returns hipSuccess or the launch error; arguments are validated by the
// ABI layer before these are called.
struct DigGlaArgs {
  const void *q, *k, *v, *g;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, o_sb, o_st, o_sh;
  void *o;
  const float *s0;
  float *s_final;
  int B, T, H, dk, dv, gh, gw, dir, chunk;
  const int *order;   // nullable: scan position -> canonical token [T]; replaces (gh, gw, dir)
  void *workspace;
  size_t workspace_bytes;
  uint32_t epoch;
  int num_cu;
};

hipError_t dig_launch_gla_bf16(const DigGlaArgs &a, hipStream_t s);
// Byte offset, inside the bf16 forward's workspace, of the error word its
// kernel sets when a wait between workgroups gives up (bit 0).
constexpr size_t DIG_GLA_ERR_WORD_OFFSET = 64;
size_t dig_gla_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk, int num_cu);
hipError_t dig_launch_gla_f32(const DigGlaArgs &a, hipStream_t s);

struct DigGlaBwdArgs {
  const void *q, *k, *v, *g, *dout;
  int64_t qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, do_sb, do_st, do_sh;
  const float *s0, *ds_final;
  void *dq, *dk_out, *dv_out;
  float *dlog_alpha, *ds0;
  int B, T, H, dk, dv, gh, gw, dir, chunk;
  const int *order;   // nullable: scan position -> canonical token [T]; replaces (gh, gw, dir)
  void *workspace;
  int num_cu;   // compute units of the device (the chunk kernel's persistent grid)
};
hipError_t dig_launch_gla_bwd(const DigGlaBwdArgs &a, hipStream_t s);
size_t dig_gla_bwd_workspace(int B, int T, int H, int dk, int dv, int chunk);
int dig_gla_bwd_chunk(int dk, int dv, int chunk);
size_t dig_gla_f32_lds_bytes(int dk, int dv, int chunk);

hipError_t dig_launch_dwconv(const void *x, int dtype, int B, int T, int C, int64_t x_sb, int64_t x_st,
                             const float *w, int gh, int gw, int dir, void *y, int64_t y_sb,
                             int64_t y_st, int num_cu, hipStream_t s);
// One DiG block forward (block.hip).
struct DigBlockArgs {
  const void *x;          // bf16 [B, T, C] canonical (residual stream in)
  const float *c;         // [B, C] conditioning (timestep + class embedding)
  const void *w_ada;      // bf16 [6C, C]
  const float *b_ada;     // [6C]
  const void *w_in;       // bf16 [4C, C]: q | k | v | gate rows
  const float *b_in;      // [4C]
  const void *w_out;      // bf16 [C, C]
  const float *b_out;     // [C]
  const void *w_ff1;      // bf16 [4C, C]
  const float *b_ff1;     // [4C]
  const void *w_ff2;      // bf16 [C, 4C]
  const float *b_ff2;     // [C]
  const float *w_conv;    // [C, 3, 3]
  void *y;                // bf16 [B, T, C] canonical (block output)
  int B, T, C, H, gh, gw, dir, chunk;
  void *workspace;
  uint32_t epoch;
  int num_cu;
};
size_t dig_block_workspace(int B, int T, int C, int H, int num_cu);
hipError_t dig_launch_block(const DigBlockArgs &a, hipStream_t s);

// Dense product Y[M][N] = alpha X[M][K] W[N][K]^T (+ bias[N]) with an
// epilogue (gemm.hip): bf16 operands, fp32 accumulation, Y bf16 or fp32.
// Needs K and N multiples of 8 and M K, N K below 2^30 (32-bit byte offsets).
enum {
  DIG_EPI_NONE = 0,      // alpha acc (+ bias)
  DIG_EPI_GELU = 1,      // tanh GELU(alpha acc + bias)
  DIG_EPI_GATE = 2,      // alpha acc + bias; columns >= gate_col -> logsigmoid(.) / 16
  DIG_EPI_RESIDUAL = 3,  // Y[r'] = res[r'] + gate[b][gate_off + n] (alpha acc + bias), r' the mapped row
};
struct DigGemmArgs {
  const void *X, *W;
  void *Y;
  bool y_f32;
  int M, N, K;
  int kind;
  float alpha;
  const float *bias;     // nullable, 16-byte aligned
  int gate_col;
  const void *res;       // RESIDUAL: bf16 [M][N], indexed by the mapped row
  const float *gate;     // RESIDUAL: fp32, row b at gate + b gate_stride + gate_off
  int gate_stride, gate_off;
  int rowmap;            // RESIDUAL: 0 identity; 1 X rows in scan order -> Y canonical; 2 canonical -> scan
  int T, dir, gh, gw;    // RESIDUAL: tokens per batch element and the scan order (rowmap != 0)
  int num_cu;
};
hipError_t dig_launch_gemm(const DigGemmArgs &a, hipStream_t s);
hipError_t dig_launch_gather_rows(const void *x, int dtype, int B, int T, int C, const int *index, void *y,
                                  int num_cu, hipStream_t s);
hipError_t dig_launch_remap(const void *x, int dtype, int B, int T, int C, int gh, int gw, int from,
                            int to, void *y, int num_cu, hipStream_t s);
hipError_t dig_launch_adaln(const void *x, int dtype, int64_t N, int C, int64_t x_sn, const float *scale,
                            const float *shift, float eps, float out_scale, void *y, int64_t y_sn,
                            hipStream_t s);
