// api.cpp -- the C ABI of libdig_gla.so (declared in include/dig_gla.h):
// argument validation (before any HIP call), device checks, dispatch to the
// kernel launchers, error codes and the thread-local error message.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/dig_gla.h"
#include "dig_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(DIG_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device facts, looked up once per device.
struct DevInfo {
  bool ok = false;
  int num_cu = 0;
};
constexpr int kMaxDev = 64;
DevInfo g_dev[kMaxDev];
std::once_flag g_dev_once[kMaxDev];

int current_device(DevInfo &out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(DIG_ENODEV, "device index %d out of range", dev);
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    g_dev[dev].ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].num_cu = prop.multiProcessorCount;
  });
  out = g_dev[dev];
  if (!out.ok) return fail(DIG_ENODEV, "device %d is not a gfx950 (MI355X) GPU", dev);
  return DIG_OK;
}

std::atomic<uint32_t> g_epoch{1};

// Fixed device scratch of gla_fwd_noalloc: the forward's workspace for callers
// that cannot allocate.  Each device the library runs on holds its own copy
// (zero at load) until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
void *g_scratch_ptr[kMaxDev];
hipError_t g_scratch_err[kMaxDev];
std::once_flag g_scratch_once[kMaxDev];

int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(DIG_ENODEV, "device index %d out of range", dev);
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress(scratch)");
  if (g_scratch_ptr[dev] == nullptr) return fail(DIG_EHIP, "hipGetSymbolAddress(scratch) gave no address");
  *out = g_scratch_ptr[dev];
  return DIG_OK;
}

int auto_chunk(int dtype, int chunk, int dk, int dv) {
  if (chunk != 0) return chunk;
  if (dtype != DIG_BF16) return 16;
  return (dk > 96 || dv > 96) ? 32 : 64;
}

int check_gla_sizes(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
  if (dtype != DIG_F32 && dtype != DIG_BF16) return fail(DIG_EINVAL, "gla_fwd: dtype must be DIG_F32 or DIG_BF16");
  if (B <= 0 || T <= 0 || H <= 0) return fail(DIG_EINVAL, "gla_fwd: B, T, H must be positive");
  if (dk <= 0 || dv <= 0 || dk > 128 || dv > 128)
    return fail(DIG_EINVAL, "gla_fwd: dk and dv must be in [1, 128] (got %d, %d)", dk, dv);
  if ((int64_t)B * H > (int64_t)1 << 30) return fail(DIG_EINVAL, "gla_fwd: B*H too large");
  const int M = auto_chunk(dtype, chunk, dk, dv);
  if (dtype == DIG_BF16) {
    if (dk % 8 || dv % 8) return fail(DIG_EINVAL, "gla_fwd: bf16 path needs dk, dv multiples of 8");
    if (M != 16 && M != 32 && M != 64 && M != 128)
      return fail(DIG_EINVAL, "gla_fwd: bf16 chunk must be 0, 16, 32, 64 or 128");
    if (M == 64 && (dk > 96 || dv > 96))
      return fail(DIG_EINVAL, "gla_fwd: bf16 chunk 64 needs dk, dv <= 96 (use 0, 16 or 32)");
    if (M == 128 && (dk > 32 || dv > 32))
      return fail(DIG_EINVAL, "gla_fwd: bf16 chunk 128 needs dk, dv <= 32 (use 0, 16, 32 or 64)");
  } else {
    if (M != 16 && M != 32 && M != 64 && M != 128)
      return fail(DIG_EINVAL, "gla_fwd: fp32 chunk must be 0, 16, 32, 64 or 128");
  }
  return DIG_OK;
}

}  // namespace

namespace {
int check_bwd_sizes(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
  if (dtype != DIG_BF16) return fail(DIG_EINVAL, "gla_bwd: dtype must be DIG_BF16");
  if (B <= 0 || T <= 0 || H <= 0) return fail(DIG_EINVAL, "gla_bwd: B, T, H must be positive");
  if (dk < 1 || dk > 128 || dv < 1 || dv > 128)
    return fail(DIG_EINVAL, "gla_bwd: dk and dv must be in [1, 128] (got %d, %d)", dk, dv);
  if (dk % 8 || dv % 8) return fail(DIG_EINVAL, "gla_bwd: dk, dv must be multiples of 8");
  if ((int64_t)B * H > (int64_t)1 << 24) return fail(DIG_EINVAL, "gla_bwd: B*H too large");
  const int M = dig_gla_bwd_chunk(dk, dv, chunk);
  if (M != 16 && M != 32 && M != 64) return fail(DIG_EINVAL, "gla_bwd: chunk must be 0, 16, 32 or 64");
  if (M == 64 && (dk > 80 || dv > 80)) return fail(DIG_EINVAL, "gla_bwd: chunk 64 needs dk, dv <= 80");
  const int64_t units_chunks = (int64_t)B * H * ((T + M - 1) / M);
  if (units_chunks >= ((int64_t)1 << 31)) return fail(DIG_EINVAL, "gla_bwd: too many chunks");
  return DIG_OK;
}
}  // namespace

extern "C" {

const char *dig_last_error(void) { return g_err.c_str(); }

const char *dig_version(void) { return "dig_gla 0.1.0 (gfx950)"; }

size_t gla_fwd_workspace_size(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
  if (check_gla_sizes(dtype, B, T, H, dk, dv, chunk) != DIG_OK) return (size_t)-1;
  if (dtype == DIG_F32) return 0;
  DevInfo di;
  const int num_cu = (current_device(di) == DIG_OK) ? di.num_cu : 256;
  return dig_gla_bf16_workspace(B, T, H, dk, dv, auto_chunk(dtype, chunk, dk, dv), num_cu);
}

}  // extern "C"

namespace {
// gla_fwd and gla_fwd_ordered: the scan order is either (gh, gw, dir) or the
// table `order` (non-null).
int gla_fwd_impl(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
                 int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
                 int B, int T, int H, int dk, int dv, int gh, int gw, int dir, const int32_t *order, int chunk,
                 const float *s0, void *o, int64_t o_sb, int64_t o_st, int64_t o_sh, float *s_final,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    int rc = check_gla_sizes(dtype, B, T, H, dk, dv, chunk);
    if (rc) return rc;
    if (!q || !k || !v || !log_alpha || !o) return fail(DIG_EINVAL, "gla_fwd: q, k, v, log_alpha and o are required");
    if (order) {
      if (reinterpret_cast<uintptr_t>(order) & 3u) return fail(DIG_EINVAL, "gla_fwd_ordered: order must be 4-byte aligned");
      gh = 1; gw = T; dir = DIG_L2R;
    }
    if (gh <= 0 || gw <= 0 || (int64_t)gh * gw != T)
      return fail(DIG_EINVAL, "gla_fwd: grid %dx%d does not hold T=%d tokens", gh, gw, T);
    if (dir < DIG_L2R || dir > DIG_B2T) return fail(DIG_EINVAL, "gla_fwd: dir must be 0..3");
    if (qk_sb < 0 || qk_st < 0 || qk_sh < 0 || v_sb < 0 || v_st < 0 || v_sh < 0 || o_sb < 0 || o_st < 0 || o_sh < 0)
      return fail(DIG_EINVAL, "gla_fwd: negative stride");
    if (o == q || o == k || o == v || o == log_alpha) return fail(DIG_EINVAL, "gla_fwd: o aliases an input");
    const int M = auto_chunk(dtype, chunk, dk, dv);
    if (dtype == DIG_BF16) {
      if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(o))
        return fail(DIG_EINVAL, "gla_fwd: bf16 path needs 16-byte aligned q, k, v, log_alpha, o");
      if ((qk_sb | qk_st | qk_sh | v_sb | v_st | v_sh) % 8)
        return fail(DIG_EINVAL, "gla_fwd: bf16 input strides must be multiples of 8 elements");
      if ((o_sb | o_st | o_sh) % 4) return fail(DIG_EINVAL, "gla_fwd: bf16 output strides must be multiples of 4");
      // the kernel addresses one (batch, head) slice with 32-bit byte offsets
      if (((int64_t)(T - 1) * qk_st + dk) * 2 >= ((int64_t)1 << 31) ||
          ((int64_t)(T - 1) * v_st + dv) * 2 >= ((int64_t)1 << 31) ||
          ((int64_t)(T - 1) * o_st + dv) * 2 >= ((int64_t)1 << 31))
        return fail(DIG_EINVAL, "gla_fwd: one (batch, head) slice of q/k/log_alpha, v or o spans 2 GiB or more");
    } else {
      if (dig_gla_f32_lds_bytes(dk, dv, M) > 160 * 1024)
        return fail(DIG_EINVAL, "gla_fwd: fp32 path LDS need exceeds 160 KiB for dk=%d dv=%d chunk=%d", dk, dv, M);
    }
    DevInfo di;
    rc = current_device(di);
    if (rc) return rc;
    const size_t need = dtype == DIG_BF16 ? dig_gla_bf16_workspace(B, T, H, dk, dv, M, di.num_cu) : 0;
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(DIG_EWORKSPACE, "gla_fwd: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return fail(DIG_EINVAL, "gla_fwd: workspace must be 256-byte aligned");

    DigGlaArgs a;
    a.q = q; a.k = k; a.v = v; a.g = log_alpha;
    a.qk_sb = qk_sb; a.qk_st = qk_st; a.qk_sh = qk_sh;
    a.v_sb = v_sb; a.v_st = v_st; a.v_sh = v_sh;
    a.o_sb = o_sb; a.o_st = o_st; a.o_sh = o_sh;
    a.o = o; a.s0 = s0; a.s_final = s_final;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.gh = gh; a.gw = gw; a.dir = dir; a.chunk = M;
    a.order = order;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    // launch tag for the workspace flags: 1 .. 2^29-1 (never 0, the zero-filled state)
    a.epoch = g_epoch.fetch_add(1, std::memory_order_relaxed) % 0x1fffffffu + 1u;
    a.num_cu = di.num_cu;
    const hipError_t e = dtype == DIG_BF16 ? dig_launch_gla_bf16(a, stream) : dig_launch_gla_f32(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gla_fwd launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "gla_fwd: unexpected C++ exception");
  }
}
}  // namespace

extern "C" {

int gla_fwd(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
            int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
            int B, int T, int H, int dk, int dv, int gh, int gw, int dir, int chunk,
            const float *s0, void *o, int64_t o_sb, int64_t o_st, int64_t o_sh, float *s_final,
            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return gla_fwd_impl(q, k, v, log_alpha, dtype, qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, B, T, H, dk, dv, gh, gw,
                      dir, nullptr, chunk, s0, o, o_sb, o_st, o_sh, s_final, workspace, workspace_bytes, stream);
}

int gla_fwd_noalloc(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv, int gh, int gw, int dir, int chunk,
                    const float *s0, void *o, int64_t o_sb, int64_t o_st, int64_t o_sh, float *s_final,
                    hipStream_t stream) {
  try {
    int rc = check_gla_sizes(dtype, B, T, H, dk, dv, chunk);
    if (rc) return rc;
    DevInfo di;
    rc = current_device(di);
    if (rc) return rc;
    const size_t need =
        dtype == DIG_BF16 ? dig_gla_bf16_workspace(B, T, H, dk, dv, auto_chunk(dtype, chunk, dk, dv), di.num_cu) : 0;
    if (need > kScratchBytes)
      return fail(DIG_EWORKSPACE, "gla_fwd_noalloc: these sizes need %zu bytes of scratch, more than its fixed %zu "
                  "(use gla_fwd with a workspace)", need, kScratchBytes);
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return gla_fwd_impl(q, k, v, log_alpha, dtype, qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, B, T, H, dk, dv, gh, gw,
                        dir, nullptr, chunk, s0, o, o_sb, o_st, o_sh, s_final, ws, kScratchBytes, stream);
  } catch (...) {
    return fail(DIG_EHIP, "gla_fwd_noalloc: unexpected C++ exception");
  }
}

int gla_fwd_ordered(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv, const int32_t *order, int chunk,
                    const float *s0, void *o, int64_t o_sb, int64_t o_st, int64_t o_sh, float *s_final,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!order) return fail(DIG_EINVAL, "gla_fwd_ordered: order is required");
  return gla_fwd_impl(q, k, v, log_alpha, dtype, qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, B, T, H, dk, dv, 1, T,
                      DIG_L2R, order, chunk, s0, o, o_sb, o_st, o_sh, s_final, workspace, workspace_bytes, stream);
}


int gla_fwd_workspace_status(void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (!workspace || workspace_bytes < DIG_GLA_ERR_WORD_OFFSET + 4)
      return fail(DIG_EINVAL, "gla_fwd_workspace_status: a gla_fwd workspace is required");
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "gla_fwd_workspace_status: hipStreamSynchronize");
    unsigned word = 0;
    char *p = static_cast<char *>(workspace) + DIG_GLA_ERR_WORD_OFFSET;
    e = hipMemcpy(&word, p, sizeof(word), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "gla_fwd_workspace_status: hipMemcpy");
    if (word == 0) return DIG_OK;
    const unsigned zero = 0;
    e = hipMemcpy(p, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "gla_fwd_workspace_status: hipMemcpy");
    return fail(DIG_EHIP, "gla_fwd: a wait between workgroups gave up (error word 0x%x): a call that used this "
                "workspace returned wrong results (workspace not zero-filled before its first use, or shared "
                "by calls in flight at the same time)", word);
  } catch (...) {
    return fail(DIG_EHIP, "gla_fwd_workspace_status: unexpected C++ exception");
  }
}

size_t gla_bwd_workspace_size(int dtype, int B, int T, int H, int dk, int dv, int chunk) {
  if (check_bwd_sizes(dtype, B, T, H, dk, dv, chunk) != DIG_OK) return (size_t)-1;
  return dig_gla_bwd_workspace(B, T, H, dk, dv, chunk);
}

}  // extern "C"

namespace {
int gla_bwd_impl(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
                 int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
                 int B, int T, int H, int dk, int dv, int gh, int gw, int dir, const int32_t *order, int chunk,
                 const float *s0, const void *d_o, int64_t do_sb, int64_t do_st, int64_t do_sh,
                 const float *ds_final, void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *ds0,
                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    int rc = check_bwd_sizes(dtype, B, T, H, dk, dv, chunk);
    if (rc) return rc;
    if (!q || !k || !v || !log_alpha || !d_o || !dq || !dk_out || !dv_out || !dlog_alpha)
      return fail(DIG_EINVAL, "gla_bwd: q, k, v, log_alpha, d_o, dq, dk, dv and dlog_alpha are required");
    if (order) {
      if (reinterpret_cast<uintptr_t>(order) & 3u) return fail(DIG_EINVAL, "gla_bwd_ordered: order must be 4-byte aligned");
      gh = 1; gw = T; dir = DIG_L2R;
    }
    if (gh <= 0 || gw <= 0 || (int64_t)gh * gw != T)
      return fail(DIG_EINVAL, "gla_bwd: grid %dx%d does not hold T=%d tokens", gh, gw, T);
    if (dir < DIG_L2R || dir > DIG_B2T) return fail(DIG_EINVAL, "gla_bwd: dir must be 0..3");
    if (qk_sb < 0 || qk_st < 0 || qk_sh < 0 || v_sb < 0 || v_st < 0 || v_sh < 0 || do_sb < 0 || do_st < 0 ||
        do_sh < 0)
      return fail(DIG_EINVAL, "gla_bwd: negative stride");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(log_alpha) || !aligned16(d_o))
      return fail(DIG_EINVAL, "gla_bwd: q, k, v, log_alpha, d_o must be 16-byte aligned");
    if ((qk_sb | qk_st | qk_sh | v_sb | v_st | v_sh | do_sb | do_st | do_sh) % 8)
      return fail(DIG_EINVAL, "gla_bwd: input strides must be multiples of 8 elements");
    if (((int64_t)(T - 1) * qk_st + dk) * 2 >= ((int64_t)1 << 31) ||
        ((int64_t)(T - 1) * v_st + dv) * 2 >= ((int64_t)1 << 31) ||
        ((int64_t)(T - 1) * do_st + dv) * 2 >= ((int64_t)1 << 31))
      return fail(DIG_EINVAL, "gla_bwd: one (batch, head) slice of an input spans 2 GiB or more");
    if ((int64_t)T * H * dk * 4 >= ((int64_t)1 << 31) || (int64_t)T * H * dv * 2 >= ((int64_t)1 << 31))
      return fail(DIG_EINVAL, "gla_bwd: one batch of an output spans 2 GiB or more");
    const void *outs[5] = {dq, dk_out, dv_out, dlog_alpha, ds0};
    const void *ins[5] = {q, k, v, log_alpha, d_o};
    for (const void *o : outs)
      for (const void *i : ins)
        if (o && o == i) return fail(DIG_EINVAL, "gla_bwd: an output aliases an input");
    DevInfo di;
    rc = current_device(di);
    if (rc) return rc;
    const size_t need = dig_gla_bwd_workspace(B, T, H, dk, dv, chunk);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(DIG_EWORKSPACE, "gla_bwd: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(DIG_EINVAL, "gla_bwd: workspace must be 256-byte aligned");
    DigGlaBwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = log_alpha; a.dout = d_o;
    a.qk_sb = qk_sb; a.qk_st = qk_st; a.qk_sh = qk_sh;
    a.v_sb = v_sb; a.v_st = v_st; a.v_sh = v_sh;
    a.do_sb = do_sb; a.do_st = do_st; a.do_sh = do_sh;
    a.s0 = s0; a.ds_final = ds_final;
    a.dq = dq; a.dk_out = dk_out; a.dv_out = dv_out; a.dlog_alpha = dlog_alpha; a.ds0 = ds0;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.gh = gh; a.gw = gw; a.dir = dir; a.chunk = chunk;
    a.order = order;
    a.workspace = workspace;
    a.num_cu = di.num_cu;
    const hipError_t e = dig_launch_gla_bwd(a, stream);
    if (e != hipSuccess) return hip_fail(e, "gla_bwd launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "gla_bwd: unexpected C++ exception");
  }
}
}  // namespace

extern "C" {

int gla_bwd(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
            int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
            int B, int T, int H, int dk, int dv, int gh, int gw, int dir, int chunk,
            const float *s0, const void *d_o, int64_t do_sb, int64_t do_st, int64_t do_sh,
            const float *ds_final, void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *ds0,
            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return gla_bwd_impl(q, k, v, log_alpha, dtype, qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, B, T, H, dk, dv, gh, gw,
                      dir, nullptr, chunk, s0, d_o, do_sb, do_st, do_sh, ds_final, dq, dk_out, dv_out, dlog_alpha,
                      ds0, workspace, workspace_bytes, stream);
}

int gla_bwd_ordered(const void *q, const void *k, const void *v, const void *log_alpha, int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh, int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv, const int32_t *order, int chunk,
                    const float *s0, const void *d_o, int64_t do_sb, int64_t do_st, int64_t do_sh,
                    const float *ds_final, void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *ds0,
                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!order) return fail(DIG_EINVAL, "gla_bwd_ordered: order is required");
  return gla_bwd_impl(q, k, v, log_alpha, dtype, qk_sb, qk_st, qk_sh, v_sb, v_st, v_sh, B, T, H, dk, dv, 1, T,
                      DIG_L2R, order, chunk, s0, d_o, do_sb, do_st, do_sh, ds_final, dq, dk_out, dv_out,
                      dlog_alpha, ds0, workspace, workspace_bytes, stream);
}

int srem_dwconv(const void *x_scan, int dtype, int B, int T, int C, int64_t x_sb, int64_t x_st,
                const float *w, int gh, int gw, int dir, void *y, int64_t y_sb, int64_t y_st,
                hipStream_t stream) {
  try {
    if (dtype != DIG_F32 && dtype != DIG_BF16) return fail(DIG_EINVAL, "srem_dwconv: bad dtype");
    if (!x_scan || !w || !y) return fail(DIG_EINVAL, "srem_dwconv: x_scan, w and y are required");
    if (B <= 0 || T <= 0 || C <= 0) return fail(DIG_EINVAL, "srem_dwconv: B, T, C must be positive");
    if (gh <= 0 || gw <= 0 || (int64_t)gh * gw != T)
      return fail(DIG_EINVAL, "srem_dwconv: grid %dx%d does not hold T=%d tokens", gh, gw, T);
    if (dir < DIG_L2R || dir > DIG_B2T) return fail(DIG_EINVAL, "srem_dwconv: dir must be 0..3");
    const int vec = dtype == DIG_BF16 ? 8 : 4;
    if (C % vec) return fail(DIG_EINVAL, "srem_dwconv: C must be a multiple of %d", vec);
    if (!aligned16(x_scan) || !aligned16(y)) return fail(DIG_EINVAL, "srem_dwconv: x and y must be 16-byte aligned");
    if ((x_sb | x_st | y_sb | y_st) % vec || x_sb < 0 || x_st < C || y_sb < 0 || y_st < C)
      return fail(DIG_EINVAL, "srem_dwconv: strides must be multiples of %d and token strides >= C", vec);
    if (x_scan == y) return fail(DIG_EINVAL, "srem_dwconv: in-place is not allowed");
    // the kernel addresses one batch slice of x with 32-bit byte offsets
    if (((int64_t)(T - 1) * x_st + C) * (dtype == DIG_BF16 ? 2 : 4) >= ((int64_t)1 << 31))
      return fail(DIG_EINVAL, "srem_dwconv: one batch slice of x spans 2 GiB or more");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    const hipError_t e = dig_launch_dwconv(x_scan, dtype, B, T, C, x_sb, x_st, w, gh, gw, dir, y, y_sb, y_st,
                                           di.num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "srem_dwconv launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "srem_dwconv: unexpected C++ exception");
  }
}

int srem_remap(const void *x, int dtype, int B, int T, int C, int gh, int gw, int from, int to, void *y,
               hipStream_t stream) {
  try {
    if (dtype != DIG_F32 && dtype != DIG_BF16) return fail(DIG_EINVAL, "srem_remap: bad dtype");
    if (!x || !y) return fail(DIG_EINVAL, "srem_remap: x and y are required");
    if (B <= 0 || T <= 0 || C <= 0) return fail(DIG_EINVAL, "srem_remap: B, T, C must be positive");
    if (gh <= 0 || gw <= 0 || (int64_t)gh * gw != T)
      return fail(DIG_EINVAL, "srem_remap: grid %dx%d does not hold T=%d tokens", gh, gw, T);
    if (from < DIG_L2R || from > DIG_B2T || to < DIG_L2R || to > DIG_B2T)
      return fail(DIG_EINVAL, "srem_remap: directions must be 0..3");
    const int vec = dtype == DIG_BF16 ? 8 : 4;
    if (C % vec) return fail(DIG_EINVAL, "srem_remap: C must be a multiple of %d", vec);
    if (!aligned16(x) || !aligned16(y)) return fail(DIG_EINVAL, "srem_remap: x and y must be 16-byte aligned");
    if (x == y) return fail(DIG_EINVAL, "srem_remap: in-place is not allowed");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    const hipError_t e = dig_launch_remap(x, dtype, B, T, C, gh, gw, from, to, y, di.num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "srem_remap launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "srem_remap: unexpected C++ exception");
  }
}

int dig_gather_rows(const void *x, int dtype, int B, int T, int C, const int32_t *index, void *y,
                    hipStream_t stream) {
  try {
    if (dtype != DIG_F32 && dtype != DIG_BF16) return fail(DIG_EINVAL, "dig_gather_rows: bad dtype");
    if (!x || !y || !index) return fail(DIG_EINVAL, "dig_gather_rows: x, index and y are required");
    if (B <= 0 || T <= 0 || C <= 0) return fail(DIG_EINVAL, "dig_gather_rows: B, T, C must be positive");
    const int vec = dtype == DIG_BF16 ? 8 : 4;
    if (C % vec) return fail(DIG_EINVAL, "dig_gather_rows: C must be a multiple of %d", vec);
    if (!aligned16(x) || !aligned16(y)) return fail(DIG_EINVAL, "dig_gather_rows: x and y must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(index) & 3u) return fail(DIG_EINVAL, "dig_gather_rows: index must be 4-byte aligned");
    if (x == y) return fail(DIG_EINVAL, "dig_gather_rows: in-place is not allowed");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    const hipError_t e = dig_launch_gather_rows(x, dtype, B, T, C, index, y, di.num_cu, stream);
    if (e != hipSuccess) return hip_fail(e, "dig_gather_rows launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "dig_gather_rows: unexpected C++ exception");
  }
}

size_t dig_linear_workspace_size(void) { return 0; }

int dig_linear(const void *x, const void *w, void *y, int M, int N, int K, void *workspace, size_t workspace_bytes,
               hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  try {
    if (!x || !w || !y) return fail(DIG_EINVAL, "dig_linear: x, w and y are required");
    if (M <= 0 || N <= 0 || K <= 0) return fail(DIG_EINVAL, "dig_linear: M, N, K must be positive");
    if (K % 8 || N % 8) return fail(DIG_EINVAL, "dig_linear: K and N must be multiples of 8");
    if ((int64_t)M * K >= ((int64_t)1 << 30) || (int64_t)N * K >= ((int64_t)1 << 30))
      return fail(DIG_EINVAL, "dig_linear: M*K and N*K must stay below 2^30 elements");
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return fail(DIG_EINVAL, "dig_linear: 16-byte alignment needed");
    if (y == x || y == w) return fail(DIG_EINVAL, "dig_linear: y aliases an input");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    DigGemmArgs g{};
    g.X = x; g.W = w; g.Y = y; g.y_f32 = false; g.M = M; g.N = N; g.K = K; g.kind = DIG_EPI_NONE; g.alpha = 1.0f;
    g.num_cu = di.num_cu;
    const hipError_t e = dig_launch_gemm(g, stream);
    if (e != hipSuccess) return hip_fail(e, "dig_linear");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "dig_linear: unexpected C++ exception");
  }
}

size_t dig_block_workspace_size(int B, int T, int C, int H) {
  if (B <= 0 || T <= 0 || C <= 0 || H <= 0 || C % H || C % 8) return (size_t)-1;
  DevInfo di;
  const int num_cu = (current_device(di) == DIG_OK) ? di.num_cu : 256;
  return dig_block_workspace(B, T, C, H, num_cu);
}

int dig_block_fwd(const void *x, const float *c, const void *w_ada, const float *b_ada, const void *w_in,
                  const float *b_in, const void *w_out, const float *b_out, const void *w_ff1, const float *b_ff1,
                  const void *w_ff2, const float *b_ff2, const float *w_conv, int B, int T, int C, int H, int gh,
                  int gw, int dir, void *y, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (!x || !c || !w_ada || !b_ada || !w_in || !b_in || !w_out || !b_out || !w_ff1 || !b_ff1 || !w_ff2 || !b_ff2 ||
        !w_conv || !y)
      return fail(DIG_EINVAL, "dig_block_fwd: every input, weight and y is required");
    if (B <= 0 || T <= 0 || C <= 0 || H <= 0 || C % H) return fail(DIG_EINVAL, "dig_block_fwd: bad B, T, C, H");
    const int d = C / H;
    if (d % 8 || d > 128) return fail(DIG_EINVAL, "dig_block_fwd: head dim C/H must be a multiple of 8, at most 128");
    if (C > 16384) return fail(DIG_EINVAL, "dig_block_fwd: C must be at most 16384");
    if ((int64_t)B * T * 4 * C >= ((int64_t)1 << 31) / 2)
      return fail(DIG_EINVAL, "dig_block_fwd: B*T*4C too large for one product");
    if (gh <= 0 || gw <= 0 || (int64_t)gh * gw != T)
      return fail(DIG_EINVAL, "dig_block_fwd: grid %dx%d does not hold T=%d tokens", gh, gw, T);
    if (dir < DIG_L2R || dir > DIG_B2T) return fail(DIG_EINVAL, "dig_block_fwd: dir must be 0..3");
    const void *al[] = {x, w_ada, w_in, w_out, w_ff1, w_ff2, y, b_ada, b_in, b_out, b_ff1, b_ff2};
    for (const void *p : al)
      if (!aligned16(p))
        return fail(DIG_EINVAL, "dig_block_fwd: bf16 tensors and the fp32 biases b_ada, b_in, b_out, b_ff1, b_ff2 "
                                "must be 16-byte aligned");
    if (y == x) return fail(DIG_EINVAL, "dig_block_fwd: y aliases x");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    const size_t need = dig_block_workspace(B, T, C, H, di.num_cu);
    if (!workspace || workspace_bytes < need)
      return fail(DIG_EWORKSPACE, "dig_block_fwd: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(DIG_EINVAL, "dig_block_fwd: workspace must be 256-byte aligned");
    DigBlockArgs a;
    a.x = x; a.c = c; a.w_ada = w_ada; a.b_ada = b_ada; a.w_in = w_in; a.b_in = b_in; a.w_out = w_out;
    a.b_out = b_out; a.w_ff1 = w_ff1; a.b_ff1 = b_ff1; a.w_ff2 = w_ff2; a.b_ff2 = b_ff2; a.w_conv = w_conv;
    a.y = y; a.B = B; a.T = T; a.C = C; a.H = H; a.gh = gh; a.gw = gw; a.dir = dir; a.chunk = 0;
    a.workspace = workspace;
    a.epoch = g_epoch.fetch_add(1, std::memory_order_relaxed) % 0x1fffffffu + 1u;
    a.num_cu = di.num_cu;
    const hipError_t e = dig_launch_block(a, stream);
    if (e != hipSuccess) return hip_fail(e, "dig_block_fwd");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "dig_block_fwd: unexpected C++ exception");
  }
}

int dig_adaln_modulate(const void *x, int dtype, int64_t N, int C, int64_t x_sn, const float *scale,
                       const float *shift, float eps, float out_scale, void *y, int64_t y_sn,
                       hipStream_t stream) {
  try {
    if (dtype != DIG_F32 && dtype != DIG_BF16) return fail(DIG_EINVAL, "dig_adaln_modulate: bad dtype");
    if (!x || !scale || !shift || !y) return fail(DIG_EINVAL, "dig_adaln_modulate: x, scale, shift, y are required");
    const int vec = dtype == DIG_BF16 ? 8 : 4;
    if (N <= 0 || C <= 0 || C % vec || C / vec > 2048)
      return fail(DIG_EINVAL, "dig_adaln_modulate: need N > 0 and C a multiple of %d with C/%d <= 2048", vec, vec);
    if (!aligned16(x) || !aligned16(y)) return fail(DIG_EINVAL, "dig_adaln_modulate: x and y must be 16-byte aligned");
    if (x_sn < C || y_sn < C || x_sn % vec || y_sn % vec)
      return fail(DIG_EINVAL, "dig_adaln_modulate: row strides must be >= C and multiples of %d", vec);
    if (!(eps >= 0.f)) return fail(DIG_EINVAL, "dig_adaln_modulate: eps must be >= 0");
    DevInfo di;
    int rc = current_device(di);
    if (rc) return rc;
    const hipError_t e = dig_launch_adaln(x, dtype, N, C, x_sn, scale, shift, eps, out_scale, y, y_sn, stream);
    if (e != hipSuccess) return hip_fail(e, "dig_adaln_modulate launch");
    return DIG_OK;
  } catch (...) {
    return fail(DIG_EHIP, "dig_adaln_modulate: unexpected C++ exception");
  }
}

}  // extern "C"
