/*
 * dig_gla.h -- C ABI of the MI355X (gfx950) GLA forward + SREM library
 *              (libdig_gla.so).
 *
 * The library computes the token mixer of a DiG block on one GPU:
 *   gla_fwd       chunk-wise Gated Linear Attention forward, scanned in one
 *                 of four SREM directions, output in scan order + final state;
 *   gla_bwd       its gradients (training);
 *   srem_dwconv   3x3 depthwise conv in the scan frame, stored back to the
 *                 canonical token order (the fused direction remap);
 *   srem_remap    the exact permutation between two scan orders;
 *   dig_adaln_modulate  the adaLN modulation that feeds the mixer.
 *
 * Sources (web pages, cited by title and section):
 *   "DiG: Scalable and Efficient Diffusion Models with Gated Linear
 *   Attention" paper notes (CVPR 2025): 关键设计 / SREM, 关键设计 / DiG
 *   Block设计, 关键设计 / 硬件友好的效率设计;
 *   the diffusers issue #20 of the same title: description bullets and the
 *   draft recurrence (state orientation, gate over key rows, readout q.S);
 *   "Scalable Diffusion Models with Transformers" notes, 3.2 (adaLN);
 *   "ZigMa" paper notes (ECCV 2024), 关键设计 / 异构逐层扫描 (arrange, scan,
 *   arrange back).
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch-owned
 *     device memory) unless stated otherwise.  The caller owns every buffer
 *     and keeps it alive until the work queued on `stream` has finished.
 *   - The library never allocates or frees device memory (gla_fwd_noalloc's
 *     fixed scratch is a static device array of the library), keeps no
 *     global mutable state beyond per-device facts looked up once, and never
 *     synchronises the stream, except gla_fwd_workspace_status, which exists
 *     to do so.  Work is queued on `stream` (NULL = the default stream of the
 *     current device); errors raised by a kernel while it runs surface at the
 *     caller's next synchronisation.
 *   - Strides are in ELEMENTS; the innermost (channel) dimension is contiguous.
 *   - Return value: 0 on success; DIG_EINVAL for invalid arguments (checked
 *     before any HIP call, nothing is queued); DIG_EWORKSPACE when the
 *     workspace is too small; DIG_EHIP when a HIP call or launch fails;
 *     DIG_ENODEV when the current device is not a gfx950.  After a non-zero
 *     return, dig_last_error() describes it.  No C++ exception crosses the ABI.
 *   - Calls on different streams are thread-safe, except that two calls in
 *     flight at the same time must not share a workspace.
 */
#ifndef DIG_GLA_H
#define DIG_GLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DIG_OK 0
#define DIG_EINVAL (-1)
#define DIG_EWORKSPACE (-2)
#define DIG_EHIP (-3)
#define DIG_ENODEV (-4)

/* Element types. */
#define DIG_F32 0
#define DIG_BF16 1

/* Scan directions over a (gh x gw) token grid whose canonical order is
 * row-major, n = r*gw + c.  Scan position p visits canonical index
 *   DIG_L2R: n = p                                  (row-major)
 *   DIG_R2L: n = T-1-p                              (row-major, reversed)
 *   DIG_T2B: n = (p mod gh)*gw + floor(p / gh)      (column-major)
 *   DIG_B2T: the DIG_T2B index of T-1-p             (column-major, reversed)
 * (DiG paper notes, 关键设计 / SREM: four scans made with a transpose of the
 * 2D token matrix and a flip of the sequence, the flip read as a reversal of
 * the whole sequence.)  A DiG stack uses direction i mod 4 in block i. */
#define DIG_L2R 0
#define DIG_R2L 1
#define DIG_T2B 2
#define DIG_B2T 3

/*
 * gla_fwd -- Gated Linear Attention forward over one scan direction.
 *
 * For each batch b and head h, with S = s0[b,h] (or 0) a dk x dv fp32 state,
 * and for scan positions p = 0..T-1 visiting canonical token n (see DIG_*):
 *     S   = diag(exp(log_alpha[b,n,h,:])) * S + k[b,n,h,:]^T v[b,n,h,:]
 *     o[b,p,h,:] = q[b,n,h,:] * S
 * (the diffusers issue #20 recurrence: head_dim x head_dim state, forget
 * gate over the key rows, current token written before the read; no feature
 * map, normaliser or internal 1/sqrt(d)).  It is evaluated chunk-wise as the
 * DiG notes (硬件友好的效率设计) describe: chunks of `chunk` tokens, causal
 * intra-chunk products on bf16 MFMA with fp32 accumulation, the state kept
 * in fp32 and handed from chunk to chunk and from segment to segment.
 *
 * Arguments
 *   q, k, log_alpha  [B, T, H, dk] in CANONICAL token order, strides
 *                    (qk_sb, qk_st, qk_sh) shared by the three tensors.
 *   v                [B, T, H, dv] canonical order, strides (v_sb, v_st, v_sh).
 *   dtype            DIG_BF16: q, k, v, log_alpha and o are bf16, the state
 *                    and all accumulation are fp32 (MFMA path);
 *                    DIG_F32: all fp32, evaluated on the vector ALUs.
 *   B, T, H, dk, dv  sizes; T = gh*gw; 1 <= dk, dv <= 128.  The bf16 path
 *                    needs dk and dv multiples of 8, 16-byte aligned q/k/v/
 *                    log_alpha/o pointers and strides that are multiples of 8
 *                    elements (o: 4), and one (batch, head) slice of q/k/
 *                    log_alpha, v or o must span less than 2 GiB; the fp32
 *                    path takes any layout.
 *   gh, gw, dir      the token grid and the scan direction.
 *   chunk            tokens per chunk: 0 = automatic (bf16: 64, or 32 when
 *                    dk or dv exceeds 96; fp32: 16); else 16, 32, 64 or
 *                    128 (bf16; 64 only for dk, dv <= 96, 128 only for dk,
 *                    dv <= 32, where its LDS plan fits) or 16, 32, 64, 128
 *                    (fp32, as long as its LDS plan -- 4 (3 M dk + M dv +
 *                    M^2 + dk dv) bytes -- fits in 160 KiB, e.g. 128 for
 *                    dk, dv <= 32).  The chunk size changes rounding only,
 *                    never the result.
 *   s0               nullable; [B, H, dk, dv] contiguous fp32 initial state.
 *   o                [B, T, H, dv] written in SCAN order (row p is scan
 *                    position p), strides (o_sb, o_st, o_sh).  Must not
 *                    overlap any input.
 *   s_final          nullable; [B, H, dk, dv] contiguous fp32, the state after
 *                    scan position T-1.  Passing it as s0 of a later call
 *                    continues the scan (state hand-off).
 *   workspace        device memory of at least gla_fwd_workspace_size(...)
 *                    bytes, 256-byte aligned, zero-filled before its first
 *                    use; the library keeps it consistent afterwards, so it
 *                    can be reused by later calls of any size up to the one
 *                    it was sized for, and by replays of a captured graph
 *                    (not by two calls in flight at once).  Its header holds
 *                    cyclic ticket counters (any content gives each piece of
 *                    work to exactly one workgroup) and launch-tagged flags;
 *                    every wait between workgroups is bounded (4 s), and a
 *                    wait that gives up -- possible only on a workspace that
 *                    was not zero-filled or is shared by calls in flight --
 *                    sets an error word that gla_fwd_workspace_status
 *                    reports.  While `stream` is capturing a graph, a small
 *                    fill kernel that clears the flags is queued before the
 *                    GLA kernel.  May be NULL when the size function
 *                    returns 0.
 *   stream           HIP stream to queue on.
 */
int gla_fwd(const void *q, const void *k, const void *v, const void *log_alpha,
            int dtype,
            int64_t qk_sb, int64_t qk_st, int64_t qk_sh,
            int64_t v_sb, int64_t v_st, int64_t v_sh,
            int B, int T, int H, int dk, int dv,
            int gh, int gw, int dir, int chunk,
            const float *s0,
            void *o, int64_t o_sb, int64_t o_st, int64_t o_sh,
            float *s_final,
            void *workspace, size_t workspace_bytes,
            hipStream_t stream);

/*
 * gla_fwd_noalloc -- gla_fwd without a workspace argument, for callers that
 * cannot allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  It allocates nothing: the
 * workspace is a fixed 16 MiB device array inside the library, one per GPU
 * (zero when the library's code is loaded on that GPU, held until the
 * process ends), whose address is looked up on the first call on each
 * device.  Arguments, outputs, constraints and errors as gla_fwd; sizes
 * whose workspace (gla_fwd_workspace_size) exceeds 16 MiB return
 * DIG_EWORKSPACE with nothing queued.  Every call on one GPU shares that
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and give wrong results -- serialise them, or use gla_fwd with a workspace
 * per stream.  The array keeps each call's state; the forward needs nothing
 * of it cleared between calls (cyclic tickets, launch-tagged flags, cleared
 * before the kernel under graph capture).
 */
int gla_fwd_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                    int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh,
                    int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv,
                    int gh, int gw, int dir, int chunk,
                    const float *s0,
                    void *o, int64_t o_sb, int64_t o_st, int64_t o_sh,
                    float *s_final,
                    hipStream_t stream);

/*
 * gla_fwd_ordered -- gla_fwd over a caller-given scan order: any permutation
 * of the T tokens, e.g. ZigMa's zigzag (snake) space-filling scans (ZigMa
 * notes, 关键设计 / Zigzag 扫描方案) or DiG's bidirectional scan (DiG notes,
 * ablation table: a forward and a reversed order).
 *
 *   order   device int32 [T]: order[p] = canonical index of the token scanned
 *           at position p; 4-byte aligned; read on the stream, so it must stay
 *           valid until the call completes.  It should be a permutation of
 *           0..T-1: an entry outside that range reads as a zero token (its
 *           output row is still written); repeated entries are allowed and
 *           simply scan that token again.
 * All other arguments, outputs (o in SCAN order, S_final), constraints,
 * workspace and errors as gla_fwd; (gh, gw, dir) are replaced by `order`.
 * With the table of one of the four grid orders it returns exactly what
 * gla_fwd returns for that direction.
 */
int gla_fwd_ordered(const void *q, const void *k, const void *v, const void *log_alpha,
                    int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh,
                    int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv,
                    const int32_t *order, int chunk,
                    const float *s0,
                    void *o, int64_t o_sb, int64_t o_st, int64_t o_sh,
                    float *s_final,
                    void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace gla_fwd needs for these sizes on the current device
 * (state hand-off records between sequence segments, their flags and a
 * ticket counter).  Returns 0 when no workspace is needed; (size_t)-1 for
 * invalid sizes. */
size_t gla_fwd_workspace_size(int dtype, int B, int T, int H, int dk, int dv, int chunk);

/* gla_fwd_workspace_status -- SYNCHRONISES `stream`, then reads and clears
 * the error word of a gla_fwd / gla_fwd_ordered workspace.  Returns DIG_OK
 * when the word is clear: no call that used the workspace since the last
 * check had a wait between workgroups give up.  Returns DIG_EHIP (with a
 * message) when one did -- that call's o and s_final are wrong -- and also
 * on the first check of a workspace that was not zero-filled before its
 * first use (the word is part of the header; the outputs of such calls are
 * still right unless a wait gave up).  DIG_EINVAL for a NULL or too small
 * workspace.  The only call of the library that waits for the stream; it is
 * meant for tests and for callers that check a workspace. */
int gla_fwd_workspace_status(void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gla_bwd -- gradients of gla_fwd (bf16 path) for training.
 *
 * With L a scalar loss, d_o = dL/do ([B, T, H, dv], SCAN order like o) and
 * ds_final = dL/dS_final, returns dL/dq, dL/dk, dL/dv, dL/dlog_alpha and
 * dL/ds0 of the forward with the same q, k, v, log_alpha, grid, dir and s0.
 * (The DiG paper notes train with this operator, 关键设计 / 硬件友好的效率设计;
 * the gradients are the reverse-mode derivative of the recurrence above:
 * G_p = q_p^T do_p + diag(alpha_{p+1}) G_{p+1}, dq_p = S_p do_p^T,
 * dk_p = G_p v_p^T, dv_p = k_p G_p, dlog_alpha_p = alpha_p * rowsum(G_p .
 * S_{p-1}), ds0 = diag(alpha_0) G_0.)  It runs chunk-wise: a forward and a
 * reverse scan over the chunk boundaries (states and state gradients, kept
 * in the workspace as bf16), then every chunk independently on bf16 MFMA
 * with fp32 accumulation; chunks whose gates are too strong for the
 * factorised exponentials are evaluated with exact exponent differences.
 *
 * Arguments
 *   q, k, log_alpha, v, strides, B, T, H, dk, dv, gh, gw, dir, s0: as gla_fwd;
 *                    dtype must be DIG_BF16 (the only path).
 *   chunk            0 = automatic (64, or 32 when dk or dv exceeds 80); else
 *                    16, 32 or 64 (64 only for dk, dv <= 80).  Rounding only.
 *   d_o              bf16 [B, T, H, dv] in SCAN order, strides (do_sb, do_st,
 *                    do_sh), multiples of 8, 16-byte aligned.
 *   ds_final         nullable (zero); fp32 [B, H, dk, dv] contiguous.
 *   dq, dk_out       bf16 [B, T, H, dk] contiguous, CANONICAL token order.
 *   dv_out           bf16 [B, T, H, dv] contiguous, canonical order.
 *   dlog_alpha       fp32 [B, T, H, dk] contiguous, canonical order.
 *   ds0              nullable; fp32 [B, H, dk, dv] contiguous.
 *   workspace        at least gla_bwd_workspace_size(...) bytes, 256-byte
 *                    aligned (no zero-filling needed); not shared by two
 *                    calls in flight at once.
 * Outputs must not overlap the inputs or each other.  Constraints as for the
 * bf16 gla_fwd.
 */
int gla_bwd(const void *q, const void *k, const void *v, const void *log_alpha,
            int dtype,
            int64_t qk_sb, int64_t qk_st, int64_t qk_sh,
            int64_t v_sb, int64_t v_st, int64_t v_sh,
            int B, int T, int H, int dk, int dv,
            int gh, int gw, int dir, int chunk,
            const float *s0,
            const void *d_o, int64_t do_sb, int64_t do_st, int64_t do_sh,
            const float *ds_final,
            void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *ds0,
            void *workspace, size_t workspace_bytes,
            hipStream_t stream);

/*
 * gla_bwd_ordered -- gla_bwd of gla_fwd_ordered: the same scan order table
 * `order` (device int32 [T], as for gla_fwd_ordered) in place of (gh, gw,
 * dir); d_o in that scan order; gradients in canonical order.  The table
 * must be a permutation for the gradients to be defined: a token listed twice
 * has one of its occurrences' gradients stored (they are not summed), and an
 * entry outside [0, T) is a zero token whose gradients are not written
 * (memory outside the outputs is never touched).  Everything else as gla_bwd.
 */
int gla_bwd_ordered(const void *q, const void *k, const void *v, const void *log_alpha,
                    int dtype,
                    int64_t qk_sb, int64_t qk_st, int64_t qk_sh,
                    int64_t v_sb, int64_t v_st, int64_t v_sh,
                    int B, int T, int H, int dk, int dv,
                    const int32_t *order, int chunk,
                    const float *s0,
                    const void *d_o, int64_t do_sb, int64_t do_st, int64_t do_sh,
                    const float *ds_final,
                    void *dq, void *dk_out, void *dv_out, float *dlog_alpha, float *ds0,
                    void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Bytes of workspace gla_bwd needs for these sizes ((size_t)-1 for invalid
 * sizes or dtypes). */
size_t gla_bwd_workspace_size(int dtype, int B, int T, int H, int dk, int dv, int chunk);

/*
 * srem_dwconv -- SREM 3x3 depthwise conv with the direction remap fused in.
 *
 * x_scan is the mixer output in SCAN order of `dir` ([B, T, C], strides
 * (x_sb, x_st), channels contiguous).  Its sequence is reshaped to the scan
 * frame, (R, Q) = (gh, gw) for L2R/R2L and (gw, gh) for T2B/B2T, X[r][c] =
 * x_scan[r*Q + c]; each channel is cross-correlated with its 3x3 kernel w[ch]
 * (fp32 [C, 3, 3], contiguous) with zero padding and no bias; the result of
 * scan position p = r*Q + c is stored at the CANONICAL index of p in y
 * ([B, T, C], strides (y_sb, y_st)).  (DiG notes, 关键设计 / DiG Block设计
 * steps 4-5 and 关键设计 / SREM; arrange-back of the ZigMa notes.)
 * Accumulation is fp32; y has the dtype of x.  With the identity kernel
 * (centre tap 1) y is exactly the canonical reordering of x.
 * Constraints: C >= 1; bf16 needs C % 8 == 0 and 16-byte aligned pointers and
 * strides; fp32 needs C % 4 == 0 and 16-byte alignment; one batch slice of x
 * ((T-1)*x_st + C elements) must span less than 2 GiB.  y must not overlap x.
 */
int srem_dwconv(const void *x_scan, int dtype, int B, int T, int C,
                int64_t x_sb, int64_t x_st,
                const float *w, int gh, int gw, int dir,
                void *y, int64_t y_sb, int64_t y_st,
                hipStream_t stream);

/*
 * srem_remap -- exact permutation of a [B, T, C] token tensor from scan order
 * `from` to scan order `to` (the transpose/flip of DiG's SREM): the token at
 * canonical index n moves from position inv_from(n) to position inv_to(n).
 * Contiguous [B, T, C] in and out; bitwise copy; element size from dtype.
 * Constraints as for srem_dwconv; y must not overlap x.
 */
int srem_remap(const void *x, int dtype, int B, int T, int C, int gh, int gw,
               int from, int to, void *y, hipStream_t stream);

/*
 * dig_gather_rows -- y[b, p, :] = x[b, index[p], :] for p < T: arranging a
 * token tensor into a scan order (index = the order table) or back to the
 * canonical order (index = its inverse), the arrange / arrange-back steps of
 * ZigMa's scans (ZigMa notes, 关键设计 / 异构逐层扫描).
 * x, y: contiguous [B, T, C], element size from dtype (DIG_BF16 or DIG_F32),
 * 16-byte aligned; C % 8 == 0 (bf16) or C % 4 == 0 (fp32).  index: device
 * int32 [T], 4-byte aligned; an entry outside [0, T) gives a zero row.
 * Bitwise copy.  y must not overlap x.
 */
int dig_gather_rows(const void *x, int dtype, int B, int T, int C,
                    const int32_t *index, void *y, hipStream_t stream);

/*
 * dig_linear -- y = x w^T for row-major bf16 x [M, K], w [N, K] (a PyTorch
 * Linear weight), y [M, N] bf16; fp32 accumulation.  The plain form of the
 * library's bf16 MFMA product that the block's projections use (DiG notes,
 * 关键设计 / DiG Block设计), queued on `stream`.  Needs K and N multiples of 8,
 * 16-byte aligned pointers and M*K, N*K below 2^30 elements.  It needs no
 * workspace: dig_linear_workspace_size() returns 0 and `workspace` may be
 * NULL (the arguments stay for the ABI).  Errors: DIG_EINVAL (null, sizes,
 * alignment, aliasing), DIG_EHIP.
 */
size_t dig_linear_workspace_size(void);
int dig_linear(const void *x, const void *w, void *y, int M, int N, int K,
               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dig_block_fwd -- one DiG block forward (DiG notes, 关键设计 / DiG Block设计:
 * adaLN -> GLA, adaLN -> FFN, the sequence as a 2-D grid through the 3x3
 * depthwise conv, the next block in another direction; adaLN-Zero
 * conditioning as DiT, DiT notes 3.2).  For each batch element b:
 *   [s1|a1|g1|s2|a2|g2] = SiLU(c[b]) w_ada^T + b_ada           (6 vectors of C)
 *   h  = LN(x)(1 + a1) + s1                                     (LN: no affine, eps 1e-6)
 *   [q|k|v|u] = h w_in^T + b_in;  q /= sqrt(C/H);  log_alpha = logsigmoid(u) / 16
 *   o  = gla_fwd over (gh, gw, dir) with H heads of C/H channels (scan order)
 *   x1 = x + g1 (.) canon(o w_out^T + b_out)                    (canon: back to canonical order)
 *   h2 = LN(x1)(1 + a2) + s2
 *   x2 = x1 + g2 (.) (GELU_tanh(h2 w_ff1^T + b_ff1) w_ff2^T + b_ff2)
 *   y  = srem_dwconv(x2 arranged in the scan order of dir, w_conv)  (canonical order)
 *
 *   x, y     bf16 [B, T, C] contiguous, canonical token order; y must not
 *            overlap x or the workspace.
 *   c        fp32 [B, C]: the conditioning (timestep + class embedding).
 *   w_ada    bf16 [6C, C], b_ada fp32 [6C]; w_in bf16 [4C, C] (rows q, k, v,
 *            u), b_in fp32 [4C]; w_out bf16 [C, C], b_out fp32 [C]; w_ff1 bf16
 *            [4C, C], b_ff1 fp32 [4C]; w_ff2 bf16 [C, 4C], b_ff2 fp32 [C];
 *            w_conv fp32 [C, 3, 3].  All contiguous; bf16 ones and b_in,
 *            b_ada, b_in, b_out, b_ff1, b_ff2 16-byte aligned.
 *   C = H * d with d a multiple of 8, at most 128; C <= 16384.
 *   workspace  at least dig_block_workspace_size(B, T, C, H) bytes, 256-byte
 *            aligned, any contents (the call clears the part it needs
 *            cleared), not shared by calls in flight at once.  The products
 *            run on the library's bf16 MFMA GEMM with the biases, the log
 *            gate, GELU and both gated residuals in its epilogues.
 * Errors as gla_fwd.
 */
size_t dig_block_workspace_size(int B, int T, int C, int H);
int dig_block_fwd(const void *x, const float *c,
                  const void *w_ada, const float *b_ada,
                  const void *w_in, const float *b_in,
                  const void *w_out, const float *b_out,
                  const void *w_ff1, const float *b_ff1,
                  const void *w_ff2, const float *b_ff2,
                  const float *w_conv,
                  int B, int T, int C, int H, int gh, int gw, int dir,
                  void *y, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * dig_adaln_modulate -- adaLN modulation of N rows (tokens) of C channels:
 *   y = ((x - mean) / sqrt(var + eps) * (1 + scale) + shift) * out_scale
 * with the population mean and variance of the row, computed in fp32.
 * (DiG notes, 关键设计 / DiG Block设计 step 2: adaLN before the GLA; DiT notes,
 * 3.2: scale/shift regressed from the conditioning, identity at init.)
 * x, y: [N, C] with row strides x_sn, y_sn (elements), same dtype; scale and
 * shift: fp32 [C].  Constraints: C % 8 == 0 (bf16) or C % 4 == 0 (fp32),
 * 16-byte alignment, C <= 16384.  y may equal x (in place) but may not
 * partially overlap it.
 */
int dig_adaln_modulate(const void *x, int dtype, int64_t N, int C, int64_t x_sn,
                       const float *scale, const float *shift, float eps, float out_scale,
                       void *y, int64_t y_sn, hipStream_t stream);

/* Thread-local description of the last non-zero return on this thread. */
const char *dig_last_error(void);

/* Library version string. */
const char *dig_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIG_GLA_H */
