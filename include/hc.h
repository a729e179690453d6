/*
 * hc.h - C ABI of the MI355X (gfx950) hyper-connection sublayer library (libhc.so).
 *
 * The library computes one forward hyper-connection sublayer per token:
 * mHC's Sinkhorn-constrained n-stream residual mixing and xHC's routed,
 * augmented extension. Sources of the definitions:
 *   [mHC]   "mHC: Manifold-Constrained Hyper-Connections" (paper notes),
 *           Eq. 3, Eq. 6, section 4.2 (Eq. 7-9), section 4.3.1 (Eq. 10-19 and
 *           the F_pre / F_post,res kernels).
 *   [xHC]   "xHC: Expanded Hyper-Connections" (paper summary), Method: temporal
 *           feature augmentation; sparse residual stream architecture, steps
 *           1-3; parameterisation and practical deployment.
 *   [xHC-R] xHC repository README, default xHC configuration table.
 *
 * Conventions shared by every call:
 *   - All tensor arguments are DEVICE pointers to caller-owned, C-contiguous,
 *     row-major buffers. Scalars and the kappa array of xhc_augment are host
 *     values. The library never allocates, frees or synchronises; every call
 *     only enqueues kernels on `stream` (a hipStream_t; NULL = default stream)
 *     and returns. Buffers must stay alive until that work completes.
 *   - Stream tensors (X, F_out, F_in, Wb, V) have dtype HC_F32 or HC_BF16;
 *     coefficient tensors, phi, biases and conv weights are always float32.
 *     Accumulation is float32; every stored stream value is rounded once
 *     (round-to-nearest-even for bfloat16).
 *   - Token state X is [T, n, C] (stream-major within a token); the flattened
 *     state vec(x) of a token is its contiguous n*C slice (index i*C + c).
 *   - Return value: HC_OK (0) or a negative status. Argument errors are found
 *     on the host before any HIP call; the outputs are then untouched.
 *     HC_ERR_DEVICE means no usable GPU; HC_ERR_LAUNCH means a kernel launch
 *     failed (outputs undefined). No call prints, aborts or throws.
 *   - T == 0 (or B*S == 0) is valid and does nothing; pointers may then be NULL.
 *   - Outputs must not overlap inputs, except where a call says otherwise.
 *   - Calls keep no global mutable state and are safe to issue from several
 *     host threads; calls that share output or workspace buffers must be
 *     ordered by the caller (same stream or events).
 *   - Workspaces: calls that take `workspace` need at least the bytes returned
 *     by the matching *_workspace_bytes query (device memory, 256-byte
 *     aligned, contents need not be initialised, reused freely between calls
 *     on one stream).
 */
#ifndef HC_H_
#define HC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HC_F32 0
#define HC_BF16 1

#define HC_OK 0
#define HC_ERR_NULL (-1)      /* a required pointer is NULL */
#define HC_ERR_SHAPE (-2)     /* a size or count is out of range */
#define HC_ERR_DTYPE (-3)     /* unknown dtype code */
#define HC_ERR_ALIGN (-4)     /* a pointer is not aligned to its element size */
#define HC_ERR_ALIAS (-5)     /* an output overlaps an input it must not */
#define HC_ERR_DEVICE (-6)    /* no usable HIP device */
#define HC_ERR_LAUNCH (-7)    /* a kernel launch failed */
#define HC_ERR_WORKSPACE (-8) /* workspace missing, misaligned or too small */
#define HC_ERR_SCRATCH (-9)   /* the sizes need more than the library's fixed scratch */

/* Limits checked by every call. */
#define HC_MAX_STREAMS 64     /* n (mHC) and N (xHC) */
#define HC_MAX_MHC_STREAMS 16 /* n for the mHC calls */
#define HC_MAX_ACTIVE 16      /* k (xHC) */
#define HC_MAX_COMPONENTS 8   /* K = r + 1 write-back components */
#define HC_MAX_KAPPA 32       /* causal conv kernel size */
#define HC_MAX_ITERS 10000    /* Sinkhorn iterations */
#define HC_MAX_BWD_ITERS 64   /* Sinkhorn iterations of hc_backward (iterates kept on chip) */
#define HC_MAX_FLASH_SUBLAYERS 4 /* L, sublayers of an xHC-Flash block */

/* Human-readable text of a status code (static string, never NULL). */
const char* hc_status_string(int status);

/* ABI version (major*100 + minor). */
int hc_version(void);

/* ------------------------------------------------------------------ mHC -- */

/* Workspace bytes needed by hc_coeffs / hc_coeffs_pre for these sizes. */
int64_t hc_coeffs_workspace_bytes(int64_t T, int n, int64_t C, int dtype);

/*
 * hc_coeffs - mHC coefficients of every token ([mHC] Eq. 7-9 and 14-19).
 *   X      [T, n, C] stream dtype.       1 <= n <= 16, C >= 1.
 *   phi    [n*C, n*n + 2n] float32, columns [pre n | post n | res n*n], the
 *          RMSNorm gain folded in (Eq. 10, 14). Row i*C + c multiplies x[i, c].
 *   bias   [n*n + 2n] float32, same column order (Eq. 13).
 *   alpha_pre, alpha_post, alpha_res: the three gates (Eq. 12).
 *   sinkhorn_iters >= 1: fixed iteration count (t_max; 20 on the pages).
 * Per token: r = ||vec x||_2 / sqrt(nC) (Eq. 15; r = 0 gives a zero
 * normalised state), z = alpha_block * (vec x @ phi) / r + bias (Eq. 16),
 * h_pre = sigmoid(z_pre), h_post = 2 sigmoid(z_post), h_res = Sinkhorn-Knopp
 * of exp(mat(z_res)) with columns then rows normalised per iteration (Eq. 9),
 * mat row-major: h_res[i][j] = z_res[i*n + j].
 * Outputs (float32): h_pre [T, n], h_post [T, n], h_res [T, n, n].
 */
int hc_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C,
              const float* phi, const float* bias,
              float alpha_pre, float alpha_post, float alpha_res, int sinkhorn_iters,
              float* h_pre, float* h_post, float* h_res,
              void* workspace, int64_t workspace_bytes, void* stream);

/*
 * hc_pre - dense pre-read F_pre = H_pre x ([mHC] 4.3.1):
 *   F_in[t, c] = sum_i h_pre[t, i] * X[t, i, c].
 *   X [T, n, C] and F_in [T, C] in the stream dtype; h_pre [T, n] float32.
 */
int hc_pre(const void* X, int dtype, int64_t T, int n, int64_t C,
           const float* h_pre, void* F_in, void* stream);

/*
 * hc_coeffs_pre - hc_coeffs followed by hc_pre, fused so that the state is
 * read from HBM once where the shape allows it. Same arguments as hc_coeffs
 * plus F_in [T, C] (stream dtype). h_pre may be NULL (then not stored).
 */
int hc_coeffs_pre(const void* X, int dtype, int64_t T, int n, int64_t C,
                  const float* phi, const float* bias,
                  float alpha_pre, float alpha_post, float alpha_res, int sinkhorn_iters,
                  float* h_pre, float* h_post, float* h_res, void* F_in,
                  void* workspace, int64_t workspace_bytes, void* stream);

/*
 * hc_backward_post, hc_backward - gradients of one mHC sublayer ([mHC] 4.3.1
 * Kernel Fusion: the backward of the Eq. 14-15 projection, two products over
 * the same x, and a Sinkhorn-Knopp backward that recomputes the iterates on
 * chip; 4.3 recomputes the forward's intermediates from x in the backward).
 *   Forward (hc_coeffs, hc_pre, hc_post with the same arguments):
 *     F_in = H_pre x,  X_next = H_res x + H_post^T F_out.
 *   Two stages, in the order a training step meets them:
 *   hc_backward_post (before the sublayer function's backward, which needs
 *     dF_out): from X [T, 4, C], F_out [T, C], dX_next [T, 4, C] (the upstream
 *     gradient of X_next) and the forward's h_post [T, 4] float32:
 *       dF_out [T, C]                = H_post dX_next (bfloat16, rounded once),
 *       dh[:, 4:8]  = dH_post[i]     = <dX_next_i, F_out>,
 *       dh[:, 8:24] = dH_res[i, j]   = <dX_next_i, x_j>  (index 8 + 4i + j).
 *   hc_backward (once dF_in [T, C], the gradient of F_in, is known): fills
 *     dh[:, 0:4] = dH_pre[i] = <dF_in, x_i>, reads dh[:, 4:24] as left by
 *     hc_backward_post, and writes
 *       dX [T, 4, C] (bfloat16, rounded once), dphi [4C, 24], dbias [24] (column
 *       order of phi), dalpha [3] (pre, post, res) float32, the last three
 *       summed over the T tokens.
 *     phi, bias, alpha_*, sinkhorn_iters as for hc_coeffs; the maps are
 *     recomputed from X. dh [T, 24] float32 is the gradient of the maps
 *     [H_pre | H_post | H_res] per token.
 *   Covered: dtype HC_BF16 (HC_F32 -> HC_ERR_DTYPE), n = 4, C a multiple of 32,
 *   1 <= sinkhorn_iters <= HC_MAX_BWD_ITERS (else HC_ERR_SHAPE). The all-zero
 *   state takes 1/r = 0 (as the forward) and passes no gradient through r.
 *   Alignment: the bfloat16 arrays and h_post 16 bytes, the other float arrays
 *   4 bytes, workspace 256 bytes and at least hc_backward_workspace_bytes (the
 *   packed phi, projection partials, recomputed maps, dP and the partial sums
 *   of dphi). No output may overlap an input, another output or the workspace
 *   (HC_ERR_ALIAS). Deterministic: every sum runs in a fixed order.
 *   hc_backward_workspace_bytes: 0 for T = 0, -1 for sizes or a dtype that
 *   hc_backward does not cover.
 */
int64_t hc_backward_workspace_bytes(int64_t T, int n, int64_t C, int dtype);
int hc_backward_post(const void* X, int dtype, int64_t T, int n, int64_t C,
                     const float* h_post, const void* F_out, const void* dX_next,
                     void* dF_out, float* dh, void* stream);
int hc_backward(const void* X, int dtype, int64_t T, int n, int64_t C,
                const float* phi, const float* bias,
                float alpha_pre, float alpha_post, float alpha_res, int sinkhorn_iters,
                const void* dX_next, const void* dF_in, float* dh,
                void* dX, float* dphi, float* dbias, float* dalpha,
                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * hc_post - fused post/res write F_post,res = H_res x + H_post^T F ([mHC] Eq. 3,
 * 4.3.1), reading (n+1)C and writing nC elements per token:
 *   X_next[t, i, c] = sum_j h_res[t, i, j] X[t, j, c] + h_post[t, i] F_out[t, c].
 *   X, X_next [T, n, C] and F_out [T, C] in the stream dtype; h_res [T, n, n]
 *   and h_post [T, n] float32. X_next may equal X (in place); any other
 *   overlap with an input is HC_ERR_ALIAS.
 */
int hc_post(const void* X, int dtype, int64_t T, int n, int64_t C,
            const float* h_res, const float* h_post, const void* F_out, void* X_next,
            void* stream);

/*
 * hc_post_coeffs - hc_post followed by hc_coeffs on the state it writes, in one
 * pass: the post/res write of sublayer l ([mHC] Eq. 3, 4.3.1) and the
 * coefficients of sublayer l+1 ([mHC] Eq. 7-9, 14-19) computed from X_next
 * while it is produced (so a chain of sublayers reads each state twice: once
 * in the pre-read, once here).
 *   X, h_res, h_post, F_out, X_next: as hc_post (X_next may equal X).
 *   phi_next, bias_next, alpha_*, sinkhorn_iters: sublayer l+1's parameters,
 *   as hc_coeffs. Outputs h_pre_next, h_post_next [T, n], h_res_next [T, n, n]
 *   (float32; all required) are the coefficients of X_next.
 *   Workspace: hc_coeffs_workspace_bytes(T, n, C, dtype).
 */
int hc_post_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C,
                   const float* h_res, const float* h_post, const void* F_out, void* X_next,
                   const float* phi_next, const float* bias_next,
                   float alpha_pre, float alpha_post, float alpha_res, int sinkhorn_iters,
                   float* h_pre_next, float* h_post_next, float* h_res_next,
                   void* workspace, int64_t workspace_bytes, void* stream);

/*
 * hc_phi_packed_bytes - bytes of phi in the packed form the fast path of the
 * coefficient calls multiplies with (n = 4, bfloat16 streams, C % 32 == 0);
 * 0 when that form does not exist for (n, C, dtype); -1 for invalid sizes.
 */
int64_t hc_phi_packed_bytes(int n, int64_t C, int dtype);

/*
 * hc_phi_pack - phi [n*C, n*n+2n] float32 -> its packed form in `packed`
 * (256-byte aligned, at least hc_phi_packed_bytes): per group of 8 rows, 48
 * columns of 8 bfloat16: columns 0..23 hold hi = bf16(phi) (round to nearest
 * even), columns 24..47 hold lo = bf16(phi - hi), so hi + lo carries about 16
 * significant bits of phi ([mHC] Eq. 10 runs this product in tf32; see the
 * notes in the source). A weight that is used many times is packed once. When
 * no packed form exists the call does nothing and returns HC_OK.
 */
int hc_phi_pack(const float* phi, int n, int64_t C, int dtype, void* packed, int64_t packed_bytes,
                void* stream);

/*
 * hc_post_pre - the whole step between sublayer l's function and sublayer
 * l+1's: hc_post_coeffs (the post/res write of sublayer l, [mHC] Eq. 3, 4.3.1,
 * and the coefficients of X_next under sublayer l+1's parameters, Eq. 7-9,
 * 14-19) followed by hc_pre on X_next (F_in_next, the input of sublayer l+1's
 * function, Eq. 3). Arguments as hc_post_coeffs, plus:
 *   phi_next_packed: NULL, or hc_phi_pack(phi_next) (16-byte aligned); when
 *     given and the fast path applies, phi_next is not packed again.
 *   h_pre_next may be NULL (not stored); F_in_next [T, C] stream dtype.
 *   Workspace: hc_coeffs_workspace_bytes(T, n, C, dtype).
 */
int hc_post_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                const void* phi_next_packed, const float* bias_next, float alpha_pre, float alpha_post,
                float alpha_res, int sinkhorn_iters, float* h_pre_next, float* h_post_next,
                float* h_res_next, void* F_in_next, void* workspace, int64_t workspace_bytes,
                void* stream);

/*
 * hc_post_pre_noalloc - hc_post_pre for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments and results as hc_post_pre (the same
 * kernels run), without workspace / workspace_bytes: the workspace is a fixed
 * device array inside the library, HC_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the first call on that GPU until the process ends. The call allocates and
 * frees nothing. Limit: hc_coeffs_workspace_bytes(T, n, C, dtype) must not
 * exceed HC_NOALLOC_SCRATCH_BYTES, else HC_ERR_SCRATCH is returned before any
 * work (32 MiB covers bfloat16 n = 4 states of C = 4096 up to about 62,000 tokens
 * and of C = 7168 up to about 37,000). The first call on a device looks up that device's copy of the
 * array (a HIP symbol query, with the device current); HC_ERR_DEVICE if that
 * fails. Every call on one GPU shares that GPU's array, whose contents persist
 * from call to call (nothing in it needs to start at zero): calls that overlap
 * in time on one GPU (different streams, unordered) race on it and must be
 * ordered by the caller.
 */
#define HC_NOALLOC_SCRATCH_BYTES (32ll << 20)
int hc_post_pre_noalloc(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res,
                        const float* h_post, const void* F_out, void* X_next, const float* phi_next,
                        const void* phi_next_packed, const float* bias_next, float alpha_pre, float alpha_post,
                        float alpha_res, int sinkhorn_iters, float* h_pre_next, float* h_post_next,
                        float* h_res_next, void* F_in_next, void* stream);

/* ------------------------------------------------------------------ xHC -- */

/* Workspace bytes needed by xhc_pre (with_router != 0 when w_router is given). */
int64_t xhc_pre_workspace_bytes(int64_t T, int N, int64_t C, int m, int with_router, int dtype);

/*
 * xhc_pre - full-state pass of an xHC sublayer ([xHC] steps 1 and 2):
 *   dense read over all N streams: h_pre = sigmoid(alpha_pre * (vec X @ phi_pre)
 *   / r + b_pre), F_in[t, c] = sum_{i<N} h_pre[t, i] X[t, i, c], and, when
 *   w_router != NULL, the router: score[t, j] = sigmoid((vec X @ w_router)[j] / r)
 *   for candidate stream m + j (j < N - m), and idx[t] = the m fixed streams
 *   0..m-1 plus the k - m candidates with the highest score (equal scores go
 *   to the lower stream index), listed in ascending stream order.
 *   X [T, N, C], F_in [T, C] stream dtype; phi_pre [N*C, N], b_pre [N],
 *   w_router [N*C, N - m] float32; outputs h_pre [T, N] float32 (may be NULL),
 *   idx [T, k] int32, score [T, N - m] float32 (both required iff w_router).
 *   1 <= m <= k <= N <= 64, k <= 16.
 */
int xhc_pre(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
            const float* phi_pre, const float* b_pre, float alpha_pre, const float* w_router,
            float* h_pre, void* F_in, int32_t* idx, float* score,
            void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes needed by xhc_route (with_router != 0 when idx_in is NULL). */
int64_t xhc_route_workspace_bytes(int64_t T, int N, int64_t C, int k, int m, int K,
                                  int with_router, int dtype);

/*
 * xhc_route - stream routing, gather, sparse mix and scatter, IN PLACE on X
 * ([xHC] steps 1 and 3; parameterisation).
 *   If idx_in is NULL the active set is selected here from the full state with
 *   w_router exactly as in xhc_pre; otherwise idx_in [T, k] (int32, k distinct
 *   stream indices in [0, N), ascending) is used and w_router is ignored.
 *   Per token: X_A = X[t, idx[a], :] (a < k, slot order); r_A = ||vec X_A|| /
 *   sqrt(kC); z = alpha * (vec X_A @ phi_act) / r_A + b_act with columns
 *   [post k*K (a*K + j) | res k*k (a*k + b)] and alpha_post / alpha_res on the
 *   two blocks; H_post_A = 2 sigmoid(z_post) [k, K]; H_res_A = Sinkhorn-Knopp
 *   of exp(z_res) [k, k]; then X[t, idx[a], :] = sum_b H_res_A[a, b] X_A[b, :]
 *   + sum_j H_post_A[a, j] Wb[t, j, :]. Streams not in idx are not written.
 *   Wb [T, K, C] stream dtype: the K write-back components (K = 1: F_out;
 *   K = r + 1: the output of xhc_augment). 1 <= K <= 8.
 *   phi_act [k*C, k*K + k*k], b_act [k*K + k*k] float32.
 *   Outputs: idx_out [T, k] int32 (required), score_out [T, N - m] float32
 *   (optional, only written when selecting), h_post_out [T, k, K] and
 *   h_res_out [T, k, k] float32 (optional).
 *   Index entries outside [0, N) in idx_in leave the token unchanged.
 */
int xhc_route(void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
              const float* w_router, const int32_t* idx_in,
              const float* phi_act, const float* b_act, float alpha_post, float alpha_res,
              int sinkhorn_iters, const void* Wb, int K,
              int32_t* idx_out, float* score_out, float* h_post_out, float* h_res_out,
              void* workspace, int64_t workspace_bytes, void* stream);

/*
 * xHC chained sublayers - the pair xhc_route (sublayer l) + xhc_pre (sublayer
 * l + 1) with one read of the full state per sublayer ([xHC] steps 1-3). The
 * maps of sublayer l + 1 are linear in the state up to the RMS factor, and
 * route l rewrites only its k active rows, so their projection splits into the
 * rows route l leaves unchanged, projected while the call before read the
 * whole state for sublayer l's pre-read (the "carry"), and the k rewritten rows,
 * projected right after the mix; the sum of squares splits the same way. The
 * outputs are those of xhc_route + xhc_pre on the same inputs, with sums added
 * in another order.
 *   xhc_pre_chain(... maps of sublayer 0 ..., phi_pre_next, w_router_next,
 *     carry_out): xhc_pre of the first sublayer (with the router: idx, score
 *     required), whose pre-read also forms carry_out for sublayer 1's maps
 *     (phi_pre_next [N*C, N], w_router_next [N*C, N - m]).
 *   xhc_route_pre(X, ..., idx_in, route of sublayer l ..., b_pre, alpha_pre of
 *     sublayer l + 1, carry_in, phi_pre_next, w_router_next, carry_out, outputs
 *     of l + 1): xhc_route with idx_in, then xhc_pre of sublayer l + 1 on the
 *     updated state: idx_out, score_out, h_pre_out (each may be NULL except
 *     idx_out), F_in. carry_in is the carry written by the call that produced
 *     idx_in (xhc_pre_chain or the previous xhc_route_pre), on this state
 *     unchanged since; it holds sublayer l + 1's phi_pre and w_router (packed)
 *     with their partial projection. With phi_pre_next and w_router_next (the
 *     maps of sublayer l + 2) carry_out is written for the next call, else (the
 *     last sublayer) phi_pre_next, w_router_next and carry_out are NULL.
 *     carry_out may be carry_in (the carry is read before it is written);
 *     idx_out may be idx_in.
 *   carry: xhc_chain_carry_bytes(T, N, C, k, m, dtype) bytes, 256-byte aligned,
 *     opaque (per-item partial projections, float32, and the maps in the
 *     projection's packed bfloat16 form).
 *   Covered: dtype HC_BF16 (HC_F32 -> HC_ERR_DTYPE), N = 16, k = 4, 1 <= m <= 4,
 *   C a multiple of 512, K <= 8, 1 <= sinkhorn_iters <= HC_MAX_ITERS (else
 *   HC_ERR_SHAPE; xhc_chain_carry_bytes returns -1). X, Wb, F_in 16-byte
 *   aligned, idx arrays 16-byte aligned, float arrays 4 (else HC_ERR_ALIGN);
 *   workspace 256-byte aligned, at least xhc_chain_workspace_bytes. The carries
 *   and outputs overlap no input (but as stated above) and no other output
 *   (HC_ERR_ALIAS). idx_in must be an active set these calls produced (k
 *   distinct streams per token, as the carry left out).
 */
int64_t xhc_chain_carry_bytes(int64_t T, int N, int64_t C, int k, int m, int dtype);
int64_t xhc_chain_workspace_bytes(int64_t T, int N, int64_t C, int k, int m, int K, int dtype);
int xhc_pre_chain(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
                  const float* phi_pre, const float* b_pre, float alpha_pre, const float* w_router,
                  const float* phi_pre_next, const float* w_router_next,
                  float* h_pre, void* F_in, int32_t* idx, float* score, void* carry_out,
                  void* workspace, int64_t workspace_bytes, void* stream);
int xhc_route_pre(void* X, int dtype, int64_t T, int N, int64_t C, int k, int m,
                  const int32_t* idx_in, const float* phi_act, const float* b_act, float alpha_post,
                  float alpha_res, int sinkhorn_iters, const void* Wb, int K,
                  const float* b_pre, float alpha_pre, const void* carry_in,
                  const float* phi_pre_next, const float* w_router_next, void* carry_out,
                  float* h_post_out, float* h_res_out, int32_t* idx_out, float* score_out, float* h_pre_out,
                  void* F_in, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * xhc_route_backward, xhc_pre_backward - gradients of the routed xHC step
 * (xhc_pre, then xhc_route with K = 1 or 4 write-back components), the
 * backward of [xHC] steps 2 and 3 with the parameterisation: on the active rows
 * the route is the mHC post/res write with maps formed from the active state
 * alone, so its backward follows the mHC one ([mHC] 4.3.1: the Sinkhorn backward
 * recomputes the iterates on chip; the maps are recomputed from X). The active
 * set is a discrete choice: it and the router weights receive no gradient.
 *   X [T, N, C]: the state both forward calls read, i.e. before xhc_route's
 *   in-place update (keep it, or its active rows, for the backward).
 *   xhc_route_backward (first; it does not need dF_in): dX [T, N, C] holds the
 *     upstream gradient dX_next on entry and the route's gradient on exit: rows
 *     outside the active set are left as they are (they pass through); the
 *     active rows become H_res_A^T dX_next_A plus the maps' terms. Also
 *     dWb = H_post_A^T dX_next_A, the gradient of the write-back components Wb
 *     [T, K, C] (bfloat16): K = 1 (Wb = F_out): dWb [T, C] bfloat16; K = 4 (Wb =
 *     xhc_augment's V): dWb = dV [T, 4, C] float32, the input of
 *     xhc_augment_backward. dphi_act [4C, 4K + 16], db_act [4K + 16], dalpha [2]
 *     (post, res), dh [T, 4K + 16] = the map gradients [dH_post (a*K + j) |
 *     dH_res (4a + b)]. idx [T, 4] as the forward used (int32, 16-byte aligned);
 *     phi_act, b_act, alpha_*, sinkhorn_iters as for xhc_route.
 *   xhc_pre_backward (once dF_in, the gradient of F_in, is known): adds the
 *     dense read's gradient to dX (in place), and writes dphi_pre [NC, N],
 *     db_pre [N], dalpha [1], dh_pre [T, N] = <dF_in, x_i> (16-byte aligned).
 *   Covered: dtype HC_BF16 (HC_F32 -> HC_ERR_DTYPE), N a multiple of 4 up to 16,
 *   k = 4, K = 1 or 4, C a multiple of 32, 1 <= sinkhorn_iters <=
 *   HC_MAX_BWD_ITERS (else HC_ERR_SHAPE). bfloat16 arrays and dWb 16 bytes
 *   aligned, float arrays 4; workspace 256 bytes, at least
 *   xhc_backward_workspace_bytes (both calls, either K). dX overlaps nothing
 *   else; no output overlaps an input, another output or the workspace
 *   (HC_ERR_ALIAS). Deterministic: every sum runs in a fixed order.
 *   xhc_backward_workspace_bytes: 0 for T = 0, -1 for what the calls do not cover.
 */
int64_t xhc_backward_workspace_bytes(int64_t T, int N, int64_t C, int k, int K, int dtype);
int xhc_route_backward(const void* X, int dtype, int64_t T, int N, int64_t C, int k, const int32_t* idx,
                       const float* phi_act, const float* b_act, float alpha_post, float alpha_res,
                       int sinkhorn_iters, const void* Wb, int K, void* dX, void* dWb, float* dphi_act,
                       float* db_act, float* dalpha, float* dh, void* workspace, int64_t workspace_bytes,
                       void* stream);
int xhc_pre_backward(const void* X, int dtype, int64_t T, int N, int64_t C, const float* phi_pre,
                     const float* b_pre, float alpha_pre, const void* dF_in, void* dX, float* dphi_pre,
                     float* db_pre, float* dalpha, float* dh_pre, void* workspace, int64_t workspace_bytes,
                     void* stream);

/* Workspace bytes needed by xhc_augment (0 when it needs none); -1 for invalid sizes. */
int64_t xhc_augment_workspace_bytes(int64_t B, int64_t S, int64_t C, const int* kappa, int r, int dtype,
                                    int v_dtype);

/*
 * xhc_augment - temporal feature augmentation ([xHC] temporal feature
 * augmentation; kernel sizes {4, 8, 12} in [xHC-R]):
 *   tokens are B sequences of S tokens ([B, S] row-major, T = B*S);
 *   g_j[t, c] = sum_{s<kappa_j} w_j[c, s] * F_out[t - kappa_j + 1 + s, c], with
 *   zeros before the start of each sequence (w_j[c, kappa_j - 1] weights the
 *   current token); then Gram-Schmidt (modified form, no normalisation):
 *   V[t, 0] = F_out[t]; V[t, j] = g_j minus its projections on V[t, 0..j-1],
 *   removed one after another. (For kappa = {4, 8, 12} the projections are
 *   formed from each token's 4x4 Gram matrix, which gives the same vectors in
 *   exact arithmetic.)
 *   F_out [T, C] stream dtype `dtype`; conv_w = [C, kappa_1] then [C, kappa_2] ...
 *   float32; kappa: HOST array of r kernel sizes (1..32); 0 <= r <= 7;
 *   V [T, r + 1, C] in `v_dtype`.
 *   Workspace: xhc_augment_workspace_bytes(B, S, C, kappa, r, dtype, v_dtype)
 *   (may be NULL when that is 0).
 */
int xhc_augment(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C,
                const float* conv_w, const int* kappa, int r,
                void* V, int v_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * xhc_augment_backward - gradients of xhc_augment ([xHC] temporal feature
 * augmentation) for the upstream gradient dV [T, 4, C] float32 of its output
 * (xhc_route_backward's dWb for K = 4): the Gram-Schmidt steps walked in
 * reverse (recomputed from each token's Gram matrix of [F_out, g_1, g_2, g_3]
 * and of dV against them, in float64), then each causal conv's transpose:
 *   dF_out[t, c] = dU_0[t, c] + sum_j sum_d w_j[c, kappa_j - 1 - d] dU_j[t + d, c]
 *     (within the sequence), stored in `dtype`, rounded once;
 *   dconv_w[j][c, s] = sum_t dU_j[t, c] F_out[t - kappa_j + 1 + s, c] (zeros before
 *     the sequence start), float32 in conv_w's layout, summed over all tokens.
 *   Covered: r = 3 convs of sizes kappa = {4, 8, 12} (else HC_ERR_SHAPE), F_out
 *   bfloat16 or float32, any C. No epsilon (as the forward): a token whose
 *   components are linearly dependent gives non-finite values.
 *   Workspace: xhc_augment_backward_workspace_bytes (0 when B*S = 0, -1 for what
 *   the call does not cover). Deterministic: every sum runs in a fixed order.
 */
int64_t xhc_augment_backward_workspace_bytes(int64_t B, int64_t S, int64_t C, const int* kappa, int r, int dtype);
int xhc_augment_backward(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C,
                         const float* conv_w, const int* kappa, int r, const float* dV,
                         void* dF_out, float* dconv_w, void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * xHC-Flash ([xHC] memory efficiency; [xHC-R] method and memory-efficiency table): a block of L
 * consecutive sublayers (L = 2: attention + MLP; L = 4: the four-sublayer
 * variant) shares one routing decision and the block-entry state's full-state
 * reads; the residual mixing of the active streams is deferred to the block's
 * last sublayer, and the later sublayers' inputs are rebuilt from the entry
 * state's dense reads without reading the state again. Readings (the pages give
 * no formulas): sublayer l has its own phi_pre^(l), b_pre^(l) (alpha_pre shared)
 * on the RMS-normalised entry state, as xhc_pre forms h_pre; the router runs
 * once at block entry; the active maps come from the entry state's active rows
 * with one post column per sublayer and one H_res; sublayers l < L-1 add
 * H_post[:, l] F_out^(l) to the active rows with no mixing and the last mixes
 * with H_res and adds its own write. A block runs:
 *   xhc_flash_pre(X_0) -> idx, h_pre, F_pre;  xhc_flash_maps(X_0, idx) -> H_post, H_res;
 *   for l: F_in^(l) = xhc_flash_input(l, ...); F_out^(l) = sublayer_l(F_in^(l));
 *   xhc_flash_post(X_0 -> X_L, F_outs).
 * X_0 is read by the first two calls and updated in place by the last.
 *
 * xhc_flash_pre: idx [T, k] (int32) from the router w_router [N*C, N-m] as
 *   xhc_pre selects it (m fixed streams + the top k-m candidates, ascending);
 *   score [T, N-m] (may be NULL); h_pre [L, T, N] float32 with phi_pre [L, N*C, N],
 *   b_pre [L, N]; F_pre [L, T, C] in X's dtype: F_pre[l] = sum_i h_pre[l, :, i] X_0[:, i]
 *   (the L dense reads come from one pass over X_0 for bfloat16 with N a
 *   multiple of 4 up to 16, C % 8 == 0 and 16-byte aligned X and F_pre).
 *   Requires 1 <= m < N, m <= k <= min(N, HC_MAX_ACTIVE), 1 <= L <=
 *   HC_MAX_FLASH_SUBLAYERS. Workspace: xhc_flash_pre_workspace_bytes.
 * The block's write-back components: the last sublayer (the MLP, which [xHC-R]'s
 * default configuration augments) may write back K_last components (its
 * xhc_augment output V, K_last = K_r = 4) instead of its F_out (K_last = 1); the
 * earlier sublayers write back their F_out. Kb = L - 1 + K_last components in
 * all, W [T, Kb, C] in the stream dtype: F_out^(0..L-2), then the last
 * sublayer's K_last components. 1 <= K_last, Kb <= HC_MAX_COMPONENTS.
 * xhc_flash_maps: H_post [T, k, Kb] (column j: the 2 sigma post map of component
 *   j) and H_res [T, k, k] (Sinkhorn, sinkhorn_iters) from the active rows of X_0
 *   (idx), phi_act [k*C, k*Kb + k*k] with columns [post (a*Kb + j) | res (a*k + b)],
 *   b_act in the same order: xhc_route's maps with K = Kb write-back columns.
 *   Workspace: xhc_flash_maps_workspace_bytes.
 * xhc_flash_input: sublayer l's input F_in [T, C] = F_pre_l + sum_{j<l} c_j
 *   W[:, j] with c_j[t] = sum_a h_pre_l[t, idx[t, a]] H_post[t, a, j];
 *   F_pre_l = F_pre[l], h_pre_l = h_pre[l] [T, N], W (F_outs) [T, Kb, C] (rows
 *   j < l read; may be NULL for l = 0). F_in may be F_pre_l itself. Computed in
 *   float32, rounded once. No workspace.
 * xhc_flash_post: X_0 -> X_L in place on the active rows:
 *   X_L,A = H_res (X_0,A + sum_{j<L-1} H_post[:, j] W_j) + sum_{j>=L-1} H_post[:, j] W_j,
 *   computed as one mix with the write maps E[:, j] = H_res H_post[:, j] (j < L-1)
 *   and E[:, j] = H_post[:, j] (j >= L-1) (kept in the workspace, T*k*Kb floats,
 *   xhc_flash_post_workspace_bytes); rows outside the active set untouched.
 *   W_last: NULL, or the last sublayer's K_last components [T, K_last, C] kept
 *   apart (e.g. xhc_augment's output as written): then they are read from W_last
 *   and F_outs' rows L-1 .. Kb-1 are not read (F_outs keeps its [T, Kb, C] layout).
 * All: dtype HC_F32 or HC_BF16; float arrays 4-byte aligned, stream arrays aligned
 * to their element size, workspaces 256 bytes; outputs overlap no input, other
 * output or workspace (HC_ERR_ALIAS). Workspace queries: -1 for invalid sizes.
 */
int64_t xhc_flash_pre_workspace_bytes(int64_t T, int N, int64_t C, int m, int L, int dtype);
int xhc_flash_pre(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int m, int L, const float* phi_pre,
                  const float* b_pre, float alpha_pre, const float* w_router, int32_t* idx, float* score,
                  float* h_pre, void* F_pre, void* workspace, int64_t workspace_bytes, void* stream);
int64_t xhc_flash_maps_workspace_bytes(int64_t T, int N, int64_t C, int k, int L, int K_last, int dtype);
int xhc_flash_maps(const void* X, int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last,
                   const int32_t* idx, const float* phi_act, const float* b_act, float alpha_post, float alpha_res,
                   int sinkhorn_iters, float* H_post, float* H_res, void* workspace, int64_t workspace_bytes,
                   void* stream);
int xhc_flash_input(int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last, int l, const void* F_pre_l,
                    const float* h_pre_l, const int32_t* idx, const float* H_post, const void* F_outs, void* F_in,
                    void* stream);
int64_t xhc_flash_post_workspace_bytes(int64_t T, int k, int L, int K_last);
int xhc_flash_post(void* X, int dtype, int64_t T, int N, int64_t C, int k, int L, int K_last, const int32_t* idx,
                   const float* H_post, const float* H_res, const void* F_outs, const void* W_last, void* workspace,
                   int64_t workspace_bytes, void* stream);

/* ----------------------------------------- HC baseline and gain diagnostic -- */

/*
 * hc_tanh_coeffs - the maps of unconstrained Hyper-Connections ([mHC] section 3
 * Preliminary, Eq. 5), for comparison with the mHC calls (apply them with
 * hc_pre and hc_post):
 *   per token t and stream i, x~_i = X[t, i] / r_i with r_i = sqrt(sum_c
 *   X[t, i, c]^2 / C) (each stream normalised over its own C channels; no gain,
 *   no epsilon; x~_i = 0 when r_i = 0);
 *   h_pre[t, i]     = alpha_pre  * tanh(theta[0]     . x~_i) + bias[i]
 *   h_post[t, i]    = alpha_post * tanh(theta[1]     . x~_i) + bias[n + i]
 *   h_res[t, j, i]  = alpha_res  * tanh(theta[2 + j] . x~_i) + bias[2n + j*n + i]
 *   X [T, n, C] stream dtype; theta [n + 2, C] float32 (rows pre, post, res_0 ..
 *   res_{n-1}); bias [n*n + 2n] float32 as for hc_coeffs; outputs float32
 *   h_pre [T, n], h_post [T, n], h_res [T, n, n] (row j = output stream j).
 *   1 <= n <= 16. No workspace.
 */
int hc_tanh_coeffs(const void* X, int dtype, int64_t T, int n, int64_t C, const float* theta,
                   const float* bias, float alpha_pre, float alpha_post, float alpha_res, float* h_pre,
                   float* h_post, float* h_res, void* stream);

/*
 * hc_amax_gain - Amax gain magnitude of a chain of residual maps ([mHC]
 * section 3.1): per token t, M = H_{L-1} ... H_1 H_0 (float32) with
 * H_l = h_res[l, t] (n x n, row = output stream), then
 *   gain_fwd[t] = max_i |sum_j M[i, j]|   (largest absolute row sum: forward)
 *   gain_bwd[t] = max_j |sum_i M[i, j]|   (largest absolute column sum: backward).
 *   h_res [L, T, n, n] float32 (layer 0 first; may be NULL when L == 0, the
 *   gains are then 1); gain_fwd, gain_bwd [T] float32. 1 <= n <= 16, L >= 0.
 */
int hc_amax_gain(const float* h_res, int64_t L, int64_t T, int n, float* gain_fwd, float* gain_bwd,
                 void* stream);

/* ------------------------------------------------------------- static mHC -- */

/*
 * Static mHC ("mHC-SSM" abstract: mHC around a state space model block with
 * one set of maps per layer, shared by every token).
 *
 * hc_static_maps - the maps from their logits (device arrays):
 *   logits [n*n + 2n] float32 (pre n | post n | res n*n row-major, the layout of
 *   the mHC bias); h_pre [n] = softmax(pre logits) and h_post [n] =
 *   softmax(post logits) (simplex-constrained pre- and post-mixing: nonnegative,
 *   summing to 1); h_res [n, n] = Sinkhorn-Knopp of exp(res logits), as in
 *   hc_coeffs ([mHC] Eq. 9). 1 <= n <= 16; 1 <= sinkhorn_iters <= HC_MAX_ITERS.
 *
 * hc_static_pre  - F_in[t] = sum_i h_pre[i] X[t, i]       ([mHC] F_pre, one h_pre for all tokens)
 * hc_static_post - X_next[t] = h_res X[t] + h_post^T F_out[t]  ([mHC] Eq. 3, F_post,res)
 *   X [T, n, C], F_in / F_out [T, C] stream dtype; h_pre, h_post [n], h_res [n, n]
 *   float32 device arrays; X_next may equal X (not partially overlap it).
 */
int hc_static_maps(const float* logits, int n, int sinkhorn_iters, float* h_pre, float* h_post, float* h_res,
                   void* stream);
int hc_static_pre(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_pre, void* F_in,
                  void* stream);
int hc_static_post(const void* X, int dtype, int64_t T, int n, int64_t C, const float* h_res, const float* h_post,
                   const void* F_out, void* X_next, void* stream);

/* ------------------------------------------------------------ measurement -- */

/*
 * hc_copy_probe - not part of the method: a plain device-to-device copy of
 * `bytes` bytes with 16-byte nontemporal loads and stores, the access pattern
 * the streaming kernels use, so that a benchmark can measure the practical HBM
 * streaming rate of the device it runs on next to the sublayer's rate.
 *   src, dst: device pointers, 16-byte aligned, not overlapping; bytes >= 0 and
 *   a multiple of 16 (bytes == 0 does nothing; pointers may then be NULL).
 *   Errors: HC_ERR_NULL, HC_ERR_SHAPE (bytes < 0), HC_ERR_ALIGN (alignment or
 *   bytes % 16), HC_ERR_ALIAS (overlap).
 */
int hc_copy_probe(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HC_H_ */
