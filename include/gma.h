/*
 * gma.h -- C ABI of libgma.so, the MI355X (gfx950) forward and backward passes of
 * Gaussian Mixture Attention (GMA).
 *
 * The operation (page "Attention par Mélange Gaussien (GMA)", gist.science paper
 * 2606.18283, section "Méthodologie", sub-section "Mécanisme Central"):
 *   item 1 "Routage Latent Probabiliste": for a routing vector x (a row of Q_X or K_X) the
 *          responsibility gamma_k(x) = p(z = k | x) is the posterior of a K-component GMM with
 *          means mu_k, diagonal covariances Sigma_k and mixing priors pi_k; rows of Gamma_Q and
 *          Gamma_K (N x K) are these posteriors.  One mixture per head routes both Q and K.
 *   item 2 "Routage de Mémoire Latente": write Vt = Gamma_K^T V (K x d_v), Z = Gamma_K^T 1 (K);
 *          read O = Gamma_Q Vt / (Gamma_Q Z + eps), one scalar denominator per query row.
 *          The N x N affinity Gamma_Q Gamma_K^T is never formed.
 *   item 3 "Variantes et Entraînement": bidirectional and causal variants (causal: prefix sums
 *          of Vt and Z, so O_i depends on j <= i only, the diagonal included); variances are
 *          softplus(raw) and priors are softmax(prior logits).
 *
 * Conventions shared by every entry point
 *   Layout     tensors are contiguous row-major: x, qx, kx [B, H, N, d_r]; v, o [B, H, N, d_v];
 *              gamma [B, H, N, K]; mu, raw_var [H, K, d_r] (fp32); prior_logits [H, K] (fp32).
 *              Parameters are the raw learned ones (softplus / softmax are applied inside).
 *   Dtypes     GMA_DTYPE_F32: x, qx, kx, v and o are fp32; all arithmetic is fp32.
 *              GMA_DTYPE_BF16: x, qx, kx, v and o are bf16; logits use fp16 matrix-core
 *              operands, responsibilities / values / states use bf16 operands, every sum and
 *              the softmax accumulate in fp32.  A (batch, head) with a row whose fp16 logits
 *              are not finite (|x| >= 256, so x^2 leaves fp16; sigma^2 < 1.1e-5 or |mu| / sigma^2
 *              > 45000, so a coefficient does) is detected by the kernels and recomputed exactly
 *              afterwards in the same call (log-density in its direct form in fp64, state in
 *              fp32): correct for every finite bf16 input, but one workgroup per such slice walks
 *              its tokens in order (milliseconds per 10^4 tokens).  fp32 storage: |x| < 1e19.
 *   Memory     every tensor pointer is a device pointer owned by the caller; the workspace is a
 *              caller-owned device buffer of at least gma_workspace_size() bytes, 16-byte
 *              aligned, whose contents need not be initialised and are clobbered.  The library
 *              never allocates, frees or synchronises device memory.  o and gamma must not
 *              overlap any input.
 *   Streams    `stream` is a hipStream_t (NULL = the legacy default stream).  Every call only
 *              enqueues kernels and returns; results are ready when the stream reaches them.
 *   Errors     invalid arguments are reported by status code before any HIP call is made.
 *              GMA_ERROR_LAUNCH reports a failed kernel launch.  gma_last_error() gives a
 *              human-readable message for the last failing call on the calling thread.
 *   Limits     1 <= d_r, K, d_v <= 256; B, H, N >= 1.  Shapes are padded internally to a compiled
 *              tile class (K, d_v, d_r): bf16 (32, 64, 64), (128, 128, 128), (256, 64, 64),
 *              (256, 128, 128); fp32 (16, 16, 16), (64, 64, 64), (128, 128, 128).  The cheapest class
 *              that covers the shape runs it (padding components get zero responsibility, padding
 *              dims zero coefficients).  A shape that no class covers (d_r or d_v in (128, 256])
 *              runs on the generic path: Gamma_Q and Gamma_K materialised in fp32 in the workspace
 *              (logits on the fp32 matrix cores, each 16-dim step added in fp64), and the write and
 *              read phases as fp32 matrix-core products (causal: 64-token chunks); slower, with a
 *              workspace of about B H N (2 K + d_v + 1) 4 bytes (+ B H N 64 4 when causal).
 *              gma_decode_step and the backward have no classes.
 *   Results    deterministic: repeated calls give bitwise identical outputs (no atomics; every
 *              reduction runs in a fixed order independent of the device).
 *   Environment GMA_CAUSAL_ROUNDS=R (measurement only; default 1): the bf16 causal pass launches its
 *              aggregate, scan and output kernels in R rounds over the sequence instead of once.
 *              Results differ from R = 1 only in the summation order of the carried state.
 */
#ifndef GMA_H_
#define GMA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GMA_DTYPE_F32 = 0, GMA_DTYPE_BF16 = 1 } gma_dtype_t;

typedef enum {
    GMA_SUCCESS = 0,
    GMA_ERROR_INVALID_VALUE = 1,
    GMA_ERROR_NOT_SUPPORTED = 2,
    GMA_ERROR_WORKSPACE_TOO_SMALL = 3,
    GMA_ERROR_LAUNCH = 4
} gma_status_t;

typedef enum {
    GMA_OP_RESPONSIBILITIES = 0,
    GMA_OP_FORWARD_BIDIR = 1,
    GMA_OP_FORWARD_CAUSAL = 2,
    GMA_OP_FORWARD_CAUSAL_STATE = 3,
    GMA_OP_RESPONSIBILITY_STATS = 4,
    GMA_OP_BACKWARD_BIDIR = 5,
    GMA_OP_BACKWARD_CAUSAL = 6
} gma_op_t;

/* Problem sizes.  eps >= 0 and finite; it is added to each row's denominator Gamma_Q Z. */
typedef struct {
    int64_t batch;     /* B */
    int64_t heads;     /* H */
    int64_t seq_len;   /* N */
    int32_t d_route;   /* d_r: width of the routing projections Q_X, K_X */
    int32_t n_comp;    /* K: number of Gaussian components */
    int32_t d_value;   /* d_v: width of V and O */
    int32_t dtype;     /* gma_dtype_t of x / qx / kx / v / o / (not gamma: always fp32) */
    float eps;
} gma_problem_t;

/* Bytes of workspace `op` needs for `problem` on its fastest path; 0 if the problem is invalid or
 * unsupported.  Pure host computation.  For GMA_OP_FORWARD_CAUSAL with bf16 storage this includes
 * the stored responsibility tiles of the keys, B * H * ceil(N / 64) * 64 * K_padded * 2 bytes
 * (K_padded: K rounded up to a power of two, at least 32).  The tiles are used only with a
 * workspace of at least this size; a smaller one is still accepted where it holds the rest, and
 * the causal pass then recomputes Gamma_K from K_X (slower). */
size_t gma_workspace_size(const gma_problem_t* problem, int op);

/* Responsibilities (item 1 above) of every row of x [B, H, N, d_r] under head h's mixture:
 * gamma [B, H, N, K] fp32, each row non-negative and summing to 1. */
gma_status_t gma_responsibilities(const gma_problem_t* problem, const void* x, const float* mu,
                                  const float* raw_var, const float* prior_logits, float* gamma,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* Responsibility diagnostics (item 1; the pages discuss how the components are used): for every
 * row of x [B, H, N, d_r] under head h's mixture,
 *   usage [B, H, K] fp32         sum over the rows of gamma_k (each row of Gamma sums to 1);
 *   hard_counts [B, H, K] uint32 number of rows whose largest gamma is at component k (ties go to the
 *                                lowest k; decided on the library's fp32 Gamma, where values within
 *                                about 2^-15 of each other count as equal, so rows whose two largest
 *                                responsibilities are that close may go either way);
 *   usage_entropy [B, H] fp32    -sum_k p_k ln p_k / ln K with p = usage / N (0 ln 0 = 0; 0 when
 *                                K = 1): the usage entropy as a fraction of its largest value, the
 *                                normalisation under which the page's interpretability figures (usage
 *                                entropy 0.933 with 104 of 128 components in use, section "Résultats
 *                                et Performance") are consistent.  Components in use: hard_counts > 0.
 * The responsibilities kernel reduces its rows as it forms them: per-segment usage sums and counts
 * (a few segments per (batch, head)) are combined in a fixed order, and Gamma is never stored.
 * Workspace: gma_workspace_size(problem, GMA_OP_RESPONSIBILITY_STATS) bytes, independent of N for the
 * compiled classes (the generic path, d_r > 128, forms Gamma, about B * H * N * K * 4 bytes).
 * d_value is ignored. */
gma_status_t gma_responsibility_stats(const gma_problem_t* problem, const void* x, const float* mu,
                                      const float* raw_var, const float* prior_logits, float* usage,
                                      uint32_t* hard_counts, float* usage_entropy, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* Bidirectional forward (items 1-2): O = Gamma_Q (Gamma_K^T V) / (Gamma_Q (Gamma_K^T 1) + eps)
 * over the whole sequence of each (b, h).  qx, kx [B, H, N, d_r]; v, o [B, H, N, d_v]. */
gma_status_t gma_forward_bidir(const gma_problem_t* problem, const void* qx, const void* kx,
                               const void* v, const float* mu, const float* raw_var,
                               const float* prior_logits, void* o, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Causal forward (item 3): O_i = Gamma_Q[i] Vt_i / (Gamma_Q[i] . Z_i + eps) with
 * Vt_i = sum_{j <= i} gamma_K[j] (x) v_j and Z_i = sum_{j <= i} gamma_K[j].  Same arguments as
 * gma_forward_bidir. */
gma_status_t gma_forward_causal(const gma_problem_t* problem, const void* qx, const void* kx,
                                const void* v, const float* mu, const float* raw_var,
                                const float* prior_logits, void* o, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Causal forward that allocates nothing, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): gma_forward_causal with
 * no workspace argument.  Its workspace is a fixed array of GMA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held from the library's first use on that GPU until the process ends; its
 * address on the current device is looked up on the first call there.  Results are those of
 * gma_forward_causal given a workspace of GMA_NOALLOC_SCRATCH_BYTES bytes (the stored Gamma_K tiles
 * are used only where they fit; otherwise Gamma_K is recomputed from K_X).
 *   Limit   the workspace the causal pass needs without the stored tiles must fit the array: about
 *           B H P (K_pad (d_v_pad + 1)) 4 + H K_pad (4 d_r_pad + 4) bytes with B H P >= 256, e.g.
 *           17 MiB for K = d_r = d_v = 128.  Larger problems return GMA_ERROR_WORKSPACE_TOO_SMALL
 *           (before any HIP call).
 *   Races   every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *           (on different streams, or from different threads without ordering) race and give wrong
 *           results.  Calls ordered on one stream are safe.  The stream's device must be current.
 *   No call of this entry point allocates or frees memory (hipMalloc, hipFree or any allocating
 *   library routine).  Other arguments and errors as gma_forward_causal. */
#define GMA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gma_status_t gma_forward_causal_noalloc(const gma_problem_t* problem, const void* qx, const void* kx,
                                        const void* v, const float* mu, const float* raw_var,
                                        const float* prior_logits, void* o, void* stream);

/* Bidirectional forward with separate query and key/value sequences (cross-attention; the pages
 * name N_q != N_k as future work, and the write / read equations of item 2 apply unchanged):
 * qx [B, H, N_q, d_r] and o [B, H, N_q, d_v] with N_q = problem->seq_len; kx [B, H, N_kv, d_r] and
 * v [B, H, N_kv, d_v] with N_kv = seq_len_kv >= 1.  Workspace: gma_workspace_size() of the same
 * problem with seq_len = max(N_q, N_kv) and op GMA_OP_FORWARD_BIDIR (the compiled classes need only
 * that of seq_len = N_kv; the generic path holds rows of both sides).  Otherwise as gma_forward_bidir. */
gma_status_t gma_forward_bidir_kv(const gma_problem_t* problem, int64_t seq_len_kv, const void* qx,
                                  const void* kx, const void* v, const float* mu, const float* raw_var,
                                  const float* prior_logits, void* o, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Causal forward with the latent memory carried across calls (item 3: the causal output is a
 * prefix sum, so everything before this call's first token enters only through [Vt | Z]).  Lets a
 * sequence be processed in consecutive pieces (streaming, or one-token decode steps) with results
 * identical, up to rounding order, to one call over the whole sequence.
 *   state_in   [B, H, K, d_v + 1] fp32 or NULL (zero): row k of (b, h) holds Vt[k, 0 .. d_v-1] and
 *              then Z[k], the memory after all earlier tokens.
 *   state_out  [B, H, K, d_v + 1] fp32 or NULL: receives the memory after this call's last token
 *              (state_in plus this call's Gamma_K^T [V | 1]).
 * state_in and state_out may be the same buffer (updated in place); otherwise they must be
 * disjoint, and neither may overlap qx, kx, v, o or the workspace.  4-byte aligned.  Other
 * arguments as gma_forward_causal; workspace: gma_workspace_size(problem,
 * GMA_OP_FORWARD_CAUSAL_STATE) bytes. */
gma_status_t gma_forward_causal_state(const gma_problem_t* problem, const void* qx, const void* kx,
                                      const void* v, const float* mu, const float* raw_var,
                                      const float* prior_logits, const float* state_in,
                                      float* state_out, void* o, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* One causal decode step (item 3, streaming): one new token per (b, h), problem->seq_len = 1.
 * qx, kx [B, H, 1, d_r]; v, o [B, H, 1, d_v]; state_in / state_out as gma_forward_causal_state
 * (either may be NULL: zero initial state / state not written; they may be the same buffer).
 * Updates [Vt | Z] with the token's gamma_K (x) [v | 1] and writes its output row, which includes
 * the token itself; the same result, up to rounding, as gma_forward_causal_state over one token.
 * Any 1 <= d_r, K, d_v <= 256 (no tile classes); needs no workspace.  Arithmetic in fp32 with
 * the log-density sums in fp64 (more precise than the bulk path's matrix-core logits). */
gma_status_t gma_decode_step(const gma_problem_t* problem, const void* qx, const void* kx,
                             const void* v, const float* mu, const float* raw_var,
                             const float* prior_logits, const float* state_in, float* state_out,
                             void* o, void* stream);

/* Decode with a prepared mixture (item 3, streaming).  gma_decode_step derives the variances and
 * the prior from the raw parameters (softplus, log, log-sum-exp over K·d_r numbers) on every token;
 * a decoder whose parameters are fixed between updates prepares them once instead:
 *   gma_decode_params_size  bytes of the prepared form for problem->heads, n_comp, d_route
 *                           (0 for an invalid problem): 1 / softplus(raw_var) [H, K, d_r] fp32, then,
 *                           at the next 256-byte boundary, c_k = log pi_k - 1/2 sum_d log sigma^2_kd
 *                           [H, K] fp64 (log pi = log-softmax of prior_logits).
 *   gma_decode_prepare      writes that form into `prepared` (caller-owned device memory, 256-byte
 *                           aligned, prepared_bytes >= gma_decode_params_size, disjoint from the
 *                           parameters), asynchronously on `stream`.  Only heads, n_comp and
 *                           d_route of the problem are read.
 *   gma_decode_step_prepared  as gma_decode_step, with the mixture given by mu and `prepared`
 *                           (raw_var and prior_logits are not read).  The log-density of a row x is
 *                           c_k - 1/2 sum_d (x_d - mu_kd)^2 / sigma^2_kd: the same quantity as
 *                           gma_decode_step's, summed in a different order (results agree to
 *                           rounding).  `prepared` must be the output of gma_decode_prepare for the
 *                           current parameters and must not overlap o or the states.
 * Errors as gma_decode_step; GMA_ERROR_WORKSPACE_TOO_SMALL when prepared_bytes is too small. */
size_t gma_decode_params_size(const gma_problem_t* problem);
gma_status_t gma_decode_prepare(const gma_problem_t* problem, const float* raw_var,
                                const float* prior_logits, void* prepared, size_t prepared_bytes,
                                void* stream);
gma_status_t gma_decode_step_prepared(const gma_problem_t* problem, const void* qx, const void* kx,
                                      const void* v, const float* mu, const void* prepared,
                                      size_t prepared_bytes, const float* state_in, float* state_out,
                                      void* o, void* stream);

/* Backward of the bidirectional (gma_backward_bidir) or causal (gma_backward_causal) forward above:
 * the gradients of a scalar loss L with respect to every input, given dout = dL/dO [B, H, N, d_v].
 * The pages train the layer end to end (item 3: softplus variances and softmax priors are the
 * learned reparameterisation), so these are the chain rule through items 1-3:
 *   read    g_i = dO_i / den_i, h_i = -(dO_i . O_i) / den_i, dGamma_Q[i] = Vt_i g_i + Z_i h_i
 *   write   dGamma_K[j] = R_j v_j + r_j and dv_j = R_j^T gamma_K[j], with R_j, r_j the sums of
 *           Gamma_Q[i] (x) g_i and Gamma_Q[i] h_i over the queries i that see key j
 *   item 1  dl = gamma (dgamma - gamma . dgamma) per row; dx_d = sum_k dl_k (mu_kd - x_d) / s_kd
 *   item 3  dmu, dsigma2 and dlog pi summed over the rows of both Q_X and K_X of every batch, then
 *           draw_var = dsigma2 * sigmoid(raw_var), dprior_logits = G - pi sum_k G_k (G = dlog pi).
 * Outputs (written, not accumulated): dqx, dkx [B, H, N, d_r] and dv [B, H, N, d_v] in the storage
 * dtype; dmu, draw_var [H, K, d_r] and dprior_logits [H, K] fp32.  The forward is recomputed from the
 * inputs (O is not an argument).  Sums accumulate in fp32.  Products run on the fp32 matrix cores for
 * fp32 storage; for bf16 storage on the bf16 matrix cores with every fp32 operand split into bf16
 * hi + lo (about 16 significant bits; bf16 inputs are exact), and the outputs are rounded once.
 * Workspace:
 * gma_workspace_size(problem, GMA_OP_BACKWARD_BIDIR or GMA_OP_BACKWARD_CAUSAL) bytes, about
 * B * H * N * (6 K + 3 (d_v + 1) + 4 d_r) * 4 bytes plus per-chunk states; causal bf16 at
 * K = d_v = 128 (fused chunk kernels) about B * H * N * (4 K * 4 + 3 d_v * 2) bytes plus one array of
 * per-chunk states, B * H * ceil(N / 64) * K * (d_v + 4) * 4 bytes (4.1 GB at B = 1, H = 16, N = 65536).
 * There, v, dout or dv rows that are not 16-byte aligned are staged through aligned copies in the
 * workspace.  No gradient may overlap an input, another gradient or the workspace. */
gma_status_t gma_backward_bidir(const gma_problem_t* problem, const void* qx, const void* kx,
                                const void* v, const float* mu, const float* raw_var,
                                const float* prior_logits, const void* dout, void* dqx, void* dkx,
                                void* dv, float* dmu, float* draw_var, float* dprior_logits,
                                void* workspace, size_t workspace_bytes, void* stream);
gma_status_t gma_backward_causal(const gma_problem_t* problem, const void* qx, const void* kx,
                                 const void* v, const float* mu, const float* raw_var,
                                 const float* prior_logits, const void* dout, void* dqx, void* dkx,
                                 void* dv, float* dmu, float* draw_var, float* dprior_logits,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* gma_status_string(gma_status_t status);

/* Message of the last failing call on this thread ("" if none). */
const char* gma_last_error(void);

/* Measurement support.  When enabled, every kernel launch is bracketed by a pair of HIP
 * events recorded on the launch stream.  gma_timing_read() waits for the recorded events of
 * kernel `kernel_id` (0 <= id < gma_kernel_count()), returns their summed elapsed time and
 * launch count, and forgets them.  Disabled by default; enabling costs two event records per
 * launch. */
gma_status_t gma_timing_enable(int enabled);
gma_status_t gma_timing_read(int kernel_id, double* total_ms, int64_t* launches);
int gma_kernel_count(void);
const char* gma_kernel_name(int kernel_id);

/* Measurement support: the measured rate of the hardware base-2 exponential on the current device,
 * in exponentials per second, written to *per_second.  The softmax of item 1 takes 2 K of them per
 * token-head.  Runs one untimed and one timed launch on `stream` (NULL: the null stream) and waits
 * for them; allocates no device memory.  GMA_ERROR_INVALID_VALUE if per_second is NULL,
 * GMA_ERROR_LAUNCH if a HIP call fails (*per_second is then 0). */
gma_status_t gma_probe_exp2_rate(double* per_second, void* stream);

/* Measurement support: the rate at which the current device reads HBM, in bytes per second, written
 * to *bytes_per_second.  Reads the first bytes / 16 16-byte pieces of the caller's device buffer `buf`
 * (16-byte aligned; its contents do not matter and are not changed) with one untimed and ten timed
 * launches of a plain grid-stride read kernel on `stream` (NULL: the null stream), and waits for them;
 * allocates no device memory.  Pass a buffer well beyond the 256 MB last-level cache (1 GiB) to measure
 * HBM.  GMA_ERROR_INVALID_VALUE if bytes_per_second or buf is NULL, bytes < 16 or buf is not 16-byte
 * aligned; GMA_ERROR_LAUNCH if a HIP call fails (*bytes_per_second is then 0). */
gma_status_t gma_probe_read_rate(const void* buf, size_t bytes, double* bytes_per_second, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMA_H_ */
