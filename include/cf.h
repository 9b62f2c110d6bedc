/*
 * cf.h -- C ABI of the MI355X (gfx950) fused GEMM-epilogue and back-to-back
 * GEMM library.
 *
 * Method: ComFuse's Stage-Stream execution model and B2BGEMM schedule, as
 * described on the pith.science review of arXiv 2608.03537, "ComFuse: Fusing
 * Complex Memory-Intensive Subgraphs with Compute-Intensive Kernels For Modern
 * GPU Architectures" (cited as "ComFuse review" below).
 *
 * Conventions for every entry point:
 *   - Every matrix is row-major; leading dimensions (ld*) and batch strides are
 *     in elements. Pointers are device pointers owned by the caller; the
 *     library never allocates, frees or synchronises the caller's memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Each call only enqueues work on that stream and returns at once.
 *   - Argument and descriptor errors are detected on the host before any HIP
 *     call and return a status; nothing is launched then. No call aborts or
 *     throws across this ABI.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (all cross-workgroup merges run in a fixed order).
 *   - Fast paths need 16-byte aligned base pointers and leading dimensions,
 *     K and N that are multiples of 8 elements (bf16) or 4 (f32); other shapes
 *     and alignments are accepted and run on element-wise load paths.
 */
#ifndef CF_H_
#define CF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CF_OK = 0,
  CF_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size/stride, bad enum      */
  CF_ERR_UNSUPPORTED = 2,      /* legal but not implemented combination         */
  CF_ERR_WORKSPACE = 3,        /* workspace missing, too small or misaligned    */
  CF_ERR_NO_DEVICE = 4,        /* no HIP device is visible                      */
  CF_ERR_HIP = 5,              /* a HIP runtime call failed; see cf_last_hip_error */
  CF_ERR_DEVICE_TIMEOUT = 6    /* a strip exchange wait hit its time limit      */
} cf_status;

typedef enum { CF_F32 = 0, CF_BF16 = 1 } cf_dtype;

typedef enum { CF_ACT_NONE = 0, CF_ACT_RELU = 1 } cf_act;

/* Row operation that forms the Stage-Stream stage boundary: a reduction over
 * the output columns n of one row m (ComFuse review, "Core claim" and Referee
 * Report major comment 1 on Eq. (1): such a reduction needs only the tiles
 * T_{m,n} that share m). */
typedef enum {
  CF_ROW_NONE = 0,
  CF_ROW_SOFTMAX = 1,   /* y = exp(x - max_n x) / sum_n exp(x - max_n x)                 */
  CF_ROW_LAYERNORM = 2, /* y = (x - mean) / sqrt(var + eps) * gamma[n] + beta[n]; var is
                           the biased (1/N) variance; gamma/beta optional (NULL = 1 / 0) */
  CF_ROW_RMSNORM = 3,   /* y = x / sqrt(mean_n x^2 + eps) * gamma[n]; gamma optional     */
  CF_ROW_ARGMAX = 4,    /* cf_gemm_epilogue only: row_index[m] = the smallest n with
                           x[m, n] = max_n x[m, n], a NaN ranking as -inf (a row of
                           NaN and -inf gives 0), row_stats[m] (if given) = that
                           maximum (-inf for a NaN); y = x is stored only when C != NULL
                           (C may be NULL: the logits of a greedy LM head are never
                           written). gamma and beta must be NULL.                      */
  CF_ROW_TOPK = 5       /* cf_gemm_epilogue only: the topk (1..8, <= N) largest x of
                           each row, largest first, equal values by column ascending
                           (a NaN ranks as -inf at its own column and is reported
                           as -inf; topk = 1 is CF_ROW_ARGMAX):
                           row_index[m * topk + j] = their columns, row_stats[m * topk
                           + j] (if given) = their values. C as for argmax (may be
                           NULL). gamma, beta and residual must be NULL; fast-path
                           layouts only (CF_ERR_UNSUPPORTED otherwise). topk = 1
                           runs as CF_ROW_ARGMAX; topk <= 4 keeps shorter lists.    */
} cf_row_op;

/* Visibility mask on the scores S of cf_b2bgemm's softmax (ignored nowhere:
 * any other use is CF_ERR_UNSUPPORTED). */
typedef enum {
  CF_MASK_NONE = 0,
  CF_MASK_CAUSAL = 1    /* key l is visible to query row m iff l <= m + (L - M): the M
                           queries are the last M of the L positions (for M = L, the
                           usual lower-triangular self-attention mask). A row that sees
                           no key (only when M > L) outputs 0.                          */
} cf_mask;

/* The axis a row operation (softmax, LayerNorm, RMSNorm) reduces over.
 * CF_AXIS_ROW: over the columns n of each row m (the default). CF_AXIS_COLUMN:
 * over the rows m of each column n, through the tiles that share n -- the
 * complementary strip of the review's Eq. (1) argument (ComFuse review,
 * Referee Report major comment 1 on Sec. III). gamma/beta stay per column n;
 * row_stats then holds one statistic per column ([N], or [N, 2] for
 * LayerNorm). Column reductions: cf_gemm_epilogue with row_op softmax,
 * LayerNorm or RMSNorm, no second row stage, fast-path layouts (N a multiple
 * of 8, 16-byte aligned operands, leading dimensions multiples of 8 elements)
 * and M <= 65536; CF_ERR_UNSUPPORTED otherwise. */
typedef enum { CF_AXIS_ROW = 0, CF_AXIS_COLUMN = 1 } cf_axis;

/* Epilogue descriptor. The stages run in this fixed order on the fp32
 * accumulator of P = A.B (ComFuse review, "What carries the argument":
 * elementwise nodes stream over the accumulator fragments, the reduction is a
 * stage boundary):
 *   1. x = alpha * P
 *   2. x += bias[n]                (if bias != NULL)
 *   3. x += residual[m, n]         (if residual != NULL)
 *   4. x = act(x)
 *   5. row operation (row_op), with gamma/beta/eps
 *   6. cast to the output dtype (round to nearest even for bf16) and store.
 * bias, gamma and beta are vectors of N elements of dtype `vec_dtype`;
 * residual is an [M, N] matrix of dtype `residual_dtype` with leading
 * dimension ld_residual.
 *
 * Second output (x_out, optional, cf_gemm_epilogue only): the result of stage
 * 4, the x that the row operation reads, is also cast to x_out_dtype and
 * stored to x_out ([M, N], leading dimension ld_x_out, caller-owned device
 * memory that must not overlap C, A, B or the residual). The epilogue is then
 * a dataflow graph with two sinks, one on each side of the reduction boundary
 * (the review's "What carries the argument": the epilogue is split into
 * chained DAGs at its reductions); a pre-norm transformer block uses it to
 * keep the new residual stream x = P + residual beside y = RMSNorm(x). In the
 * stored X only the cast rounds: x is the same fp32 value the row operation
 * consumes. NULL (the default from cf_epilogue_init) stores nothing.
 *
 * Row statistics (row_stats, optional, fp32, caller-owned device memory): the
 * per-row result of the reduction stage itself (the review's "Reading between
 * the lines": other single-axis reductions such as log-sum-exp), as a
 * backward pass needs it:
 *   CF_ROW_SOFTMAX   row_stats[m]         = ln sum_n exp(x[m, n])  (log-sum-exp)
 *   CF_ROW_LAYERNORM row_stats[2m], [2m+1] = mean, 1 / sqrt(var + eps)
 *   CF_ROW_RMSNORM   row_stats[m]         = 1 / sqrt(mean_n x^2 + eps)
 *   CF_ROW_ARGMAX    row_stats[m]         = max_n x[m, n]
 * cf_b2bgemm (softmax only): row_stats[b * M + m] = ln sum_l exp(alpha * S[m, l])
 * over the visible keys; -inf for a causal row that sees none.
 * Must be 4-byte aligned; CF_ERR_INVALID_ARGUMENT with CF_ROW_NONE.
 *
 * Second row stage (row_op2, optional, cf_gemm_epilogue only): a second
 * reduction boundary in the same epilogue (the review's "What carries the
 * argument": an epilogue is a chain of DAGs cut at each reduction). With y the
 * output of the first row operation (after its gamma/beta), C receives
 *   z = row_op2(y) over the same row, with gamma2, beta2 and eps2
 * (meanings as for the first stage; vec_dtype for both vector sets). row_op
 * must then be CF_ROW_SOFTMAX, CF_ROW_LAYERNORM or CF_ROW_RMSNORM and row_op2
 * one of these three (CF_ERR_INVALID_ARGUMENT otherwise, also for gamma2/beta2
 * or eps2 set without row_op2 and beta2 without CF_ROW_LAYERNORM). row_stats,
 * if given, holds the first stage's statistics and x_out the first stage's
 * input x. The workspace then holds a second set of exchange slots
 * (cf_gemm_epilogue_workspace_size counts them). Two stages run only where
 * the fast path does: N, K and every leading dimension multiples of 8 (of 4
 * for fp32 inputs), 16-byte aligned matrices, no fp32 residual
 * (CF_ERR_UNSUPPORTED otherwise). cf_b2bgemm: row_op2 must be CF_ROW_NONE
 * (CF_ERR_UNSUPPORTED). */
typedef struct cf_epilogue {
  uint32_t struct_size;     /* must be sizeof(cf_epilogue)                        */
  float alpha;
  const void* bias;
  const void* residual;
  int64_t ld_residual;
  cf_dtype residual_dtype;
  cf_dtype vec_dtype;       /* dtype of bias, gamma and beta                      */
  cf_act act;
  cf_row_op row_op;
  const void* gamma;
  const void* beta;
  float eps;
  void* x_out;              /* optional second output: x after stage 4 (see above) */
  int64_t ld_x_out;         /* leading dimension of x_out in elements, >= N       */
  cf_dtype x_out_dtype;     /* CF_BF16 or CF_F32                                  */
  cf_mask mask;             /* cf_b2bgemm with row_op CF_ROW_SOFTMAX only         */
  float* row_stats;         /* optional fp32 per-row statistics of the row op (see below) */
  int32_t* row_index;       /* CF_ROW_ARGMAX: [M] column of each row's maximum (required) */
  cf_row_op row_op2;        /* optional second row stage on the first one's output (below) */
  const void* gamma2;       /* its LayerNorm gamma / RMSNorm weight, N of vec_dtype, or NULL */
  const void* beta2;        /* its LayerNorm beta, or NULL                               */
  float eps2;
  int32_t topk;             /* CF_ROW_TOPK: k (1..8); 0 otherwise                  */
  cf_axis axis;             /* the row op's reduction axis (CF_AXIS_ROW unless set) */
} cf_epilogue;

/* Fills *epi with the identity epilogue (alpha 1, no bias/residual/act/row op). */
void cf_epilogue_init(cf_epilogue* epi);

/* Bytes of device workspace cf_gemm_epilogue needs for this problem. Zero when
 * no exchange between workgroups is needed (no row operation, or N fits in one
 * 256-column tile). The workspace holds the per-strip partial row statistics
 * (level 3 of the review's three-level reduction, Fig. 4), a launch counter and
 * an error word. */
size_t cf_gemm_epilogue_workspace_size(int64_t M, int64_t N, int64_t K, const cf_epilogue* epi);

/* Clears a workspace (enqueued on `stream`). Must be called once after the
 * workspace is allocated and before its first use; a workspace may then be
 * reused by any number of calls of any shape on one stream at a time. Calls
 * that share a workspace on different streams concurrently race.
 * ws must be 256-byte aligned and ws_bytes >= 4096. */
cf_status cf_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Reads the workspace error word (blocking copy; call after the stream has
 * synchronised). Returns CF_ERR_DEVICE_TIMEOUT if a strip exchange wait timed
 * out since the last cf_workspace_init, otherwise CF_OK. The rows whose wait
 * timed out are NaN in every output of that call (row_index -1), so a timeout
 * is visible in the results without this check. Waits time out only when the
 * workgroups of one row strip do not run at the same time: the grid never
 * exceeds the kernel's co-resident capacity, but kernels of other streams or
 * processes on the same GPU can hold compute units meanwhile. */
cf_status cf_workspace_status(const void* ws, void* stream);

/* C[M,N] = epilogue(A[M,K] . B) -- one fused kernel; P is never written to
 * memory (ComFuse review, "The pith" and "If this is right": the MatMul's output
 * tiles flow into the normalisation while still on chip).
 *   A       [M, K] with leading dimension lda, dtype ab_dtype.
 *   B       [K, N] (b_is_nk = 0) or [N, K] (b_is_nk = 1, the nn.Linear weight
 *           layout) with leading dimension ldb, dtype ab_dtype.
 *   C       [M, N] with leading dimension ldc, dtype c_dtype. Must not overlap
 *           the inputs. May be NULL (ldc then unused) with CF_ROW_ARGMAX.
 *   ab_dtype CF_BF16 (bf16 MFMA, fp32 accumulation) or CF_F32 (fp32 MFMA).
 *   epi     epilogue descriptor (NULL = identity).
 *   ws      workspace of at least cf_gemm_epilogue_workspace_size() bytes,
 *           cleared once by cf_workspace_init(); may be NULL when that size is 0.
 *   epi->x_out (optional) receives x before the row operation, [M, N] with
 *           leading dimension epi->ld_x_out >= N, dtype epi->x_out_dtype,
 *           aligned to its element size; CF_ERR_INVALID_ARGUMENT otherwise.
 * M, N or K may be 0 (nothing is launched when M or N is 0; K = 0 gives P = 0).
 * Row operations need N <= 65536. */
cf_status cf_gemm_epilogue(int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda,
                           const void* B, int64_t ldb, int b_is_nk, cf_dtype ab_dtype,
                           void* C, int64_t ldc, cf_dtype c_dtype,
                           const cf_epilogue* epi, void* ws, size_t ws_bytes, void* stream);

/* cf_gemm_epilogue without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels, results and
 * errors as cf_gemm_epilogue, minus ws/ws_bytes: the strip exchange uses a
 * static device array of the library (16 MiB = 16777216 bytes per GPU, held
 * by each GPU the library runs on until the process ends). A problem whose
 * cf_gemm_epilogue_workspace_size() exceeds 16 MiB returns CF_ERR_WORKSPACE
 * before any HIP call. The first call on a device enqueues a clear of the
 * array on `stream`; no call allocates or frees memory. All calls on one GPU
 * share that array: calls that overlap in time on one GPU (concurrent
 * streams, or threads) race and must be serialised by the caller. A strip
 * exchange that times out leaves the rows concerned NaN (as in
 * cf_gemm_epilogue); its status word is not readable through this entry. */
cf_status cf_gemm_epilogue_noalloc(int64_t M, int64_t N, int64_t K,
                                   const void* A, int64_t lda,
                                   const void* B, int64_t ldb, int b_is_nk, cf_dtype ab_dtype,
                                   void* C, int64_t ldc, cf_dtype c_dtype,
                                   const cf_epilogue* epi, void* stream);

/* Back-to-back GEMM, one fused kernel per call (ComFuse review, Referee Report
 * major comment 2, paper Sec. IV-A, Eqs. (2)-(5); Fig. 5):
 *   S = alpha * A . B0 (+ bias[l]),  P = F(S),  O = P . B1
 * for each of `batch` independent problems. The intermediate S/P [M, L] stays
 * in registers and LDS and is never written to memory.
 *   A   [M, K], leading dimension lda, batch stride sa.
 *   B0  [K, L] (b0_is_lk = 0) or [L, K] (b0_is_lk = 1, e.g. attention keys),
 *       leading dimension ldb0, batch stride sb0 (0 = shared by all batches).
 *   B1  [L, N], leading dimension ldb1, batch stride sb1 (0 = shared).
 *   O   [M, N], leading dimension ldo, batch stride so.
 *   mid epilogue on S: alpha, bias (vector of L), act, and row_op in
 *       {CF_ROW_NONE, CF_ROW_SOFTMAX}; residual/gamma/beta/x_out must be NULL
 *       (CF_ERR_UNSUPPORTED otherwise: S is never stored). With row_op
 *       CF_ROW_SOFTMAX, bias and act must be unset (CF_ERR_UNSUPPORTED: the
 *       softmax takes alpha * S as it is); mask = CF_MASK_CAUSAL hides the scores of keys
 *       l > m + L - M before the softmax (causal attention; the review's
 *       Self-Attention workload, Referee Report major comment 3); key segments
 *       that no row of a tile can see are not computed.
 * The second GEMM takes P in bf16 (the MFMA operand type); for the softmax the
 * operand is round(2^(t - c)) with t = log2(e) * S and an integer per-row c,
 * and the row sum used for normalisation is taken before rounding.
 * in_dtype must be CF_BF16; out_dtype CF_BF16 or CF_F32.
 * Any M, K, L, N and batch (each batch entry's operands below 2 GiB). K above
 * 128 is contracted in blocks of 128; N above 128 is computed in column
 * blocks of 128, each of which evaluates S and F again (the softmax gives
 * identical terms in every block). */
cf_status cf_b2bgemm(int64_t batch, int64_t M, int64_t K, int64_t L, int64_t N,
                     const void* A, int64_t lda, int64_t sa,
                     const void* B0, int64_t ldb0, int64_t sb0, int b0_is_lk,
                     const void* B1, int64_t ldb1, int64_t sb1,
                     void* O, int64_t ldo, int64_t so,
                     cf_dtype in_dtype, cf_dtype out_dtype, const cf_epilogue* mid,
                     void* stream);

/* Human-readable name of a status. Never NULL. */
const char* cf_status_string(cf_status s);

/* hipError_t of the last failing HIP call made by this thread (0 if none). */
int cf_last_hip_error(void);

/* Library version string. */
const char* cf_version(void);

/* Upper bound, in microseconds, of each strip-exchange wait (default 2e6).
 * A wait that exceeds it records CF_ERR_DEVICE_TIMEOUT in the workspace,
 * makes the rows concerned NaN and lets the kernel finish. Returns the
 * previous value. */
uint64_t cf_set_exchange_timeout_us(uint64_t us);

/* Default of cf_set_exchange_leader_tiles: 0, peer-to-peer for every strip.
 * On MI355X leader-follower measured slower at every strip width tried (16 to
 * 256 column tiles, K = 256 and 2048): its followers wait for two exchange
 * latencies, while the extra partials peer-to-peer reads come from L2 and the
 * last-level cache. */
#define CF_DEFAULT_LEADER_TILES 0

/* Aggregation mode of the strip exchange (ComFuse review, Referee Report minor
 * comment 4 on Sec. III-A and "Assumptions & free parameters": a dual-mode
 * scheme, peer-to-peer or leader-follower, switched at a strip width C_N the
 * pages leave open). In peer-to-peer mode every workgroup of a row strip reads
 * every other workgroup's per-row partial statistics; in leader-follower mode
 * the workgroup of column tile 0 merges them all and publishes the merged
 * statistics, which the others read. Both merge in column-tile order, so the
 * outputs are bit-identical; the mode changes only the exchange's traffic
 * (tiles^2 against 2 tiles partials per strip) and latency (one hop against
 * two). Exchange groups (row strips, or tile columns for a column
 * reduction) of at least `min_tiles` tiles of 256 use leader-follower,
 * narrower ones peer-to-peer; 0 means never (C_N here; default
 * CF_DEFAULT_LEADER_TILES). A negative value changes nothing. Returns the
 * previous value. Process-wide; applies to the first row stage (a second row
 * stage and top-k keep their own schemes). */
int cf_set_exchange_leader_tiles(int min_tiles);

/* Schedule of cf_b2bgemm's softmax (ComFuse review, "Assumptions & free
 * parameters": the Sec. III-C PingPong pipeline, two groups alternating
 * tensor-core and CUDA-core work). on = 1 selects, where it applies (row_op
 * CF_ROW_SOFTMAX without mask, K = N = 64, at least one 512-row tile per CU),
 * a workgroup of eight waves per CU whose two groups of four alternate an
 * MFMA phase and a softmax phase, a workgroup barrier between phases, with the
 * A rows and the B0/B1 segments in LDS. on = 0 (the default) keeps two
 * independent four-wave workgroups per CU whose MFMA blocks run at raised
 * wave priority. Both give the same results up to the order of the row-sum
 * additions. On MI355X at batch 512, M = L = 1024, the ping-pong schedule
 * measured no faster (each phase waits at the barrier for the slowest of eight
 * waves, and the softmax phase alone takes about as long as both MFMA GEMMs).
 * A negative value changes nothing. Returns the previous value. Process-wide. */
int cf_set_b2b_pingpong(int on);

#ifdef __cplusplus
}
#endif

#endif /* CF_H_ */
