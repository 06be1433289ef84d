/*
 * lmhead.h -- C ABI of liblmhead.so: the LM output layer with FP32 logits and
 * a fused FP32 vocabulary cross-entropy, hand-written HIP for gfx950 (MI355X).
 *
 * Sources the operations follow (cited by page title and section):
 *  [MIXED] Megatron-LM pull request "Add mixed-precision (FP32) LM output
 *          logits": section "What does this PR do?" (the output-layer GEMM
 *          keeps its FP32 accumulator as FP32 logits instead of rounding each
 *          logit to BF16; the backward casts the logits gradient to BF16 for
 *          the GEMMs that follow) and section "Tests" (the logit dtype option
 *          accepts bf16 and fp32 and rejects fp16).
 *  [XENT]  Transformer Engine issue "[Pytorch] change fused cross entropy
 *          backward grad to fp32 and reduce one read/...": sections
 *          "Description" and "Changes" (the backward gradient is computed in
 *          FP32; one logits read is removed) and the discussion (the forward
 *          keeps the input, an n_rows x 1 target and an n_rows x 4 m_d_X_y
 *          record; the original kernel wrote the gradient over its input).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers on the current HIP device.  The
 *    caller owns every buffer; the library allocates nothing and keeps no
 *    state between calls.  Calls are thread-safe.
 *  - Matrices are row-major with a leading dimension `ld*` in ELEMENTS
 *    (row r starts at base + r * ld).  BF16 tensors are raw 16-bit words
 *    (the top half of an IEEE binary32).
 *  - Every call validates its arguments on the host first and returns a
 *    non-zero LMH_ERR_* code WITHOUT touching the GPU when they are invalid.
 *    Otherwise it enqueues its kernels on `stream` (a hipStream_t passed as
 *    void*, NULL = the default stream) and returns at once; LMH_ERR_LAUNCH
 *    reports a failed launch.  Results are ready when the stream reaches
 *    that point.
 *  - Alignment: every pointer 16-byte aligned; `ld` a multiple of 8 for BF16
 *    and of 4 for FP32 (LMH_ERR_ALIGN).  ld must be >= the row length, and
 *    a matrix may span at most 2^44 elements ((rows - 1) * ld + row length;
 *    the same for a stride between blocks of records) (LMH_ERR_SHAPE).  Sizes
 *    are >= 0; a zero-size output is a no-op.
 *    The GEMMs run fastest with 128-byte aligned rows (BF16 ld a multiple
 *    of 64); rows only 16-byte aligned are accepted but measured up to a
 *    third slower.
 *  - Padding between a row's end and the next row (ld > row length) is never
 *    written.
 *  - Results are bitwise deterministic run to run; no kernel uses floating
 *    point atomics.
 *  - No entry point allocates device memory, waits on the stream or the
 *    device, or enqueues a memset: calls made under stream capture record
 *    kernel launches only.
 *  - Launch limits: one kernel launch holds at most 2^31 work-items.  The
 *    cross-entropy calls that would need more (e.g. 2^25 rows, or 64-column
 *    blocks of 8192 x 131072 logits) run as several launches over row ranges,
 *    with the same results.  A GEMM call whose R x C output (logits: V x M,
 *    dgrad: K x M, wgrad: K x V) has ceil(R / 128) * ceil(C / 32) > 2^23
 *    (with a split V sum also 16 ceil(R / 256) ceil(C / 128) > 2^22 or
 *    C ceil(R / 4) > 2^31) returns LMH_ERR_SHAPE before anything is enqueued;
 *    such outputs are larger than a GPU's memory.
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  LMH_FP16 exists only so that it can be rejected ([MIXED],
 * "Tests": the logit dtype accepts bf16 and fp32 and rejects fp16). */
enum lmh_dtype { LMH_BF16 = 0, LMH_FP32 = 1, LMH_FP16 = 2 };

enum lmh_status {
    LMH_OK = 0,
    LMH_ERR_DTYPE = 1,  /* unsupported element type (fp16 or unknown)        */
    LMH_ERR_SHAPE = 2,  /* negative size, ld too small, bad stride or limit  */
    LMH_ERR_NULL = 3,   /* required pointer is NULL                          */
    LMH_ERR_ALIGN = 4,  /* pointer not 16-B aligned or ld not a multiple     */
    LMH_ERR_ALIAS = 5,  /* an output overlaps an input in an unsupported way */
    LMH_ERR_LAUNCH = 6, /* the HIP launch failed (see hipGetLastError)       */
    LMH_ERR_SCRATCH = 7 /* needs more than the fixed scratch array holds     */
};

/* Human-readable name of a status code (static string, never NULL). */
const char *lmhead_status_str(int32_t status);

/* Library ABI version (major * 100 + minor). */
int32_t lmhead_version(void);

/*
 * lmhead_logits -- logits[M x V] = x[M x K] . W[V x K]^T        ([MIXED])
 *
 *  x    BF16 activations, row-major [M x K], leading dimension ldx >= K.
 *  W    BF16 vocabulary weights, row-major [V x K] (K contiguous), ldw >= K.
 *  out  logits, row-major [M x V], ldo >= V, element type out_dtype:
 *         LMH_FP32 -- the FP32 MFMA accumulator stored as is (the new path);
 *         LMH_BF16 -- the same accumulator rounded to BF16, nearest-even (the
 *                     legacy path kept for comparison);
 *         LMH_FP16 or anything else -- LMH_ERR_DTYPE.
 *  Products of BF16 values are exact in FP32 and every sum is FP32; with
 *  integer operands whose partial sums stay below 2^24 the FP32 result is
 *  exact, independent of summation order.  K == 0 writes zeros.
 *  `out` must not overlap x or W (LMH_ERR_ALIAS).
 */
int32_t lmhead_logits(const void *x, int64_t ldx, const void *W, int64_t ldw,
                      void *out, int64_t ldo, int32_t out_dtype,
                      int64_t M, int64_t K, int64_t V, void *stream);

/*
 * lmhead_logits_xent -- FP32 logits plus their cross-entropy block records
 *
 *  The FP32 logits of lmhead_logits (out_dtype LMH_FP32) and, from the same
 *  FP32 accumulators, the records lmhead_xent_partial would write for those
 *  logits with block_cols = 256 and col0 = 0: for each 256-column block b of
 *  the vocabulary and each token i, part[b * part_stride + 4 i + {0..3}] =
 *  {m_b, d_b, X_b, own_b}.  lmhead_xent_merge (n_parts = ceil(V / 256),
 *  vocab = V) then gives the forward's stats without reading the logits:
 *  [XENT]'s point of removing a logits read ("Description"), carried into
 *  the GEMM's epilogue -- an extension the pages do not describe.  For
 *  shapes whose GEMM kernel lacks this epilogue (M <= 256, or operands too
 *  large for 32-bit tile offsets) the records are computed from the stored
 *  logits by a second kernel (one extra read), with the same meaning.
 *
 *  x, W, out as lmhead_logits (out FP32, ldo a multiple of 4).  target int32
 *  [M], global vocabulary indices; ignore_index as in the forward.
 *  part_stride >= 4 M and a multiple of 4; part 16-byte aligned.  out, part
 *  and target must not overlap each other or the operands.
 */
int32_t lmhead_logits_xent(const void *x, int64_t ldx, const void *W, int64_t ldw,
                           float *out, int64_t ldo, int64_t M, int64_t K, int64_t V,
                           const int32_t *target, int32_t ignore_index,
                           float *part, int64_t part_stride, void *stream);

/*
 * lmhead_xent_fwd -- fused cross-entropy forward over FP32 logits  ([XENT])
 *
 *  logits  FP32 [n_rows x n_cols], leading dimension ld >= n_cols; read once.
 *  target  int32 [n_rows]; a row whose target equals ignore_index is ignored.
 *  loss    FP32 [n_rows] per-row loss, or NULL to skip it.
 *  stats   FP32 [n_rows x 4], one 16-byte record per row:
 *            stats[i] = { m_i   = max_j z_ij,
 *                         d_i   = sum_j exp(z_ij - m_i),
 *                         X_i   = z_i,target_i,
 *                         loss_i = (m_i - X_i) + log d_i }.
 *          An ignored row stores {m_i, d_i, 0, 0} and loss 0.  A target that is
 *          neither ignore_index nor in [0, n_cols) cannot be reported from the
 *          kernel: that row stores X = NaN and loss = NaN.
 *  n_cols >= 1 when n_rows > 0.  stats and loss must not overlap the logits.
 */
int32_t lmhead_xent_fwd(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                        const int32_t *target, int32_t ignore_index,
                        float *loss, float *stats, void *stream);

/*
 * lmhead_xent_partial -- split-vocabulary CE forward, step 1        ([XENT])
 *
 *  The per-shard half of vocabulary-parallel cross entropy ([XENT],
 *  "Description", names Megatron's vocabulary-parallel CE as the FP32
 *  reference): the statistics of a slice of each logits row, per column
 *  block, to be combined by lmhead_xent_merge.  The same call serves a vocab
 *  shard of a larger model (col0 = the shard's first global column) and a
 *  single GPU that splits long rows into blocks so that few rows still fill
 *  the chip.
 *
 *  logits  FP32 [n_rows x n_cols], leading dimension ld; the slice holds the
 *          global columns [col0, col0 + n_cols).  Read once.
 *  block_cols  columns per block, a positive multiple of 4, at most
 *          INT32_MAX; the slice is cut into n_blocks = ceil(n_cols /
 *          block_cols) blocks (the last one may be shorter).  n_blocks * n_rows must not exceed INT32_MAX
 *          (LMH_ERR_SHAPE).
 *  target  int32 [n_rows], GLOBAL column indices; ignore_index as in the
 *          forward.
 *  part    FP32 output, n_blocks arrays of n_rows 16-byte records:
 *          part[b * part_stride + 4 i + {0,1,2,3}] =
 *            { m_b   = max of the row's block,
 *              d_b   = sum over the block of exp(z - m_b),
 *              X_b   = the target logit if col0 <= target_i - b block_cols
 *                      < col0 + (width of block b), else 0,
 *              own_b = 1 in that case, else 0 }   (ignored rows: X = own = 0).
 *          part_stride (elements) >= 4 n_rows and a multiple of 4.  part must
 *          not overlap the logits or the target.
 */
int32_t lmhead_xent_partial(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                            int64_t col0, int64_t block_cols, const int32_t *target,
                            int32_t ignore_index, float *part, int64_t part_stride,
                            void *stream);

/*
 * lmhead_xent_merge -- split-vocabulary CE forward, step 2          ([XENT])
 *
 *  Combines n_parts partial records per row (from one or more
 *  lmhead_xent_partial calls, at part + p * part_stride + 4 i for part p) in
 *  a fixed order (64 interleaved running pairs, then a butterfly), so the
 *  result is deterministic:  m = max m_p,  d = sum_p d_p exp(m_p - m),  X_y
 *  from the one part that owns the target,  loss = (m - X_y) + log d.
 *  Writes the same stats record and loss as lmhead_xent_fwd, so that
 *  lmhead_xent_bwd can run on the merged statistics.
 *
 *  vocab   total number of columns; a target outside [0, vocab) that is not
 *          ignore_index, or one owned by no part or by several, gives
 *          X = loss = NaN (m and d are still merged).  Ignored rows: X = loss = 0.
 *  loss    FP32 [n_rows] or NULL;  stats FP32 [n_rows x 4].
 *  n_parts >= 1, vocab >= 1, part_stride >= 4 n_rows and a multiple of 4.
 *  stats and loss must not overlap the parts or the target.
 */
int32_t lmhead_xent_merge(const float *part, int64_t n_parts, int64_t part_stride,
                          int64_t n_rows, const int32_t *target, int32_t ignore_index,
                          int64_t vocab, float *loss, float *stats, void *stream);

/*
 * lmhead_xent_mean -- mean reduction of the per-row loss
 *
 *  Not an operation the pages describe: they state no reduction.  The
 *  workloads this library is measured on take the mean loss over the rows
 *  whose target is not ignore_index (-100 there), the usual language-model
 *  training loss, and its 1 / n_valid is the upstream gradient of every row.
 *
 *  loss     FP32 [n_rows]; target int32 [n_rows] (rows equal to ignore_index
 *           are excluded).  loss may be NULL when mean_out is NULL: 1 / n_valid
 *           depends on the targets only, so it can be had before the forward
 *           (for lmhead_xent_fused).
 *  mean_out FP32 scalar: sum of valid losses / n_valid (0 if n_valid == 0),
 *           or NULL.
 *  inv_nvalid_out FP32 scalar: 1 / n_valid (0 if n_valid == 0), or NULL; it is
 *           the upstream gradient of every row of a mean loss and can be passed
 *           to lmhead_xent_bwd as `dloss` with dloss_stride 0.
 *  One workgroup sums in a fixed order (FP64), so the result is
 *  deterministic.  Both outputs NULL is a no-op.
 */
int32_t lmhead_xent_mean(const float *loss, const int32_t *target, int32_t ignore_index,
                         int64_t n_rows, float *mean_out, float *inv_nvalid_out,
                         void *stream);

/*
 * lmhead_xent_bwd -- fused cross-entropy backward in FP32          ([XENT])
 *
 *  dlogits_ij = dloss_i * (exp(z_ij - m_i) / d_i - [j == target_i]),
 *  computed in FP32 from the logits (read once more) and the stats record of
 *  lmhead_xent_fwd; rows whose target is ignore_index get zeros.
 *
 *  logits   FP32 [n_rows x n_cols], leading dimension ld.
 *  stats    FP32 [n_rows x 4] from lmhead_xent_fwd (m and d are used).
 *  target   int32 [n_rows]; ignore_index as in the forward.
 *  dloss    FP32 device pointer: dloss_i = dloss[dloss_stride * i] with
 *           dloss_stride 0 (one scalar for every row, e.g. the inv_nvalid
 *           output of lmhead_xent_mean) or 1 (one value per row).
 *  dlogits  [n_rows x n_cols], leading dimension ldg, type grad_dtype:
 *             LMH_FP32 -- FP32 gradient;
 *             LMH_BF16 -- the same FP32 value rounded to BF16 (nearest-even),
 *                         the cast the backward applies before the GEMMs
 *                         ([MIXED]);
 *           In place: dlogits == logits with ldg == ld and LMH_FP32 writes the
 *           gradient over the logits (each element is read, then overwritten
 *           by the same thread).  Any other overlap with logits, stats, target
 *           or dloss, or BF16 in place, is LMH_ERR_ALIAS.
 *  A target outside [0, n_cols) that is not ignore_index yields a NaN row.
 */
int32_t lmhead_xent_bwd(const float *logits, int64_t ld, const float *stats,
                        const int32_t *target, int32_t ignore_index,
                        const float *dloss, int64_t dloss_stride,
                        void *dlogits, int64_t ldg, int32_t grad_dtype,
                        int64_t n_rows, int64_t n_cols, void *stream);

/*
 * lmhead_xent_fused -- forward and backward in one read of the logits ([XENT])
 *
 *  For an upstream gradient known before the forward (a mean loss: dloss =
 *  1 / n_valid, which lmhead_xent_mean gives from the targets alone): writes
 *  the forward's loss and stats record (as lmhead_xent_fwd) and the
 *  backward's dlogits (as lmhead_xent_bwd) while reading the logits once.
 *  [XENT]'s discussion: the original fused kernel wrote the gradient over its
 *  input during the forward; the FP32 backward of [XENT] "Changes" is kept.
 *  Rows of up to 65536 columns are held in registers by one workgroup per
 *  row (8 bytes of traffic per element with FP32 gradients instead of 12);
 *  longer rows run the forward and then the backward (two reads).
 *
 *  Arguments as lmhead_xent_fwd (logits, ld, n_rows, n_cols, target,
 *  ignore_index, loss (may be NULL), stats) and lmhead_xent_bwd (dloss,
 *  dloss_stride, dlogits, ldg, grad_dtype, in place when dlogits == logits
 *  with ldg == ld and LMH_FP32).  The stats, loss and dlogits outputs must not
 *  overlap each other, the target or dloss; stats and loss must not overlap
 *  the logits.  Results agree with lmhead_xent_fwd + lmhead_xent_bwd to
 *  rounding (the row reduction runs over a different thread layout).
 */
int32_t lmhead_xent_fused(const float *logits, int64_t ld, int64_t n_rows, int64_t n_cols,
                          const int32_t *target, int32_t ignore_index,
                          const float *dloss, int64_t dloss_stride,
                          float *loss, float *stats,
                          void *dlogits, int64_t ldg, int32_t grad_dtype, void *stream);

/*
 * lmhead_dgrad -- input gradient dX[M x K] = dlogits[M x V] . W[V x K]
 *
 *  The GEMM that consumes the BF16 logits gradient ([MIXED]: the backward
 *  casts the gradient to BF16 for the following GEMMs).
 *  dlogits BF16 [M x V], ldd >= V;  W BF16 [V x K], ldw >= K;
 *  dX [M x K], ldx >= K, dx_dtype LMH_BF16 (nearest-even) or LMH_FP32.
 *  FP32 accumulation; V == 0 writes zeros.  dX must not overlap the inputs.
 */
int32_t lmhead_dgrad(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                     void *dX, int64_t ldx, int32_t dx_dtype,
                     int64_t M, int64_t K, int64_t V, void *stream);

/*
 * lmhead_dgrad_workspace_bytes / lmhead_dgrad_ws -- lmhead_dgrad with the sum
 * over V split in parts ([MIXED] "What does this PR do?", the GEMMs after the
 * BF16 cast: the same product dX = dlogits . W).
 *
 *  When M x K has too few 256 x 256 output tiles to fill the chip (fewer than
 *  256, e.g. M = 1024, K = 8192, or few tokens), the V sum is split `splits`
 *  ways; every part writes an FP32 partial dX into `workspace`, and a second
 *  kernel adds the partials in split order and stores dX (FP32, or BF16
 *  rounded to nearest-even once, from the FP32 sum).  splits == 0 picks the
 *  shape's default (1 - 16 parts, for ~256 workgroups); 1 <= splits <= 16
 *  asks for that many parts of whole 64-deep stages (fewer when V is small).
 *  The result is deterministic run to run; its summation order differs from
 *  lmhead_dgrad's, so the two agree within the FP32 tolerance, and bitwise on
 *  integer inputs.
 *
 *  lmhead_dgrad_workspace_bytes returns the workspace bytes that
 *  lmhead_dgrad_ws needs for (M, K, V, splits): parts x M x K4 x 4 with K4 =
 *  K rounded up to a multiple of 4, or 0 when the shape runs unsplit; a
 *  negative LMH_ERR_SHAPE for negative sizes, splits outside [0, 16], or a dX
 *  of more than 2^44 elements.
 *
 *  lmhead_dgrad_ws takes lmhead_dgrad's arguments plus splits and the
 *  caller's device workspace (16-byte aligned, workspace_bytes >= the size
 *  above, else LMH_ERR_ALIGN / LMH_ERR_SHAPE; NULL -> LMH_ERR_NULL).  The
 *  workspace must not overlap dlogits, W or dX (LMH_ERR_ALIAS); its contents
 *  on entry do not matter and are garbage afterwards.  When the size above is
 *  0 the call is lmhead_dgrad and the workspace is not touched.  Two calls that
 *  share a workspace must be ordered on one stream.
 */
int64_t lmhead_dgrad_workspace_bytes(int64_t M, int64_t K, int64_t V, int32_t splits);
int32_t lmhead_dgrad_ws(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                        void *dX, int64_t ldx, int32_t dx_dtype,
                        int64_t M, int64_t K, int64_t V, int32_t splits,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * lmhead_dgrad_noalloc -- lmhead_dgrad_ws with no workspace argument and no
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 *  Same arguments, split choice, kernels and results as lmhead_dgrad_ws
 *  (bitwise, for the same splits); the FP32 partial sums go to a fixed device
 *  array of LMH_DGRAD_NOALLOC_MAX_BYTES (64 MiB) that the library holds on
 *  each GPU it runs on until the process ends.  Shapes whose split needs more
 *  than that (lmhead_dgrad_workspace_bytes(M, K, V, splits) >
 *  LMH_DGRAD_NOALLOC_MAX_BYTES) return LMH_ERR_SCRATCH before anything is
 *  enqueued; shapes that run unsplit are lmhead_dgrad.  The first call on a
 *  device looks up the array's device address (with that device current); the
 *  call never allocates, frees or clears memory.  Every call on one GPU
 *  shares that GPU's array: calls that may overlap on one GPU (different
 *  streams, or host threads without ordering) race and must be serialised
 *  by the caller.  Nothing needs the array zeroed: every partial is written
 *  before it is read.
 */
#define LMH_DGRAD_NOALLOC_MAX_BYTES (((int64_t)64) << 20)
int32_t lmhead_dgrad_noalloc(const void *dlogits, int64_t ldd, const void *W, int64_t ldw,
                             void *dX, int64_t ldx, int32_t dx_dtype,
                             int64_t M, int64_t K, int64_t V, int32_t splits, void *stream);

/*
 * lmhead_wgrad -- weight gradient dW[V x K] (+)= dlogits[M x V]^T . x[M x K]
 *
 *  The other GEMM that consumes the BF16 logits gradient ([MIXED] "What does
 *  this PR do?": the backward casts the gradient to BF16 for the GEMMs that
 *  follow).  The pages say nothing of dW's type; it is kept in FP32 (the
 *  GEMM's accumulator), so that it can be accumulated over micro-batches.
 *
 *  dlogits BF16 [M x V], ldd >= V;  x BF16 [M x K], ldx >= K;
 *  dW FP32 [V x K], ldw >= K.  accumulate == 0 overwrites dW; accumulate != 0
 *  adds the product to the FP32 values already in dW.  FP32 accumulation over
 *  M; M == 0 writes zeros (or leaves dW unchanged when accumulating).
 *  dW must not overlap the inputs.
 */
int32_t lmhead_wgrad(const void *dlogits, int64_t ldd, const void *x, int64_t ldx,
                     float *dW, int64_t ldw, int32_t accumulate,
                     int64_t M, int64_t K, int64_t V, void *stream);

/*
 * lmhead_diag_mfma_loop -- diagnostic: the sustained BF16 matrix-core rate.
 *
 *  Not a step of the method: a register-only loop that the benchmark runs
 *  beside the GEMMs so their throughput can be compared with what the chip
 *  sustains under full matrix load at its power limit (the datasheet peak
 *  assumes 2.4 GHz).  n_workgroups workgroups of 256 threads (4 waves) each
 *  run 8 independent chains of `iters` 32x32x16 BF16 MFMAs:
 *  2 * 32 * 32 * 16 * 8 * iters FLOP per wave, 4 waves per workgroup.
 *  operands selects the data, which sets how much the multipliers switch and
 *  so the power drawn:
 *    0  every operand 1.0.  sink FP32 [n_workgroups * 256] receives, per
 *       thread, 128 * iters exactly (the sum of element 0 of its 8
 *       accumulators), which checks that every MFMA ran.
 *    1  pseudo-random BF16 operands (random sign and 7 mantissa bits, |v| in
 *       [1, 2), a different set per lane) cycling through (A1, B1), (A2, B2),
 *       (A1, -B1), (A2, -B2), so every accumulator returns to exactly 0 each
 *       fourth MFMA of its chain (all partial sums are exact in FP32).  sink
 *       receives, per thread, element 0 of its 8 accumulators weighted
 *       1 ... 8: 0 when iters % 4 == 0, and for other iters a value that
 *       depends only on iters % 4.
 *  Limits: operands in {0, 1}, 0 <= iters, 128 * iters < 2^24 and
 *  0 <= n_workgroups <= 65536, else LMH_ERR_SHAPE; n_workgroups == 0 is a
 *  no-op.  sink must not be NULL (LMH_ERR_NULL) and 16-byte aligned.
 */
int32_t lmhead_diag_mfma_loop(int64_t iters, int64_t n_workgroups, int32_t operands,
                              float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
