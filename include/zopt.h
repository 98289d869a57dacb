/*
 * zopt.h -- one data-parallel rank's optimizer step under ZeRO-style
 * sharding, on AMD Instinct MI355X (gfx950).
 *
 * libzopt holds two optimizers that a ZeRO-sharded trainer runs on each rank
 * after its gradients are in place:
 *
 *  - zopt_adamw_shard_step: AdamW over the rank's flat, bucket-padded fp32
 *    master shard, in one pass that reads the bf16 gradient, updates the fp32
 *    master and both fp32 moments, and writes the bf16 compute weights;
 *  - zopt_muon_step: Muon on whole 2-D matrices the rank owns (momentum with
 *    Nesterov look-ahead, Newton-Schulz orthogonalisation on bf16 matrix
 *    cores, a decayed and scaled update of the fp32 master), and
 *    zopt_muon_step_groups, the same on several shapes in one call, with
 *    zopt_muon_step_groups_guarded adding the Newton-Schulz health checks,
 *    and zopt_muon_graph_* capturing a call once for replay each step;
 *  - zopt_round_bf16: the fp32 -> bf16 round-to-nearest-even write-back on
 *    its own;
 *  - zopt_grad_sq_norm, zopt_grad_clip_stats and zopt_adamw_shard_step_clipped:
 *    the gradient norm of the shard, the clip statistics, and the AdamW step
 *    taking its gradient scale from them in device memory.
 *
 * Conventions common to every call
 * --------------------------------
 *  - Every buffer is device memory owned by the caller.  The library
 *    allocates no device memory at run time and keeps no state between calls,
 *    with five exceptions: a captured Muon graph is a handle the caller owns;
 *    zopt_set_ns_workgroup_limit is a process-wide setting that every later
 *    call in the process uses (one thread's setting changes the launch plan,
 *    never the results, of another's calls); zopt_set_ns_form is another,
 *    which selects how Newton-Schulz is computed (and so changes results
 *    within bf16 rounding, and the workspace size); zopt_grad_sq_norm_noalloc
 *    uses a 16 KiB array per GPU that the library holds for the life of the
 *    process; and a grouped Muon call whose Newton-Schulz launches are short
 *    (see zopt_muon_step_groups) uses a second stream per GPU, with two
 *    events, that the library creates at the first such call and holds for
 *    the life of the process.  Every other call is reentrant.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without synchronising.  All launch parameters travel
 *    as kernel arguments, so back-to-back calls need no host sync.
 *  - Arguments are checked before anything is enqueued.  On any status other
 *    than ZOPT_OK nothing has been enqueued and no buffer has been touched,
 *    except ZOPT_ERR_DEVICE, which reports a failed launch.
 *  - NaN and Inf in the data are not reported; they propagate as IEEE
 *    arithmetic dictates.
 *  - Buffers must not overlap.  No alignment is required; bases aligned to
 *    16 bytes take the 128-bit vector path.
 *  - bf16 is the upper half of an IEEE binary32, carried as uint16_t.
 *  - Rounding to bf16 is round-to-nearest, ties to even, with no flush of
 *    subnormals; a value beyond the largest finite bf16 becomes infinity and
 *    a NaN becomes 0x7FC0 -- what a cast of an fp32 tensor to bf16 yields
 *    [DEG zero.py, ZeroMaster docstring and gather_params: the updated shard
 *    is rounded to bf16, bitwise the unsharded trainer's copy of the master
 *    into the bf16 weights].
 *  - Per-step scalars derived from the hyperparameters are formed in double
 *    on the host and rounded once to binary32; the elementwise arithmetic is
 *    binary32 with no fused multiply-adds, in the order stated below.
 */
#ifndef ZOPT_H
#define ZOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZOPT_OK = 0,
    ZOPT_ERR_NULL = 1,      /* a required pointer is NULL                       */
    ZOPT_ERR_SIZE = 2,      /* a size, count, rank or shard length is invalid   */
    ZOPT_ERR_HYPER = 3,     /* a hyperparameter is out of its domain            */
    ZOPT_ERR_WORKSPACE = 4, /* workspace too small or not 256-byte aligned      */
    ZOPT_ERR_DEVICE = 5     /* the HIP runtime reported a launch failure        */
} zopt_status;

/* A static, human-readable name of a status code. */
const char *zopt_status_string(zopt_status status);

/*
 * zopt_adamw_shard_step -- one AdamW step over rank `rank`'s shard.
 *
 * Layout [DEG zero.py: ZeroMaster module docstring, ZeroMaster.__init__,
 * reduce_scatter, gather_params].  The trainable parameters lie end to end in
 * a flat vector of N elements.  The bucket length is lowered to a multiple of
 * `world` (never below `world`): B = max(world, bucket - bucket % world).
 * Buckets [s, e) tile [0, N); bucket b has padded length
 * L_b = ceil((e - s) / world) * world and is cut into `world` equal pieces
 * of p_b = L_b / world elements.  Rank r owns piece r of every bucket; its
 * shard is those pieces concatenated, so shard_len = sum_b p_b.  Shard
 * element j of bucket b (shard offset o_b = sum of earlier pieces) is flat
 * element f = s_b + r * p_b + (j - o_b); it is padding when f >= e_b.
 *
 * Per shard element, in this order [dmuon PR #16, commit "foreach AdamW":
 * decoupled weight decay, then the moments, then the bias-corrected addcdiv,
 * bias corrections being per-step scalars of the post-increment step;
 * BluScript trainer source, optimizer-precision note: the decay is a
 * (1 - lr*wd) multiply on fp32 masters and moments; DeepSpeed PR #9021,
 * commits "bf16 gradients of fp32 params" (the bf16 gradient is promoted in
 * registers) and "grad_scale" (multiplied as each element is loaded, after
 * the promotion)]:
 *
 *   g  = fp32(grad[f]) * grad_scale          (g = 0 on padding)
 *   p  = p * decay
 *   m  = beta1 * m + omb1 * g
 *   v  = beta2 * v + (omb2 * g) * g
 *   p  = p - step_size * (m / (sqrt(v) / bc2_sqrt + eps))
 *   weight[f] = bf16(p)                      (real elements only)
 *
 * with t = step and, in double rounded once to binary32,
 *   step_size = lr / (1 - beta1^t),  bc2_sqrt = sqrt(1 - beta2^t),
 *   decay = 1 - lr * weight_decay,   omb1 = 1 - beta1,  omb2 = 1 - beta2.
 * The gradient here is this rank's contribution as it stands: the sum over
 * ranks (a reduce-scatter) is not part of this call; an average over ranks
 * is grad_scale = 1/world.
 *
 * Arguments
 *   master, exp_avg, exp_avg_sq  fp32 [shard_len], device, read and written.
 *                                Padding positions are stepped with g = 0.
 *   grad      bf16 [N] flat gradient, device, read only at this rank's real
 *             elements.
 *   weight    bf16 [N] flat compute weights, device, written only at this
 *             rank's real elements; NULL skips the write-back.
 *   N, bucket, world, rank, shard_len   the layout above; shard_len must equal
 *             the value it derives from (N, bucket, world).
 *   lr, beta1, beta2, eps, weight_decay, step, grad_scale   as above; step
 *             is 1 on the first update (already incremented by the caller).
 *   stream    hipStream_t or NULL.
 *
 * Errors: ZOPT_ERR_NULL (master, exp_avg, exp_avg_sq or grad NULL);
 * ZOPT_ERR_SIZE (N < 1, bucket < 1, world < 1, rank outside [0, world),
 * shard_len wrong); ZOPT_ERR_HYPER (lr < 0 or not finite, beta outside
 * [0, 1), eps <= 0 or not finite, weight_decay < 0 or not finite, step < 1,
 * grad_scale not finite); ZOPT_ERR_DEVICE.
 */
zopt_status zopt_adamw_shard_step(float *master, float *exp_avg, float *exp_avg_sq,
                                  const uint16_t *grad, uint16_t *weight,
                                  int64_t N, int64_t bucket, int32_t world,
                                  int32_t rank, int64_t shard_len,
                                  float lr, float beta1, float beta2, float eps,
                                  float weight_decay, int64_t step, float grad_scale,
                                  void *stream);

/*
 * Gradient clipping without a host round trip.  A ZeRO rank clips on the
 * norm of the whole summed gradient: each rank squares and sums its own real
 * gradient elements, the ranks' sums are added (an all-reduce, not part of
 * this library), and the clip coefficient derived from the total scales the
 * gradient as the AdamW step loads it [DEG zero.py: ZeroMaster.grad_sq_norm;
 * BluScript trainer source, cross-group global clipping block: coefficient
 * min(1, clip / (norm + 1e-6)), and the Muon path does not apply it; DeepSpeed
 * PR #9021, commit "grad_scale": the factor is multiplied in as each gradient
 * element is loaded].  The statistics stay in device memory as binary32
 * scalars, so nothing waits for the host [dmuon PR #16, commit "device-tensor
 * stats": total_norm / clip_coef / clipped / found_inf as device scalars,
 * finiteness judged on the norm, so an infinite norm reports found_inf and
 * not clipped].  A clipped step is three calls on one stream:
 *
 *   zopt_grad_sq_norm(grad, ..., sq, ws, &ws_bytes, s);     per rank
 *   (all-reduce sq over ranks, or pass the per-rank sums to the next call)
 *   zopt_grad_clip_stats(sq, 1, max_norm, inv_scale, stats, s);
 *   zopt_adamw_shard_step_clipped(..., stats, skip_nonfinite, s);
 */

/* Layout of the clip statistics: ZOPT_CLIP_STATS binary32 values. */
enum {
    ZOPT_CLIP_TOTAL_NORM = 0, /* fp32(sqrt(sum of squares) * inv_scale)            */
    ZOPT_CLIP_COEF = 1,       /* min(1, max_norm / (total_norm + 1e-6)), binary32   */
    ZOPT_CLIP_CLIPPED = 2,    /* 1 if !found_inf and clip_coef < 1, else 0          */
    ZOPT_CLIP_FOUND_INF = 3,  /* 1 if total_norm is not finite, else 0              */
    ZOPT_CLIP_GRAD_SCALE = 4, /* inv_scale * clip_coef: the AdamW gradient factor   */
    ZOPT_CLIP_STATS = 5
};

/*
 * zopt_grad_sq_norm -- *sq = the sum of the squares of rank `rank`'s real
 * gradient elements (the layout of zopt_adamw_shard_step; padding and other
 * ranks' positions are not read).  Each square is exact in double and the sum
 * is double, in an order fixed by shard_len alone: the result is the same on
 * every run.
 *
 * Arguments
 *   grad      bf16 [N] flat gradient, device, read.
 *   N, bucket, world, rank, shard_len   as for zopt_adamw_shard_step.
 *   sq        one double, device, written.
 *   workspace device scratch, 256-byte aligned, of at least the size the
 *             NULL-workspace query writes to *workspace_bytes (at most 16 KiB);
 *             with workspace == NULL the call only writes that size.
 *   stream    hipStream_t or NULL.
 *
 * Errors: ZOPT_ERR_NULL (workspace_bytes NULL; grad or sq NULL with a
 * workspace); ZOPT_ERR_SIZE (the layout arguments as for
 * zopt_adamw_shard_step); ZOPT_ERR_WORKSPACE; ZOPT_ERR_DEVICE.
 */
zopt_status zopt_grad_sq_norm(const uint16_t *grad, int64_t N, int64_t bucket, int32_t world,
                              int32_t rank, int64_t shard_len, double *sq, void *workspace,
                              size_t *workspace_bytes, void *stream);

/*
 * zopt_grad_sq_norm_noalloc -- zopt_grad_sq_norm for callers that cannot
 * allocate device memory (code under stream capture, tight training loops,
 * harnesses that forbid allocation): the same sum, bit for bit, with the
 * partial sums kept in a scratch array inside the library instead of a
 * caller's workspace.  The array is 16 KiB per GPU (2048 doubles, the most
 * partials any shard length needs), allocated when the library is loaded and
 * held until the process ends; the call itself allocates nothing.  Every
 * call on one GPU uses that GPU's one array, so calls that may overlap on a
 * GPU (different streams, or different host threads without ordering) race
 * and must not be issued; calls in one stream are ordered and safe.  The
 * array needs no clearing: each call writes every partial it reads.
 *
 * Arguments as zopt_grad_sq_norm, without workspace and workspace_bytes.
 *
 * Errors: ZOPT_ERR_NULL (grad or sq NULL); ZOPT_ERR_SIZE (the layout
 * arguments as for zopt_adamw_shard_step); ZOPT_ERR_WORKSPACE (the partials
 * would exceed the array -- no valid layout does); ZOPT_ERR_DEVICE (the
 * array's address could not be found on the current device, or a launch
 * failed).
 */
zopt_status zopt_grad_sq_norm_noalloc(const uint16_t *grad, int64_t N, int64_t bucket,
                                      int32_t world, int32_t rank, int64_t shard_len,
                                      double *sq, void *stream);

/*
 * zopt_grad_clip_stats -- the clip statistics (layout above) from `count`
 * sums of squares, added in index order in double:
 *   total_norm = fp32(sqrt(sum) * inv_scale)
 *   clip_coef  = min(1, max_norm / (total_norm + 1e-6f)), binary32; an
 *                infinite norm gives 0, a NaN norm gives NaN
 *   clipped    = !found_inf && clip_coef < 1,  found_inf = !isfinite(total_norm)
 *   grad_scale = inv_scale * clip_coef
 *
 * Arguments
 *   sq         `count` doubles, device, read (per-rank sums, or one total).
 *   count      1 .. 65536.
 *   max_norm   > 0 (+inf reports the norm without clipping).
 *   inv_scale  finite, > 0: the gradients are a loss scale times the true
 *              ones; 1 = none.
 *   stats      ZOPT_CLIP_STATS floats, device, written.
 *   stream     hipStream_t or NULL.
 *
 * Errors: ZOPT_ERR_NULL; ZOPT_ERR_SIZE (count); ZOPT_ERR_HYPER (max_norm,
 * inv_scale); ZOPT_ERR_DEVICE.
 */
zopt_status zopt_grad_clip_stats(const double *sq, int32_t count, float max_norm,
                                 float inv_scale, float *stats, void *stream);

/*
 * zopt_adamw_shard_step_clipped -- zopt_adamw_shard_step with grad_scale
 * read from device memory when the kernel runs: grad_scale =
 * clip_stats[ZOPT_CLIP_GRAD_SCALE].  With skip_nonfinite = 1 a step whose
 * clip_stats[ZOPT_CLIP_FOUND_INF] is non-zero writes nothing (master, moments
 * and weights keep their values); the step count is the caller's, who may
 * read found_inf later and not count that step.  Every other argument,
 * and the arithmetic, as zopt_adamw_shard_step: given the same grad_scale
 * value the two calls give the same bits.
 *
 * Errors: those of zopt_adamw_shard_step; ZOPT_ERR_NULL also for clip_stats
 * NULL; ZOPT_ERR_HYPER also for skip_nonfinite not 0/1.
 */
zopt_status zopt_adamw_shard_step_clipped(float *master, float *exp_avg, float *exp_avg_sq,
                                          const uint16_t *grad, uint16_t *weight, int64_t N,
                                          int64_t bucket, int32_t world, int32_t rank,
                                          int64_t shard_len, float lr, float beta1, float beta2,
                                          float eps, float weight_decay, int64_t step,
                                          const float *clip_stats, int32_t skip_nonfinite,
                                          void *stream);

/*
 * zopt_shard_len -- the shard length every rank holds for a flat vector of N
 * elements in buckets of `bucket` over `world` ranks (the layout above:
 * sum over buckets of ceil(len_b / world)).  Host-only; enqueues nothing.
 * Returns -1 if N < 1, bucket < 1 or world < 1.
 */
int64_t zopt_shard_len(int64_t N, int64_t bucket, int32_t world);

/*
 * zopt_muon_step -- one Muon step on `batch` matrices of one stored shape
 * [rows, cols] (row-major, PyTorch's [out, in]), each owned whole by this
 * rank [BluScript trainer source, ShardedMuon comment block: Newton-Schulz is
 * a whole-matrix operator, so Muon shards by whole parameter, the owner
 * holding the matrix's fp32 master and momentum; dmuon PR #16, commit "NS
 * CUDA-graph replay": Newton-Schulz runs on a small stable set of shapes,
 * lr / wd / momentum stay in the pre- and post-steps around it].
 *
 * Per matrix, in this order:
 *   1. Momentum [BluScript trainer source, Muon config block: momentum 0.95,
 *      Nesterov; the buffer is an exponential moving average]:
 *        g = fp32(grad);  M = mu * M + omm * g;
 *        U = omm * g + mu * M  (nesterov)   or   U = M   (otherwise)
 *      with mu = momentum_beta and omm = fp32(1 - mu) formed in double.
 *   2. Pre-scale: X0 = s U, s = 1 / (||U||_F + ns_eps), ||U||_F^2 a
 *      fixed-order (run-to-run deterministic) fp64 sum of the exact squares
 *      and s formed in double; X0 is taken transposed when rows > cols, so X
 *      is m x n with m = min(rows, cols).  With ns_steps = 0,
 *      X0 = bf16(U * s) (the product in double) is the result.  Otherwise,
 *      when 2^-60 <= ||U||_F^2 <= 2^100, X0 is never stored: the first
 *      iteration reads bf16(U) and applies s in fp32 to its products (s^2 to
 *      X X^T, s to B X), which in that range can neither overflow nor lose
 *      precision to underflow; outside it (huge or tiny gradients, Inf, NaN)
 *      X0 = bf16(U * s) is written first and the iteration reads that.
 *   3. ns_steps Newton-Schulz iterations [BluScript trainer source, ShardedMuon
 *      comment block: X <- aX + (bXX' + c(XX')^2)X]:
 *        A = X X^T;  B = b A + c A A;  X = a X + B X
 *      on bf16 matrix cores with fp32 accumulation; A, B and X are rounded to
 *      bf16 after each product; only the upper triangle of the symmetric A
 *      and B is computed and mirrored.  Where the long side is at least twice
 *      the short one (n >= 2 m), m <= 4096 and the group is large enough for
 *      the flops saved to pay for two more launches (batch m^2 (n - m) >=
 *      2^29; a rule on the group alone) the same polynomial map runs in
 *      segments of
 *      up to three steps on the m x m Gram matrix: with A_j = X_j X_j^T and
 *      P_j = a I + b A_j + c A_j^2, X_{j+1} = P_j X_j gives A_{j+1} =
 *      P_j^2 A_j and X_L = (P_{L-1} ... P_0) X_0, so a segment forms X X^T
 *      once and multiplies X by one m x m matrix; every other product is of
 *      two commuting symmetric m x m matrices (upper triangle computed), and
 *      the chain of them is held in fp16 where the coefficients allow
 *      (zopt_set_ns_form), with the final m x m factor rounded to bf16.  Five
 *      steps are segments of 3 and 2: 6 m^2 n + 14 m^3 flops against
 *      15 m^2 n + 5 m^3.  Each segment restarts from its X, which keeps the
 *      bf16 rounding of the m x m chain from compounding.  The two forms
 *      agree to within bf16 rounding, not bit for bit; zopt_set_ns_form
 *      selects plain iterations for every matrix.  Every symmetric m x m
 *      matrix is held as a bf16 off-diagonal part and an fp32 diagonal.
 *   4. Post-step [BluScript trainer source, Muon config block (weight decay
 *      pinned to AdamW's) and the note beside the MuonAdjustLr choice]:
 *        P = P * decay - step_lr * fp32(O),  weight = bf16(P)
 *      with O the result of step 3 in the stored orientation and, in double
 *      rounded once to binary32, decay = 1 - lr * weight_decay and
 *      step_lr = lr * scale, scale = 0.2 * sqrt(max(rows, cols)) when
 *      adjust_lr = 1 (the update's entry RMS matches AdamW's 0.2) or
 *      sqrt(max(1, rows / cols)) when adjust_lr = 0 (the original convention).
 *
 * Arguments
 *   batch        1 .. 64 matrices.
 *   rows, cols   the stored shape, >= 1, rows * cols < 2^31 and
 *                max(rows, cols) <= 2^21 (2,097,152: the kernels address a
 *                row panel of the padded matrix with 32-bit byte offsets).
 *   master, momentum   host arrays of `batch` device pointers, fp32
 *                [rows * cols] each, read and written.
 *   grad         host array of `batch` device pointers, bf16 [rows * cols].
 *   weight       host array of `batch` device pointers, bf16 [rows * cols],
 *                written; NULL skips the write-back (if non-NULL, every entry
 *                must be non-NULL).
 *   lr, momentum_beta, nesterov (0/1), weight_decay, ns_steps (0 .. 100),
 *   ns_a, ns_b, ns_c, ns_eps, adjust_lr (0/1)   as above.
 *   workspace    device scratch, 256-byte aligned, of at least the size the
 *                NULL-workspace query returns.  With workspace == NULL the call
 *                only writes that size to *workspace_bytes and returns ZOPT_OK.
 *                Otherwise *workspace_bytes is the size provided.  The
 *                workspace's contents need no initialisation; after the call,
 *                zopt_muon_output_view locates the step-3 result in it.
 *   stream       hipStream_t or NULL.
 *
 * Errors: ZOPT_ERR_NULL (a pointer array or one of its entries NULL,
 * workspace_bytes NULL); ZOPT_ERR_SIZE (batch, rows, cols out of range);
 * ZOPT_ERR_HYPER (lr or weight_decay < 0 or not finite, momentum_beta outside
 * [0, 1), nesterov or adjust_lr not 0/1, ns_steps outside [0, 100], a
 * coefficient not finite, ns_eps < 0 or not finite); ZOPT_ERR_WORKSPACE;
 * ZOPT_ERR_DEVICE.
 */
zopt_status zopt_muon_step(int32_t batch, int64_t rows, int64_t cols,
                           float *const *master, float *const *momentum,
                           const uint16_t *const *grad, uint16_t *const *weight,
                           float lr, float momentum_beta, int32_t nesterov,
                           float weight_decay, int32_t ns_steps,
                           float ns_a, float ns_b, float ns_c, float ns_eps,
                           int32_t adjust_lr, void *workspace, size_t *workspace_bytes,
                           void *stream);

/*
 * zopt_muon_output_view -- where the orthogonalised update O of matrix
 * `index` lies in a workspace that zopt_muon_step(batch, rows, cols, ...,
 * ns_steps, ...) has filled: bf16 O[r][c] (stored orientation, [rows, cols])
 * is at (*out)[r * (*row_stride) + c].  Host-only; enqueues nothing.  The view
 * is valid until the workspace is reused, and assumes the Newton-Schulz form
 * (zopt_set_ns_form) in effect when the workspace was filled: the form decides
 * which buffer holds the result.  Errors: ZOPT_ERR_NULL,
 * ZOPT_ERR_SIZE (batch, rows, cols or index out of range), ZOPT_ERR_HYPER
 * (ns_steps out of range).
 */
zopt_status zopt_muon_output_view(int32_t batch, int64_t rows, int64_t cols,
                                  int32_t ns_steps, const void *workspace,
                                  int32_t index, const uint16_t **out,
                                  int64_t *row_stride);

/*
 * zopt_muon_step_groups -- zopt_muon_step on `ngroups` groups of matrices in
 * one call.  A rank's Muon parameters fall into a few stored shapes, and
 * launch count is what limits a per-shape loop of small steps [dmuon PR #16,
 * commit "NS CUDA-graph replay": one rank steps tens of Muon matrices of a
 * small, stable set of shapes, and the launches issued per step dominated its
 * host time].  Here every Newton-Schulz product of every group whose short
 * side selects the same output tile is one launch, so small groups share the
 * GPU instead of running one after another.  Each matrix gets exactly the
 * arithmetic zopt_muon_step gives it; the call equals ngroups separate
 * zopt_muon_step calls, except that the groups' Newton-Schulz products
 * interleave in time.
 *
 * Short launches on two streams: when the groups on 256 x 256 output tiles
 * give the X X^T launch fewer than two rounds of workgroups (2 x 256 on a
 * 256-CU GPU), each product's launch would leave much of the GPU idle in its
 * last round.  The groups then run on `stream` and on a second stream of the
 * library's.  In a call that mixes the two forms of step 3, the groups of one
 * form and output tile stay on one stream (they share its launches), these
 * classes placed by Newton-Schulz work (largest first, each to the stream
 * with less); in a call of one form the groups are placed so one by one.  The
 * side estimated to take longer runs on `stream`.  Each group's momentum
 * pass, iterations and (with no health pass) post-step run on its side's
 * stream: the second stream waits (an event) for everything enqueued on
 * `stream` before the call and for the momentum passes of `stream`'s groups,
 * and `stream` waits for the second stream's last launch (another event)
 * before the health pass, or at the end of the call, so the call is ordered
 * on `stream` as any other.  The results are the same bit for bit.  The
 * second stream is
 * created at the first such call on the GPU that is not under stream capture
 * (a call under capture before that runs on one stream) and by
 * zopt_muon_graph_create before its capture; calls from several host threads
 * enqueue this part one at a time (a lock), and their work on the second
 * stream runs in that order.  Measured on the 1B rank-0 share (12 matrices,
 * four groups): 2.81 -> 2.58 ms per five-step call with the division by
 * class (3.49 -> 3.05 ms when two streams first replaced one).
 *
 * Arguments
 *   ngroups      1 .. 16.
 *   batch, rows, cols   host arrays of `ngroups` entries; group g has
 *                batch[g] (1 .. 64) matrices of stored shape
 *                [rows[g], cols[g]] with the limits of zopt_muon_step.
 *   master, momentum, grad, weight   host arrays of sum(batch) device
 *                pointers, group 0's matrices first, then group 1's, ...;
 *                weight may be NULL (no write-back for any group).
 *   lr ... stream      as for zopt_muon_step, shared by all groups.
 *   workspace    as for zopt_muon_step; the NULL-workspace query returns the
 *                size for all groups together (the sum of the per-group sizes).
 *
 * Errors: those of zopt_muon_step; ZOPT_ERR_NULL also if batch, rows or cols
 * is NULL, ZOPT_ERR_SIZE if ngroups is out of range.
 */
zopt_status zopt_muon_step_groups(int32_t ngroups, const int32_t *batch, const int64_t *rows,
                                  const int64_t *cols, float *const *master,
                                  float *const *momentum, const uint16_t *const *grad,
                                  uint16_t *const *weight, float lr, float momentum_beta,
                                  int32_t nesterov, float weight_decay, int32_t ns_steps,
                                  float ns_a, float ns_b, float ns_c, float ns_eps,
                                  int32_t adjust_lr, void *workspace, size_t *workspace_bytes,
                                  void *stream);

/*
 * zopt_muon_step_groups_guarded -- zopt_muon_step_groups with the Newton-Schulz
 * health checks [BluScript trainer source, per-step report: nsratio, the
 * worst ||update||_F / sqrt(min(rows, cols)) among the applied updates (about
 * 1 when healthy), and nsrej, the updates the divergence guard refused because
 * an element exceeded 1000 in magnitude; dmuon PR #16, commit "device-tensor
 * stats": diagnostics stay device scalars, read back on the caller's
 * schedule].  After step 3, per matrix i of the call (in call order), from its
 * bf16 result O:
 *   ratio_i    = ||O||_F / sqrt(min(rows, cols)), the squares summed exactly
 *                in double in a fixed order, formed in double, rounded once
 *   absmax_i   = max |O_jk| (NaN if an element is NaN)
 *   rejected_i = !(absmax_i <= ns_guard)
 * A rejected matrix is not updated: step 4 leaves its master and weight as
 * they were (its momentum has taken step 1).  The other matrices get exactly
 * what zopt_muon_step_groups gives them.
 *
 * Arguments: those of zopt_muon_step_groups, and
 *   ns_guard   > 0; 1000 is the pages' value; +inf only reports.
 *   ns_health  device floats, written: [0] the number of matrices rejected,
 *              [1] the worst ratio among those not rejected (0 if none), then
 *              [2 + 3i .. 4 + 3i] = ratio_i, absmax_i, rejected_i (0 / 1) for
 *              each of the sum(batch) matrices.
 *
 * Errors: those of zopt_muon_step_groups; with a workspace, ZOPT_ERR_NULL also
 * for ns_health NULL and ZOPT_ERR_HYPER for ns_guard not > 0.
 */
zopt_status zopt_muon_step_groups_guarded(int32_t ngroups, const int32_t *batch,
                                          const int64_t *rows, const int64_t *cols,
                                          float *const *master, float *const *momentum,
                                          const uint16_t *const *grad, uint16_t *const *weight,
                                          float lr, float momentum_beta, int32_t nesterov,
                                          float weight_decay, int32_t ns_steps, float ns_a,
                                          float ns_b, float ns_c, float ns_eps, int32_t adjust_lr,
                                          float ns_guard, float *ns_health, void *workspace,
                                          size_t *workspace_bytes, void *stream);

/*
 * Captured Muon calls.  One Muon call is tens of kernel launches; issued one
 * by one per step they cost host time that a graph replay does not [dmuon PR
 * #16, commit "NS CUDA-graph replay": the launches of a Newton-Schulz call
 * captured once per shape and replayed, cutting the host cost of a call from
 * milliseconds to tens of microseconds; lr / wd / momentum are kept out of
 * the captured part so a schedule needs no re-capture].  Here the whole call
 * (pre-step, Newton-Schulz, optional health pass, post-step) is one hipGraph,
 * and lr, momentum_beta and weight_decay live in device memory, read by the
 * kernels each time the graph runs: a caller changes them with an ordinary
 * device write (a copy or a fill on the stream) before a launch.
 *
 *   scalars  device float[3] = {lr, momentum_beta, weight_decay}.  Read when
 *            the kernels run; the library cannot check these values (they
 *            should satisfy zopt_muon_step's limits).  Every derived scalar
 *            (1 - mu, 1 - lr*wd, lr*scale) is formed in double on the device
 *            exactly as the host forms it, so a replay gives the bits a
 *            zopt_muon_step_groups(_guarded) call with the same values gives.
 *
 * zopt_muon_graph_create captures one call with the arguments of
 * zopt_muon_step_groups_guarded (ns_health NULL: no health pass, ns_guard
 * ignored) -- the buffers, shapes, workspace and fixed hyperparameters are
 * baked in and must stay valid while the graph is used -- and returns a
 * handle.  Capture runs on a stream of its own and enqueues nothing (a call
 * split over two streams is captured with its fork and join).
 * workspace_bytes is the size provided (the query of zopt_muon_step_groups
 * gives the size needed).  Errors: ZOPT_ERR_NULL (graph, workspace, scalars
 * or a buffer pointer NULL); ZOPT_ERR_SIZE; ZOPT_ERR_HYPER (nesterov,
 * ns_steps, a coefficient, ns_eps, adjust_lr, or ns_guard with ns_health);
 * ZOPT_ERR_WORKSPACE; ZOPT_ERR_DEVICE (capture or instantiation failed).
 *
 * zopt_muon_graph_launch enqueues one replay on `stream` (hipStream_t or
 * NULL).  Replays on one workspace must not overlap (one stream, or ordered).
 *
 * zopt_muon_graph_destroy frees the handle (NULL is a no-op); no replay may
 * still be pending (synchronise the stream first).  The handle is host
 * memory owned by the caller until then; the library holds no other state.
 */
typedef struct zopt_muon_graph zopt_muon_graph;

zopt_status zopt_muon_graph_create(int32_t ngroups, const int32_t *batch, const int64_t *rows,
                                   const int64_t *cols, float *const *master,
                                   float *const *momentum, const uint16_t *const *grad,
                                   uint16_t *const *weight, const float *scalars,
                                   int32_t nesterov, int32_t ns_steps, float ns_a, float ns_b,
                                   float ns_c, float ns_eps, int32_t adjust_lr, float ns_guard,
                                   float *ns_health, void *workspace, size_t workspace_bytes,
                                   zopt_muon_graph **graph);
zopt_status zopt_muon_graph_launch(const zopt_muon_graph *graph, void *stream);
zopt_status zopt_muon_graph_destroy(zopt_muon_graph *graph);

/*
 * zopt_muon_groups_output_view -- zopt_muon_output_view for matrix `index` of
 * group `group` of a workspace that zopt_muon_step_groups(ngroups, batch,
 * rows, cols, ..., ns_steps, ...) has filled.  Host-only.  Errors as
 * zopt_muon_output_view; ZOPT_ERR_SIZE also for `group` out of range.
 */
zopt_status zopt_muon_groups_output_view(int32_t ngroups, const int32_t *batch,
                                         const int64_t *rows, const int64_t *cols,
                                         int32_t ns_steps, const void *workspace, int32_t group,
                                         int32_t index, const uint16_t **out,
                                         int64_t *row_stride);

/*
 * zopt_round_bf16 -- dst[i] = bf16(src[i]) for i in [0, n), round to
 * nearest even as above [DEG zero.py, gather_params: the updated fp32 shard
 * cast to the bf16 compute dtype].
 *   src  fp32 [n], device, read.   dst  bf16 [n], device, written.
 *   n    >= 0; n = 0 enqueues nothing.
 * Errors: ZOPT_ERR_NULL (src or dst NULL with n > 0); ZOPT_ERR_SIZE (n < 0);
 * ZOPT_ERR_DEVICE.
 */
zopt_status zopt_round_bf16(const float *src, uint16_t *dst, int64_t n, void *stream);

/*
 * zopt_set_ns_workgroup_limit -- caps the workgroups that the Newton-Schulz
 * X' = a X + B X launches keep resident.  Those launches are persistent: one
 * round of workgroups walks all the tiles, each starting its next tile's
 * loads while it finishes the current one.  n = 0 restores the default, one
 * full round of the device (one 256 x 256-tile workgroup per compute unit);
 * n > 0 caps it at max(8, n rounded down to a multiple of 8), which leaves
 * compute units free for work running beside the optimizer (collectives on
 * another stream, say) at a cost in Newton-Schulz time.  Process-wide; it
 * applies to calls enqueued, and graphs captured, after it.  Results do not
 * depend on it: every tile is computed the same way by whichever workgroup.
 * Errors: ZOPT_ERR_SIZE (n < 0).
 */
zopt_status zopt_set_ns_workgroup_limit(int32_t n);

/*
 * zopt_set_ns_form -- the Newton-Schulz form of later calls:
 *   0 (the default) runs the groups that zopt_muon_step's step 3 names
 *     (n >= 2 m, m <= 4096, batch m^2 (n - m) >= 2^29) in segments on the
 *     Gram matrix,
 *     holding a segment's m x m chain in fp16 (3 more mantissa bits than
 *     bf16, the same matrix-core rate) when the coefficients keep every
 *     matrix of the chain below 2^13 in magnitude (checked on the scalar
 *     map over singular values in [0, 1.05]; true for the usual quintic and
 *     cubic coefficients), else in bf16; plain iterations hold A in fp16
 *     under the same condition for m <= 4096 (fp16's subnormal range
 *     begins near the off-diagonal entries of larger matrices' A), in bf16
 *     otherwise;
 *   1 runs plain iterations for every matrix;
 *   2 is form 0 with the chain always in bf16 (for comparison: less
 *     accurate than both others on some inputs).
 * Process-wide; it applies to workspace queries, calls and graph captures
 * made after it.  Forms 0 and 2 need more workspace for those shapes (three
 * more m x m 16-bit matrices and fp32 diagonals per matrix), so a workspace
 * sized under form 1 fails their size check (ZOPT_ERR_WORKSPACE).
 * Errors: ZOPT_ERR_HYPER (form not 0, 1 or 2).
 */
zopt_status zopt_set_ns_form(int32_t form);

#ifdef __cplusplus
}
#endif

#endif /* ZOPT_H */
