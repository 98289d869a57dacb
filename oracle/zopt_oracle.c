/*
 * zopt_oracle.c -- the CPU oracle for one rank's ZeRO-style optimizer step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (-ffp-contract=off: every + - * / below is one correctly rounded IEEE
 * binary32 operation; no fused multiply-adds).
 *
 * What is here (all binary32 unless stated; all scalar loops):
 *   - the flat bucketed shard layout        [DEG zero.py: ZeroMaster docstring,
 *                                            ZeroMaster.__init__ bucket loop,
 *                                            reduce_scatter, gather_params]
 *   - AdamW with decoupled weight decay and bias correction
 *                                           [dmuon PR #16, commit "foreach AdamW":
 *                                            op order decay -> moments ->
 *                                            bias-corrected addcdiv, per-step
 *                                            scalars on the post-increment step;
 *                                            BluScript trainer source, optimizer-
 *                                            precision note: decay is a
 *                                            (1 - lr*wd) multiply on fp32 state]
 *   - bf16 gradient promotion and grad_scale on load
 *                                           [DeepSpeed PR #9021, commits "bf16
 *                                            gradients of fp32 params" and
 *                                            "grad_scale"]
 *   - round-to-nearest-even fp32 -> bf16    [DEG zero.py: ZeroMaster docstring /
 *                                            gather_params, the bf16 cast of the
 *                                            updated shard]
 *   - Muon momentum (EMA form) + Nesterov, and the scaled, decayed post-step
 *                                           [BluScript trainer source: Muon config
 *                                            block (momentum 0.95, nesterov, wd
 *                                            pinned to AdamW's) and the ShardedMuon
 *                                            note on adjust_lr conventions]
 *   - the squared gradient norm of a rank's shard, and the clip statistics
 *     (total norm, clip coefficient, clipped, found_inf) derived from the
 *     summed squares              [DEG zero.py: ZeroMaster.grad_sq_norm;
 *                                  BluScript trainer source, cross-group
 *                                  global clipping block (coefficient
 *                                  min(1, clip / (norm + 1e-6))); dmuon PR
 *                                  #16, commit "device-tensor stats"
 *                                  (finiteness judged on the norm)]
 *   - Newton-Schulz health: the update-size ratio ||O||_F / sqrt(min(r, c))
 *     and the element-magnitude divergence guard
 *                                 [BluScript trainer source, per-step report:
 *                                  the nsrej / nsratio diagnostics]
 * Newton-Schulz itself is in ns.py (fp64, numpy).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16 <-> fp32                                                              */
/* ------------------------------------------------------------------------- */

/* A bf16 value is the upper 16 bits of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to the nearest bf16, ties to even, with integer arithmetic
 * only.  Adding 0x7FFF plus the lowest kept bit, then truncating, rounds to
 * nearest with ties going to the even neighbour.  Values beyond the largest
 * finite bf16 carry into the exponent and become infinity; infinities stay
 * infinities; subnormals are rounded like any other value (no flush).
 * A NaN becomes the positive quiet NaN 0x7FC0 (the sign and payload are not
 * kept), as a cast of an fp32 tensor to bf16 produces. */
uint16_t orc_rne_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)0x7FC0u;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void orc_rne_bf16_array(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_rne_bf16(src[i]);
}

/* ------------------------------------------------------------------------- */
/* Flat bucketed shard layout                                                 */
/* ------------------------------------------------------------------------- */
/* The trainable parameters lie end to end in a flat vector of N elements.
 * The bucket length is first lowered to a multiple of world (never below
 * world).  Buckets [s, e) tile [0, N); bucket b has padded length
 * L_b = ceil((e - s) / world) * world and is cut into world equal pieces of
 * L_b / world elements.  Rank r owns piece r of every bucket; its shard is
 * those pieces concatenated in bucket order.  Shard positions whose flat
 * index falls at or beyond the bucket's real end e are padding. */

int64_t orc_bucket_adjust(int64_t bucket, int32_t world)
{
    int64_t w = world;
    int64_t b = bucket - bucket % w;
    return b > w ? b : w;
}

int64_t orc_num_buckets(int64_t n, int64_t bucket, int32_t world)
{
    int64_t b = orc_bucket_adjust(bucket, world);
    int64_t count = 0;
    for (int64_t s = 0; s < n; s += b)
        ++count;
    return count;
}

int64_t orc_shard_len(int64_t n, int64_t bucket, int32_t world)
{
    int64_t b = orc_bucket_adjust(bucket, world);
    int64_t total = 0;
    for (int64_t s = 0; s < n; s += b) {
        int64_t e = s + b < n ? s + b : n;
        int64_t len = e - s;
        int64_t padded = ((len + world - 1) / world) * world;
        total += padded / world;
    }
    return total;
}

/* For each shard index j[i] of rank r: its flat index flat[i] and whether it
 * is a real element (real[i] = 1) or padding (real[i] = 0).  A padding
 * position still gets the flat index it would have had.  Returns 0, or -1 if
 * some j is outside [0, shard_len). */
int orc_shard_index_map(int64_t n, int64_t bucket, int32_t world, int32_t rank,
                        int64_t count, const int64_t *j, int64_t *flat,
                        uint8_t *real)
{
    int64_t b = orc_bucket_adjust(bucket, world);
    for (int64_t i = 0; i < count; ++i) {
        int64_t want = j[i];
        int64_t offset = 0; /* shard offset of the current bucket's piece */
        int found = 0;
        for (int64_t s = 0; s < n && !found; s += b) {
            int64_t e = s + b < n ? s + b : n;
            int64_t padded = ((e - s + world - 1) / world) * world;
            int64_t piece = padded / world;
            if (want >= offset && want < offset + piece) {
                int64_t f = s + (int64_t)rank * piece + (want - offset);
                flat[i] = f;
                real[i] = f < e ? 1 : 0;
                found = 1;
            }
            offset += piece;
        }
        if (!found || want < 0)
            return -1;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* AdamW                                                                      */
/* ------------------------------------------------------------------------- */
/* Per-step scalars.  t is the 1-based step count after the increment.  They
 * are formed in double from the binary32 hyperparameters and each rounded
 * to binary32 once:
 *   step_size = lr / (1 - beta1^t)
 *   bc2_sqrt  = sqrt(1 - beta2^t)
 *   decay     = 1 - lr * wd
 *   omb1      = 1 - beta1,  omb2 = 1 - beta2                                 */
void orc_adamw_scalars(float lr, float beta1, float beta2, float wd, int64_t step,
                       float out[5])
{
    double t = (double)step;
    double bc1 = 1.0 - pow((double)beta1, t);
    double bc2 = 1.0 - pow((double)beta2, t);
    out[0] = (float)((double)lr / bc1);
    out[1] = (float)sqrt(bc2);
    out[2] = (float)(1.0 - (double)lr * (double)wd);
    out[3] = (float)(1.0 - (double)beta1);
    out[4] = (float)(1.0 - (double)beta2);
}

/* One AdamW update of one element, in this order: decoupled decay, first and
 * second moments, bias-corrected addcdiv with eps added after the bias
 * correction of the root.  Every operation is one rounded binary32 op. */
static void adamw_elem(float *p, float *m, float *v, float g, const float sc[5],
                       float beta1, float beta2, float eps)
{
    float step_size = sc[0], bc2_sqrt = sc[1], decay = sc[2];
    float omb1 = sc[3], omb2 = sc[4];
    float pp = *p, mm = *m, vv = *v;
    pp = pp * decay;
    mm = beta1 * mm + omb1 * g;
    vv = beta2 * vv + (omb2 * g) * g;
    float denom = sqrtf(vv) / bc2_sqrt + eps;
    pp = pp - step_size * (mm / denom);
    *p = pp;
    *m = mm;
    *v = vv;
}

/* The whole shard of rank r for one step.
 *   master, exp_avg, exp_avg_sq : [shard_len] binary32, updated in place
 *   grad                        : [n] bf16 flat gradient; only this rank's
 *                                 real positions are read
 *   weight                      : [n] bf16 flat compute weights; only this
 *                                 rank's real positions are written; may be 0
 * Padding positions step with a zero gradient and write no weight. */
void orc_adamw_shard_step(float *master, float *exp_avg, float *exp_avg_sq,
                          const uint16_t *grad, uint16_t *weight, int64_t n,
                          int64_t bucket, int32_t world, int32_t rank,
                          float lr, float beta1, float beta2, float eps,
                          float wd, int64_t step, float grad_scale)
{
    float sc[5];
    orc_adamw_scalars(lr, beta1, beta2, wd, step, sc);
    int64_t b = orc_bucket_adjust(bucket, world);
    int64_t offset = 0;
    for (int64_t s = 0; s < n; s += b) {
        int64_t e = s + b < n ? s + b : n;
        int64_t padded = ((e - s + world - 1) / world) * world;
        int64_t piece = padded / world;
        for (int64_t k = 0; k < piece; ++k) {
            int64_t j = offset + k;
            int64_t f = s + (int64_t)rank * piece + k;
            int is_real = f < e;
            float g = 0.0f;
            if (is_real)
                g = bf16_to_f32(grad[f]) * grad_scale;
            adamw_elem(&master[j], &exp_avg[j], &exp_avg_sq[j], g, sc, beta1,
                       beta2, eps);
            if (is_real && weight)
                weight[f] = orc_rne_bf16(master[j]);
        }
        offset += piece;
    }
}

/* Independent elements: count points with binary32 gradients already scaled
 * (g[i] is the value fed to the moments).  p, m, v updated in place; w[i]
 * receives the bf16 of the new p[i]. */
void orc_adamw_points(int64_t count, float *p, float *m, float *v, const float *g,
                      uint16_t *w, float lr, float beta1, float beta2, float eps,
                      float wd, int64_t step)
{
    float sc[5];
    orc_adamw_scalars(lr, beta1, beta2, wd, step, sc);
    for (int64_t i = 0; i < count; ++i) {
        adamw_elem(&p[i], &m[i], &v[i], g[i], sc, beta1, beta2, eps);
        if (w)
            w[i] = orc_rne_bf16(p[i]);
    }
}

/* ------------------------------------------------------------------------- */
/* Muon pre-step and post-step (binary32)                                     */
/* ------------------------------------------------------------------------- */
/* Momentum as an exponential moving average of the gradient, then the
 * Nesterov look-ahead:
 *   M <- mu * M + (1 - mu) * g
 *   U  = (1 - mu) * g + mu * M     (nesterov)   or   U = M   (otherwise)
 * g is the bf16 gradient widened to binary32.  count = rows * cols, in the
 * caller's row-major order; the transpose for Newton-Schulz is not done here. */
void orc_muon_pre(int64_t count, float *momentum, const uint16_t *grad, float mu,
                  int nesterov, float *u)
{
    float omm = (float)(1.0 - (double)mu);
    for (int64_t i = 0; i < count; ++i) {
        float g = bf16_to_f32(grad[i]);
        float mm = mu * momentum[i] + omm * g;
        momentum[i] = mm;
        u[i] = nesterov ? omm * g + mu * mm : mm;
    }
}

/* The update scale of an orthogonalised [rows, cols] matrix.
 *   adjust = 1 (match AdamW's update RMS): 0.2 * sqrt(max(rows, cols)); a
 *            semi-orthogonal O has entry RMS 1/sqrt(max(rows, cols)), so the
 *            scaled update has entry RMS 0.2.
 *   adjust = 0 (the original convention): sqrt(max(1, rows / cols)).
 * Computed in double. */
double orc_muon_scale(int64_t rows, int64_t cols, int adjust)
{
    if (adjust) {
        double big = (double)(rows > cols ? rows : cols);
        return 0.2 * sqrt(big);
    }
    double ratio = (double)rows / (double)cols;
    return sqrt(ratio > 1.0 ? ratio : 1.0);
}

/* P <- P * fp32(1 - lr * wd) - fp32(lr * scale) * O, then W = bf16(P).
 * O is the orthogonalised update in binary32, [rows, cols] row-major.
 * w may be 0. */
void orc_muon_post(int64_t rows, int64_t cols, float *master, const float *o,
                   uint16_t *w, float lr, float wd, int adjust)
{
    float decay = (float)(1.0 - (double)lr * (double)wd);
    float step = (float)((double)lr * orc_muon_scale(rows, cols, adjust));
    int64_t count = rows * cols;
    for (int64_t i = 0; i < count; ++i) {
        float pp = master[i] * decay - step * o[i];
        master[i] = pp;
        if (w)
            w[i] = orc_rne_bf16(pp);
    }
}

/* ------------------------------------------------------------------------- */
/* Gradient norm and clip statistics                                          */
/* ------------------------------------------------------------------------- */
/* Sum of the squares of rank r's real gradient elements (padding and other
 * ranks' positions are never read).  Each square of a bf16 value is exact in
 * double; the sum runs in index order in long double (x86 extended, 64-bit
 * significand), so the returned double is within about n * 2^-64 of the exact
 * sum plus one final rounding. */
double orc_grad_sq_norm(const uint16_t *grad, int64_t n, int64_t bucket, int32_t world,
                        int32_t rank)
{
    int64_t b = orc_bucket_adjust(bucket, world);
    long double acc = 0.0L;
    for (int64_t s = 0; s < n; s += b) {
        int64_t e = s + b < n ? s + b : n;
        int64_t padded = ((e - s + world - 1) / world) * world;
        int64_t piece = padded / world;
        for (int64_t k = 0; k < piece; ++k) {
            int64_t f = s + (int64_t)rank * piece + k;
            if (f < e) {
                double g = (double)bf16_to_f32(grad[f]);
                acc += (long double)(g * g);
            }
        }
    }
    return (double)acc;
}

/* Clip statistics from summed squares.  sq[0..count) are partial sums (one
 * per rank, say), added in index order in double.
 *   total_norm = fp32( sqrt(sum) * inv_scale )           (inv_scale undoes a
 *                                                         loss scale; 1 = none)
 *   found_inf  = total_norm is not finite                 (judged on the norm)
 *   clip_coef  = min(1, max_norm / (total_norm + 1e-6))  binary32; a NaN
 *                quotient stays NaN, an infinite norm gives 0
 *   clipped    = !found_inf && clip_coef < 1
 *   grad_scale = inv_scale * clip_coef                    binary32: the factor
 *                the AdamW step multiplies each promoted gradient by
 * out = {total_norm, clip_coef, clipped, found_inf, grad_scale}, flags as
 * 0.0 / 1.0. */
void orc_clip_stats(const double *sq, int32_t count, float max_norm, float inv_scale,
                    float out[5])
{
    double total = 0.0;
    for (int32_t i = 0; i < count; ++i)
        total += sq[i];
    float norm = (float)(sqrt(total) * (double)inv_scale);
    int found_inf = !isfinite(norm);
    float coef = max_norm / (norm + 1e-6f);
    if (coef > 1.0f)
        coef = 1.0f;
    out[0] = norm;
    out[1] = coef;
    out[2] = (!found_inf && coef < 1.0f) ? 1.0f : 0.0f;
    out[3] = found_inf ? 1.0f : 0.0f;
    out[4] = inv_scale * coef;
}

/* ------------------------------------------------------------------------- */
/* Newton-Schulz health                                                       */
/* ------------------------------------------------------------------------- */
/* For one orthogonalised update O ([rows, cols] binary32):
 *   ratio    = ||O||_F / sqrt(min(rows, cols)), 1 for a semi-orthogonal O
 *              (its min(rows, cols) singular values are all 1); the squares
 *              are summed in long double, the ratio formed in double and
 *              rounded to binary32 once
 *   absmax   = max |O_ij| (NaN if any element is NaN)
 *   rejected = 1 unless absmax <= guard: the divergence guard refuses the
 *              update of a matrix with an element beyond the guard or not a
 *              number
 * out = {ratio, absmax, rejected}. */
void orc_ns_health(int64_t rows, int64_t cols, const float *o, float guard, float out[3])
{
    long double acc = 0.0L;
    float amax = 0.0f;
    int nan_seen = 0;
    int64_t count = rows * cols;
    for (int64_t i = 0; i < count; ++i) {
        double x = (double)o[i];
        acc += (long double)(x * x);
        float a = fabsf(o[i]);
        if (isnan(a))
            nan_seen = 1;
        else if (a > amax)
            amax = a;
    }
    double mn = (double)(rows < cols ? rows : cols);
    out[0] = (float)(sqrt((double)acc) / sqrt(mn));
    out[1] = nan_seen ? NAN : amax;
    out[2] = (out[1] <= guard) ? 0.0f : 1.0f;
}
