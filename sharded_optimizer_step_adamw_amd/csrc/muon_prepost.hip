// muon_prepost.hip -- the bandwidth-bound passes around Newton-Schulz.
//
// Pre-step [BluScript trainer source, Muon config block: momentum 0.95 with
// Nesterov; the momentum buffer is an exponential moving average of the
// gradient; dmuon PR #16, commit "NS CUDA-graph replay": momentum, lr and wd
// stay in the eager pre/post steps around the fixed-shape Newton-Schulz]:
//   pass 1  M = mu M + (1-mu) g, U = (1-mu) g + mu M (or U = M); write M,
//           bf16(U) in the Newton-Schulz orientation (zero padding), and
//           fixed-order fp64 partial sums of U^2 (exact squares)  (12 B/elem)
//   final   per matrix, s = 1 / (sqrt(sum of partials) + eps) in double, the
//           partials summed in a fixed order (deterministic); the first
//           Newton-Schulz iteration applies s to its products when ||U||_F^2
//           lies in [2^-60, 2^100], where those fp32 products of bf16(U)
//           neither overflow nor lose precision to underflow; outside that
//           range (huge or tiny gradients, Inf, NaN) this kernel rewrites X
//           as X0 = bf16(U s) itself and the iteration applies 1
// A call with no iterations returns X0 = bf16(U s) itself, so it runs
//   pass 1  M and the partials only                              (10 B/elem)
//   pass 2  recompute U from the new M (bitwise the same U), write
//           X0 = bf16(U s) (U s formed in double) in the Newton-Schulz
//           orientation and, for a matrix stored transposed, X0^T,
//           zero-filling the tile padding                        (8 B/elem)
// Health [BluScript trainer source, per-step report: nsratio, the update's
// ||O||_F / sqrt(min(rows, cols)), about 1 when healthy, and nsrej, the
// updates the divergence guard refused for an element above 1000]:
//   pass    fp64 sum of squares and max |x| of X, per workgroup    (2 B/elem)
//   final   per matrix: ratio, absmax, rejected = !(absmax <= guard)
// Post-step [BluScript trainer source: Muon weight decay pinned to AdamW's;
// the adjust_lr note on the update scale]:
//   P = P * decay - step_lr * O, W = bf16(P)                      (12 B/elem)
//   (a rejected matrix is left as it is)
#include "zopt_internal.h"

// M, U and P are bit-exact binary32 arithmetic: no contraction.
#pragma clang fp contract(off)

namespace zopt {
namespace {

// Elements per thread and sweeps per workgroup of the streaming passes.
// Measured on MI355X (GPT-2-small and 8B-share Muon calls): one sweep of 8
// per thread in pass 1 and 4 per thread in the post-step beat four sweeps of
// 8 and 8 (pre/post 4% faster) and one element per thread (34% slower).
constexpr int kThreads = 256;
constexpr int kPreEPT = 8;          // pass 1 of a call with no iterations: elements per thread per sweep
constexpr int kSweeps = 1;          // sweeps per workgroup in that pass
constexpr int kChunk = kThreads * kPreEPT * kSweeps;  // elements / workgroup
constexpr int kPostEPT = 4;         // post-step: elements per thread (1, 4 or 8)
constexpr int kTile = 64;           // pass-2 transpose tile
constexpr int kFallbackBlocks = 32; // workgroups per matrix of the norm launch (X0 rewrite)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E consecutive fp32 (E = 1, 4 or 8; 16-byte aligned for E > 1).
template <int E, bool NT>
__device__ __forceinline__ void ld_f32(const float *p, float (&x)[E]) {
    if constexpr (E == 1) {
        x[0] = NT ? __builtin_nontemporal_load(p) : *p;
    } else {
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            const f32x4 *q = reinterpret_cast<const f32x4 *>(p) + h;
            const f32x4 v = NT ? __builtin_nontemporal_load(q) : *q;
            x[4 * h] = v.x; x[4 * h + 1] = v.y; x[4 * h + 2] = v.z; x[4 * h + 3] = v.w;
        }
    }
}
template <int E, bool NT>
__device__ __forceinline__ void st_f32(float *p, const float (&x)[E]) {
    if constexpr (E == 1) {
        if (NT) __builtin_nontemporal_store(x[0], p); else *p = x[0];
    } else {
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            f32x4 *q = reinterpret_cast<f32x4 *>(p) + h;
            const f32x4 v{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
            if (NT) __builtin_nontemporal_store(v, q); else *q = v;
        }
    }
}
// E consecutive bf16 as fp32 (8 / 16-byte aligned for E = 4 / 8).
template <int E>
__device__ __forceinline__ void ld_bf16(const uint16_t *p, float (&x)[E]) {
    if constexpr (E == 1) {
        x[0] = bf16_bits_to_float(__builtin_nontemporal_load(p));
    } else {
        uint32_t w[E / 2];
        if constexpr (E == 4) {
            const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            w[0] = v.x; w[1] = v.y;
        } else {
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = bf16_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
}
// E values rounded to bf16 and stored (8 / 16-byte aligned for E = 4 / 8).
template <int E>
__device__ __forceinline__ void st_bf16(uint16_t *p, const float (&x)[E]) {
    if constexpr (E == 1) {
        __builtin_nontemporal_store((uint16_t)rne_bf16_bits(x[0]), p);
    } else if constexpr (E == 4) {
        __builtin_nontemporal_store(u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])},
                                    reinterpret_cast<u32x2 *>(p));
    } else {
        __builtin_nontemporal_store(u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                          pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])},
                                    reinterpret_cast<u32x4 *>(p));
    }
}

// Fixed-order sum of fp64 values over the workgroup: butterfly within each
// 64-wide wave, then the four wave sums in order.
__device__ double block_sum_d(double x, double *lds4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds4[wave] = x;
    __syncthreads();
    double s = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    __syncthreads();
    return s;
}

// u^2 added to an fp64 sum: the square of a binary32 value is exact in
// binary64, so the fused form rounds once, as a separate add would.
__device__ __forceinline__ void add_sq(double &acc, float u) {
    const double d = (double)u;
    acc = __builtin_fma(d, d, acc);
}

// The sum of the exact squares of E (4 or 8) binary32 values in fp64, added
// pairwise (a short dependency chain: the streaming passes that use it keep
// several groups of loads in flight per thread).
template <int E>
__device__ __forceinline__ double sum_sq(const float (&u)[E]) {
    double s[E];
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] = (double)u[e] * (double)u[e];
#pragma unroll
    for (int w = 1; w < E; w *= 2)
#pragma unroll
        for (int e = 0; e < E; e += 2 * w) s[e] += s[e + w];
    return s[0];
}

// The range of ||U||_F^2 over which the first Newton-Schulz iteration applies
// the pre-scale s to its fp32 products of bf16(U): every entry of U U^T is at
// most ||U||_F^2 <= 2^100 and every accumulator of B U at most ~10 ||U||_F, far
// inside binary32; s and s^2 stay normal; and with ||U||_F^2 >= 2^-60 a
// typical product of two entries (about ||U||_F^2 / (m n) >= 2^-91 for
// m n < 2^31) is a normal binary32, so only entries ~1e-9 of the typical one
// or smaller could underflow.
constexpr double kFoldMin = 0x1p-60, kFoldMax = 0x1p100;

struct PreArgs {
    int32_t count;        // rows * cols
    int32_t vec;          // 8-element vector path allowed
    float mu, omm;
    int32_t nesterov;
    const float *dev;     // device scalars [lr, momentum_beta, weight_decay], or NULL
};

// mu and omm = fp32(1 - mu), formed in double as the host forms them, from
// the device scalars when the launch carries them.
__device__ __forceinline__ void device_momentum(const float *dev, float &mu, float &omm) {
    if (dev) {
        mu = dev[kDevMomentum];
        omm = (float)(1.0 - (double)mu);
    }
}

__device__ __forceinline__ void momentum_update(float &m, float g, float &u,
                                                const PreArgs &a) {
    m = a.mu * m + a.omm * g;
    u = a.nesterov ? a.omm * g + a.mu * m : m;
}

__global__ __launch_bounds__(kThreads) void muon_momentum_kernel(
    MuonPtrs ptrs, PreArgs a, double *__restrict__ partials, int32_t norm_blocks) {
    __shared__ double lds4[4];
    device_momentum(a.dev, a.mu, a.omm);
    const int b = blockIdx.y;
    float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    double sumsq = 0.0;
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    for (int s = 0; s < kSweeps; ++s) {
        const int64_t i0 = base + ((int64_t)s * kThreads + threadIdx.x) * kPreEPT;
        if (i0 >= a.count) break;
        if (a.vec && i0 + kPreEPT <= a.count) {
            float m[kPreEPT], g[kPreEPT];
            ld_f32<kPreEPT, false>(mom + i0, m);
            ld_bf16<kPreEPT>(grad + i0, g);
            float us[kPreEPT];
#pragma unroll
            for (int e = 0; e < kPreEPT; ++e) momentum_update(m[e], g[e], us[e], a);
            sumsq += sum_sq(us);
            st_f32<kPreEPT, false>(mom + i0, m);
        } else {
            for (int e = 0; e < kPreEPT && i0 + e < a.count; ++e) {
                float g = bf16_bits_to_float(grad[i0 + e]);
                float m = mom[i0 + e], u;
                momentum_update(m, g, u, a);
                mom[i0 + e] = m;
                add_sq(sumsq, u);
            }
        }
    }
    const double total = block_sum_d(sumsq, lds4);
    if (threadIdx.x == 0) partials[(int64_t)b * norm_blocks + blockIdx.x] = total;
}

struct ScaleArgs {
    int32_t rows, cols;     // stored shape
    int32_t transposed;     // X = U^T
    int32_t mp, np;         // padded Newton-Schulz shape (X is mp x np)
    int32_t tiles_c;        // tiles along the stored columns (padded)
    float mu, omm;
    int32_t nesterov;
    int32_t vec;            // cols % 8 == 0 and every base 16-byte aligned
    const float *dev;       // device scalars, or NULL
    int32_t want_t;         // also write X0^T
};

// X0 = bf16(U sd) on one 64 x 64 tile (index t) of the padded
// stored-orientation matrix b, U recomputed from the momentum pass 1 wrote
// (bitwise the U pass 1 formed) and U sd formed in double.  The stored
// orientation is X when rows <= cols and X^T otherwise; it is written straight
// out (for X^T only when a.want_t), and the LDS-transposed tile goes to the
// other.  Zeros in the padding.  Every thread of the workgroup calls it.
__device__ __forceinline__ void x0_tile(const MuonPtrs &ptrs, const ScaleArgs &a,
                                        const PreArgs &pa, int b, int t, double sd,
                                        uint16_t *__restrict__ x_base,
                                        uint16_t *__restrict__ xt_base, int64_t x_stride,
                                        int64_t xt_stride, uint16_t (*tile)[kTile + 2]) {
    const int tr = t / a.tiles_c, tc = t % a.tiles_c;
    const float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    // the stored-orientation output and its padded leading dimension
    uint16_t *direct = a.transposed ? xt_base + (int64_t)b * xt_stride
                                    : x_base + (int64_t)b * x_stride;
    uint16_t *other = a.transposed ? x_base + (int64_t)b * x_stride
                                   : xt_base + (int64_t)b * xt_stride;
    const int64_t ld_direct = a.transposed ? a.mp : a.np;
    const int64_t ld_other = a.transposed ? a.np : a.mp;

    // 64 rows x 8 groups of 8 columns = 512 groups; two per thread
    for (int q = 0; q < 2; ++q) {
        const int grp = threadIdx.x + q * kThreads;
        const int lr = grp >> 3, lc = (grp & 7) * 8;
        const int r = tr * kTile + lr, c0 = tc * kTile + lc;
        uint32_t packed[4];
        if (a.vec && r < a.rows && c0 + 8 <= a.cols) {
            // the 8 columns are inside the matrix: 128-bit loads
            const int64_t i = (int64_t)r * a.cols + c0;
            const u32x4 gw = *reinterpret_cast<const u32x4 *>(grad + i);
            const f32x4 m0 = *reinterpret_cast<const f32x4 *>(mom + i);
            const f32x4 m1 = *reinterpret_cast<const f32x4 *>(mom + i + 4);
            const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            const uint32_t gb[4] = {gw.x, gw.y, gw.z, gw.w};
            float xs[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = bf16_bits_to_float((gb[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
                const float u = pa.nesterov ? pa.omm * g + pa.mu * mv[e] : mv[e];
                xs[e] = (float)((double)u * sd);
            }
#pragma unroll
            for (int e = 0; e < 8; e += 2) packed[e >> 1] = pack_bf16x2(xs[e], xs[e + 1]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                float x2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = c0 + e + h;
                    float x = 0.0f;
                    if (r < a.rows && c < a.cols) {
                        const int64_t i = (int64_t)r * a.cols + c;
                        float g = bf16_bits_to_float(grad[i]);
                        float m = mom[i];  // already updated by pass 1
                        float u = pa.nesterov ? pa.omm * g + pa.mu * m : m;
                        x = (float)((double)u * sd);
                    }
                    x2[h] = x;
                }
                packed[e >> 1] = pack_bf16x2(x2[0], x2[1]);
            }
        }
        // X0^T is the stored orientation of a transposed matrix: written only
        // when wanted
        if (!a.transposed || a.want_t)
            *reinterpret_cast<u32x4 *>(direct + (int64_t)r * ld_direct + c0) =
                u32x4{packed[0], packed[1], packed[2], packed[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            tile[lr][lc + e] = (uint16_t)((packed[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
    if (!a.transposed && !a.want_t) return;  // uniform: X0 alone is wanted
    __syncthreads();
    // transposed: output row = stored column, output columns = stored rows
    for (int q = 0; q < 2; ++q) {
        const int grp = threadIdx.x + q * kThreads;
        const int lc = grp >> 3, lr0 = (grp & 7) * 8;
        uint32_t packed[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            packed[e >> 1] = (uint32_t)tile[lr0 + e][lc] | ((uint32_t)tile[lr0 + e + 1][lc] << 16);
        const int64_t orow = (int64_t)tc * kTile + lc;
        const int64_t ocol = (int64_t)tr * kTile + lr0;
        *reinterpret_cast<u32x4 *>(other + orow * ld_other + ocol) =
            u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
    __syncthreads();  // the tile is free for the caller's next one
}

// Per matrix b = blockIdx.y: s = 1 / (||U||_F + eps) in double from the fp64
// partials, summed in a fixed order (every workgroup of the matrix forms the
// same value), stored as sd[b]; xs[b] is the factor the first Newton-Schulz
// iteration applies to its products of X.  With fold (iterations follow and
// pass 1 left bf16(U) in X): xs[b] = s when ||U||_F^2 lies in [kFoldMin,
// kFoldMax]; otherwise xs[b] = 1 and the workgroups of the matrix rewrite X
// as X0 = bf16(U s), tiles blockIdx.x, blockIdx.x + gridDim.x, ...  Without
// fold one workgroup per matrix only forms s (pass 2 writes X0).
__global__ __launch_bounds__(kThreads) void muon_norm_kernel(
    MuonPtrs ptrs, ScaleArgs a, const double *__restrict__ partials, int32_t norm_blocks,
    int32_t count, double *__restrict__ sd, float *__restrict__ xs, float ns_eps, int32_t fold,
    int32_t tiles, uint16_t *__restrict__ x_base, int64_t x_stride) {
    __shared__ double lds4[4];
    __shared__ uint16_t tile[kTile][kTile + 2];
    const int b = blockIdx.y;
    const double *p = partials + (int64_t)b * norm_blocks;
    // four loads in flight per thread (tens of thousands of partials for the
    // largest matrices); the same fixed order in every workgroup
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int i = threadIdx.x;
    for (; i + 3 * kThreads < count; i += 4 * kThreads) {
        a0 += p[i];
        a1 += p[i + kThreads];
        a2 += p[i + 2 * kThreads];
        a3 += p[i + 3 * kThreads];
    }
    for (; i < count; i += kThreads) a0 += p[i];
    const double total = block_sum_d((a0 + a1) + (a2 + a3), lds4);
    const double s = 1.0 / (__builtin_sqrt(total) + (double)ns_eps);
    // (NaN and infinity compare false: such a matrix takes the rewrite)
    const bool folded = total >= kFoldMin && total <= kFoldMax;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        sd[b] = s;
        xs[b] = (fold && folded) ? (float)s : 1.0f;
    }
    if (!fold || folded) return;  // uniform
    PreArgs pa{0, 0, a.mu, a.omm, a.nesterov, nullptr};
    device_momentum(a.dev, pa.mu, pa.omm);
    for (int t = blockIdx.x; t < tiles; t += gridDim.x)
        x0_tile(ptrs, a, pa, b, t, s, x_base, x_base, x_stride, x_stride, tile);
}

// Pass 2 of a call with no iterations.  One workgroup per 64 x 64 tile of
// the padded stored-orientation matrix: X0 = bf16(U s), and X0^T where wanted.
__global__ __launch_bounds__(kThreads) void muon_scale_kernel(
    MuonPtrs ptrs, ScaleArgs a, const double *__restrict__ sd,
    uint16_t *__restrict__ x_base, uint16_t *__restrict__ xt_base,
    int64_t x_stride, int64_t xt_stride) {
    __shared__ uint16_t tile[kTile][kTile + 2];
    const int b = blockIdx.y;
    PreArgs pa{0, 0, a.mu, a.omm, a.nesterov, nullptr};
    device_momentum(a.dev, pa.mu, pa.omm);
    x0_tile(ptrs, a, pa, b, blockIdx.x, sd[b], x_base, xt_base, x_stride, xt_stride, tile);
}

// Pass 1 of a call that runs Newton-Schulz iterations, fused with the write
// of its input, for a matrix stored transposed: one workgroup per T x T tile
// of the padded stored-orientation matrix (T = 128 where both padded sides
// allow, else 64) updates M there, writes bf16(U) (not yet scaled) in the
// Newton-Schulz orientation through the LDS tile, with zeros in the padding,
// and leaves the tile's sum of U^2 (a fixed order: each thread's elements,
// then the workgroup sum) as a partial.  The first iteration applies
// s = 1 / (||U||_F + eps) to the products it forms from this X (s^2 to X X^T,
// s to B X), so X0 = s U is never stored: 12 bytes per element in all,
// against 10 + 8 for pass 1 and a separate scaling pass.
template <int T>
__global__ __launch_bounds__(kThreads) void muon_momentum_x_kernel(
    MuonPtrs ptrs, ScaleArgs a, double *__restrict__ partials, int32_t norm_blocks,
    uint16_t *__restrict__ x_base, int64_t x_stride) {
    constexpr int GPR = T / 8;                  // 8-element groups per tile row
    constexpr int PER = T * GPR / kThreads;     // groups per thread
    __shared__ uint16_t tile[T][T + 2];
    __shared__ double lds4[4];
    const int b = blockIdx.y;
    const int tiles_c = a.transposed ? a.mp / T : a.np / T;  // tiles along the stored columns
    const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
    float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    uint16_t *x = x_base + (int64_t)b * x_stride;
    PreArgs pa{0, 0, a.mu, a.omm, a.nesterov, nullptr};
    device_momentum(a.dev, pa.mu, pa.omm);
    double sumsq = 0.0;
    // bf16(U) of the group of 8 at tile row lr, column lc: to X (rows <= cols)
    // or to the LDS tile (transposed)
    auto put = [&](int lr, int lc, int r, int c0, const float (&us)[8]) __attribute__((always_inline)) {
        const uint32_t packed[4] = {pack_bf16x2(us[0], us[1]), pack_bf16x2(us[2], us[3]),
                                    pack_bf16x2(us[4], us[5]), pack_bf16x2(us[6], us[7])};
        if (!a.transposed)
            *reinterpret_cast<u32x4 *>(x + (int64_t)r * a.np + c0) =
                u32x4{packed[0], packed[1], packed[2], packed[3]};
        else
#pragma unroll
            for (int e = 0; e < 8; ++e)
                tile[lr][lc + e] = (uint16_t)((packed[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    };

    if (a.vec && (tr + 1) * T <= a.rows && (tc + 1) * T <= a.cols) {
        // a tile inside the matrix (uniform): the loads of LB groups leave
        // together, before any of them is used (the pass is latency-bound
        // with one group in flight per thread)
        constexpr int LB = PER < 4 ? PER : 4;
        for (int q0 = 0; q0 < PER; q0 += LB) {
            float m[LB][8], g[LB][8];
#pragma unroll
            for (int k = 0; k < LB; ++k) {
                const int grp = threadIdx.x + (q0 + k) * kThreads;
                const int r = tr * T + grp / GPR, c0 = tc * T + (grp % GPR) * 8;
                const int64_t i = (int64_t)r * a.cols + c0;
                ld_f32<8, true>(mom + i, m[k]);  // read once, next by the next step
                ld_bf16<8>(grad + i, g[k]);
            }
#pragma unroll
            for (int k = 0; k < LB; ++k) {
                const int grp = threadIdx.x + (q0 + k) * kThreads;
                const int lr = grp / GPR, lc = (grp % GPR) * 8;
                const int r = tr * T + lr, c0 = tc * T + lc;
                float us[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) momentum_update(m[k][e], g[k][e], us[e], pa);
                st_f32<8, true>(mom + (int64_t)r * a.cols + c0, m[k]);
                sumsq += sum_sq(us);
                put(lr, lc, r, c0, us);
            }
        }
    } else {
    // T rows x GPR groups of 8 columns; PER per thread
    for (int q = 0; q < PER; ++q) {
        const int grp = threadIdx.x + q * kThreads;
        const int lr = grp / GPR, lc = (grp % GPR) * 8;
        const int r = tr * T + lr, c0 = tc * T + lc;
        float us[8];
        if (a.vec && r < a.rows && c0 + 8 <= a.cols) {
            const int64_t i = (int64_t)r * a.cols + c0;
            float m[8], g[8];
            ld_f32<8, true>(mom + i, m);  // read once, next by the next step
            ld_bf16<8>(grad + i, g);
#pragma unroll
            for (int e = 0; e < 8; ++e) momentum_update(m[e], g[e], us[e], pa);
            st_f32<8, true>(mom + i, m);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = c0 + e;
                float u = 0.0f;
                if (r < a.rows && c < a.cols) {
                    const int64_t i = (int64_t)r * a.cols + c;
                    float m = mom[i];
                    momentum_update(m, bf16_bits_to_float(grad[i]), u, pa);
                    mom[i] = m;
                }
                us[e] = u;
            }
        }
        sumsq += sum_sq(us);
        put(lr, lc, r, c0, us);
    }
    }
    const double total = block_sum_d(sumsq, lds4);  // its barriers also order the tile writes
    if (threadIdx.x == 0) partials[(int64_t)b * norm_blocks + blockIdx.x] = total;
    if (!a.transposed) return;  // uniform
    // transposed: X row = stored column, X columns = stored rows
    for (int q = 0; q < PER; ++q) {
        const int grp = threadIdx.x + q * kThreads;
        const int lc = grp / GPR, lr0 = (grp % GPR) * 8;
        uint32_t packed[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2)
            packed[e >> 1] = (uint32_t)tile[lr0 + e][lc] | ((uint32_t)tile[lr0 + e + 1][lc] << 16);
        const int64_t orow = (int64_t)tc * T + lc;
        const int64_t ocol = (int64_t)tr * T + lr0;
        *reinterpret_cast<u32x4 *>(x + orow * a.np + ocol) =
            u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
}

// The same pass for a matrix stored in the Newton-Schulz orientation (rows
// <= cols): a flat stream of consecutive stored elements (kFlatEPT per
// thread), M updated in place and bf16(U) written to X's row at the padded
// stride np, one fixed-order partial of U^2 per workgroup.  (LDS-transpose
// tiles read 64-128 row pieces of 256-512 bytes per workgroup; this reads
// whole runs.)  The padding of X is zeroed by muon_x_pad_kernel.
// elements per thread of the flat pass: 4 (1024 per workgroup) measured ~1% faster than 8 on
// a one-iteration GPT-2-small call, like the post-step's 4
constexpr int kFlatEPT = 4;
__global__ __launch_bounds__(kThreads) void muon_momentum_xflat_kernel(
    MuonPtrs ptrs, ScaleArgs a, double *__restrict__ partials, int32_t norm_blocks,
    uint16_t *__restrict__ x_base, int64_t x_stride) {
    constexpr int E = kFlatEPT;
    __shared__ double lds4[4];
    const int b = blockIdx.y;
    float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    uint16_t *x = x_base + (int64_t)b * x_stride;
    PreArgs pa{0, 0, a.mu, a.omm, a.nesterov, nullptr};
    device_momentum(a.dev, pa.mu, pa.omm);
    const uint32_t count = (uint32_t)a.rows * (uint32_t)a.cols;  // < 2^31
    const uint32_t i0 = (blockIdx.x * kThreads + threadIdx.x) * E;
    double sumsq = 0.0;
    if (a.vec && i0 + E <= count) {
        // cols % 8 == 0: the elements share one row
        float m[E], g[E], us[E];
        ld_f32<E, true>(mom + i0, m);
        ld_bf16<E>(grad + i0, g);
        const uint32_t r = i0 / (uint32_t)a.cols, c = i0 - r * (uint32_t)a.cols;
#pragma unroll
        for (int e = 0; e < E; ++e) momentum_update(m[e], g[e], us[e], pa);
        st_f32<E, true>(mom + i0, m);
        sumsq += sum_sq(us);
        st_bf16<E>(x + (int64_t)r * a.np + c, us);
    } else {
        for (uint32_t e = 0; e < (uint32_t)E && i0 + e < count; ++e) {
            const uint32_t i = i0 + e, r = i / (uint32_t)a.cols, c = i - r * (uint32_t)a.cols;
            float m = mom[i], u;
            momentum_update(m, bf16_bits_to_float(grad[i]), u, pa);
            mom[i] = m;
            add_sq(sumsq, u);
            x[(int64_t)r * a.np + c] = (uint16_t)rne_bf16_bits(u);
        }
    }
    const double total = block_sum_d(sumsq, lds4);
    if (threadIdx.x == 0) partials[(int64_t)b * norm_blocks + blockIdx.x] = total;
}

// Zeros of X's padding for the flat pass: columns [cols, np) of rows
// [0, rows), then rows [rows, mp) whole; `pad` elements per matrix, walked by
// a grid of at most kPadBlocks workgroups per matrix.
constexpr int64_t kPadBlocks = 4096;
__global__ __launch_bounds__(kThreads) void muon_x_pad_kernel(
    int32_t rows, int32_t cols, int32_t np, int64_t pad, uint16_t *__restrict__ x_base,
    int64_t x_stride) {
    uint16_t *x = x_base + (int64_t)blockIdx.y * x_stride;
    const int64_t wpad = np - cols, side = (int64_t)rows * wpad;
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < pad;
         k += (int64_t)gridDim.x * kThreads) {
        if (k < side) {
            const int64_t r = k / wpad;
            x[r * np + cols + (k - r * wpad)] = 0;
        } else {
            x[(int64_t)rows * np + (k - side)] = 0;
        }
    }
}

struct PostArgs {
    int32_t rows, cols;
    int32_t vec;
    float decay, step_lr;
    int64_t o_ld;
    int64_t o_stride;
    const int32_t *reject;  // per-matrix flags, or NULL
    const float *dev;       // device scalars, or NULL
    double scale;           // the update scale of this shape (for dev)
};

__global__ __launch_bounds__(kThreads) void muon_post_kernel(
    MuonPtrs ptrs, PostArgs a, const uint16_t *__restrict__ o_base) {
    const int b = blockIdx.y;
    if (a.reject && a.reject[b]) return;
    if (a.dev) {
        // decay = fp32(1 - lr wd), step_lr = fp32(lr scale), formed in double
        // as the host forms them
        const double lr = (double)a.dev[kDevLr], wd = (double)a.dev[kDevWeightDecay];
        a.decay = (float)(1.0 - lr * wd);
        a.step_lr = (float)(lr * a.scale);
    }
    const uint32_t count = (uint32_t)a.rows * (uint32_t)a.cols;  // < 2^31
    const uint32_t i0 = (blockIdx.x * kThreads + threadIdx.x) * kPostEPT;
    if (i0 >= count) return;
    float *__restrict__ P = ptrs.master[b];
    uint16_t *__restrict__ W = ptrs.weight[b];
    const uint16_t *__restrict__ O = o_base + (int64_t)b * a.o_stride;
    if (a.vec && i0 + kPostEPT <= count) {
        // cols % 8 == 0: the elements share one row
        float p[kPostEPT], o[kPostEPT];
        ld_f32<kPostEPT, true>(P + i0, p);
        const uint32_t r = i0 / (uint32_t)a.cols, c = i0 - r * (uint32_t)a.cols;
        ld_bf16<kPostEPT>(O + (int64_t)r * a.o_ld + c, o);
#pragma unroll
        for (int e = 0; e < kPostEPT; ++e) p[e] = p[e] * a.decay - a.step_lr * o[e];
        st_f32<kPostEPT, true>(P + i0, p);
        if (W) st_bf16<kPostEPT>(W + i0, p);
        return;
    }
    for (uint32_t e = 0; e < (uint32_t)kPostEPT && i0 + e < count; ++e) {
        const uint32_t i = i0 + e;
        const uint32_t r = i / (uint32_t)a.cols, c = i - r * (uint32_t)a.cols;
        float o = bf16_bits_to_float(O[(int64_t)r * a.o_ld + c]);
        float p = P[i] * a.decay - a.step_lr * o;
        P[i] = p;
        if (W) W[i] = (uint16_t)rne_bf16_bits(p);
    }
}

// ------------------------------------------------------------------ health

constexpr int kHealthLoads = 4;      // 16-byte loads in flight per thread
constexpr int kHealthMaxBlocks = 256;

// One health launch covers the groups of a launch bin (at most
// kMaxCallGroups), described by this table in the kernel arguments.
struct HealthGroup {
    const uint16_t *x;     // X of matrix 0; matrix b at x + b * x_stride
    int64_t x_stride, count;
    double *psum;
    float *pmax;
    int32_t *flags;
    float *health;         // this group's first [ratio, absmax, rejected] triple
    int32_t hblocks, short_side;
    int32_t block0, mat0;  // first workgroup / matrix of this group in the grid
};
struct HealthLaunch {
    HealthGroup g[kMaxCallGroups];
    int32_t ngroups;
    float guard;
};

__device__ __forceinline__ void health_add(uint32_t bits, double &acc, float &amax) {
    const float x = bf16_bits_to_float(bits);
    const double xd = (double)x;
    acc = __builtin_fma(xd, xd, acc);  // the square is exact in double
    amax = __builtin_fmaxf(amax, __builtin_fabsf(x));  // a NaN shows in acc instead
}

// Partial sums of squares (fp64) and maxima of |x| over X of every matrix of
// the groups in the table: count = m * np contiguous bf16 per matrix (the
// padding columns are zero); hblocks workgroups per matrix, the groups'
// workgroups one after the other in the grid.  Sums in a fixed order: each
// thread's run, a wave butterfly, the waves in order.
__global__ __launch_bounds__(kThreads) void ns_health_kernel(HealthLaunch h) {
    __shared__ double lsum[kThreads / 64];
    __shared__ float lmax[kThreads / 64];
    int gi = 0;
    while (gi + 1 < h.ngroups && (int)blockIdx.x >= h.g[gi + 1].block0) ++gi;
    const HealthGroup &G = h.g[gi];
    const int local = (int)blockIdx.x - G.block0;
    const int b = local / G.hblocks, blk = local - b * G.hblocks;
    const uint16_t *__restrict__ X = G.x + (int64_t)b * G.x_stride;
    const int64_t step = (int64_t)G.hblocks * kThreads * 8;
    const int64_t count = G.count;
    int64_t i = ((int64_t)blk * kThreads + threadIdx.x) * 8;
    double acc = 0.0;
    float amax = 0.0f;
    for (; i + (kHealthLoads - 1) * step < count; i += kHealthLoads * step) {
        u32x4 w[kHealthLoads];
#pragma unroll
        for (int q = 0; q < kHealthLoads; ++q)
            w[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X + i + q * step));
#pragma unroll
        for (int q = 0; q < kHealthLoads; ++q) {
            const uint32_t v[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                health_add(v[e] & 0xFFFFu, acc, amax);
                health_add(v[e] >> 16, acc, amax);
            }
        }
    }
    for (; i < count; i += step) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X + i));
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            health_add(v[e] & 0xFFFFu, acc, amax);
            health_add(v[e] >> 16, acc, amax);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        acc += __shfl_xor(acc, off, 64);
        amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, 64));
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lsum[wave] = acc;
        lmax[wave] = amax;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = 0.0;
        float mx = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) {
            s += lsum[w];
            mx = __builtin_fmaxf(mx, lmax[w]);
        }
        G.psum[(int64_t)b * G.hblocks + blk] = s;
        G.pmax[(int64_t)b * G.hblocks + blk] = mx;
    }
}

// Per matrix (one wave each, matrices of the table's groups one after the
// other): the partials in a fixed order (each lane's run, then a butterfly),
// ratio = ||X||_F / sqrt(min(rows, cols)) formed in double and rounded once,
// absmax (NaN if any element is NaN, which the sum of squares carries),
// rejected = !(absmax <= guard).
__global__ __launch_bounds__(64) void ns_health_matrix_kernel(HealthLaunch h) {
    int gi = 0;
    while (gi + 1 < h.ngroups && (int)blockIdx.x >= h.g[gi + 1].mat0) ++gi;
    const HealthGroup &G = h.g[gi];
    const int b = (int)blockIdx.x - G.mat0;
    double s = 0.0;
    float mx = 0.0f;
    for (int i = threadIdx.x; i < G.hblocks; i += 64) {
        s += G.psum[(int64_t)b * G.hblocks + i];
        mx = __builtin_fmaxf(mx, G.pmax[(int64_t)b * G.hblocks + i]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        s += __shfl_xor(s, off, 64);
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (threadIdx.x != 0) return;
    if (__builtin_isnan(s)) mx = __builtin_nanf("");
    const float ratio = (float)(__builtin_sqrt(s) / __builtin_sqrt((double)G.short_side));
    const bool rejected = !(mx <= h.guard);
    G.flags[b] = rejected ? 1 : 0;
    G.health[3 * b] = ratio;
    G.health[3 * b + 1] = mx;
    G.health[3 * b + 2] = rejected ? 1.0f : 0.0f;
}

// The call's totals from its per-matrix triples (one wave; a count of 0/1
// flags and a maximum, both exact in any order).
__global__ __launch_bounds__(64) void ns_health_total_kernel(float *__restrict__ health,
                                                             int32_t nmat) {
    float rejected = 0.0f, worst = 0.0f;
    for (int i = threadIdx.x; i < nmat; i += 64) {
        const float *t = health + 2 + 3 * i;
        if (t[2] != 0.0f) rejected += 1.0f;
        else worst = __builtin_fmaxf(worst, t[0]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        rejected += __shfl_xor(rejected, off, 64);
        worst = __builtin_fmaxf(worst, __shfl_xor(worst, off, 64));
    }
    if (threadIdx.x == 0) {
        health[0] = rejected;
        health[1] = worst;
    }
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

int32_t ns_health_blocks(int64_t count) {
    const int64_t per = (int64_t)kThreads * 8 * kHealthLoads;
    const int64_t b = (count + per - 1) / per;
    return (int32_t)(b < 1 ? 1 : b > kHealthMaxBlocks ? kHealthMaxBlocks : b);
}

hipError_t launch_ns_health(const NsGroupRef *refs, const int *mat_first, int nrefs,
                            int ns_steps, float guard, float *health, hipStream_t stream) {
    HealthLaunch h{};
    h.ngroups = nrefs;
    h.guard = guard;
    int blocks = 0, mats = 0;
    for (int i = 0; i < nrefs; ++i) {
        const MuonGeom &g = *refs[i].geom;
        const MuonWorkspace &L = *refs[i].layout;
        char *ws = refs[i].base;
        HealthGroup &G = h.g[i];
        G.x = reinterpret_cast<const uint16_t *>(ws + ((ns_segments(g, ns_steps) & 1) ? L.xt0 : L.x));
        G.x_stride = (int64_t)(L.x_stride / 2);
        G.count = (int64_t)g.m * g.np;  // a multiple of 8: np is a multiple of 64
        G.psum = reinterpret_cast<double *>(ws + L.hsum);
        G.pmax = reinterpret_cast<float *>(ws + L.hmax);
        G.flags = reinterpret_cast<int32_t *>(ws + L.hflag);
        G.health = health + 2 + 3 * mat_first[i];
        G.hblocks = g.health_blocks;
        G.short_side = g.m;
        G.block0 = blocks;
        G.mat0 = mats;
        blocks += g.batch * g.health_blocks;
        mats += g.batch;
    }
    hipLaunchKernelGGL(ns_health_kernel, dim3(blocks), dim3(kThreads), 0, stream, h);
    hipLaunchKernelGGL(ns_health_matrix_kernel, dim3(mats), dim3(64), 0, stream, h);
    return hipGetLastError();
}

hipError_t launch_ns_health_total(float *health, int32_t nmat, hipStream_t stream) {
    hipLaunchKernelGGL(ns_health_total_kernel, dim3(1), dim3(64), 0, stream, health, nmat);
    return hipGetLastError();
}

int32_t muon_norm_blocks(int64_t count) {
    // room for the partials of either pass-1 form
    const int64_t a = (count + kChunk - 1) / kChunk;
    const int64_t b = (count + kThreads * kFlatEPT - 1) / (kThreads * kFlatEPT);
    return (int32_t)(a > b ? a : b);
}

int32_t muon_pre_tiles(const MuonGeom &g) {
    const int srows = g.transposed ? g.np : g.mp;
    const int scols = g.transposed ? g.mp : g.np;
    return (srows / kTile) * (scols / kTile);
}

hipError_t launch_muon_pre(const MuonGeom &g, const MuonPtrs &ptrs, float mu,
                           int32_t nesterov, float ns_eps, char *ws,
                           const MuonWorkspace &L, bool no_iterations, const float *dev,
                           hipStream_t stream) {
    const int64_t count = (int64_t)g.rows * g.cols;
    const float omm = (float)(1.0 - (double)mu);
    bool vec = (count % 8) == 0;
    for (int b = 0; b < g.batch; ++b)
        vec = vec && aligned16(ptrs.momentum[b]) && aligned16(ptrs.grad[b]);
    double *partials = reinterpret_cast<double *>(ws + L.partials);
    double *sd = muon_sd_ptr(ws, g, L);
    float *xs = muon_scale_ptr(ws, g, L);
    uint16_t *x = reinterpret_cast<uint16_t *>(ws + L.x);
    const int64_t xstr = (int64_t)(L.x_stride / 2);
    // stored-orientation padded extent
    const int scols = g.transposed ? g.mp : g.np;
    const int tiles = muon_pre_tiles(g);
    ScaleArgs sa{g.rows, g.cols, g.transposed, g.mp, g.np, scols / kTile, mu, omm, nesterov,
                 (vec && g.cols % 8 == 0) ? 1 : 0, dev, (no_iterations && g.transposed) ? 1 : 0};
    const int32_t chunks = (int32_t)((count + kChunk - 1) / kChunk);  // the separate pass 1
    if (!no_iterations) {
        int32_t parts = tiles;
        if (g.transposed && g.mp % 128 == 0 && g.np % 128 == 0) {
            // 128 x 128 tiles: 512-byte runs of M read and 256-byte runs of X written
            parts = (g.np / 128) * (g.mp / 128);
            hipLaunchKernelGGL(muon_momentum_x_kernel<128>, dim3(parts, g.batch), dim3(kThreads),
                               0, stream, ptrs, sa, partials, g.norm_blocks, x, xstr);
        } else if (g.transposed) {
            hipLaunchKernelGGL(muon_momentum_x_kernel<kTile>, dim3(tiles, g.batch), dim3(kThreads),
                               0, stream, ptrs, sa, partials, g.norm_blocks, x, xstr);
        } else {
            const int32_t fchunks = (int32_t)((count + kThreads * kFlatEPT - 1) / (kThreads * kFlatEPT));
            hipLaunchKernelGGL(muon_momentum_xflat_kernel, dim3(fchunks, g.batch), dim3(kThreads),
                               0, stream, ptrs, sa, partials, g.norm_blocks, x, xstr);
            parts = fchunks;
            const int64_t pad = (int64_t)g.rows * (g.np - g.cols) + (int64_t)(g.mp - g.rows) * g.np;
            if (pad > 0) {
                const int64_t blocks = (pad + kThreads - 1) / kThreads;
                hipLaunchKernelGGL(muon_x_pad_kernel,
                                   dim3((uint32_t)(blocks < kPadBlocks ? blocks : kPadBlocks),
                                        g.batch),
                                   dim3(kThreads), 0, stream, g.rows, g.cols, g.np, pad, x, xstr);
            }
        }
        // the norm, and the rewrite of X for a matrix whose ||U||_F^2 is out of
        // the first iteration's range (the other workgroups leave at once).
        // Every workgroup of a matrix sums all its partials, so matrices with
        // many get fewer workgroups (at least 4 for the rewrite)
        int fb = 16384 / (parts > 0 ? parts : 1);
        fb = fb < 4 ? 4 : fb > kFallbackBlocks ? kFallbackBlocks : fb;
        if (fb > tiles) fb = tiles;
        hipLaunchKernelGGL(muon_norm_kernel, dim3(fb, g.batch), dim3(kThreads), 0, stream, ptrs,
                           sa, partials, g.norm_blocks, parts, sd, xs, ns_eps, 1, tiles, x, xstr);
        return hipGetLastError();
    }
    PreArgs pa{(int32_t)count, vec ? 1 : 0, mu, omm, nesterov, dev};
    hipLaunchKernelGGL(muon_momentum_kernel, dim3(chunks, g.batch), dim3(kThreads),
                       0, stream, ptrs, pa, partials, g.norm_blocks);
    hipLaunchKernelGGL(muon_norm_kernel, dim3(1, g.batch), dim3(kThreads), 0, stream, ptrs, sa,
                       partials, g.norm_blocks, chunks, sd, xs, ns_eps, 0, tiles, x, xstr);
    hipLaunchKernelGGL(muon_scale_kernel, dim3(tiles, g.batch), dim3(kThreads), 0, stream,
                       ptrs, sa, sd, x, reinterpret_cast<uint16_t *>(ws + L.xt1), xstr,
                       (int64_t)(L.x_stride / 2));
    return hipGetLastError();
}

hipError_t launch_muon_post(const MuonGeom &g, const MuonPtrs &ptrs,
                            const uint16_t *o_base, int64_t o_ld, size_t o_stride,
                            float decay, float step_lr, const int32_t *reject,
                            const float *dev, double scale, hipStream_t stream) {
    const int64_t count = (int64_t)g.rows * g.cols;
    bool vec = (g.cols % 8) == 0;
    for (int b = 0; b < g.batch; ++b)
        vec = vec && aligned16(ptrs.master[b]) &&
              (ptrs.weight[b] == nullptr || aligned16(ptrs.weight[b]));
    PostArgs pa{g.rows, g.cols, vec ? 1 : 0, decay, step_lr, o_ld, (int64_t)(o_stride / 2),
                reject, dev, scale};
    const int64_t units = (count + kPostEPT - 1) / kPostEPT;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(muon_post_kernel, dim3((uint32_t)blocks, g.batch), dim3(kThreads), 0,
                       stream, ptrs, pa, o_base);
    return hipGetLastError();
}

}  // namespace zopt
