// muon_prepost.hip -- the bandwidth-bound passes around Newton-Schulz.
//
// Pre-step [BluScript trainer source, Muon config block: momentum 0.95 with
// Nesterov; the momentum buffer is an exponential moving average of the
// gradient; dmuon PR #16, commit "NS CUDA-graph replay": momentum, lr and wd
// stay in the eager pre/post steps around the fixed-shape Newton-Schulz]:
//   pass 1  M = mu M + (1-mu) g, U = (1-mu) g + mu M (or U = M); write M,
//           one fp32 partial sum of U^2 per workgroup            (10 B/elem)
//   final   per matrix, s = 1 / (sqrt(sum of partials) + eps), the partials
//           summed in a fixed order (deterministic)
//   pass 2  recompute U from the new M (bitwise the same U), write
//           X0 = bf16(U s) in the Newton-Schulz orientation and its transpose,
//           zero-filling the tile padding                        (10 B/elem)
// Post-step [BluScript trainer source: Muon weight decay pinned to AdamW's;
// the adjust_lr note on the update scale]:
//   P = P * decay - step_lr * O, W = bf16(P)                      (12 B/elem)
#include "zopt_internal.h"

// M, U and P are bit-exact binary32 arithmetic: no contraction.
#pragma clang fp contract(off)

namespace zopt {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 8;       // elements per thread per sweep
constexpr int kSweeps = 4;          // sweeps per workgroup in pass 1
constexpr int kChunk = kThreads * kPerThread * kSweeps;  // elements / workgroup
constexpr int kTile = 64;           // pass-2 transpose tile

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Fixed-order sum over the workgroup: butterfly within each 64-wide wave,
// then the four wave sums in order.
__device__ float block_sum(float x, float *lds4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds4[wave] = x;
    __syncthreads();
    float s = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
    __syncthreads();
    return s;
}

struct PreArgs {
    int32_t count;        // rows * cols
    int32_t vec;          // 8-element vector path allowed
    float mu, omm;
    int32_t nesterov;
};

__device__ __forceinline__ void momentum_update(float &m, float g, float &u,
                                                const PreArgs &a) {
    m = a.mu * m + a.omm * g;
    u = a.nesterov ? a.omm * g + a.mu * m : m;
}

__global__ __launch_bounds__(kThreads) void muon_momentum_kernel(
    MuonPtrs ptrs, PreArgs a, float *__restrict__ partials, int32_t norm_blocks) {
    __shared__ float lds4[4];
    const int b = blockIdx.y;
    float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    float sumsq = 0.0f;
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    for (int s = 0; s < kSweeps; ++s) {
        const int64_t i0 = base + ((int64_t)s * kThreads + threadIdx.x) * kPerThread;
        if (i0 >= a.count) break;
        if (a.vec && i0 + kPerThread <= a.count) {
            f32x4 *M = reinterpret_cast<f32x4 *>(mom + i0);
            u32x4 gw = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(grad + i0));
            f32x4 m0 = M[0], m1 = M[1];
            float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
            uint32_t gb[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float g = bf16_bits_to_float((gb[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
                float u;
                momentum_update(m[e], g, u, a);
                sumsq += u * u;
            }
            M[0] = f32x4{m[0], m[1], m[2], m[3]};
            M[1] = f32x4{m[4], m[5], m[6], m[7]};
        } else {
            for (int e = 0; e < kPerThread && i0 + e < a.count; ++e) {
                float g = bf16_bits_to_float(grad[i0 + e]);
                float m = mom[i0 + e], u;
                momentum_update(m, g, u, a);
                mom[i0 + e] = m;
                sumsq += u * u;
            }
        }
    }
    float total = block_sum(sumsq, lds4);
    if (threadIdx.x == 0) partials[(int64_t)b * norm_blocks + blockIdx.x] = total;
}

// One workgroup per matrix: s = 1 / (||U||_F + eps) from the partials.
__global__ __launch_bounds__(kThreads) void muon_norm_kernel(
    float *__restrict__ partials, int32_t norm_blocks, float *__restrict__ scale,
    float ns_eps) {
    __shared__ float lds4[4];
    const int b = blockIdx.x;
    const float *p = partials + (int64_t)b * norm_blocks;
    float s = 0.0f;
    for (int i = threadIdx.x; i < norm_blocks; i += kThreads) s += p[i];
    float total = block_sum(s, lds4);
    if (threadIdx.x == 0) scale[b] = 1.0f / (__builtin_sqrtf(total) + ns_eps);
}

struct ScaleArgs {
    int32_t rows, cols;     // stored shape
    int32_t transposed;     // X = U^T
    int32_t mp, np;         // padded Newton-Schulz shape (X is mp x np)
    int32_t tiles_c;        // tiles along the stored columns (padded)
    float mu, omm;
    int32_t nesterov;
    int32_t vec;            // cols % 8 == 0 and every base 16-byte aligned
};

// Pass 2.  One workgroup per 64 x 64 tile of the padded stored-orientation
// matrix.  The stored orientation is X when rows <= cols and X^T otherwise;
// it is written straight out, and the LDS-transposed tile goes to the other.
__global__ __launch_bounds__(kThreads) void muon_scale_kernel(
    MuonPtrs ptrs, ScaleArgs a, const float *__restrict__ scale,
    uint16_t *__restrict__ x_base, uint16_t *__restrict__ xt_base,
    int64_t x_stride, int64_t xt_stride) {
    __shared__ uint16_t tile[kTile][kTile + 2];
    const int b = blockIdx.y;
    const int tr = blockIdx.x / a.tiles_c, tc = blockIdx.x % a.tiles_c;
    const float s = scale[b];
    const float *__restrict__ mom = ptrs.momentum[b];
    const uint16_t *__restrict__ grad = ptrs.grad[b];
    // the stored-orientation output and its padded leading dimension
    uint16_t *direct = a.transposed ? xt_base + (int64_t)b * xt_stride
                                    : x_base + (int64_t)b * x_stride;
    uint16_t *other = a.transposed ? x_base + (int64_t)b * x_stride
                                   : xt_base + (int64_t)b * xt_stride;
    const int64_t ld_direct = a.transposed ? a.mp : a.np;
    const int64_t ld_other = a.transposed ? a.np : a.mp;
    PreArgs pa{0, 0, a.mu, a.omm, a.nesterov};

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
                const float u = a.nesterov ? pa.omm * g + pa.mu * mv[e] : mv[e];
                xs[e] = u * s;
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
                        float u = a.nesterov ? pa.omm * g + pa.mu * m : m;
                        x = u * s;
                    }
                    x2[h] = x;
                }
                packed[e >> 1] = pack_bf16x2(x2[0], x2[1]);
            }
        }
        *reinterpret_cast<u32x4 *>(direct + (int64_t)r * ld_direct + c0) =
            u32x4{packed[0], packed[1], packed[2], packed[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            tile[lr][lc + e] = (uint16_t)((packed[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
    }
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
}

struct PostArgs {
    int32_t rows, cols;
    int32_t vec;
    float decay, step_lr;
    int64_t o_ld;
    int64_t o_stride;
};

__global__ __launch_bounds__(kThreads) void muon_post_kernel(
    MuonPtrs ptrs, PostArgs a, const uint16_t *__restrict__ o_base) {
    const int b = blockIdx.y;
    const int64_t count = (int64_t)a.rows * a.cols;
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kPerThread;
    if (i0 >= count) return;
    float *__restrict__ P = ptrs.master[b];
    uint16_t *__restrict__ W = ptrs.weight[b];
    const uint16_t *__restrict__ O = o_base + (int64_t)b * a.o_stride;
    if (a.vec && i0 + kPerThread <= count) {
        // cols % 8 == 0: the 8 elements share one row
        const int64_t r = i0 / a.cols, c = i0 - r * a.cols;
        u32x4 ow = *reinterpret_cast<const u32x4 *>(O + r * a.o_ld + c);
        f32x4 *Pv = reinterpret_cast<f32x4 *>(P + i0);
        f32x4 p0 = __builtin_nontemporal_load(Pv), p1 = __builtin_nontemporal_load(Pv + 1);
        float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        uint32_t ob[4] = {ow.x, ow.y, ow.z, ow.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float o = bf16_bits_to_float((ob[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
            p[e] = p[e] * a.decay - a.step_lr * o;
        }
        __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, Pv);
        __builtin_nontemporal_store(f32x4{p[4], p[5], p[6], p[7]}, Pv + 1);
        if (W) {
            u32x4 w{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                    pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(W + i0));
        }
        return;
    }
    for (int e = 0; e < kPerThread && i0 + e < count; ++e) {
        const int64_t i = i0 + e;
        const int64_t r = i / a.cols, c = i - r * a.cols;
        float o = bf16_bits_to_float(O[r * a.o_ld + c]);
        float p = P[i] * a.decay - a.step_lr * o;
        P[i] = p;
        if (W) W[i] = (uint16_t)rne_bf16_bits(p);
    }
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

int32_t muon_norm_blocks(int64_t count) { return (int32_t)((count + kChunk - 1) / kChunk); }

hipError_t launch_muon_pre(const MuonGeom &g, const MuonPtrs &ptrs, float mu,
                           int32_t nesterov, float ns_eps, char *ws,
                           const MuonWorkspace &L, hipStream_t stream) {
    const int64_t count = (int64_t)g.rows * g.cols;
    const float omm = (float)(1.0 - (double)mu);
    bool vec = (count % 8) == 0;
    for (int b = 0; b < g.batch; ++b)
        vec = vec && aligned16(ptrs.momentum[b]) && aligned16(ptrs.grad[b]);
    PreArgs pa{(int32_t)count, vec ? 1 : 0, mu, omm, nesterov};
    float *partials = reinterpret_cast<float *>(ws + L.partials);
    float *scale = partials + (int64_t)g.batch * g.norm_blocks;
    hipLaunchKernelGGL(muon_momentum_kernel, dim3(g.norm_blocks, g.batch), dim3(kThreads),
                       0, stream, ptrs, pa, partials, g.norm_blocks);
    hipLaunchKernelGGL(muon_norm_kernel, dim3(g.batch), dim3(kThreads), 0, stream, partials,
                       g.norm_blocks, scale, ns_eps);
    // stored-orientation padded extent
    const int srows = g.transposed ? g.np : g.mp;
    const int scols = g.transposed ? g.mp : g.np;
    ScaleArgs sa{g.rows, g.cols, g.transposed, g.mp, g.np, scols / kTile, mu, omm, nesterov,
                 (vec && g.cols % 8 == 0) ? 1 : 0};
    const int tiles = (srows / kTile) * (scols / kTile);
    hipLaunchKernelGGL(muon_scale_kernel, dim3(tiles, g.batch), dim3(kThreads), 0, stream,
                       ptrs, sa, scale, reinterpret_cast<uint16_t *>(ws + L.x),
                       reinterpret_cast<uint16_t *>(ws + L.xt0),
                       (int64_t)(L.x_stride / 2), (int64_t)(L.x_stride / 2));
    return hipGetLastError();
}

hipError_t launch_muon_post(const MuonGeom &g, const MuonPtrs &ptrs,
                            const uint16_t *o_base, int64_t o_ld, size_t o_stride,
                            float decay, float step_lr, hipStream_t stream) {
    const int64_t count = (int64_t)g.rows * g.cols;
    bool vec = (g.cols % 8) == 0;
    for (int b = 0; b < g.batch; ++b)
        vec = vec && aligned16(ptrs.master[b]) &&
              (ptrs.weight[b] == nullptr || aligned16(ptrs.weight[b]));
    PostArgs pa{g.rows, g.cols, vec ? 1 : 0, decay, step_lr, o_ld, (int64_t)(o_stride / 2)};
    const int64_t units = (count + kPerThread - 1) / kPerThread;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(muon_post_kernel, dim3((uint32_t)blocks, g.batch), dim3(kThreads), 0,
                       stream, ptrs, pa, o_base);
    return hipGetLastError();
}

}  // namespace zopt
