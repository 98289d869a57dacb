// adamw_shard.hip -- the fused one-pass AdamW over a rank's flat shard, and
// the standalone fp32 -> bf16 write-back.
//
// AdamW per element, in the order of dmuon PR #16 (commit "foreach AdamW":
// decoupled decay, then moments, then the bias-corrected addcdiv), on fp32
// state (BluScript trainer source, optimizer-precision note) with the bf16
// gradient promoted in registers and grad_scale applied on load (DeepSpeed
// PR #9021, commits "bf16 gradients of fp32 params" and "grad_scale").  The
// shard-to-flat index map is the bucket layout of DEG zero.py (ZeroMaster).
//
// The step is bound by HBM bandwidth: per shard element it reads 2 B of
// gradient and 12 B of fp32 state and writes 12 B of state and 2 B of bf16
// weight (28 B).  Each thread takes one unit of 8 consecutive shard elements:
// three pairs of 128-bit loads and stores for master / exp_avg / exp_avg_sq,
// one 128-bit gradient load and one 128-bit weight store.  Nothing is
// re-read, so every access is a streaming (non-temporal) one.
#include "zopt_internal.h"

// Bit-exact arithmetic: every + - * / below is one correctly rounded binary32
// operation; no contraction into fused multiply-adds.
#pragma clang fp contract(off)

namespace zopt {
namespace {

constexpr int kUnit = 8;            // shard elements per thread
constexpr int kThreads = 256;       // threads per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld_stream(const T *p) {
    return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void st_stream(T *p, T v) {
    __builtin_nontemporal_store(v, p);
}

__device__ __forceinline__ void adamw_update(float &p, float &m, float &v, float g,
                                             const AdamWParams &a) {
    p = p * a.decay;
    m = a.beta1 * m + a.omb1 * g;
    v = a.beta2 * v + (a.omb2 * g) * g;
    float denom = __builtin_sqrtf(v) / a.bc2_sqrt + a.eps;
    p = p - a.step_size * (m / denom);
}

// Flat index of shard element j and whether it is a real element.
__device__ __forceinline__ int64_t flat_of(int64_t j, const AdamWParams &a, bool &real) {
    if (j < a.full_len) {
        int64_t b = (int64_t)((uint64_t)j / (uint64_t)a.piece);
        real = true;
        return j + b * a.gap + a.rank_off;
    }
    int64_t f = a.last_flat0 + (j - a.full_len);
    real = f < a.n;
    return f;
}

// One element at a time: any unit that straddles a bucket edge, touches
// padding, is misaligned, or runs past the end of the shard.
__device__ void adamw_unit_scalar(float *__restrict__ master, float *__restrict__ exp_avg,
                                  float *__restrict__ exp_avg_sq,
                                  const uint16_t *__restrict__ grad,
                                  uint16_t *__restrict__ weight, int64_t j0,
                                  const AdamWParams &a) {
    for (int e = 0; e < kUnit; ++e) {
        int64_t j = j0 + e;
        if (j >= a.shard_len) return;
        bool real;
        int64_t f = flat_of(j, a, real);
        float g = 0.0f;
        if (real) g = bf16_bits_to_float(grad[f]) * a.grad_scale;
        float p = master[j], m = exp_avg[j], v = exp_avg_sq[j];
        adamw_update(p, m, v, g, a);
        master[j] = p;
        exp_avg[j] = m;
        exp_avg_sq[j] = v;
        if (real && weight) weight[f] = (uint16_t)rne_bf16_bits(p);
    }
}

__global__ __launch_bounds__(kThreads) void adamw_shard_kernel(
    float *__restrict__ master, float *__restrict__ exp_avg, float *__restrict__ exp_avg_sq,
    const uint16_t *__restrict__ grad, uint16_t *__restrict__ weight, AdamWParams a) {
    const int64_t unit = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t j0 = unit * kUnit;
    if (j0 >= a.shard_len) return;

    // Decide whether the 8 elements map to 8 consecutive, real, 8-aligned
    // flat positions inside one bucket.
    bool fast = false;
    int64_t f0 = 0;
    if (a.vec && j0 + kUnit <= a.shard_len) {
        if (j0 + kUnit <= a.full_len) {
            uint64_t b0 = (uint64_t)j0 / (uint64_t)a.piece;
            uint64_t b7 = (uint64_t)(j0 + kUnit - 1) / (uint64_t)a.piece;
            f0 = j0 + (int64_t)b0 * a.gap + a.rank_off;
            fast = (b0 == b7) && ((f0 & (kUnit - 1)) == 0);
        } else if (j0 >= a.full_len) {
            f0 = a.last_flat0 + (j0 - a.full_len);
            fast = (f0 + kUnit <= a.n) && ((f0 & (kUnit - 1)) == 0);
        }
    }
    if (!fast) {
        adamw_unit_scalar(master, exp_avg, exp_avg_sq, grad, weight, j0, a);
        return;
    }

    const f32x4 *P = reinterpret_cast<const f32x4 *>(master + j0);
    const f32x4 *M = reinterpret_cast<const f32x4 *>(exp_avg + j0);
    const f32x4 *V = reinterpret_cast<const f32x4 *>(exp_avg_sq + j0);
    const u32x4 *G = reinterpret_cast<const u32x4 *>(grad + f0);
    f32x4 p0 = ld_stream(P), p1 = ld_stream(P + 1);
    f32x4 m0 = ld_stream(M), m1 = ld_stream(M + 1);
    f32x4 v0 = ld_stream(V), v1 = ld_stream(V + 1);
    u32x4 gw = ld_stream(G);

    float p[kUnit] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
    float m[kUnit] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float v[kUnit] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t gbits[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
    for (int e = 0; e < kUnit; ++e) {
        uint32_t h = (gbits[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
        float g = bf16_bits_to_float(h) * a.grad_scale;
        adamw_update(p[e], m[e], v[e], g, a);
    }
    f32x4 *Pw = reinterpret_cast<f32x4 *>(master + j0);
    f32x4 *Mw = reinterpret_cast<f32x4 *>(exp_avg + j0);
    f32x4 *Vw = reinterpret_cast<f32x4 *>(exp_avg_sq + j0);
    st_stream(Pw, f32x4{p[0], p[1], p[2], p[3]});
    st_stream(Pw + 1, f32x4{p[4], p[5], p[6], p[7]});
    st_stream(Mw, f32x4{m[0], m[1], m[2], m[3]});
    st_stream(Mw + 1, f32x4{m[4], m[5], m[6], m[7]});
    st_stream(Vw, f32x4{v[0], v[1], v[2], v[3]});
    st_stream(Vw + 1, f32x4{v[4], v[5], v[6], v[7]});
    if (weight) {
        u32x4 w{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        st_stream(reinterpret_cast<u32x4 *>(weight + f0), w);
    }
}

// dst[i] = bf16(src[i]); 8 elements per thread, 6 bytes of traffic each.
__global__ __launch_bounds__(kThreads) void round_bf16_kernel(
    const float *__restrict__ src, uint16_t *__restrict__ dst, int64_t n, int32_t vec) {
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * kUnit;
    if (i0 >= n) return;
    if (vec && i0 + kUnit <= n) {
        const f32x4 *S = reinterpret_cast<const f32x4 *>(src + i0);
        f32x4 a = ld_stream(S), b = ld_stream(S + 1);
        u32x4 w{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y),
                pack_bf16x2(b.z, b.w)};
        st_stream(reinterpret_cast<u32x4 *>(dst + i0), w);
        return;
    }
    for (int e = 0; e < kUnit && i0 + e < n; ++e)
        dst[i0 + e] = (uint16_t)rne_bf16_bits(src[i0 + e]);
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_adamw_shard(float *master, float *exp_avg, float *exp_avg_sq,
                              const uint16_t *grad, uint16_t *weight,
                              const AdamWParams &p_in, hipStream_t stream) {
    AdamWParams p = p_in;
    p.vec = aligned16(master) && aligned16(exp_avg) && aligned16(exp_avg_sq) &&
            aligned16(grad) && (weight == nullptr || aligned16(weight));
    const int64_t units = (p.shard_len + kUnit - 1) / kUnit;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(adamw_shard_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, master, exp_avg, exp_avg_sq, grad, weight, p);
    return hipGetLastError();
}

hipError_t launch_round_bf16(const float *src, uint16_t *dst, int64_t n,
                             hipStream_t stream) {
    const int32_t vec = aligned16(src) && aligned16(dst);
    const int64_t units = (n + kUnit - 1) / kUnit;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(round_bf16_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, src, dst, n, vec);
    return hipGetLastError();
}

}  // namespace zopt
