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
// weight (28 B).  A workgroup of 256 threads streams one tile of 256 shard
// elements, one element per thread, so a wave-wide instruction covers 256
// contiguous bytes of a state array.  When the buckets' pieces hold whole
// tiles, the full buckets are one launch of a (tiles per piece) x (buckets)
// grid whose flat index needs no division, so all four loads of a thread
// leave at once (adamw_bucket_grid_kernel); the rest of the shard is mapped
// through the bucket layout tile by tile (adamw_shard_kernel).  Measured on
// MI355X at 2.5e8 elements: 81% of the HBM peak, against 70% for
// 2048-element tiles of 16-byte vectors and 76-79% for 512-1024-element
// tiles -- on this part the many-stream step runs faster the smaller each
// workgroup's span of every array.  Nothing is re-read, so every access is a
// streaming (non-temporal) one.
//
// Also here: the squared gradient norm of the same shard (2 B read per
// element) and the clip statistics derived from it [DEG zero.py:
// ZeroMaster.grad_sq_norm; BluScript trainer source, cross-group global
// clipping block; dmuon PR #16, commit "device-tensor stats"], which a
// device-scale variant of the AdamW kernel reads as its grad_scale without
// any host round trip.
#include "zopt_internal.h"

// Bit-exact arithmetic: every + - * / below is one correctly rounded binary32
// operation; no contraction into fused multiply-adds.
#pragma clang fp contract(off)

namespace zopt {
namespace {

constexpr int kThreads = 256;            // threads per workgroup
constexpr int kTile = kThreads;          // shard elements per workgroup: one per thread
// Workgroups per launch: a dispatch's grid counts work-items in 32 bits, so
// longer shards are stepped by several launches, each from a tile offset.
constexpr int64_t kMaxLaunchTiles = int64_t(1) << 22;
constexpr int64_t kMaxGridY = 65535;     // buckets per bucket-grid launch

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

// Bucket of shard element j (j < full_len): j / piece through a double
// reciprocal, corrected by one step either way (exact for j < 2^52).
__device__ __forceinline__ int64_t bucket_of(int64_t j, const AdamWParams &a) {
    int64_t b = (int64_t)((double)j * a.inv_piece);
    if (b * a.piece > j) --b;
    else if ((b + 1) * a.piece <= j) ++b;
    return b;
}

// Flat index of shard element j and whether it is a real element.
__device__ __forceinline__ int64_t flat_of(int64_t j, const AdamWParams &a, bool &real) {
    if (j < a.full_len) {
        real = true;
        return j + bucket_of(j, a) * a.gap + a.rank_off;
    }
    const int64_t f = a.last_flat0 + (j - a.full_len);
    real = f < a.n;
    return f;
}

// Bucket of tile `tile` of [0, full_len) when a piece holds tpp whole tiles:
// tile / tpp through a double reciprocal, corrected by one step either way
// (exact for 32-bit tile indices).  Wave-uniform and short, so the gradient
// load it gates follows the state loads closely.
__device__ __forceinline__ uint32_t bucket_of_tile(uint32_t tile, const AdamWParams &a) {
    uint32_t b = (uint32_t)((double)tile * a.inv_tpp);
    if ((uint64_t)b * a.tpp > tile) --b;
    else if ((uint64_t)(b + 1) * a.tpp <= tile) ++b;
    return b;
}

// Flat index of the first element of tile [t0, t0 + tile) when the whole
// tile maps to consecutive real flat positions (one bucket's piece, no
// padding, inside the shard), else -1.
__device__ __forceinline__ int64_t tile_flat(int64_t t0, int64_t tile, const AdamWParams &a) {
    const int64_t t1 = t0 + tile;
    if (t1 <= a.full_len) {
        const int64_t b = bucket_of(t0, a);
        return bucket_of(t1 - 1, a) == b ? t0 + b * a.gap + a.rank_off : -1;
    }
    if (t0 >= a.full_len && t1 <= a.shard_len) {
        const int64_t f0 = a.last_flat0 + (t0 - a.full_len);
        return f0 + tile <= a.n ? f0 : -1;
    }
    return -1;
}

// One workgroup per tile of kTile shard elements, one element per thread,
// starting at tile `tile0`.  When the whole tile maps to consecutive real flat
// positions (the common case: buckets' pieces are long) the flat index is the
// tile's plus the thread's; a tile that straddles a bucket edge, touches
// padding or ends the shard maps each element through the bucket layout.
// kDevScale: grad_scale is read from the clip statistics in device memory
// (a.stats), and with a.skip_nonfinite a found_inf there leaves every output
// untouched.
template <bool kDevScale>
__global__ __launch_bounds__(kThreads) void adamw_shard_kernel(
    float *__restrict__ master, float *__restrict__ exp_avg, float *__restrict__ exp_avg_sq,
    const uint16_t *__restrict__ grad, uint16_t *__restrict__ weight, AdamWParams a,
    int64_t tile0) {
    if constexpr (kDevScale) {
        if (a.skip_nonfinite && a.stats[kClipFoundInf] != 0.0f) return;
        a.grad_scale = a.stats[kClipGradScale];
    }
    const int64_t tile = tile0 + (int64_t)blockIdx.x;
    const int64_t t0 = tile * kTile;
    const int64_t j = t0 + threadIdx.x;
    if (j >= a.shard_len) return;
    // the state loads depend on the shard index alone: issue them before the
    // layout arithmetic, which then runs while they are in flight
    float p = ld_stream(master + j), m = ld_stream(exp_avg + j), v = ld_stream(exp_avg_sq + j);
    int64_t f0;
    if (a.tpp && tile < a.full_tiles)
        f0 = t0 + (int64_t)bucket_of_tile((uint32_t)tile, a) * a.gap + a.rank_off;
    else
        f0 = tile_flat(t0, kTile, a);
    bool real = true;
    int64_t f;
    if (f0 >= 0)
        f = f0 + threadIdx.x;
    else
        f = flat_of(j, a, real);
    float g = 0.0f;
    if (real) g = bf16_bits_to_float(ld_stream(grad + f)) * a.grad_scale;
    adamw_update(p, m, v, g, a);
    st_stream(master + j, p);
    st_stream(exp_avg + j, m);
    st_stream(exp_avg_sq + j, v);
    if (real && weight) st_stream(weight + f, (uint16_t)rne_bf16_bits(p));
}

// The per-step scalars of the AdamW update, alone (the bucket-grid kernel's
// small argument block).
struct AdamWScalars {
    float beta1, beta2, eps, step_size, bc2_sqrt, decay, omb1, omb2, grad_scale;
    int32_t skip_nonfinite;
    const float *stats;
};

// The full buckets of the shard as a grid of (tiles per piece) x (buckets):
// blockIdx.y is the bucket, blockIdx.x the tile within this rank's piece of
// it.  grad_r and weight_r are the flat arrays advanced to this rank's piece
// of bucket 0, so the flat index of a tile is blockIdx.y * bstride +
// blockIdx.x * kTile from them, with bstride the adjusted bucket length:
// scalar arithmetic on the launch indices, and all four loads leave at once.
template <bool kDevScale>
__global__ __launch_bounds__(kThreads) void adamw_bucket_grid_kernel(
    float *__restrict__ master, float *__restrict__ exp_avg, float *__restrict__ exp_avg_sq,
    const uint16_t *__restrict__ grad_r, uint16_t *__restrict__ weight_r, int64_t bstride,
    uint32_t tpp, AdamWScalars s) {
    const int64_t j = ((int64_t)blockIdx.y * tpp + blockIdx.x) * kTile + threadIdx.x;
    const int64_t f = (int64_t)blockIdx.y * bstride + (int64_t)blockIdx.x * kTile + threadIdx.x;
    float p = ld_stream(master + j), m = ld_stream(exp_avg + j), v = ld_stream(exp_avg_sq + j);
    const float gb = bf16_bits_to_float(ld_stream(grad_r + f));
    if constexpr (kDevScale) {
        if (s.skip_nonfinite && s.stats[kClipFoundInf] != 0.0f) return;
        s.grad_scale = s.stats[kClipGradScale];
    }
    AdamWParams a;
    a.beta1 = s.beta1;
    a.beta2 = s.beta2;
    a.eps = s.eps;
    a.step_size = s.step_size;
    a.bc2_sqrt = s.bc2_sqrt;
    a.decay = s.decay;
    a.omb1 = s.omb1;
    a.omb2 = s.omb2;
    adamw_update(p, m, v, gb * s.grad_scale, a);
    st_stream(master + j, p);
    st_stream(exp_avg + j, m);
    st_stream(exp_avg_sq + j, v);
    if (weight_r) st_stream(weight_r + f, (uint16_t)rne_bf16_bits(p));
}

// ------------------------------------------------------------------ norm

constexpr int kNormLoads = 4;                              // 16-byte loads per thread per tile
constexpr int kNormTile = kThreads * 8 * kNormLoads;       // 8192 shard elements
typedef double f64;

// acc + x^2 for the bf16 value x: the square is exact in double (16
// significant bits, exponent in range), so one fused multiply-add rounds
// exactly as the separate multiply and add would.
__device__ __forceinline__ f64 add_sq_bf16(f64 acc, uint32_t bits) {
    const f64 x = (f64)bf16_bits_to_float(bits);
    return __builtin_fma(x, x, acc);
}

// Sum over the workgroup, the same in every run: a butterfly within each
// wave, then the waves' sums in wave order.  Valid in thread 0.
__device__ __forceinline__ f64 block_sum(f64 v, f64 *lds) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    f64 s = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < kThreads / 64; ++w) s += lds[w];
    return s;
}

// Partial sums of squares of the real gradient elements of the shard.  The
// grid is fixed by the shard length alone, so the summation order (each
// thread's running sum over its tiles, then the workgroup sum) is the same on
// every run and every device.  A tile of consecutive real flat positions is
// read with 16-byte loads, one contiguous kilobyte per wave instruction, four
// in flight per thread; any other tile element by element.
__global__ __launch_bounds__(kThreads) void grad_sq_norm_kernel(
    const uint16_t *__restrict__ grad, AdamWParams a, int64_t tiles, f64 *__restrict__ partials) {
    __shared__ f64 lds[kThreads / 64];
    f64 acc = 0.0;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t t0 = t * kNormTile;
        const int64_t f0 = a.vec ? tile_flat(t0, kNormTile, a) : -1;
        if (f0 >= 0 && (f0 & 7) == 0) {
            u32x4 g[kNormLoads];
#pragma unroll
            for (int q = 0; q < kNormLoads; ++q)
                g[q] = ld_stream(reinterpret_cast<const u32x4 *>(
                    grad + f0 + (int64_t)q * kThreads * 8 + threadIdx.x * 8));
#pragma unroll
            for (int q = 0; q < kNormLoads; ++q) {
                const uint32_t w[4] = {g[q].x, g[q].y, g[q].z, g[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = add_sq_bf16(acc, w[e] & 0xFFFFu);
                    acc = add_sq_bf16(acc, w[e] >> 16);
                }
            }
        } else {
            for (int k = 0; k < kNormTile / kThreads; ++k) {
                const int64_t j = t0 + (int64_t)k * kThreads + threadIdx.x;
                if (j >= a.shard_len) break;
                bool real;
                const int64_t f = flat_of(j, a, real);
                if (real) acc = add_sq_bf16(acc, grad[f]);
            }
        }
    }
    const f64 s = block_sum(acc, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

// sq[0] = the partials added in a fixed order (one workgroup).
__global__ __launch_bounds__(kThreads) void sq_norm_final_kernel(
    const f64 *__restrict__ partials, int32_t count, f64 *__restrict__ sq) {
    __shared__ f64 lds[kThreads / 64];
    f64 acc = 0.0;
    for (int i = threadIdx.x; i < count; i += kThreads) acc += partials[i];
    const f64 s = block_sum(acc, lds);
    if (threadIdx.x == 0) sq[0] = s;
}

// The clip statistics from `count` summed-square partials (in index order):
//   total_norm = fp32(sqrt(sum) * inv_scale); found_inf = total_norm not
//   finite; clip_coef = min(1, max_norm / (total_norm + 1e-6)) in binary32,
//   NaN staying NaN; clipped = !found_inf && clip_coef < 1;
//   grad_scale = inv_scale * clip_coef.
__global__ __launch_bounds__(64) void clip_stats_kernel(const f64 *__restrict__ sq, int32_t count,
                                                        float max_norm, float inv_scale,
                                                        float *__restrict__ stats) {
    if (threadIdx.x != 0) return;
    f64 total = 0.0;
    for (int i = 0; i < count; ++i) total += sq[i];
    const float norm = (float)(__builtin_sqrt(total) * (f64)inv_scale);
    const bool found_inf = !__builtin_isfinite(norm);
    float coef = max_norm / (norm + 1e-6f);
    if (coef > 1.0f) coef = 1.0f;
    stats[kClipTotalNorm] = norm;
    stats[kClipCoef] = coef;
    stats[kClipClipped] = (!found_inf && coef < 1.0f) ? 1.0f : 0.0f;
    stats[kClipFoundInf] = found_inf ? 1.0f : 0.0f;
    stats[kClipGradScale] = inv_scale * coef;
}

// dst[i] = bf16(src[i]), 6 bytes of traffic per element: 2048 elements per
// workgroup, two 16-byte loads and two 8-byte stores per thread (one
// contiguous kilobyte of fp32 per wave instruction), starting at tile
// `tile0`; element by element when the bases are not 16/8-byte aligned or
// at the end.  (Unlike the AdamW step's eight streams, this two-stream pass
// measured fastest with these larger tiles: 81% of the HBM peak against 77%
// for 1024-element and 38% for 256-element tiles.)
constexpr int kRoundGroups = 2;
constexpr int kRoundTile = kThreads * 4 * kRoundGroups;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kThreads) void round_bf16_kernel(
    const float *__restrict__ src, uint16_t *__restrict__ dst, int64_t n, int32_t vec,
    int64_t tile0) {
    const int64_t t0 = (tile0 + (int64_t)blockIdx.x) * kRoundTile;
    if (vec && t0 + kRoundTile <= n) {
#pragma unroll
        for (int q = 0; q < kRoundGroups; ++q) {
            const int64_t o = t0 + (int64_t)q * kThreads * 4 + threadIdx.x * 4;
            const f32x4 x = ld_stream(reinterpret_cast<const f32x4 *>(src + o));
            st_stream(reinterpret_cast<u32x2 *>(dst + o),
                      u32x2{pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w)});
        }
        return;
    }
    for (int k = 0; k < kRoundTile / kThreads; ++k) {
        const int64_t i = t0 + (int64_t)k * kThreads + threadIdx.x;
        if (i >= n) return;
        dst[i] = (uint16_t)rne_bf16_bits(src[i]);
    }
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_adamw_shard(float *master, float *exp_avg, float *exp_avg_sq,
                              const uint16_t *grad, uint16_t *weight,
                              const AdamWParams &p_in, hipStream_t stream) {
    AdamWParams p = p_in;
    p.inv_piece = 1.0 / (double)p.piece;
    const int64_t tiles = (p.shard_len + kTile - 1) / kTile;
    p.tpp = 0;
    if (p.piece % kTile == 0 && p.piece / kTile <= (int64_t)UINT32_MAX &&
        tiles <= (int64_t)UINT32_MAX) {
        p.tpp = (uint32_t)(p.piece / kTile);
        p.full_tiles = (uint32_t)(p.full_len / kTile);
        p.inv_tpp = 1.0 / (double)p.tpp;
    }
    int64_t t = 0;
    if (p.tpp && p.full_tiles > 0 && p.tpp <= kMaxLaunchTiles &&
        p.full_tiles / p.tpp <= kMaxGridY) {
        // the full buckets as one (tiles per piece) x (buckets) grid
        const dim3 grid(p.tpp, p.full_tiles / p.tpp);
        const AdamWScalars sc{p.beta1, p.beta2,    p.eps,  p.step_size, p.bc2_sqrt,
                              p.decay, p.omb1,     p.omb2, p.grad_scale, p.skip_nonfinite,
                              p.stats};
        const int64_t bstride = p.gap + p.piece;
        const uint16_t *grad_r = grad + p.rank_off;
        uint16_t *weight_r = weight ? weight + p.rank_off : nullptr;
        if (p.stats)
            hipLaunchKernelGGL(adamw_bucket_grid_kernel<true>, grid, dim3(kThreads), 0, stream,
                               master, exp_avg, exp_avg_sq, grad_r, weight_r, bstride, p.tpp, sc);
        else
            hipLaunchKernelGGL(adamw_bucket_grid_kernel<false>, grid, dim3(kThreads), 0, stream,
                               master, exp_avg, exp_avg_sq, grad_r, weight_r, bstride, p.tpp, sc);
        t = p.full_tiles;
    }
    for (; t < tiles; t += kMaxLaunchTiles) {
        const uint32_t blocks = (uint32_t)(tiles - t < kMaxLaunchTiles ? tiles - t : kMaxLaunchTiles);
        if (p.stats)
            hipLaunchKernelGGL(adamw_shard_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream,
                               master, exp_avg, exp_avg_sq, grad, weight, p, t);
        else
            hipLaunchKernelGGL(adamw_shard_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream,
                               master, exp_avg, exp_avg_sq, grad, weight, p, t);
    }
    return hipGetLastError();
}

int32_t grad_sq_norm_blocks(int64_t shard_len) {
    const int64_t tiles = (shard_len + kNormTile - 1) / kNormTile;
    return (int32_t)(tiles < kNormBlocksMax ? tiles : kNormBlocksMax);
}

hipError_t launch_grad_sq_norm(const uint16_t *grad, const AdamWParams &p_in, double *partials,
                               double *sq, hipStream_t stream) {
    AdamWParams p = p_in;
    p.vec = aligned16(grad);
    p.inv_piece = 1.0 / (double)p.piece;
    const int64_t tiles = (p.shard_len + kNormTile - 1) / kNormTile;
    const int32_t blocks = grad_sq_norm_blocks(p.shard_len);
    hipLaunchKernelGGL(grad_sq_norm_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                       grad, p, tiles, partials);
    hipLaunchKernelGGL(sq_norm_final_kernel, dim3(1), dim3(kThreads), 0, stream, partials, blocks,
                       sq);
    return hipGetLastError();
}

hipError_t launch_clip_stats(const double *sq, int32_t count, float max_norm, float inv_scale,
                             float *stats, hipStream_t stream) {
    hipLaunchKernelGGL(clip_stats_kernel, dim3(1), dim3(64), 0, stream, sq, count, max_norm,
                       inv_scale, stats);
    return hipGetLastError();
}

hipError_t launch_round_bf16(const float *src, uint16_t *dst, int64_t n,
                             hipStream_t stream) {
    const int32_t vec = aligned16(src) && ((uintptr_t)dst & 7u) == 0;
    const int64_t tiles = (n + kRoundTile - 1) / kRoundTile;
    for (int64_t t = 0; t < tiles; t += kMaxLaunchTiles) {
        const uint32_t blocks = (uint32_t)(tiles - t < kMaxLaunchTiles ? tiles - t : kMaxLaunchTiles);
        hipLaunchKernelGGL(round_bf16_kernel, dim3(blocks), dim3(kThreads), 0, stream, src, dst,
                           n, vec, t);
    }
    return hipGetLastError();
}

}  // namespace zopt
