// zopt_api.hip -- the C-ABI entry points of libzopt (declared in zopt.h).
//
// Each entry point checks its arguments, derives the launch parameters on the
// host (layout of the flat shard, per-step scalars in double rounded once to
// binary32, workspace carve-up), and enqueues its kernels on the caller's
// stream without synchronising.  Nothing is enqueued unless every check
// passes.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "zopt.h"
#include "zopt_internal.h"

#define ZOPT_EXPORT extern "C" __attribute__((visibility("default")))

namespace zopt {

int32_t muon_norm_blocks(int64_t count);  // muon_prepost.hip

namespace {

inline bool finite(float x) { return std::isfinite(x); }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t round_up64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Flat bucketed shard layout [DEG zero.py, ZeroMaster.__init__]: the bucket
// is lowered to a multiple of world (never below world); every bucket but
// possibly the last has that full length and no padding; the last is padded
// to a multiple of world.  Fills the shard-region fields of p and returns
// the shard length.
int64_t adamw_layout(int64_t n, int64_t bucket, int32_t world, int32_t rank,
                     AdamWParams &p) {
    const int64_t w = world;
    int64_t B = bucket - bucket % w;
    if (B < w) B = w;
    const int64_t nb = (n + B - 1) / B;
    const int64_t piece = B / w;
    const int64_t last_len = n - (nb - 1) * B;
    p.piece = piece;
    p.gap = B - piece;
    p.rank_off = (int64_t)rank * piece;
    p.n = n;
    if (last_len == B) {
        p.full_len = nb * piece;
        p.last_flat0 = 0;
        return p.full_len;
    }
    const int64_t last_piece = (last_len + w - 1) / w;  // ceil(len / w) * w / w
    p.full_len = (nb - 1) * piece;
    p.last_flat0 = (nb - 1) * B + (int64_t)rank * last_piece;
    return p.full_len + last_piece;
}

}  // namespace

// The Newton-Schulz form (zopt_set_ns_form): 0 on the Gram matrix where the
// shape favours it (its m x m chain in fp16 where the coefficients allow), 1
// plain iterations throughout, 2 as 0 with the chain always in bf16.
std::atomic<int> g_ns_form{0};

MuonGeom muon_geometry(int32_t batch, int64_t rows, int64_t cols) {
    MuonGeom g{};
    g.batch = batch;
    g.rows = (int32_t)rows;
    g.cols = (int32_t)cols;
    g.transposed = rows > cols ? 1 : 0;
    g.m = (int32_t)(rows < cols ? rows : cols);
    g.n = (int32_t)(rows < cols ? cols : rows);
    // 256 x 256 tiles from m = 1024 on, and from m = 768 on where they pad m
    // no further than 128 x 128 tiles would (m = 768, or 897 .. 1023): 6
    // upper-triangle tiles per 768-row matrix instead of 21.  On GPT-2-small's
    // three 768-row groups (432 X X^T workgroups, under two rounds, so the
    // iterations run on two streams) Newton-Schulz took 1.630 ms per call
    // against 1.718 on 128 tiles; on one stream the 256 tiles alone took 1.743.
    const bool big = g.m >= 1024 || (g.m >= 768 && round_up64(g.m, 256) == round_up64(g.m, 128));
    g.tile = big ? 256 : g.m >= 256 ? 128 : 64;
    g.mp = (int32_t)round_up64(g.m, g.tile);
    g.np = (int32_t)round_up64(g.n, g.tile);
    // B X has 2 m^2 n of the 3 m^2 n + m^3 flops: where the padded sizes allow,
    // it takes the larger tile, which does more work per byte staged
    g.tile_bx = (g.tile == 128 && g.mp % 256 == 0 && g.np % 256 == 0) ? 256 : g.tile;
    // X X^T and A A touch only the upper-triangle tiles: a group with fewer
    // than 128 of them at 256 x 256 would leave most of the GPU idle, so it
    // takes 128 x 128 tiles (four times as many) for those two products
    const int64_t t256 = g.mp / 256;
    if (g.tile == 256 && (int64_t)batch * (t256 * (t256 + 1) / 2) < 128) g.tile = 128;
    const int32_t chunks = muon_norm_blocks(rows * cols), tiles = muon_pre_tiles(g);
    g.norm_blocks = chunks > tiles ? chunks : tiles;
    // X X^T of a group with a long reduction and fewer upper-triangle tiles of
    // 256 than the GPU has compute units is split along K in two: its tiles
    // would otherwise set the length of the launch.  The rule depends on the
    // group alone, so a group's result is the same in any call.
    const int64_t u256 = (g.mp + 255) / 256;
    g.ksplit = (g.np >= 8192 && (int64_t)batch * (u256 * (u256 + 1) / 2) < 256) ? 2 : 1;
    g.health_blocks = ns_health_blocks((int64_t)g.m * g.np);
    // Newton-Schulz on the Gram matrix where the long side is at least twice
    // the short one: a segment of L steps costs 3 m^2 n + (4 L - 3) m^3 flops
    // against L (3 m^2 n + m^3) for plain iterations (five steps in segments
    // of 3 and 2: 6 m^2 n + 14 m^3 against 15 m^2 n + 5 m^3), and two more
    // launches, so only for groups where the flops saved, 9 batch m^2 (n - m)
    // for five steps, are worth more than those (batch m^2 (n - m) >= 2^29;
    // 2 x [128, 512] stays plain: 0.099 ms per call against 0.107)
    const double saved = (double)batch * g.m * g.m * ((double)g.n - g.m);
    g.gram = (g_ns_form.load(std::memory_order_relaxed) != 1 && (int64_t)g.n >= 2 * (int64_t)g.m &&
              saved >= (double)(1 << 29) && g.m <= kNsF16MaxM) ? 1 : 0;
    return g;
}

MuonWorkspace muon_workspace_layout(const MuonGeom &g) {
    MuonWorkspace L{};
    L.x_stride = round_up((size_t)g.mp * g.np * 2, 256);
    L.a_stride = round_up((size_t)g.mp * g.mp * 2, 256);
    L.d_stride = round_up((size_t)g.mp * 4, 256);
    size_t off = 0;
    L.x = off;   off += L.x_stride * g.batch;
    L.xt0 = off; off += L.x_stride * g.batch;
    L.xt1 = off; off += L.x_stride * g.batch;
    L.nslots = g.gram ? kNsSlots : 2;
    for (int k = 0; k < L.nslots; ++k) {
        L.sm[k] = off;
        off += L.a_stride * g.batch;
    }
    for (int k = 0; k < L.nslots; ++k) {
        L.sd[k] = off;
        off += L.d_stride * g.batch;
    }
    L.part = off;
    if (g.ksplit > 1) off += round_up((size_t)g.ksplit * g.batch * g.mp * g.mp * 4, 256);
    L.partials = off;
    off += round_up(((size_t)g.batch * g.norm_blocks + g.batch) * sizeof(double) +
                        (size_t)g.batch * sizeof(float), 256);
    const size_t hparts = (size_t)g.batch * g.health_blocks;
    L.hsum = off;  off += round_up(hparts * sizeof(double), 256);
    L.hmax = off;  off += round_up(hparts * sizeof(float), 256);
    L.hflag = off; off += round_up((size_t)g.batch * sizeof(int32_t), 256);
    L.total = off;
    return L;
}

}  // namespace zopt

using namespace zopt;

ZOPT_EXPORT const char *zopt_status_string(zopt_status s) {
    switch (s) {
        case ZOPT_OK: return "ZOPT_OK";
        case ZOPT_ERR_NULL: return "ZOPT_ERR_NULL: a required pointer is NULL";
        case ZOPT_ERR_SIZE: return "ZOPT_ERR_SIZE: a size, count, rank or shard length is invalid";
        case ZOPT_ERR_HYPER: return "ZOPT_ERR_HYPER: a hyperparameter is out of its domain";
        case ZOPT_ERR_WORKSPACE: return "ZOPT_ERR_WORKSPACE: workspace too small or misaligned";
        case ZOPT_ERR_DEVICE: return "ZOPT_ERR_DEVICE: the HIP runtime reported a launch failure";
    }
    return "unknown zopt_status";
}

namespace {

// Checks of the AdamW arguments common to both entry points and the launch
// parameters they derive (the per-step scalars in double, rounded once).
zopt_status adamw_prepare(const float *master, const float *exp_avg, const float *exp_avg_sq,
                          const uint16_t *grad, int64_t N, int64_t bucket, int32_t world,
                          int32_t rank, int64_t shard_len, float lr, float beta1, float beta2,
                          float eps, float weight_decay, int64_t step, AdamWParams &p) {
    if (!master || !exp_avg || !exp_avg_sq || !grad) return ZOPT_ERR_NULL;
    if (N < 1 || bucket < 1 || world < 1 || rank < 0 || rank >= world) return ZOPT_ERR_SIZE;
    // sizes the index arithmetic is written for (a step is issued as
    // launches of at most 2^30 shard elements each)
    if (N > ((int64_t)1 << 40)) return ZOPT_ERR_SIZE;
    if (!finite(lr) || lr < 0.0f || !(beta1 >= 0.0f && beta1 < 1.0f) ||
        !(beta2 >= 0.0f && beta2 < 1.0f) || !finite(eps) || eps <= 0.0f ||
        !finite(weight_decay) || weight_decay < 0.0f || step < 1)
        return ZOPT_ERR_HYPER;
    p = AdamWParams{};
    const int64_t want = adamw_layout(N, bucket, world, rank, p);
    if (shard_len != want) return ZOPT_ERR_SIZE;
    p.shard_len = shard_len;

    const double t = (double)step;
    const double bc1 = 1.0 - std::pow((double)beta1, t);
    const double bc2 = 1.0 - std::pow((double)beta2, t);
    p.beta1 = beta1;
    p.beta2 = beta2;
    p.eps = eps;
    p.step_size = (float)((double)lr / bc1);
    p.bc2_sqrt = (float)std::sqrt(bc2);
    p.decay = (float)(1.0 - (double)lr * (double)weight_decay);
    p.omb1 = (float)(1.0 - (double)beta1);
    p.omb2 = (float)(1.0 - (double)beta2);
    p.grad_scale = 1.0f;
    return ZOPT_OK;
}

}  // namespace

ZOPT_EXPORT zopt_status zopt_adamw_shard_step(float *master, float *exp_avg, float *exp_avg_sq,
                                              const uint16_t *grad, uint16_t *weight, int64_t N,
                                              int64_t bucket, int32_t world, int32_t rank,
                                              int64_t shard_len, float lr, float beta1,
                                              float beta2, float eps, float weight_decay,
                                              int64_t step, float grad_scale, void *stream) {
    AdamWParams p;
    const zopt_status st = adamw_prepare(master, exp_avg, exp_avg_sq, grad, N, bucket, world,
                                         rank, shard_len, lr, beta1, beta2, eps, weight_decay,
                                         step, p);
    if (st != ZOPT_OK) return st;
    if (!finite(grad_scale)) return ZOPT_ERR_HYPER;
    p.grad_scale = grad_scale;
    hipError_t e = launch_adamw_shard(master, exp_avg, exp_avg_sq, grad, weight, p,
                                      (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_adamw_shard_step_clipped(
    float *master, float *exp_avg, float *exp_avg_sq, const uint16_t *grad, uint16_t *weight,
    int64_t N, int64_t bucket, int32_t world, int32_t rank, int64_t shard_len, float lr,
    float beta1, float beta2, float eps, float weight_decay, int64_t step,
    const float *clip_stats, int32_t skip_nonfinite, void *stream) {
    AdamWParams p;
    const zopt_status st = adamw_prepare(master, exp_avg, exp_avg_sq, grad, N, bucket, world,
                                         rank, shard_len, lr, beta1, beta2, eps, weight_decay,
                                         step, p);
    if (st != ZOPT_OK) return st;
    if (!clip_stats) return ZOPT_ERR_NULL;
    if (skip_nonfinite != 0 && skip_nonfinite != 1) return ZOPT_ERR_HYPER;
    p.stats = clip_stats;
    p.skip_nonfinite = skip_nonfinite;
    hipError_t e = launch_adamw_shard(master, exp_avg, exp_avg_sq, grad, weight, p,
                                      (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_grad_sq_norm(const uint16_t *grad, int64_t N, int64_t bucket,
                                          int32_t world, int32_t rank, int64_t shard_len,
                                          double *sq, void *workspace, size_t *workspace_bytes,
                                          void *stream) {
    if (!workspace_bytes) return ZOPT_ERR_NULL;
    if (N < 1 || bucket < 1 || world < 1 || rank < 0 || rank >= world) return ZOPT_ERR_SIZE;
    if (N > ((int64_t)1 << 40)) return ZOPT_ERR_SIZE;
    AdamWParams p{};
    if (shard_len != adamw_layout(N, bucket, world, rank, p)) return ZOPT_ERR_SIZE;
    p.shard_len = shard_len;
    const size_t need = round_up((size_t)grad_sq_norm_blocks(shard_len) * sizeof(double), 256);
    if (!workspace) {
        *workspace_bytes = need;
        return ZOPT_OK;
    }
    if (!grad || !sq) return ZOPT_ERR_NULL;
    if (*workspace_bytes < need || ((uintptr_t)workspace & 255u)) return ZOPT_ERR_WORKSPACE;
    hipError_t e = launch_grad_sq_norm(grad, p, (double *)workspace, sq, (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

// The scratch of zopt_grad_sq_norm_noalloc: the fp64 partials of the norm
// pass (at most kNormBlocksMax, 16 KiB).  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: host code uses the address
// hipGetSymbolAddress gives for the current device (scratch_address).
static __device__ __align__(256) double scratch[kNormBlocksMax];

namespace {

constexpr int kScratchDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kScratchDevices];  // per device, set at its first call

// The device address of `scratch` on the current device, looked up once per
// device with that device current.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

ZOPT_EXPORT zopt_status zopt_grad_sq_norm_noalloc(const uint16_t *grad, int64_t N,
                                                  int64_t bucket, int32_t world, int32_t rank,
                                                  int64_t shard_len, double *sq, void *stream) {
    if (!grad || !sq) return ZOPT_ERR_NULL;
    if (N < 1 || bucket < 1 || world < 1 || rank < 0 || rank >= world) return ZOPT_ERR_SIZE;
    if (N > ((int64_t)1 << 40)) return ZOPT_ERR_SIZE;
    AdamWParams p{};
    if (shard_len != adamw_layout(N, bucket, world, rank, p)) return ZOPT_ERR_SIZE;
    p.shard_len = shard_len;
    const size_t need = (size_t)grad_sq_norm_blocks(shard_len) * sizeof(double);
    if (need > sizeof(scratch)) return ZOPT_ERR_WORKSPACE;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return ZOPT_ERR_DEVICE;
    hipError_t e = launch_grad_sq_norm(grad, p, (double *)ws, sq, (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_grad_clip_stats(const double *sq, int32_t count, float max_norm,
                                             float inv_scale, float *stats, void *stream) {
    if (!sq || !stats) return ZOPT_ERR_NULL;
    if (count < 1 || count > 65536) return ZOPT_ERR_SIZE;
    if (!(max_norm > 0.0f) || !finite(inv_scale) || !(inv_scale > 0.0f)) return ZOPT_ERR_HYPER;
    hipError_t e = launch_clip_stats(sq, count, max_norm, inv_scale, stats, (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT int64_t zopt_shard_len(int64_t N, int64_t bucket, int32_t world) {
    if (N < 1 || bucket < 1 || world < 1) return -1;
    AdamWParams p{};
    return adamw_layout(N, bucket, world, 0, p);
}

ZOPT_EXPORT zopt_status zopt_round_bf16(const float *src, uint16_t *dst, int64_t n,
                                        void *stream) {
    if (n < 0 || n > ((int64_t)1 << 40)) return ZOPT_ERR_SIZE;
    if (n == 0) return ZOPT_OK;
    if (!src || !dst) return ZOPT_ERR_NULL;
    hipError_t e = launch_round_bf16(src, dst, n, (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_set_ns_workgroup_limit(int32_t n) {
    if (n < 0) return ZOPT_ERR_SIZE;
    ns_set_workgroup_limit(n);
    return ZOPT_OK;
}

ZOPT_EXPORT zopt_status zopt_set_ns_form(int32_t form) {
    if (form < 0 || form > 2) return ZOPT_ERR_HYPER;
    g_ns_form.store(form, std::memory_order_relaxed);
    return ZOPT_OK;
}

namespace {

// The Newton-Schulz kernels address a panel of up to 256 rows of the padded
// m x np matrix, and a 32-row stage of its columns, with 32-bit byte offsets
// (256 * np * 2 < 2^31 needs np < 2^22); the longer side is held to 2^21,
// which leaves every such offset below 2^30, and the element count to
// below 2^31 (the streaming passes index a matrix in 32 bits).
constexpr int64_t kMuonMaxSide = (int64_t)1 << 21;

zopt_status muon_check_shape(int32_t batch, int64_t rows, int64_t cols) {
    if (batch < 1 || batch > kMaxBatch || rows < 1 || cols < 1) return ZOPT_ERR_SIZE;
    if (rows > kMuonMaxSide || cols > kMuonMaxSide) return ZOPT_ERR_SIZE;
    if (rows * cols >= ((int64_t)1 << 31)) return ZOPT_ERR_SIZE;
    return ZOPT_OK;
}

// Where the Newton-Schulz result of a call lies, in the stored orientation:
// X alternates between the x and xt0 regions (x after an even number of
// segments), and matrices stored transposed (rows > cols) find X^T in xt1,
// which the last segment (or, with no iterations, the pre-step) writes.
void muon_output(const MuonGeom &g, const MuonWorkspace &L, int32_t ns_steps, size_t &base,
                 int64_t &ld) {
    if (!g.transposed) {
        base = (ns_segments(g, ns_steps) % 2) ? L.xt0 : L.x;
        ld = g.np;
    } else {
        base = L.xt1;
        ld = g.mp;
    }
}

// The groups of a call, each with its own workspace carve-up, laid out one
// after the other in the caller's workspace.
struct GroupPlan {
    MuonGeom g;
    MuonWorkspace L;
    size_t base;
};

zopt_status plan_groups(int32_t ngroups, const int32_t *batch, const int64_t *rows,
                        const int64_t *cols, GroupPlan *plans, size_t &total, int &nmat) {
    if (!batch || !rows || !cols) return ZOPT_ERR_NULL;
    if (ngroups < 1 || ngroups > kMaxCallGroups) return ZOPT_ERR_SIZE;
    total = 0;
    nmat = 0;
    for (int i = 0; i < ngroups; ++i) {
        const zopt_status st = muon_check_shape(batch[i], rows[i], cols[i]);
        if (st != ZOPT_OK) return st;
        plans[i].g = muon_geometry(batch[i], rows[i], cols[i]);
        plans[i].L = muon_workspace_layout(plans[i].g);
        plans[i].base = total;
        total += plans[i].L.total;
        nmat += batch[i];
    }
    return ZOPT_OK;
}

// Everything a Muon call enqueues from: the groups' geometry and workspace
// carve-up, their pointer tables, where each group's matrices start in the
// call, and the launch bins.
struct MuonCallPlan {
    GroupPlan plans[kMaxCallGroups];
    MuonPtrs ptrs[kMaxCallGroups];
    NsGroupRef refs[kMaxCallGroups];
    int firsts[kMaxCallGroups];
    int bins[kMaxCallGroups + 1][kMaxCallGroups];
    int bin_size[kMaxCallGroups + 1];
    int ngroups, nmat, nbins;
    size_t total;
};

// The pointer checks of a Muon call (the shapes are checked by plan_groups).
zopt_status muon_check_ptrs(int nmat, float *const *master, float *const *momentum,
                            const uint16_t *const *grad, uint16_t *const *weight) {
    if (!master || !momentum || !grad) return ZOPT_ERR_NULL;
    for (int b = 0; b < nmat; ++b) {
        if (!master[b] || !momentum[b] || !grad[b]) return ZOPT_ERR_NULL;
        if (weight && !weight[b]) return ZOPT_ERR_NULL;
    }
    return ZOPT_OK;
}

// The hyperparameters of a Muon call that never live in device memory.
bool muon_fixed_hypers_ok(int32_t nesterov, int32_t ns_steps, float ns_a, float ns_b,
                          float ns_c, float ns_eps, int32_t adjust_lr) {
    return (nesterov == 0 || nesterov == 1) && ns_steps >= 0 && ns_steps <= 100 &&
           finite(ns_a) && finite(ns_b) && finite(ns_c) && finite(ns_eps) && ns_eps >= 0.0f &&
           (adjust_lr == 0 || adjust_lr == 1);
}

// Pointer tables and launch bins of a planned call whose workspace starts at
// ws.  All groups share one bin, so that their tiles fill each other's
// partial rounds.  A group whose symmetric products were given 128 x 128
// tiles for having too few 256 x 256 upper-triangle tiles to fill the GPU on
// its own goes back to 256 x 256 tiles when the bin holds groups on those:
// its short tiles then run in the partial last rounds of their launches
// instead of in launches of their own (the results are the same bit for bit:
// every element is accumulated over K in the same order on either tile).
// Measured on the 8B rank-0 share (8 x [1024, 4096] beside 4096-row groups):
// 52.95 ms per call against 53.40 ms with that group in a bin of its own on
// 128-tiles.
void muon_bin_call(MuonCallPlan &c, char *ws, float *const *master, float *const *momentum,
                   const uint16_t *const *grad, uint16_t *const *weight, const int32_t *batch) {
    for (int i = 0, first = 0; i < c.ngroups; first += batch[i], ++i) {
        c.firsts[i] = first;
        MuonPtrs &p = c.ptrs[i];
        for (int b = 0; b < batch[i]; ++b) {
            p.master[b] = master[first + b];
            p.momentum[b] = momentum[first + b];
            p.grad[b] = grad[first + b];
            p.weight[b] = weight ? weight[first + b] : nullptr;
        }
        c.refs[i] = NsGroupRef{&c.plans[i].g, &c.plans[i].L, ws + c.plans[i].base};
    }
    c.nbins = 1;
    c.bin_size[0] = c.ngroups;
    bool any256 = false;
    for (int i = 0; i < c.ngroups; ++i) {
        c.bins[0][i] = i;
        any256 = any256 || c.plans[i].g.tile == 256;
    }
    for (int i = 0; any256 && i < c.ngroups; ++i) {
        MuonGeom &g = c.plans[i].g;
        if (g.tile == 128 && g.m >= 768 && g.mp % 256 == 0) g.tile = 256;
    }
}

}  // namespace

bool zopt::ns_split_streams(const NsGroupRef *refs, int nrefs) {
    if (nrefs < 2) return false;
    int64_t wg = 0;
    for (int i = 0; i < nrefs; ++i) {
        const MuonGeom &g = *refs[i].geom;
        if (g.tile != 256) continue;
        const int64_t tm = g.mp / 256;
        wg += (int64_t)g.batch * (tm * (tm + 1) / 2) * g.ksplit;
    }
    return wg > 0 && wg < 2 * (int64_t)ns_round_tiles(256);
}

namespace {

// The second stream of Muon calls whose Newton-Schulz iterations are split
// over two streams (ns_split_streams): one per device, default priority,
// created at the first such call on that device that is not being captured
// (creating a stream inside a capture is not done), with the two events that
// fork it from the caller's stream and join it back.  g_aux_mutex is held
// while a call enqueues its fork ... join, so that calls from several host
// threads take the events one at a time; the work of those calls on the
// second stream is then ordered as their enqueues were.
struct AuxStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool failed = false;  // creation failed once: calls run on one stream
};
std::mutex g_aux_mutex;
AuxStream g_aux[kScratchDevices];

// The current device's second stream (g_aux_mutex held), or nullptr: not
// created yet and `caller` is capturing, or creation failed.
AuxStream *aux_stream(hipStream_t caller) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    AuxStream &a = g_aux[dev];
    if (a.s != nullptr) return &a;
    if (a.failed) return nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return nullptr;
    if (hipStreamCreateWithFlags(&a.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&a.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&a.join, hipEventDisableTiming) != hipSuccess) {
        if (a.s) (void)hipStreamDestroy(a.s);
        if (a.fork) (void)hipEventDestroy(a.fork);
        a = AuxStream{};
        a.failed = true;
        return nullptr;
    }
    return &a;
}

// The sides of a bin whose Newton-Schulz launches run on two streams: side[k]
// is 0 (the caller's stream) or 1 (the second).  Groups that run the same
// program (plain iterations or Gram segments, on the same tile) share its
// launches when they are on one side, while a plain and a Gram group on one
// side make a merged program longer than either (15 and 17 launches for five
// steps merge into 23).  So in a call that mixes the two forms, whole classes
// of such groups are placed, in order of Newton-Schulz work, each on the side
// with less work so far; in a call of one form the groups are placed so one
// by one.  Measured on the 1B rank-0 share (two 2048-row Gram groups, the
// square plain group, the 512-row Gram group on 128 tiles): 2.58 ms per call
// against 2.81 ms with the groups placed one by one; all four in plain
// iterations, one by one, Newton-Schulz 3.01 ms per call against 3.22 ms by
// class (the three 2048-row groups on one stream).
// Newton-Schulz multiply-adds of a group: 3 m^2 n + (4 L - 3) m^3 per matrix
// and segment of L steps (a plain step is a segment of one)
double ns_work(const MuonGeom &g, int ns_steps) {
    const double m = g.m, n = g.n;
    const int nseg = ns_segments(g, ns_steps);
    return g.batch * (nseg * 3.0 * m * m * n + (4.0 * ns_steps - 3.0 * nseg) * m * m * m);
}

void split_sides(const NsGroupRef *refs, int nb, int ns_steps, int *side) {
    bool mixed = false;
    for (int k = 1; k < nb; ++k) mixed = mixed || refs[k].geom->gram != refs[0].geom->gram;
    // the items placed: classes (form and tile) in a mixed call, else groups
    int item[kMaxCallGroups], key[kMaxCallGroups], nitems = 0;
    double work[kMaxCallGroups];
    for (int k = 0; k < nb; ++k) {
        const MuonGeom &g = *refs[k].geom;
        const int kk = mixed ? g.gram * 1024 + g.tile : k;
        int c = 0;
        while (c < nitems && key[c] != kk) ++c;
        if (c == nitems) {
            key[nitems] = kk;
            work[nitems++] = 0.0;
        }
        item[k] = c;
        work[c] += ns_work(g, ns_steps);
    }
    // largest first, each to the side with less work so far
    int order[kMaxCallGroups], iside[kMaxCallGroups];
    for (int c = 0; c < nitems; ++c) order[c] = c;
    std::stable_sort(order, order + nitems, [&](int x, int y) { return work[x] > work[y]; });
    double w[2] = {0.0, 0.0};
    for (int t = 0; t < nitems; ++t) {
        const int c = order[t], d = w[0] <= w[1] ? 0 : 1;
        iside[c] = d;
        w[d] += work[c];
    }
    for (int k = 0; k < nb; ++k) side[k] = iside[item[k]];
}

// Enqueues a planned call on stream s.  With dev (device scalars [lr,
// momentum_beta, weight_decay]) the kernels read those when they run and
// lr / mu / wd here are unused; with health the Newton-Schulz health pass
// runs and rejected matrices are not updated.
hipError_t muon_enqueue(const MuonCallPlan &c, char *ws, float lr, float mu, int32_t nesterov,
                        float wd, int32_t ns_steps, float ns_a, float ns_b, float ns_c,
                        float ns_eps, int32_t adjust_lr, float guard, float *health,
                        const float *dev, hipStream_t s) {
    const double lr_d = (double)lr, wd_d = (double)wd;
    hipError_t e = hipSuccess;
    for (int bi = 0; bi < c.nbins && e == hipSuccess; ++bi) {
        const int nb = c.bin_size[bi];
        NsGroupRef brefs[kMaxCallGroups];
        for (int k = 0; k < nb; ++k) brefs[k] = c.refs[c.bins[bi][k]];
        // A bin whose Newton-Schulz launches are short runs on two streams:
        // each group's pre-pass, iterations and (with no health pass) post-step
        // on its side's stream; the second stream forks from the caller's
        // after the caller's side's pre-passes and joins it before the health
        // pass, or at the end.  The lock makes the fork ... join enqueue of one
        // call atomic.
        std::unique_lock<std::mutex> lock(g_aux_mutex, std::defer_lock);
        AuxStream *aux = nullptr;
        int side[kMaxCallGroups] = {};
        if (ns_steps > 0 && ns_split_streams(brefs, nb)) {
            lock.lock();
            aux = aux_stream(s);
            if (aux != nullptr)
                split_sides(brefs, nb, ns_steps, side);
            else
                lock.unlock();
        }
        // each side's groups in one merged sequence of launches.  The side
        // estimated to take longer runs on the caller's stream, whose work
        // starts first, and its pre-passes run before the second stream
        // forks, so that they have the memory to themselves and its
        // iterations start as early as they can; the other side's pre-passes
        // then run beside those iterations.  The estimate: 24 bytes per
        // element of pre-pass and post-step at 6 TB/s, the multiply-adds at
        // 0.6 T/s (1.2 PFLOP/s) and 40 us per launch.  It puts GPT-2-small's
        // Gram groups (17 launches) before its plain group (15), and the 1B
        // share's 2048-row Gram groups (69 M elements) before its square and
        // 512-row groups (21 M elements in 30 launches): 1.741 -> 1.721 and
        // 2.588 -> 2.581 ms per call against the longer merged program first
        // and the fork before every pre-pass.
        NsGroupRef r[2][kMaxCallGroups];
        int n[2] = {0, 0};
        std::vector<NsSchedule> sch(2);
        if (ns_steps > 0) {
            const bool f16 = g_ns_form.load(std::memory_order_relaxed) == 0 &&
                             ns_gram_f16_safe(ns_steps, ns_a, ns_b, ns_c);
            auto plan_sides = [&]() {
                n[0] = n[1] = 0;
                for (int k = 0; k < nb; ++k) {
                    const int d = aux != nullptr ? side[k] : 0;
                    r[d][n[d]++] = brefs[k];
                }
                for (int d = 0; d < 2; ++d)
                    if (n[d] > 0) ns_schedule(r[d], n[d], ns_steps, f16, sch[d]);
            };
            plan_sides();
            auto cost = [&](int d) {
                double elems = 0.0, work = 0.0;
                for (int k = 0; k < n[d]; ++k) {
                    const MuonGeom &g = *r[d][k].geom;
                    elems += (double)g.batch * g.rows * g.cols;
                    work += ns_work(g, ns_steps);
                }
                int launches = 0;
                for (int t = 0; t < sch[d].nsteps; ++t) {
                    int tiles = 0;  // bit set of the step's tile sizes
                    bool split = false;
                    for (int k = 0; k < n[d]; ++k) {
                        const MuonGeom &g = *r[d][k].geom;
                        if (sch[d].idx[g.gram ? 1 : 0][t] < 0) continue;
                        tiles |= sch[d].kind[t] == kNsKindBX ? g.tile_bx : g.tile;
                        split = split || (sch[d].kind[t] == kNsKindXXT && g.ksplit > 1);
                    }
                    launches += __builtin_popcount(tiles) + (split ? 1 : 0);
                }
                return elems * 24.0 / 6e12 + work / 0.6e15 + launches * 40e-6;
            };
            if (aux != nullptr && n[0] > 0 && n[1] > 0 && cost(1) > cost(0)) {
                for (int k = 0; k < nb; ++k) side[k] ^= 1;
                plan_sides();
            }
        }
        auto on = [&](int k) { return aux != nullptr && side[k] ? aux->s : s; };
        bool joined = aux == nullptr;
        auto join = [&]() {
            // (enqueued whatever happened before, so that s never runs ahead
            // of work already on the second stream)
            if (joined) return;
            joined = true;
            const hipError_t ej = hipEventRecord(aux->join, aux->s);
            const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(s, aux->join, 0) : ej;
            if (e == hipSuccess) e = ew;
        };
        // the pre-passes of side d (all groups with one stream)
        auto pre = [&](int d) {
            for (int k = 0; k < nb && e == hipSuccess; ++k) {
                if ((aux != nullptr ? side[k] : 0) != d) continue;
                const int i = c.bins[bi][k];
                e = launch_muon_pre(c.plans[i].g, c.ptrs[i], mu, nesterov, ns_eps,
                                    ws + c.plans[i].base, c.plans[i].L, ns_steps == 0, dev, on(k));
            }
        };
        pre(0);
        if (aux != nullptr && e == hipSuccess) {
            e = hipEventRecord(aux->fork, s);
            if (e == hipSuccess) e = hipStreamWaitEvent(aux->s, aux->fork, 0);
        }
        pre(1);
        if (ns_steps > 0 && e == hipSuccess) {
            // the two sides' launches enqueued in turn
            const int steps = std::max(n[0] > 0 ? sch[0].nsteps : 0, n[1] > 0 ? sch[1].nsteps : 0);
            for (int t = 0; t < steps && e == hipSuccess; ++t)
                for (int d = 0; d < 2 && e == hipSuccess; ++d)
                    if (n[d] > 0 && t < sch[d].nsteps)
                        e = launch_ns_step(r[d], n[d], sch[d], t, ns_a, ns_b, ns_c, d ? aux->s : s);
        }
        if (health) {
            join();
            if (e == hipSuccess) {
                int bfirst[kMaxCallGroups];
                for (int k = 0; k < nb; ++k) bfirst[k] = c.firsts[c.bins[bi][k]];
                e = launch_ns_health(brefs, bfirst, nb, ns_steps, guard, health, s);
            }
        }
        for (int k = 0; k < nb && e == hipSuccess; ++k) {
            const int i = c.bins[bi][k];
            const MuonGeom &g = c.plans[i].g;
            const double big = (double)(g.rows > g.cols ? g.rows : g.cols);
            const double scale = adjust_lr
                                     ? 0.2 * std::sqrt(big)
                                     : std::sqrt(std::fmax(1.0, (double)g.rows / (double)g.cols));
            const float decay = (float)(1.0 - lr_d * wd_d);
            const float step_lr = (float)(lr_d * scale);
            size_t obase;
            int64_t old;
            muon_output(g, c.plans[i].L, ns_steps, obase, old);
            const int32_t *reject =
                health ? reinterpret_cast<const int32_t *>(ws + c.plans[i].base + c.plans[i].L.hflag)
                       : nullptr;
            e = launch_muon_post(g, c.ptrs[i],
                                 reinterpret_cast<const uint16_t *>(ws + c.plans[i].base + obase),
                                 old, c.plans[i].L.x_stride, decay, step_lr, reject, dev, scale,
                                 health ? s : on(k));
        }
        join();
    }
    if (health && e == hipSuccess) e = launch_ns_health_total(health, c.nmat, s);
    return e;
}

zopt_status muon_step_groups(int32_t ngroups, const int32_t *batch, const int64_t *rows,
                             const int64_t *cols, float *const *master, float *const *momentum,
                             const uint16_t *const *grad, uint16_t *const *weight, float lr,
                             float momentum_beta, int32_t nesterov, float weight_decay,
                             int32_t ns_steps, float ns_a, float ns_b, float ns_c, float ns_eps,
                             int32_t adjust_lr, float guard, float *health, void *workspace,
                             size_t *workspace_bytes, void *stream) {
    if (!workspace_bytes) return ZOPT_ERR_NULL;
    MuonCallPlan c;
    c.ngroups = ngroups;
    zopt_status st = plan_groups(ngroups, batch, rows, cols, c.plans, c.total, c.nmat);
    if (st != ZOPT_OK) return st;
    if (!workspace) {
        *workspace_bytes = c.total;
        return ZOPT_OK;
    }
    st = muon_check_ptrs(c.nmat, master, momentum, grad, weight);
    if (st != ZOPT_OK) return st;
    if (!finite(lr) || lr < 0.0f || !(momentum_beta >= 0.0f && momentum_beta < 1.0f) ||
        !finite(weight_decay) || weight_decay < 0.0f ||
        !muon_fixed_hypers_ok(nesterov, ns_steps, ns_a, ns_b, ns_c, ns_eps, adjust_lr))
        return ZOPT_ERR_HYPER;
    if (*workspace_bytes < c.total || ((uintptr_t)workspace & 255u) != 0)
        return ZOPT_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    muon_bin_call(c, ws, master, momentum, grad, weight, batch);
    const hipError_t e = muon_enqueue(c, ws, lr, momentum_beta, nesterov, weight_decay, ns_steps,
                                      ns_a, ns_b, ns_c, ns_eps, adjust_lr, guard, health, nullptr,
                                      (hipStream_t)stream);
    return e == hipSuccess ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

zopt_status muon_output_view(int32_t ngroups, const int32_t *batch, const int64_t *rows,
                             const int64_t *cols, int32_t ns_steps, const void *workspace,
                             int32_t group, int32_t index, const uint16_t **out,
                             int64_t *row_stride) {
    if (!workspace || !out || !row_stride) return ZOPT_ERR_NULL;
    GroupPlan plans[kMaxCallGroups];
    size_t total = 0;
    int nmat = 0;
    const zopt_status st = plan_groups(ngroups, batch, rows, cols, plans, total, nmat);
    if (st != ZOPT_OK) return st;
    if (group < 0 || group >= ngroups || index < 0 || index >= batch[group]) return ZOPT_ERR_SIZE;
    if (ns_steps < 0 || ns_steps > 100) return ZOPT_ERR_HYPER;
    const GroupPlan &p = plans[group];
    size_t base;
    int64_t ld;
    muon_output(p.g, p.L, ns_steps, base, ld);
    *out = reinterpret_cast<const uint16_t *>(static_cast<const char *>(workspace) + p.base + base +
                                              (size_t)index * p.L.x_stride);
    *row_stride = ld;
    return ZOPT_OK;
}

}  // namespace

ZOPT_EXPORT zopt_status zopt_muon_step(int32_t batch, int64_t rows, int64_t cols,
                                       float *const *master, float *const *momentum,
                                       const uint16_t *const *grad, uint16_t *const *weight,
                                       float lr, float momentum_beta, int32_t nesterov,
                                       float weight_decay, int32_t ns_steps, float ns_a,
                                       float ns_b, float ns_c, float ns_eps, int32_t adjust_lr,
                                       void *workspace, size_t *workspace_bytes, void *stream) {
    return muon_step_groups(1, &batch, &rows, &cols, master, momentum, grad, weight, lr,
                            momentum_beta, nesterov, weight_decay, ns_steps, ns_a, ns_b, ns_c,
                            ns_eps, adjust_lr, 0.0f, nullptr, workspace, workspace_bytes,
                            stream);
}

ZOPT_EXPORT zopt_status zopt_muon_step_groups(
    int32_t ngroups, const int32_t *batch, const int64_t *rows, const int64_t *cols,
    float *const *master, float *const *momentum, const uint16_t *const *grad,
    uint16_t *const *weight, float lr, float momentum_beta, int32_t nesterov, float weight_decay,
    int32_t ns_steps, float ns_a, float ns_b, float ns_c, float ns_eps, int32_t adjust_lr,
    void *workspace, size_t *workspace_bytes, void *stream) {
    return muon_step_groups(ngroups, batch, rows, cols, master, momentum, grad, weight, lr,
                            momentum_beta, nesterov, weight_decay, ns_steps, ns_a, ns_b, ns_c,
                            ns_eps, adjust_lr, 0.0f, nullptr, workspace, workspace_bytes,
                            stream);
}

ZOPT_EXPORT zopt_status zopt_muon_step_groups_guarded(
    int32_t ngroups, const int32_t *batch, const int64_t *rows, const int64_t *cols,
    float *const *master, float *const *momentum, const uint16_t *const *grad,
    uint16_t *const *weight, float lr, float momentum_beta, int32_t nesterov, float weight_decay,
    int32_t ns_steps, float ns_a, float ns_b, float ns_c, float ns_eps, int32_t adjust_lr,
    float ns_guard, float *ns_health, void *workspace, size_t *workspace_bytes, void *stream) {
    if (workspace) {
        if (!ns_health) return ZOPT_ERR_NULL;
        if (!(ns_guard > 0.0f)) return ZOPT_ERR_HYPER;  // +inf: report only, NaN rejected
    }
    return muon_step_groups(ngroups, batch, rows, cols, master, momentum, grad, weight, lr,
                            momentum_beta, nesterov, weight_decay, ns_steps, ns_a, ns_b, ns_c,
                            ns_eps, adjust_lr, ns_guard, ns_health, workspace, workspace_bytes,
                            stream);
}

// A captured Muon call: the graph and its executable instance.
struct zopt_muon_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

ZOPT_EXPORT zopt_status zopt_muon_graph_create(
    int32_t ngroups, const int32_t *batch, const int64_t *rows, const int64_t *cols,
    float *const *master, float *const *momentum, const uint16_t *const *grad,
    uint16_t *const *weight, const float *scalars, int32_t nesterov, int32_t ns_steps, float ns_a,
    float ns_b, float ns_c, float ns_eps, int32_t adjust_lr, float ns_guard, float *ns_health,
    void *workspace, size_t workspace_bytes, zopt_muon_graph **graph) {
    if (!graph) return ZOPT_ERR_NULL;
    *graph = nullptr;
    MuonCallPlan c;
    c.ngroups = ngroups;
    zopt_status st = plan_groups(ngroups, batch, rows, cols, c.plans, c.total, c.nmat);
    if (st != ZOPT_OK) return st;
    if (!workspace || !scalars) return ZOPT_ERR_NULL;
    st = muon_check_ptrs(c.nmat, master, momentum, grad, weight);
    if (st != ZOPT_OK) return st;
    if (!muon_fixed_hypers_ok(nesterov, ns_steps, ns_a, ns_b, ns_c, ns_eps, adjust_lr) ||
        (ns_health && !(ns_guard > 0.0f)))
        return ZOPT_ERR_HYPER;
    if (workspace_bytes < c.total || ((uintptr_t)workspace & 255u) != 0)
        return ZOPT_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    muon_bin_call(c, ws, master, momentum, grad, weight, batch);

    // capture on a private stream (the caller's may be the null stream, which
    // cannot be captured); the kernels read lr / momentum / weight decay from
    // `scalars` when they run, so one capture serves every step
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return ZOPT_ERR_DEVICE;
    if (ns_steps > 0) {
        // a call split over two streams: the second stream exists before the
        // capture begins (none is created inside it)
        for (int bi = 0; bi < c.nbins; ++bi) {
            NsGroupRef brefs[kMaxCallGroups];
            for (int k = 0; k < c.bin_size[bi]; ++k) brefs[k] = c.refs[c.bins[bi][k]];
            if (ns_split_streams(brefs, c.bin_size[bi])) {
                std::lock_guard<std::mutex> lock(g_aux_mutex);
                (void)aux_stream(cs);
            }
        }
    }
    hipGraph_t g = nullptr;
    hipGraphExec_t ex = nullptr;
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        const hipError_t e1 = muon_enqueue(c, ws, 0.0f, 0.0f, nesterov, 0.0f, ns_steps, ns_a, ns_b,
                                           ns_c, ns_eps, adjust_lr, ns_guard, ns_health, scalars,
                                           cs);
        const hipError_t e2 = hipStreamEndCapture(cs, &g);
        e = e1 != hipSuccess ? e1 : e2;
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    if (hipStreamDestroy(cs) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
    if (e != hipSuccess) {
        if (ex) (void)hipGraphExecDestroy(ex);
        if (g) (void)hipGraphDestroy(g);
        return ZOPT_ERR_DEVICE;
    }
    *graph = new zopt_muon_graph{g, ex};
    return ZOPT_OK;
}

ZOPT_EXPORT zopt_status zopt_muon_graph_launch(const zopt_muon_graph *graph, void *stream) {
    if (!graph) return ZOPT_ERR_NULL;
    return hipGraphLaunch(graph->exec, (hipStream_t)stream) == hipSuccess ? ZOPT_OK
                                                                         : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_muon_graph_destroy(zopt_muon_graph *graph) {
    if (!graph) return ZOPT_OK;
    const hipError_t e1 = hipGraphExecDestroy(graph->exec);
    const hipError_t e2 = hipGraphDestroy(graph->graph);
    delete graph;
    return (e1 == hipSuccess && e2 == hipSuccess) ? ZOPT_OK : ZOPT_ERR_DEVICE;
}

ZOPT_EXPORT zopt_status zopt_muon_output_view(int32_t batch, int64_t rows, int64_t cols,
                                              int32_t ns_steps, const void *workspace,
                                              int32_t index, const uint16_t **out,
                                              int64_t *row_stride) {
    return muon_output_view(1, &batch, &rows, &cols, ns_steps, workspace, 0, index, out,
                            row_stride);
}

ZOPT_EXPORT zopt_status zopt_muon_groups_output_view(int32_t ngroups, const int32_t *batch,
                                                     const int64_t *rows, const int64_t *cols,
                                                     int32_t ns_steps, const void *workspace,
                                                     int32_t group, int32_t index,
                                                     const uint16_t **out, int64_t *row_stride) {
    return muon_output_view(ngroups, batch, rows, cols, ns_steps, workspace, group, index, out,
                            row_stride);
}
