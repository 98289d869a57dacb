// zopt_internal.h -- shared declarations inside libzopt (not installed).
//
// Device helpers used by more than one kernel file, the launch-parameter
// structs the host entry points fill, and the launchers each kernel file
// exports to the entry points in zopt_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace zopt {

// ------------------------------------------------------------------ bf16

// fp32 -> bf16, round to nearest with ties to even, by integer arithmetic on
// the bit pattern: adding 0x7FFF plus the lowest kept bit and truncating
// rounds to nearest-even, carries overflow into infinity, and keeps
// subnormals.  A NaN (exponent all ones, mantissa non-zero) becomes the
// positive quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t rne_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? 0x7FC0u : r;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
    return __uint_as_float(h << 16);
}

// Two fp32 -> two bf16 packed low-first into one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return rne_bf16_bits(lo) | (rne_bf16_bits(hi) << 16);
}

// ------------------------------------------------------------------ AdamW

// Everything one AdamW launch needs; filled by zopt_adamw_shard_step.
// The shard is read as two regions: shard elements [0, full_len) lie in
// buckets of the full adjusted length B (piece = B / world each, never any
// padding); [full_len, shard_len) is the last, shorter bucket, whose piece
// starts at flat index last_flat0 and whose positions at or past n are
// padding.
struct AdamWParams {
    int64_t shard_len;
    int64_t full_len;
    int64_t piece;       // piece of a full bucket
    int64_t gap;         // B - piece: flat advance per full bucket past its piece
    int64_t rank_off;    // rank * piece
    int64_t last_flat0;  // flat index of shard element full_len
    int64_t n;           // flat length N
    float beta1, beta2, eps;
    float step_size, bc2_sqrt, decay, omb1, omb2;
    float grad_scale;
    int32_t vec;         // gradient base 16-byte aligned (the norm pass's vector loads)
    double inv_piece;    // 1 / piece, for the bucket index
    // When a piece holds a whole number of AdamW tiles (tpp tiles, tpp > 0),
    // no tile of [0, full_len) straddles a bucket edge and the bucket of such
    // a tile is tile / tpp (tiles [0, full_tiles)); tpp = 0 otherwise.
    uint32_t tpp;
    uint32_t full_tiles;
    double inv_tpp;      // 1 / tpp
    const float *stats;  // clip statistics in device memory: grad_scale read there (or NULL)
    int32_t skip_nonfinite;  // with stats: a found_inf there skips the step
};

// Indices of the clip statistics (binary32 each; flags 0 / 1).
enum : int { kClipTotalNorm = 0, kClipCoef = 1, kClipClipped = 2, kClipFoundInf = 3,
             kClipGradScale = 4, kClipStats = 5 };

// Workgroups (and fp64 partials) of the gradient-norm pass: fixed by the
// shard length, at most kNormBlocksMax.
constexpr int kNormBlocksMax = 2048;
int32_t grad_sq_norm_blocks(int64_t shard_len);

// sq[0] = sum of squares of the shard's real gradient elements; partials
// holds grad_sq_norm_blocks(shard_len) doubles of scratch.
hipError_t launch_grad_sq_norm(const uint16_t *grad, const AdamWParams &p, double *partials,
                               double *sq, hipStream_t stream);

hipError_t launch_clip_stats(const double *sq, int32_t count, float max_norm, float inv_scale,
                             float *stats, hipStream_t stream);

hipError_t launch_adamw_shard(float *master, float *exp_avg, float *exp_avg_sq,
                              const uint16_t *grad, uint16_t *weight,
                              const AdamWParams &p, hipStream_t stream);

hipError_t launch_round_bf16(const float *src, uint16_t *dst, int64_t n,
                             hipStream_t stream);

// ------------------------------------------------------------------ Muon

constexpr int kMaxBatch = 64;       // matrices per same-shape group
constexpr int kMaxCallGroups = 16;  // groups per Muon call
constexpr int kMaxGroups = 8;       // groups per Newton-Schulz launch (kernel argument space)

// Per-call Muon geometry.  m x n is the Newton-Schulz orientation
// (m = min(rows, cols)); mp x np are m and n padded up to the tile size.
struct MuonGeom {
    int32_t batch;
    int32_t rows, cols;
    int32_t transposed;  // rows > cols: X = U^T
    int32_t m, n;
    int32_t mp, np;
    int32_t tile;        // square output tile of the Newton-Schulz products X X^T and A A
    int32_t tile_bx;     // and of B X
    int32_t norm_blocks; // norm partials per matrix (room for either form of pass 1)
    int32_t ksplit;      // X X^T reduction split in this many parts (1: none)
    int32_t health_blocks;  // workgroups (and partials) per matrix of the health pass
    int32_t gram;        // 1: Newton-Schulz in segments of up to kNsMaxSegment steps on the
                         // Gram matrix (n >= 2 m); 0: plain iterations
};

struct MuonPtrs {
    float *master[kMaxBatch];
    float *momentum[kMaxBatch];
    const uint16_t *grad[kMaxBatch];
    uint16_t *weight[kMaxBatch];
};

// Symmetric mp x mp matrices a group's Newton-Schulz keeps at once: A = X X^T
// and P = a I + b A + c A A for plain iterations; up to five for a segment on
// the Gram matrix (A, P, Q and the products on the way to the next A).
constexpr int kNsSlots = 5;
constexpr int kNsMaxSegment = 3;
// The largest short side m for which the symmetric m x m matrices may be held
// in fp16 (the Gram form's chain, plain iterations' A): fp16 keeps 11 bits
// only down to 2^-14, and the off-diagonal entries of A = X X^T of a
// normalised m x n X are ~1 / (m sqrt(n)), subnormal in fp16 at m = 4096
// (~2e-6 for n = 14336) and smaller beyond.  Measured at full size, the Gram
// form with segments of 3 and 2 holds its error at 3.1e-3 up to m = 4096
// (the plain bf16 iteration: 5e-3), while a first segment of four steps
// degrades with m (3.2e-3 at m = 256, 4.9e-3 at 2048, 9.0e-3 at 4096).  Larger
// matrices run plain iterations with every matrix in bf16.
constexpr int kNsF16MaxM = 4096;

// Workspace carve-up (byte offsets; every region 256-byte aligned).  x and
// xt0 hold X (mp x np) in turn, one per Newton-Schulz segment; xt1 holds the
// result transposed (np x mp) for matrices stored transposed.  Slot k of the
// symmetric pool is sm[k] (bf16 off-diagonal part, diagonal 0) with its fp32
// diagonal at sd[k]; a group has nslots of them.
struct MuonWorkspace {
    size_t x, xt0, xt1, partials;
    size_t sm[kNsSlots], sd[kNsSlots];
    int32_t nslots;
    size_t part;       // X X^T split: ksplit fp32 mp x mp partial products per matrix
    size_t hsum, hmax, hflag;  // health pass: fp64 / fp32 partials, per-matrix reject flags
    size_t total;
    size_t x_stride, a_stride, d_stride;  // bytes per matrix of each region kind
};

MuonGeom muon_geometry(int32_t batch, int64_t rows, int64_t cols);
MuonWorkspace muon_workspace_layout(const MuonGeom &g);

// Device scalars of a Muon launch whose lr / momentum / weight decay live in
// device memory (read when the kernels run): float[3] at these indices.
enum : int { kDevLr = 0, kDevMomentum = 1, kDevWeightDecay = 2, kDevScalars = 3 };

// dev: device scalars (mu is read there and omm formed from it) or NULL (mu
// as given).
// Steps the momentum and forms s = 1 / (||U||_F + eps) per matrix (at
// muon_sd_ptr).  With iterations to follow, the x region receives bf16(U) in
// the Newton-Schulz orientation and the first iteration applies s (the factor
// at muon_scale_ptr), or, for a matrix whose ||U||_F^2 is too large or too
// small for that, X0 = bf16(U s) and the factor is 1; with no_iterations,
// X0 = bf16(U s) itself (the call's result), and X0^T in xt1 as well for
// matrices stored transposed.
hipError_t launch_muon_pre(const MuonGeom &g, const MuonPtrs &ptrs, float mu,
                           int32_t nesterov, float ns_eps, char *ws,
                           const MuonWorkspace &L, bool no_iterations, const float *dev,
                           hipStream_t stream);

// 64 x 64 tiles of the padded stored-orientation matrix (the fused pass 1's
// workgroups and norm partials per matrix).
int32_t muon_pre_tiles(const MuonGeom &g);

// The partials region of a group: batch * norm_blocks fp64 partial sums of
// U^2, then per matrix the pre-scale s = 1 / (||U||_F + eps) in fp64, then
// per matrix the binary32 factor the first Newton-Schulz iteration applies to
// its products of X (s, or 1 where the pre-step wrote X0 = bf16(U s) itself).
inline double *muon_sd_ptr(char *ws, const MuonGeom &g, const MuonWorkspace &L) {
    return reinterpret_cast<double *>(ws + L.partials) + (int64_t)g.batch * g.norm_blocks;
}
inline float *muon_scale_ptr(char *ws, const MuonGeom &g, const MuonWorkspace &L) {
    return reinterpret_cast<float *>(muon_sd_ptr(ws, g, L) + g.batch);
}

// reject: per-matrix flags (non-zero: leave that matrix untouched) or NULL.
// dev: device scalars, from which decay and step_lr = lr * scale are formed
// when the kernel runs, or NULL (decay and step_lr as given).
hipError_t launch_muon_post(const MuonGeom &g, const MuonPtrs &ptrs,
                            const uint16_t *o_base, int64_t o_ld, size_t o_stride,
                            float decay, float step_lr, const int32_t *reject,
                            const float *dev, double scale, hipStream_t stream);

int32_t ns_health_blocks(int64_t count);

// A group of a Muon call as the Newton-Schulz launches see it: its geometry,
// its workspace carve-up and where its workspace starts.
struct NsGroupRef {
    const MuonGeom *geom;
    const MuonWorkspace *layout;
    char *base;
};

// Health of each matrix's Newton-Schulz result X (in the workspaces, after
// ns_steps iterations) for the nrefs groups, in two launches: writes [ratio,
// absmax, rejected] for matrix b of group i to health + 2 + 3 * (mat_first[i]
// + b) and the reject flags to the workspaces.
hipError_t launch_ns_health(const NsGroupRef *refs, const int *mat_first, int nrefs,
                            int ns_steps, float guard, float *health, hipStream_t stream);

// health[0] = matrices rejected, health[1] = worst ratio among the others
// (0 if none), from the nmat triples at health + 2.
hipError_t launch_ns_health_total(float *health, int32_t nmat, hipStream_t stream);

// The segments of a group's ns_steps Newton-Schulz steps: steps of one each
// for plain iterations; on the Gram matrix, ceil(ns_steps / kNsMaxSegment)
// segments as even as possible, longer ones first (5 -> 3, 2).  Writes the
// lengths to len (if not NULL; room for ns_steps) and returns the count.  X
// lies in the workspace's x region before even segments and in xt0 before odd
// ones; the result is where the count's parity puts it.
int ns_segments(const MuonGeom &g, int ns_steps, int *len = nullptr);

// One step of a group's Newton-Schulz program: one kind of product, once or
// twice, on slots of the group's symmetric pool.
//   kind 0  X X^T        -> out                        (a segment's first step)
//   kind 1  a I + b A + c A A of A = in1 -> out        (P)
//   kind 2  X' = P X, P = in1                          (a segment's last step)
//   kind 3  L R of two commuting symmetric matrices in1, in2 -> out
struct NsStep {
    int8_t kind, nprod;
    int8_t in1[2], in2[2], out[2];
    int8_t f16in;      // the symmetric products' operands are fp16 (else bf16)
    int8_t f16out[2];  // each product's output is fp16
    int16_t seg;      // segment of the step
    int8_t last_seg;  // 1: the segment is the last
};
constexpr int kNsKindXXT = 0, kNsKindBX = 2;  // the kinds above by name
constexpr int kNsMaxProgram = 4 * 100;
constexpr int kNsMaxMerged = 2 * kNsMaxProgram;
struct NsProgram {
    int len;
    NsStep step[kNsMaxProgram];
};
// The launches of a set of groups: their programs (0: plain, 1: Gram), merged
// into one sequence of steps in which each launch computes the same kind of
// product for every group whose program has that step next (the shortest
// common supersequence of the two programs' kinds).  idx[p][t] is program p's
// step in merged step t, or -1.
struct NsSchedule {
    NsProgram prog[2];
    int used[2];  // whether any group runs program p
    int nsteps;
    int16_t idx[2][kNsMaxMerged];
    int8_t kind[kNsMaxMerged];
};
// f16: segments of more than one step hold their m x m chain in fp16
// (ns_gram_f16_safe), else in bf16.
void ns_schedule(const NsGroupRef *refs, int nrefs, int ns_steps, bool f16, NsSchedule &s);

// Whether fp16 holds every m x m matrix of the Gram segments of ns_steps steps
// with coefficients (a, b, c) with room to spare (see the definition).
bool ns_gram_f16_safe(int ns_steps, float a, float b, float c);

// Merged step t of a schedule for every group: one launch per tile size in
// use (more if over kMaxGroups products share a tile size).
hipError_t launch_ns_step(const NsGroupRef *refs, int nrefs, const NsSchedule &s, int t, float a,
                          float b, float c, hipStream_t stream);

// Workgroups of the Newton-Schulz kernel with the given tile size that the
// current device holds at once (one round of tiles).
int ns_round_tiles(int tile);

// Whether the Newton-Schulz iterations of these groups (one launch bin) run
// on two streams, the groups divided between them by work: when the bin's
// 256-tile X X^T launch (split parts included) holds fewer than two rounds of
// workgroups, so that each product's launch leaves much of the GPU idle in
// its last round and the other stream's launches fill it.  Per-matrix
// arithmetic is the same either way (results equal bit for bit).
bool ns_split_streams(const NsGroupRef *refs, int nrefs);

// Caps the workgroups that the persistent B X launches keep resident (n <= 0:
// a full round; otherwise max(8, n rounded down to a multiple of 8)).
void ns_set_workgroup_limit(int n);

}  // namespace zopt
