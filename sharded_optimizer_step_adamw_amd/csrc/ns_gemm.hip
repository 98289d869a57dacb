// ns_gemm.hip -- the Newton-Schulz engine on bf16 matrix cores (gfx950).
//
// One iteration [BluScript trainer source, ShardedMuon comment block:
// X <- aX + (bXX' + c(XX')^2)X] is three products, all of the form
// C = P Q^T with both operands row-major and contiguous along the reduction
// index, so every operand is read with 128-bit loads and no transposition:
//
//   A  = X X^T           P = Q = X     (m x n, K = n)   upper tiles only
//   B  = b A + c A A     P = Q = A     (A symmetric: A A = A A^T), upper tiles
//   X' = a X + B X       P = B, Q = X^T (K = m); writes X' in place and X'^T
//
// A and B are symmetric, so only tiles on or above the diagonal are computed
// and each is stored twice (itself and its mirror), from the upper triangle
// of the tile, which keeps A and B exactly symmetric.
//
// Diagonals in fp32.  The diagonals of A and B are their largest entries (A
// is positive semi-definite; once X is near-orthogonal, B is close to
// (b + c) I = -2.74 I), and a X + B X cancels them to about 0.7 X, which
// turns bf16 rounding of B's diagonal into the dominant error.  So A and B
// are stored as bf16 off-diagonal parts (zero diagonal) plus fp32 diagonal
// vectors dA, dB, and the products are regrouped exactly:
//   A A      = Aoff Aoff + dA_i Aoff_ij + Aoff_ij dA_j + delta_ij dA_i^2
//   B        = b (Aoff + diag dA) + c A A   ->  Boff, dB
//   a X + B X = (a + dB_i) X_ij + (Boff X)_ij
// Only the rounding points move; on every shape tried this lowers the error
// against float64 by 1.5-4x (bf16 emulation).
//
// The transposed copy
// X'^T written by the third product is the Q operand of the next iteration's
// third product (dmuon PR #16 prior art ran X X^T as a separate SYRK kernel;
// here all three products share one kernel template).
#include "zopt_internal.h"

namespace zopt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;

enum Mode : int { kSyrkXXT = 0, kSyrkAA = 1, kGemmBX = 2 };

struct NsArgs {
    const uint16_t *P;   // left operand rows (M x K)
    const uint16_t *Q;   // right operand rows (N x K)
    int64_t p_stride, q_stride;  // elements between batch entries
    int32_t ldp, ldq, K;
    int32_t tiles_m, tiles_n;    // tile grid (SYRK: tiles_m == tiles_n)
    uint16_t *C;                 // A or B (SYRK) / X, updated in place (GEMM)
    int64_t c_stride;
    int32_t ldc;
    const uint16_t *E;           // SYRK_AA: Aoff (for b*A); unused otherwise
    float *dIn;                  // SYRK_AA: dA; GEMM_BX: dB
    float *dOut;                 // SYRK_XXT: dA; SYRK_AA: dB
    int64_t d_stride;            // floats between batch entries of dA / dB
    uint16_t *CT;                // GEMM_BX: X'^T
    int64_t ct_stride;
    int32_t ldct;
    float a, b, c;
};

__device__ __forceinline__ uint16_t to_bf16(float x) { return (uint16_t)rne_bf16_bits(x); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return bf16_bits_to_float(h); }

// The tile of this workgroup: row-major over the tile grid for the full
// product, and over the upper triangle (ti <= tj) for the symmetric ones.
template <int MODE>
__device__ __forceinline__ void tile_of(const NsArgs &args, int &ti, int &tj) {
    if (MODE == kGemmBX) {
        ti = blockIdx.x / args.tiles_n;
        tj = blockIdx.x % args.tiles_n;
    } else {
        int t = blockIdx.x;
        ti = 0;
        while (t >= args.tiles_m - ti) {
            t -= args.tiles_m - ti;
            ++ti;
        }
        tj = ti + t;
    }
}

// ----------------------------------------------------------------------------
// The kernel.  A BM x BM output tile per workgroup of WR x WC waves; each wave
// owns a (BM/WR) x (BM/WC) sub-tile built from MFMA 16x16x32 bf16 blocks
// with fp32 accumulators:
//   BM = 256: 8 waves (two per SIMD) of 128 x 64 -- the large shapes
//   BM = 128: 4 waves of 64 x 64 (two workgroups per CU)
//   BM =  64: 4 waves of 32 x 32
// K advances 64 columns per stage through two LDS stages of 2 x BM x 128
// bytes.  Operands go from global memory straight to LDS (global_load_lds,
// 16 bytes per lane, each wave instruction filling one contiguous kilobyte =
// 8 rows of 64 K-columns); a lane fetches the chunk that the XOR swizzle
// (chunk c of row r at position c ^ (r & 7)) puts at its LDS slot, so
// fragment reads of 16 consecutive rows spread over the banks without
// padding.  Within a stage the next stage's global loads and the next
// 32-column sub-step's fragment reads are interleaved with the MFMAs, and the
// MFMA clusters run at raised wave priority so that waves sharing a SIMD
// overlap memory work with matrix work.
#define LDS_ADDR(p) ((__attribute__((address_space(3))) void *)(p))

template <int BM>
struct Cfg;
template <>
struct Cfg<256> { static constexpr int WR = 2, WC = 4; };
template <>
struct Cfg<128> { static constexpr int WR = 2, WC = 2; };
template <>
struct Cfg<64> { static constexpr int WR = 2, WC = 2; };

// Swizzled byte offset of element (i, j) in an LDS block whose rows hold
// `chunks` 16-byte chunks (chunks is a power of two).
template <int CHUNKS>
__device__ __forceinline__ int swz(int i, int j) {
    return i * (CHUNKS * 16) + (((j >> 3) ^ (i & (CHUNKS - 1))) << 4) + ((j & 7) << 1);
}

// Epilogue: the accumulators are completed in place (A A: b Aoff + c (acc +
// (dA_i + dA_j) Aoff), its diagonal b dA_i + c (acc + dA_i^2); B X:
// (a + dB_i) X + acc; the inputs staged through LDS), then leave through the
// wave's LDS region as coalesced 16-byte row stores: row order to the
// sub-block itself, transposed to X^T (B X) or to the mirror position (the
// symmetric products).  A symmetric sub-block that crosses the diagonal is
// stored element by element from its upper triangle, so the mirror of each
// value is that same bf16 value; below the diagonal nothing is stored; the
// diagonal goes to the fp32 vector (its bf16 entry is 0).  Every wave passes
// the same barriers.
template <int MODE, int FM, int FN>
__device__ __forceinline__ void epilogue(const NsArgs &args, f32x4 (&acc)[FM][FN], int batch,
                                         int R0, int C0, int wave, int lane, uint8_t *lds_all) {
    constexpr int SR = FM * 16, SC = FN * 16;      // sub-block rows, columns
    constexpr int RCH = SC / 8, TCH = SR / 8;      // chunks per row: row order, transposed
    uint8_t *W = lds_all + wave * (SR * SC * 2);
    constexpr bool sym = MODE != kGemmBX;
    const bool below = sym && R0 >= C0 + SC;
    const bool above = !sym || R0 + SR <= C0;
    const bool cross = sym && !below && !above;
    const int64_t ldc = args.ldc;
    uint16_t *Cm = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
    const int col = lane & 15, quad = lane >> 4;
    constexpr int RCHUNKS = SR * RCH, TCHUNKS = SC * TCH;   // 16-byte chunks per layout

    // 1. stage the input sub-block (row order) and complete the accumulators
    if (MODE != kSyrkXXT && !below) {
        const uint16_t *E = MODE == kSyrkAA ? args.E + batch * args.c_stride : Cm;
#pragma unroll 4
        for (int k = 0; k < RCHUNKS / 64; ++k) {
            const int id = k * 64 + lane, i = id / RCH, c = id % RCH;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(E + (int64_t)(R0 + i) * ldc + C0 + c * 8);
            *reinterpret_cast<u32x4 *>(W + i * (RCH * 16) + ((c ^ (i & (RCH - 1))) << 4)) = v;
        }
    }
    __syncthreads();
    if (MODE != kSyrkXXT && !below) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int lj = j * 16 + col, gj = C0 + lj;
                const float da_j = MODE == kSyrkAA ? dIn[gj] : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int li = i * 16 + quad * 4 + r, gi = R0 + li;
                    const float in = from_bf16(*reinterpret_cast<const uint16_t *>(W + swz<RCH>(li, lj)));
                    const float v = acc[i][j][r];
                    float x;
                    if (MODE == kGemmBX) {
                        x = (args.a + dIn[gi]) * in + v;
                    } else {
                        const float da_i = dIn[gi];
                        x = args.b * in + args.c * (v + (da_i + da_j) * in);
                        if (gi == gj) x = args.b * da_i + args.c * (v + da_i * da_i);
                    }
                    acc[i][j][r] = x;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();

    if (cross) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int gj = C0 + j * 16 + col;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gi = R0 + i * 16 + quad * 4 + r;
                    const float x = acc[i][j][r];
                    if (gi < gj) {
                        const uint16_t h = to_bf16(x);
                        Cm[(int64_t)gi * ldc + gj] = h;
                        Cm[(int64_t)gj * ldc + gi] = h;
                    } else if (gi == gj) {
                        dOut[gi] = x;
                        Cm[(int64_t)gi * ldc + gi] = 0;
                    }
                }
            }
    }
    const bool coalesced = !below && !cross;
    // 2. transposed: T[lj][li], four consecutive rows per 8-byte write
    if (coalesced) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                *reinterpret_cast<u32x2 *>(W + swz<TCH>(j * 16 + col, i * 16 + quad * 4)) =
                    u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
    }
    __syncthreads();
    if (coalesced) {
        uint16_t *dst = MODE == kGemmBX ? args.CT + batch * args.ct_stride : Cm;
        const int64_t ld = MODE == kGemmBX ? (int64_t)args.ldct : ldc;
#pragma unroll 4
        for (int k = 0; k < TCHUNKS / 64; ++k) {
            const int id = k * 64 + lane, i = id / TCH, c = id % TCH;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(W + i * (TCH * 16) + ((c ^ (i & (TCH - 1))) << 4));
            *reinterpret_cast<u32x4 *>(dst + (int64_t)(C0 + i) * ld + R0 + c * 8) = v;
        }
    }
    __syncthreads();
    // 3. row order
    if (coalesced) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<uint16_t *>(W + swz<RCH>(i * 16 + quad * 4 + r, j * 16 + col)) =
                        to_bf16(acc[i][j][r]);
    }
    __syncthreads();
    if (coalesced) {
#pragma unroll 4
        for (int k = 0; k < RCHUNKS / 64; ++k) {
            const int id = k * 64 + lane, i = id / RCH, c = id % RCH;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(W + i * (RCH * 16) + ((c ^ (i & (RCH - 1))) << 4));
            *reinterpret_cast<u32x4 *>(Cm + (int64_t)(R0 + i) * ldc + C0 + c * 8) = v;
        }
    }
}

template <int BM, int MODE>
__global__ __launch_bounds__(Cfg<BM>::WR * Cfg<BM>::WC * 64) void ns_gemm_kernel(NsArgs args) {
    constexpr int WR = Cfg<BM>::WR, WC = Cfg<BM>::WC, NW = WR * WC;
    constexpr int WTM = BM / WR, WTN = BM / WC, FM = WTM / 16, FN = WTN / 16, ROW = 128;
    constexpr int OPER = BM * ROW;               // bytes per operand per stage
    constexpr int LOADS = OPER / 1024 / NW;      // kilobyte instructions per operand per wave
    static_assert(LOADS * NW * 1024 == OPER, "tile");
    static_assert(BM * BM * 2 <= 4 * OPER, "epilogue regions fit in the stages");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][OPER];

    const int batch = blockIdx.y;
    int ti, tj;
    tile_of<MODE>(args, ti, tj);
    const int m0 = ti * BM, n0 = tj * BM;
    const uint16_t *P = args.P + batch * args.p_stride + (int64_t)m0 * args.ldp;
    const uint16_t *Q = args.Q + batch * args.q_stride + (int64_t)n0 * args.ldq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // global -> LDS: instruction q of this wave fills kilobyte block
    // k = q * NW + wave (rows 8k .. 8k+7); lane l takes row 8k + l / 8 and the
    // global chunk that the swizzle places at slot l % 8
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lrow & 7);
    const uint16_t *pl = P + (int64_t)lrow * args.ldp + lchunk * 8;
    const uint16_t *ql = Q + (int64_t)lrow * args.ldq + lchunk * 8;
    auto gload = [&](int st, int k0) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int k = q * NW + wave;
            __builtin_amdgcn_global_load_lds((const void *)(pl + (int64_t)(8 * k) * args.ldp + k0),
                                             LDS_ADDR(&lds[st][0][k * 1024]), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void *)(ql + (int64_t)(8 * k) * args.ldq + k0),
                                             LDS_ADDR(&lds[st][1][k * 1024]), 16, 0, 0);
        }
    };
    // MFMA 16x16x32 operand: lane l holds row l % 16, K-chunk l / 16 of the
    // 32-column sub-step (chunk 4 ks + l / 16 of the stage)
    const int fr = lane & 15, fh = lane >> 4;
    auto frag = [&](int st, int op, int rowbase, int ks) {
        const int r = rowbase + fr, c = 4 * ks + fh;
        return *reinterpret_cast<const bf16x8 *>(&lds[st][op][r * ROW + ((c ^ (r & 7)) << 4)]);
    };

    const int KT = args.K / kBK;
    gload(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < KT) gload(st ^ 1, (kt + 1) * kBK);
        bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) af[0][i] = frag(st, 0, wr * WTM + i * 16, 0);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[0][j] = frag(st, 1, wc * WTN + j * 16, 0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int cb = ks & 1, nb = cb ^ 1;
            if (ks == 0) {
#pragma unroll
                for (int i = 0; i < FM; ++i) af[nb][i] = frag(st, 0, wr * WTM + i * 16, 1);
#pragma unroll
                for (int j = 0; j < FN; ++j) bfr[nb][j] = frag(st, 1, wc * WTN + j * 16, 1);
            }
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[cb][i], bfr[cb][j], acc[i][j],
                                                                        0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
            if (ks == 0) {
                // the next stage's global loads and the next sub-step's
                // fragment reads, one after each MFMA
                constexpr int NV = (2 * LOADS < FM * FN) ? 2 * LOADS : FM * FN;
                constexpr int ND = (FM + FN < FM * FN - NV) ? FM + FN : FM * FN - NV;
#pragma unroll
                for (int x = 0; x < NV; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
#pragma unroll
                for (int x = 0; x < ND; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    epilogue<MODE, FM, FN>(args, acc, batch, m0 + wr * WTM, n0 + wc * WTN, wave, lane, &lds[0][0][0]);
}

template <int T>
constexpr int kThreadsOf = Cfg<T>::WR * Cfg<T>::WC * 64;

template <int T>
hipError_t run_iteration(const MuonGeom &g, char *ws, const MuonWorkspace &L, int cur_xt,
                         float a, float b, float c, hipStream_t stream) {
    uint16_t *X = reinterpret_cast<uint16_t *>(ws + L.x);
    uint16_t *XT = reinterpret_cast<uint16_t *>(ws + (cur_xt ? L.xt1 : L.xt0));
    uint16_t *XTn = reinterpret_cast<uint16_t *>(ws + (cur_xt ? L.xt0 : L.xt1));
    uint16_t *A = reinterpret_cast<uint16_t *>(ws + L.a);
    uint16_t *B = reinterpret_cast<uint16_t *>(ws + L.b);
    float *dA = reinterpret_cast<float *>(ws + L.da);
    float *dB = reinterpret_cast<float *>(ws + L.db);
    const int64_t ds = (int64_t)(L.d_stride / 4);
    const int64_t xs = (int64_t)(L.x_stride / 2), as = (int64_t)(L.a_stride / 2);
    const int tm = g.mp / T, tn = g.np / T;
    const int tri = tm * (tm + 1) / 2;

    NsArgs s1{};
    s1.P = X; s1.Q = X; s1.p_stride = xs; s1.q_stride = xs;
    s1.ldp = g.np; s1.ldq = g.np; s1.K = g.np; s1.tiles_m = tm; s1.tiles_n = tm;
    s1.C = A; s1.c_stride = as; s1.ldc = g.mp;
    s1.dIn = dA; s1.dOut = dA; s1.d_stride = ds;
    hipLaunchKernelGGL((ns_gemm_kernel<T, kSyrkXXT>), dim3(tri, g.batch), dim3(kThreadsOf<T>), 0,
                       stream, s1);

    NsArgs s2{};
    s2.P = A; s2.Q = A; s2.p_stride = as; s2.q_stride = as;
    s2.ldp = g.mp; s2.ldq = g.mp; s2.K = g.mp; s2.tiles_m = tm; s2.tiles_n = tm;
    s2.C = B; s2.c_stride = as; s2.ldc = g.mp; s2.E = A; s2.b = b; s2.c = c;
    s2.dIn = dA; s2.dOut = dB; s2.d_stride = ds;
    hipLaunchKernelGGL((ns_gemm_kernel<T, kSyrkAA>), dim3(tri, g.batch), dim3(kThreadsOf<T>), 0,
                       stream, s2);

    NsArgs s3{};
    s3.P = B; s3.Q = XT; s3.p_stride = as; s3.q_stride = xs;
    s3.ldp = g.mp; s3.ldq = g.mp; s3.K = g.mp; s3.tiles_m = tm; s3.tiles_n = tn;
    s3.C = X; s3.c_stride = xs; s3.ldc = g.np;
    s3.CT = XTn; s3.ct_stride = xs; s3.ldct = g.mp; s3.a = a;
    s3.dIn = dB; s3.dOut = dB; s3.d_stride = ds;
    hipLaunchKernelGGL((ns_gemm_kernel<T, kGemmBX>), dim3(tm * tn, g.batch), dim3(kThreadsOf<T>),
                       0, stream, s3);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_iteration(const MuonGeom &g, char *ws, const MuonWorkspace &L,
                               int cur_xt, float a, float b, float c, hipStream_t stream) {
    switch (g.tile) {
        case 64: return run_iteration<64>(g, ws, L, cur_xt, a, b, c, stream);
        case 128: return run_iteration<128>(g, ws, L, cur_xt, a, b, c, stream);
        case 256: return run_iteration<256>(g, ws, L, cur_xt, a, b, c, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zopt
