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
//
// Tiling: a workgroup of 4 waves computes a BM x BN tile; each wave a
// (BM/2) x (BN/2) sub-tile from 32x32x16 bf16 MFMAs with fp32 accumulation.
// K advances BK = 64 at a time through double-buffered LDS (rows padded by 16
// bytes so the 16-byte operand reads of a wave fall in distinct banks).
#include "zopt_internal.h"

namespace zopt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kPad = 8;  // bf16 elements of row padding in LDS

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

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(NsArgs args) {
    constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32; // MFMA tiles per wave
    constexpr int LDK = kBK + kPad;
    constexpr int CPR = kBK / 8;                // 16-byte chunks per tile row
    constexpr int CP = BM * CPR / kThreads;     // P chunks per thread
    constexpr int CQ = BN * CPR / kThreads;     // Q chunks per thread
    static_assert(CP * kThreads == BM * CPR && CQ * kThreads == BN * CPR, "tile");

    __shared__ __attribute__((aligned(16))) uint16_t Ps[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Qs[2][BN][LDK];

    const int batch = blockIdx.y;
    int ti, tj;
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
    const int m0 = ti * BM, n0 = tj * BN;
    const uint16_t *__restrict__ P = args.P + batch * args.p_stride + (int64_t)m0 * args.ldp;
    const uint16_t *__restrict__ Q = args.Q + batch * args.q_stride + (int64_t)n0 * args.ldq;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 1, wc = wave & 1;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    u32x4 pr[CP], qr[CQ];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < CP; ++q) {
            const int ch = tid + q * kThreads, row = ch / CPR, col = (ch % CPR) * 8;
            pr[q] = *reinterpret_cast<const u32x4 *>(P + (int64_t)row * args.ldp + k0 + col);
        }
#pragma unroll
        for (int q = 0; q < CQ; ++q) {
            const int ch = tid + q * kThreads, row = ch / CPR, col = (ch % CPR) * 8;
            qr[q] = *reinterpret_cast<const u32x4 *>(Q + (int64_t)row * args.ldq + k0 + col);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < CP; ++q) {
            const int ch = tid + q * kThreads, row = ch / CPR, col = (ch % CPR) * 8;
            *reinterpret_cast<u32x4 *>(&Ps[buf][row][col]) = pr[q];
        }
#pragma unroll
        for (int q = 0; q < CQ; ++q) {
            const int ch = tid + q * kThreads, row = ch / CPR, col = (ch % CPR) * 8;
            *reinterpret_cast<u32x4 *>(&Qs[buf][row][col]) = qr[q];
        }
    };

    const int KT = args.K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            bf16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(
                    &Ps[cur][wr * WTM + i * 32 + (lane & 31)][kc]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *reinterpret_cast<const bf16x8 *>(
                    &Qs[cur][wc * WTN + j * 32 + (lane & 31)][kc]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator layout of a 32x32 MFMA tile: lane l, register r
    // holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
    uint16_t *C = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gj = n0 + wc * WTN + j * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = m0 + wr * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const float v = acc[i][j][r];
                if (MODE == kGemmBX) {
                    const int64_t o = (int64_t)gi * args.ldc + gj;
                    const float x = (args.a + dIn[gi]) * from_bf16(C[o]) + v;
                    const uint16_t h = to_bf16(x);
                    C[o] = h;
                    args.CT[batch * args.ct_stride + (int64_t)gj * args.ldct + gi] = h;
                } else if (gi <= gj) {
                    float x = v;
                    if (MODE == kSyrkAA) {
                        const uint16_t *E = args.E + batch * args.c_stride;
                        const float da_i = dIn[gi];
                        if (gi == gj) {
                            x = args.b * da_i + args.c * (v + da_i * da_i);
                        } else {
                            const float aoff = from_bf16(E[(int64_t)gi * args.ldc + gj]);
                            x = args.b * aoff + args.c * (v + (da_i + dIn[gj]) * aoff);
                        }
                    }
                    if (gi == gj) {
                        dOut[gi] = x;
                        C[(int64_t)gi * args.ldc + gi] = 0;
                    } else {
                        const uint16_t h = to_bf16(x);
                        C[(int64_t)gi * args.ldc + gj] = h;
                        C[(int64_t)gj * args.ldc + gi] = h;
                    }
                }
            }
        }
    }
}

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
    hipLaunchKernelGGL((ns_gemm_kernel<T, T, kSyrkXXT>), dim3(tri, g.batch), dim3(kThreads), 0,
                       stream, s1);

    NsArgs s2{};
    s2.P = A; s2.Q = A; s2.p_stride = as; s2.q_stride = as;
    s2.ldp = g.mp; s2.ldq = g.mp; s2.K = g.mp; s2.tiles_m = tm; s2.tiles_n = tm;
    s2.C = B; s2.c_stride = as; s2.ldc = g.mp; s2.E = A; s2.b = b; s2.c = c;
    s2.dIn = dA; s2.dOut = dB; s2.d_stride = ds;
    hipLaunchKernelGGL((ns_gemm_kernel<T, T, kSyrkAA>), dim3(tri, g.batch), dim3(kThreads), 0,
                       stream, s2);

    NsArgs s3{};
    s3.P = B; s3.Q = XT; s3.p_stride = as; s3.q_stride = xs;
    s3.ldp = g.mp; s3.ldq = g.mp; s3.K = g.mp; s3.tiles_m = tm; s3.tiles_n = tn;
    s3.C = X; s3.c_stride = xs; s3.ldc = g.np;
    s3.CT = XTn; s3.ct_stride = xs; s3.ldct = g.mp; s3.a = a;
    s3.dIn = dB; s3.dOut = dB; s3.d_stride = ds;
    hipLaunchKernelGGL((ns_gemm_kernel<T, T, kGemmBX>), dim3(tm * tn, g.batch), dim3(kThreads),
                       0, stream, s3);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_iteration(const MuonGeom &g, char *ws, const MuonWorkspace &L,
                               int cur_xt, float a, float b, float c, hipStream_t stream) {
    switch (g.tile) {
        case 64: return run_iteration<64>(g, ws, L, cur_xt, a, b, c, stream);
        case 128: return run_iteration<128>(g, ws, L, cur_xt, a, b, c, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace zopt
