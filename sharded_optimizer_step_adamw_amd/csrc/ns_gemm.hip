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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Epilogue shared by the kernels.  Accumulator layout of a 32x32 MFMA tile:
// lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// For the symmetric products the triangle test is made per 32x32 sub-tile
// (uniform across the wave): sub-tiles below the diagonal are skipped, those
// above it store each value and its mirror, and only the diagonal sub-tiles
// test element by element.
template <int MODE, int FM, int FN, int WTM, int WTN>
__device__ __forceinline__ void epilogue(const NsArgs &args, f32x16 (&acc)[FM][FN], int batch,
                                         int m0, int n0, int wr, int wc, int lane) {
    uint16_t *C = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
    const uint16_t *E = args.E + batch * args.c_stride;
    const int64_t ldc = args.ldc;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int R0 = m0 + wr * WTM + i * 32, C0 = n0 + wc * WTN + j * 32;
            const int gj = C0 + (lane & 31);
            if (MODE == kGemmBX) {
                uint16_t *CT = args.CT + batch * args.ct_stride;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi = R0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const int64_t o = (int64_t)gi * ldc + gj;
                    const uint16_t h = to_bf16((args.a + dIn[gi]) * from_bf16(C[o]) + acc[i][j][r]);
                    C[o] = h;
                    CT[(int64_t)gj * args.ldct + gi] = h;
                }
                continue;
            }
            if (R0 > C0) continue;            // below the diagonal
            const bool diag = R0 == C0;
            const float da_j = MODE == kSyrkAA ? dIn[gj] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gi = R0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const float v = acc[i][j][r];
                float x = v;
                if (MODE == kSyrkAA) {
                    // Aoff's diagonal is stored as zero, so this is c v there,
                    // replaced below by the diagonal's own formula
                    const float da_i = dIn[gi];
                    const float aoff = from_bf16(E[(int64_t)gi * ldc + gj]);
                    x = args.b * aoff + args.c * (v + (da_i + da_j) * aoff);
                    if (gi == gj) x = args.b * da_i + args.c * (v + da_i * da_i);
                }
                const uint16_t h = to_bf16(x);
                if (!diag || gi < gj) {
                    C[(int64_t)gi * ldc + gj] = h;
                    C[(int64_t)gj * ldc + gi] = h;
                } else if (gi == gj) {
                    dOut[gi] = x;
                    C[(int64_t)gi * ldc + gi] = 0;
                }
            }
        }
    }
}

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
    tile_of<MODE>(args, ti, tj);
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

    epilogue<MODE, FM, FN, WTM, WTN>(args, acc, batch, m0, n0, wr, wc, lane);
}


// ----------------------------------------------------------------------------
// 256 x 256 tiles for the large shapes.
//
// Eight waves (two per SIMD) each own a 128 x 64 sub-tile built from 8 x 4
// MFMA 16x16x32 bf16 tiles (128 fp32 accumulators per lane).  K advances 64
// columns per stage through two LDS stages of 2 x 32 KB.  Operands go from
// global memory straight to LDS (global_load_lds, 16 bytes per lane, each
// wave instruction filling one contiguous kilobyte = 8 rows of 64 K-columns);
// a lane fetches the chunk that the XOR swizzle (chunk c of row r at
// position c ^ (r & 7)) puts at its LDS slot, so fragment reads of 16
// consecutive rows spread over all banks without padding.  Within a stage
// the fragment reads of the next 32-column sub-step and the global loads of
// the next stage are interleaved with the MFMAs, and the MFMA clusters run at
// raised wave priority so one wave's matrix work overlaps the other wave's
// memory work on the same SIMD.
constexpr int kWaves256 = 8;

#define LDS_ADDR(p) ((__attribute__((address_space(3))) void *)(p))

// Swizzled byte offsets inside a wave's epilogue region: R holds the 128 x 64
// sub-block row by row (128-byte rows of 8 chunks), T holds it transposed
// (64 rows of 256 bytes, 16 chunks).
__device__ __forceinline__ int swz_r(int i, int j) {
    return i * 128 + (((j >> 3) ^ (i & 7)) << 4) + ((j & 7) << 1);
}
__device__ __forceinline__ int swz_t(int i, int j) {
    return i * 256 + (((j >> 3) ^ (i & 15)) << 4) + ((j & 7) << 1);
}

// Epilogue: the accumulators are completed in place (A A: b Aoff + c (acc +
// (dA_i + dA_j) Aoff), its diagonal b dA_i + c (acc + dA_i^2); B X:
// (a + dB_i) X + acc; the inputs staged through LDS), then leave through the
// wave's 16 KB LDS region as coalesced 16-byte row stores: row order to the
// sub-block itself, transposed to X^T (B X) or to the mirror position (the
// symmetric products).  A symmetric sub-block that crosses the diagonal is
// stored element by element from its upper triangle, so the mirror of each
// value is that same bf16 value; below the diagonal nothing is stored; the
// diagonal goes to the fp32 vector (its bf16 entry is 0).  Every wave passes
// the same barriers.
template <int MODE>
__device__ __forceinline__ void epilogue256(const NsArgs &args, f32x4 (&acc)[8][4], int batch,
                                            int m0, int n0, int wr, int wc, int wave, int lane,
                                            uint8_t *lds_all) {
    constexpr int SR = 128, SC = 64;
    uint8_t *W = lds_all + wave * (SR * SC * 2);
    const int R0 = m0 + wr * SR, C0 = n0 + wc * SC;
    constexpr bool sym = MODE != kGemmBX;
    const bool below = sym && R0 >= C0 + SC;
    const bool above = !sym || R0 + SR <= C0;
    const bool cross = sym && !below && !above;
    const int64_t ldc = args.ldc;
    uint16_t *Cm = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
    const int col = lane & 15, quad = lane >> 4;

    // 1. stage the input sub-block (row order) and complete the accumulators
    if (MODE != kSyrkXXT && !below) {
        const uint16_t *E = MODE == kSyrkAA ? args.E + batch * args.c_stride : Cm;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int id = k * 64 + lane, i = id >> 3, c = id & 7;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(E + (int64_t)(R0 + i) * ldc + C0 + c * 8);
            *reinterpret_cast<u32x4 *>(W + i * 128 + ((c ^ (i & 7)) << 4)) = v;
        }
    }
    __syncthreads();
    if (!below) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int lj = j * 16 + col, gj = C0 + lj;
                const float da_j = MODE == kSyrkAA ? dIn[gj] : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int li = i * 16 + quad * 4 + r, gi = R0 + li;
                    float x = acc[i][j][r];
                    if (MODE == kGemmBX) {
                        const float xv = from_bf16(*reinterpret_cast<const uint16_t *>(W + swz_r(li, lj)));
                        x = (args.a + dIn[gi]) * xv + x;
                    } else if (MODE == kSyrkAA) {
                        const float da_i = dIn[gi];
                        const float aoff = from_bf16(*reinterpret_cast<const uint16_t *>(W + swz_r(li, lj)));
                        const float v = x;
                        x = args.b * aoff + args.c * (v + (da_i + da_j) * aoff);
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
        // element by element, upper triangle and its mirror
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
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
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int lj = j * 16 + col, li = i * 16 + quad * 4;
                *reinterpret_cast<u32x2 *>(W + swz_t(lj, li)) =
                    u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
            }
    }
    __syncthreads();
    if (coalesced) {
        uint16_t *dst = MODE == kGemmBX ? args.CT + batch * args.ct_stride : Cm;
        const int64_t ld = MODE == kGemmBX ? (int64_t)args.ldct : ldc;
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int id = k * 64 + lane, i = id >> 4, c = id & 15;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(W + i * 256 + ((c ^ (i & 15)) << 4));
            *reinterpret_cast<u32x4 *>(dst + (int64_t)(C0 + i) * ld + R0 + c * 8) = v;
        }
    }
    __syncthreads();
    // 3. row order
    if (coalesced) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int lj = j * 16 + col;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    *reinterpret_cast<uint16_t *>(W + swz_r(i * 16 + quad * 4 + r, lj)) = to_bf16(acc[i][j][r]);
            }
    }
    __syncthreads();
    if (coalesced) {
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int id = k * 64 + lane, i = id >> 3, c = id & 7;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(W + i * 128 + ((c ^ (i & 7)) << 4));
            *reinterpret_cast<u32x4 *>(Cm + (int64_t)(R0 + i) * ldc + C0 + c * 8) = v;
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(kWaves256 * 64) void ns_gemm256_kernel(NsArgs args) {
    constexpr int BM = 256, WTM = 128, WTN = 64, FM = 8, FN = 4, ROW = 128;
    constexpr int OPER = BM * ROW;            // 32 KB per operand per stage
    constexpr int LOADS = 32 / kWaves256;      // kilobyte instructions per operand per wave
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2][2][OPER];

    const int batch = blockIdx.y;
    int ti, tj;
    tile_of<MODE>(args, ti, tj);
    const int m0 = ti * BM, n0 = tj * BM;
    const uint16_t *P = args.P + batch * args.p_stride + (int64_t)m0 * args.ldp;
    const uint16_t *Q = args.Q + batch * args.q_stride + (int64_t)n0 * args.ldq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave >> 2, wc = wave & 3;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // global -> LDS: instruction q of this wave fills kilobyte block
    // k = q * 8 + wave (rows 8k .. 8k+7); lane l takes row 8k + l / 8 and the
    // global chunk that the swizzle places at slot l % 8
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lrow & 7);
    const uint16_t *pl = P + (int64_t)lrow * args.ldp + lchunk * 8;
    const uint16_t *ql = Q + (int64_t)lrow * args.ldq + lchunk * 8;
    auto gload = [&](int st, int k0) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int k = q * kWaves256 + wave;
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
#pragma unroll
                for (int x = 0; x < 2 * LOADS; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
#pragma unroll
                for (int x = 0; x < FM + FN; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    epilogue256<MODE>(args, acc, batch, m0, n0, wr, wc, wave, lane, &lds[0][0][0]);
}

template <int T, int MODE>
void launch(dim3 grid, const NsArgs &a, hipStream_t stream) {
    if constexpr (T == 256)
        hipLaunchKernelGGL((ns_gemm256_kernel<MODE>), grid, dim3(kWaves256 * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((ns_gemm_kernel<T, T, MODE>), grid, dim3(kThreads), 0, stream, a);
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
    launch<T, kSyrkXXT>(dim3(tri, g.batch), s1, stream);

    NsArgs s2{};
    s2.P = A; s2.Q = A; s2.p_stride = as; s2.q_stride = as;
    s2.ldp = g.mp; s2.ldq = g.mp; s2.K = g.mp; s2.tiles_m = tm; s2.tiles_n = tm;
    s2.C = B; s2.c_stride = as; s2.ldc = g.mp; s2.E = A; s2.b = b; s2.c = c;
    s2.dIn = dA; s2.dOut = dB; s2.d_stride = ds;
    launch<T, kSyrkAA>(dim3(tri, g.batch), s2, stream);

    NsArgs s3{};
    s3.P = B; s3.Q = XT; s3.p_stride = as; s3.q_stride = xs;
    s3.ldp = g.mp; s3.ldq = g.mp; s3.K = g.mp; s3.tiles_m = tm; s3.tiles_n = tn;
    s3.C = X; s3.c_stride = xs; s3.ldc = g.np;
    s3.CT = XTn; s3.ct_stride = xs; s3.ldct = g.mp; s3.a = a;
    s3.dIn = dB; s3.dOut = dB; s3.d_stride = ds;
    launch<T, kGemmBX>(dim3(tm * tn, g.batch), s3, stream);
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
