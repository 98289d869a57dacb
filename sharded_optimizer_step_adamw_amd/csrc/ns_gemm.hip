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


// Epilogue of the 256 x 256 kernel, staged through LDS (free once the K loop
// has ended).  Each wave owns a 128 x 128 sub-block and a 32 KB LDS region
// holding it as bf16, rows of 256 bytes whose sixteen 16-byte chunks are
// XOR-swizzled by the row index.  The accumulators are completed in place
// from a staged input (A A: from Aoff; B X: the (a + dB_i) X term).  They
// are written
// to LDS once transposed (8-byte writes of four consecutive rows) and once
// in row order, and each layout leaves as coalesced 16-byte row stores: the
// transposed one to X^T (full product) or to the mirror sub-block (symmetric
// products), the row-order one to the sub-block itself.  Sub-blocks of the
// symmetric products below the diagonal do nothing; those on it are filled
// symmetrically from their upper triangle, store once, and send their
// diagonal to the fp32 vector.  Every wave passes the same barriers.
__device__ __forceinline__ int swz(int i, int j) {
    return i * 256 + (((j >> 3) ^ (i & 15)) << 4) + ((j & 7) << 1);
}

// Coalesced copy of the 128 x 128 bf16 sub-block at (R0, C0) of M (row
// stride ld) into the wave's LDS region, row order.
__device__ __forceinline__ void stage_in(uint8_t *T, const uint16_t *M, int64_t ld, int R0, int C0,
                                         int lane) {
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
        const int id = k * 64 + lane, i = id >> 4, c = id & 15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(M + (int64_t)(R0 + i) * ld + C0 + c * 8);
        *reinterpret_cast<u32x4 *>(T + i * 256 + ((c ^ (i & 15)) << 4)) = v;
    }
}

// Coalesced store of the wave's LDS region (row order) to M at (R0, C0).
__device__ __forceinline__ void stage_out(const uint8_t *T, uint16_t *M, int64_t ld, int R0, int C0,
                                          int lane) {
#pragma unroll 8
    for (int k = 0; k < 32; ++k) {
        const int id = k * 64 + lane, i = id >> 4, c = id & 15;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(T + i * 256 + ((c ^ (i & 15)) << 4));
        *reinterpret_cast<u32x4 *>(M + (int64_t)(R0 + i) * ld + C0 + c * 8) = v;
    }
}

template <int MODE>
__device__ __forceinline__ void epilogue256(const NsArgs &args, f32x16 (&acc)[4][4], int batch,
                                            int m0, int n0, int wr, int wc, int lane,
                                            uint8_t *lds_all) {
    constexpr int S = 128;
    uint8_t *T = lds_all + ((wr << 1) | wc) * (S * S * 2);
    const int R0 = m0 + wr * S, C0 = n0 + wc * S;
    constexpr bool sym = MODE != kGemmBX;
    const bool below = sym && R0 > C0;
    const bool diag = sym && R0 == C0;
    const int64_t ldc = args.ldc;
    uint16_t *Cm = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
    const int h = lane >> 5, col = lane & 31;

    // 1. complete the accumulators (A A: b Aoff + c (acc + (dA_i + dA_j) Aoff);
    //    B X: (a + dB_i) X + acc; diagonals of the symmetric products go to the
    //    fp32 vector)
    if (MODE == kSyrkAA && !below) stage_in(T, args.E + batch * args.c_stride, ldc, R0, C0, lane);
    if (MODE == kGemmBX) stage_in(T, Cm, ldc, R0, C0, lane);
    __syncthreads();
    if (!below) {
#pragma unroll
        for (int is = 0; is < 4; ++is)
#pragma unroll
            for (int js = 0; js < 4; ++js) {
                const int lj = js * 32 + col, gj = C0 + lj;
                const float da_j = MODE == kSyrkAA ? dIn[gj] : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int li = is * 32 + 8 * (r >> 2) + 4 * h + (r & 3), gi = R0 + li;
                    float x = acc[is][js][r];
                    if (MODE == kGemmBX)
                        x = (args.a + dIn[gi]) *
                                from_bf16(*reinterpret_cast<const uint16_t *>(T + swz(li, lj))) + x;
                    if (MODE == kSyrkAA) {
                        // Aoff's diagonal is stored as zero: on it this is c v,
                        // replaced by the diagonal's own formula
                        const float da_i = dIn[gi];
                        const float aoff = from_bf16(*reinterpret_cast<const uint16_t *>(T + swz(li, lj)));
                        const float v = x;
                        x = args.b * aoff + args.c * (v + (da_i + da_j) * aoff);
                        if (gi == gj) x = args.b * da_i + args.c * (v + da_i * da_i);
                    }
                    if (diag && gi == gj) {
                        dOut[gi] = x;
                        x = 0.0f;
                    }
                    acc[is][js][r] = x;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    __syncthreads();

    // 2. transposed layout T[lj][li]; on the diagonal, the symmetric fill
    if (!below) {
#pragma unroll
        for (int is = 0; is < 4; ++is)
#pragma unroll
            for (int js = 0; js < 4; ++js) {
                const int lj = js * 32 + col;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int li = is * 32 + 8 * q + 4 * h;
                    const uint32_t lo = pack_bf16x2(acc[is][js][4 * q], acc[is][js][4 * q + 1]);
                    const uint32_t hi = pack_bf16x2(acc[is][js][4 * q + 2], acc[is][js][4 * q + 3]);
                    if (!diag) {
                        *reinterpret_cast<u32x2 *>(T + swz(lj, li)) = u32x2{lo, hi};
                    } else {
#pragma unroll
                        for (int s2 = 0; s2 < 4; ++s2) {
                            const int i2 = li + s2;
                            if (i2 > lj) continue;
                            const uint16_t hv = (uint16_t)((s2 < 2 ? lo : hi) >> ((s2 & 1) * 16));
                            *reinterpret_cast<uint16_t *>(T + swz(lj, i2)) = hv;
                            *reinterpret_cast<uint16_t *>(T + swz(i2, lj)) = hv;
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    __syncthreads();
    if (!below) {
        // rows of T: X^T rows (full product), the mirror sub-block, or the
        // symmetric diagonal sub-block itself
        if (MODE == kGemmBX)
            stage_out(T, args.CT + batch * args.ct_stride, args.ldct, C0, R0, lane);
        else
            stage_out(T, Cm, ldc, C0, R0, lane);
    }
    __syncthreads();

    // 3. row order for the sub-block itself (not needed on the diagonal)
    const bool direct = !below && !diag;
    if (direct) {
#pragma unroll
        for (int is = 0; is < 4; ++is)
#pragma unroll
            for (int js = 0; js < 4; ++js) {
                const int lj = js * 32 + col;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int li = is * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    *reinterpret_cast<uint16_t *>(T + swz(li, lj)) = to_bf16(acc[is][js][r]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
    }
    __syncthreads();
    if (direct) stage_out(T, Cm, ldc, R0, C0, lane);
}

// 256 x 256 tiles for the large shapes.  Four waves each own a 128 x 128
// sub-tile (4 x 4 MFMA tiles, 256 fp32 accumulators per lane), so each
// 16-byte operand fragment read from LDS feeds four MFMAs.  The K loop moves
// 64 columns per stage through two 64 KB LDS stages.  LDS rows are 128 bytes
// with no padding; the eight 16-byte chunks of row r are stored XOR-swizzled
// (chunk c at position c ^ (r & 7)), so the 32 lanes of an operand read,
// which take one chunk from each of 32 consecutive rows, spread over all
// banks.  Global loads for stage k+2 are issued while stage k is multiplied.
template <int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm256_kernel(NsArgs args) {
    constexpr int BM = 256, BN = 256, WTM = 128, WTN = 128, FM = 4, FN = 4;
    constexpr int ROW_BYTES = kBK * 2;                  // 128
    constexpr int OPER_BYTES = BM * ROW_BYTES;          // 32 KB per operand per stage
    constexpr int LOADS = BM * (kBK / 8) / kThreads;    // 8 chunks per thread per operand
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][OPER_BYTES];

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

    // chunk ch = tid + 256 q: tile row ch / 8, 16-byte chunk ch % 8 of the
    // row's 64 K-columns; eight consecutive threads read one 128-byte row
    u32x4 pr[LOADS], qr[LOADS];
    int soff[LOADS];  // swizzled LDS byte offset of each chunk (same for P and Q)
    const uint16_t *pg[LOADS], *qg[LOADS];
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int ch = tid + q * kThreads, row = ch >> 3, c = ch & 7;
        soff[q] = row * ROW_BYTES + ((c ^ (row & 7)) << 4);
        pg[q] = P + (int64_t)row * args.ldp + c * 8;
        qg[q] = Q + (int64_t)row * args.ldq + c * 8;
    }
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q) pr[q] = *reinterpret_cast<const u32x4 *>(pg[q] + k0);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) qr[q] = *reinterpret_cast<const u32x4 *>(qg[q] + k0);
    };
    auto lstore = [&](int st) {
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            *reinterpret_cast<u32x4 *>(&lds[st][0][soff[q]]) = pr[q];
#pragma unroll
        for (int q = 0; q < LOADS; ++q)
            *reinterpret_cast<u32x4 *>(&lds[st][1][soff[q]]) = qr[q];
    };
    // operand fragment: rows base + lane % 32, chunk 2 ks + lane / 32
    const int fr = lane & 31, fh = lane >> 5;
    auto frag = [&](int st, int op, int rowbase, int ks) {
        const int r = rowbase + fr, c = 2 * ks + fh;
        return *reinterpret_cast<const bf16x8 *>(&lds[st][op][r * ROW_BYTES + ((c ^ (r & 7)) << 4)]);
    };

    const int KT = args.K / kBK;
    gload(0);
    lstore(0);
    if (KT > 1) gload(kBK);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = frag(st, 0, wr * WTM + i * 32, ks);
#pragma unroll
            for (int j = 0; j < FN; ++j) bfr[j] = frag(st, 1, wc * WTN + j * 32, ks);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < KT) {
            lstore(st ^ 1);
            if (kt + 2 < KT) gload((kt + 2) * kBK);
        }
        __syncthreads();
    }
    epilogue256<MODE>(args, acc, batch, m0, n0, wr, wc, lane, &lds[0][0][0]);
}

template <int T, int MODE>
void launch(dim3 grid, const NsArgs &a, hipStream_t stream) {
    if constexpr (T == 256)
        hipLaunchKernelGGL((ns_gemm256_kernel<MODE>), grid, dim3(kThreads), 0, stream, a);
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
