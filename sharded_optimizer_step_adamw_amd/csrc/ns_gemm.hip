// ns_gemm.hip -- the Newton-Schulz engine on bf16 matrix cores (gfx950).
//
// One iteration [BluScript trainer source, ShardedMuon comment block:
// X <- aX + (bXX' + c(XX')^2)X] is three products.  The symmetric ones are
// C = P Q^T with both operands row-major along the reduction index; the
// third reads X as it is, down its columns:
//
//   A  = X X^T           P = Q = X     (m x n, K = n)   upper tiles only
//   B  = b A + c A A     P = Q = A     (A symmetric: A A = A A^T), upper tiles
//   X' = a X + B X       P = B (K = m), Q = X read k-major; X' goes to the
//                        other buffer of a pair (X is still being read)
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
// B X stages X's rows [k, k + 32) x [n0, n0 + BM) as they lie in memory and
// reads the MFMA B operand out of LDS with ds_read_b64_tr_b16, which
// transposes 4 x 16 blocks of 16-bit values across each 16-lane group, so no
// transposed copy of X is ever written; the last iteration alone also writes
// X'^T for matrices stored transposed (their update is read in that
// orientation).  (dmuon PR #16 prior art ran X X^T as a separate SYRK kernel;
// here all three products share one kernel template.)
//
// Grouped launches.  One launch computes one product for every matrix of up
// to kMaxGroups same-tile groups (e.g. all of a model's Muon matrices whose
// short side selects the same tile), so that small groups fill the GPU
// together and the launch count per iteration stays at three per tile size.
// Workgroups are numbered group by group (longest reduction first), matrix by
// matrix, tile by tile.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <vector>

#include "zopt_internal.h"

namespace zopt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Mode : int { kSyrkXXT = 0, kSyrkAA = 1, kGemmBX = 2, kSymLR = 3 };

// One group of same-shape matrices in a launch.
struct NsGroup {
    const uint16_t *P;           // left operand rows (M x K)
    const uint16_t *Q;           // right operand: rows (N x K); B X: X (K x N)
    int64_t p_stride, q_stride;  // elements between matrices of the group
    int32_t ld, K;               // operand row stride (P; Q too but B X), reduction length
    int32_t ldq;                 // B X: row stride of X
    int32_t tiles_m, tiles_n;    // tile grid (SYRK: tiles_m == tiles_n)
    int32_t tiles_pm, tile0;     // tiles per matrix; first workgroup of the group
    int32_t tiles, padded;       // tiles of the group, rounded up to a multiple of 8
    int32_t round_tiles;         // tiles resident at once on the GPU (8 XCDs), a multiple of 8
    int32_t ldc, ldct;
    uint16_t *C;                 // A or B (SYRK) / X, updated in place (GEMM)
    int64_t c_stride;
    const uint16_t *E;           // SYRK_AA: Aoff (for b*A); unused otherwise
    const float *dIn;            // SYRK_AA: dA; GEMM_BX: dP; SYM_LR: the left operand's diagonal
    const float *dIn2;           // SYM_LR: the right operand's diagonal
    float *dOut;                 // SYRK_XXT: dA; SYRK_AA: dP; SYM_LR: the product's diagonal
    int64_t d_stride;            // floats between matrices of dA / dB
    uint16_t *CT;                // GEMM_BX: X'^T, or NULL (not wanted)
    int64_t ct_stride;
    // First iteration: X holds bf16(U) and the matrix's pre-scale s is
    // applied here, s^2 to X X^T and s to B X (one float per matrix); NULL
    // otherwise.
    const float *xs;
    // X X^T split along K: this entry's fp32 partial product (mp x mp per
    // matrix, row stride ldc), written whole for every computed tile; the
    // fix-up kernel forms A from the parts.  NULL: the normal epilogue.
    float *part;
    int64_t part_stride;
    // Symmetric products: the output's 16-bit element type (0 bf16, 1 fp16)
    int32_t out_f16;
};

struct NsLaunch {
    NsGroup g[kMaxGroups];
    int32_t ngroups;
    int32_t total;  // slots of all groups (B X: the persistent walk's end)
    int32_t xpf;    // B X: every group's K >= kStages * 32 (pipeline across tiles)
    float a, b, c;
};

// an LDS pointer in the LDS address space (for the direct-to-LDS loads)
#define LDS_ADDR(p) ((__attribute__((address_space(3))) void *)(p))

// lo, hi -> two bf16, round to nearest even, in one gfx950 instruction
// (v_cvt_pk_bf16_f32).  Equal to rne_bf16_bits for every non-NaN input; a NaN
// stays a NaN.  Used for the Newton-Schulz operands (X, A, B), which never
// meet the weight write-back's NaN convention.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
__device__ __forceinline__ uint16_t cvt_bf16(float x) { return (uint16_t)cvt_pk_bf16(x, 0.0f); }
__device__ __forceinline__ float from_bf16(uint16_t h) { return bf16_bits_to_float(h); }

// The same for fp16 (v_cvt_pk_f16_f32, round to nearest even), the element
// type of a Gram segment's m x m chain.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
__device__ __forceinline__ float from_f16(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
template <bool F16>
__device__ __forceinline__ float from_el(uint16_t h) {
    return F16 ? from_f16(h) : from_bf16(h);
}
// two values of a symmetric product's output, in its element type
__device__ __forceinline__ uint32_t pack_el(float lo, float hi, bool f16) {
    return f16 ? cvt_pk_f16(lo, hi) : cvt_pk_bf16(lo, hi);
}

// Tile t of a matrix, in bands of kBand tile rows taken column by column, so
// that the tiles an XCD runs at the same time share few operand row panels
// (kBand rows of P and the columns' rows of Q).  The full product walks the
// whole grid; the symmetric ones walk only tiles on or above the diagonal
// (ti <= tj), each band starting at its own diagonal.
constexpr int kBand = 4;
template <int MODE>
__device__ __forceinline__ void tile_coords(const NsGroup &G, int t, int &ti, int &tj) {
    const int tm = G.tiles_m;
    int b0 = 0;
    if (MODE == kGemmBX) {
        const int tn = G.tiles_n;
        for (;;) {
            const int h = tm - b0 < kBand ? tm - b0 : kBand;
            if (t < h * tn) {
                tj = t / h;
                ti = b0 + t % h;
                return;
            }
            t -= h * tn;
            b0 += kBand;
        }
    }
    for (;;) {
        const int h = tm - b0 < kBand ? tm - b0 : kBand;
        // band rows b0 .. b0+h-1, columns b0 .. tm-1; column c holds rows
        // b0 .. min(c, b0+h-1): a triangle of h(h+1)/2 then full columns
        const int tri = h * (h + 1) / 2, size = tri + h * (tm - b0 - h);
        if (t < size) {
            if (t < tri) {
                int c = 0;
                while (t > c) {
                    t -= c + 1;
                    ++c;
                }
                tj = b0 + c;
                ti = b0 + t;
            } else {
                t -= tri;
                tj = b0 + h + t / h;
                ti = b0 + t % h;
            }
            return;
        }
        t -= size;
        b0 += kBand;
    }
}

// ----------------------------------------------------------------------------
// Tiles.  A BM x BM output tile per workgroup of WR x WC waves; each wave
// owns a (BM/WR) x (BM/WC) sub-tile built from MFMA 16x16x32 bf16 blocks
// with fp32 accumulators:
//   BM = 256: 8 waves (two per SIMD) of 128 x 64 -- the large shapes
//   BM = 128: 4 waves of 64 x 64 (two workgroups per CU)
//   BM =  64: 4 waves of 32 x 32 (four workgroups per CU)
// WPE is the waves per SIMD that residency needs, which caps the registers.
template <int BM>
struct Cfg;
template <>
struct Cfg<256> { static constexpr int WR = 2, WC = 4, WPE = 2, SYM_STAGES = 4, SYM_WPE = 2; };
template <>
struct Cfg<128> { static constexpr int WR = 2, WC = 2, WPE = 2, SYM_STAGES = 3, SYM_WPE = 3; };
template <>
struct Cfg<64> { static constexpr int WR = 2, WC = 2, WPE = 4, SYM_STAGES = 4, SYM_WPE = 4; };

// Swizzled byte offset of element (i, j) in an LDS block whose rows hold
// `chunks` 16-byte chunks (chunks is a power of two).
template <int CHUNKS>
__device__ __forceinline__ int swz(int i, int j) {
    return i * (CHUNKS * 16) + (((j >> 3) ^ (i & (CHUNKS - 1))) << 4) + ((j & 7) << 1);
}

// Epilogue of the symmetric products: the accumulators are completed in
// place (A A: b Aoff + c (acc + (dA_i + dA_j) Aoff), its diagonal
// b dA_i + c (acc + dA_i^2), with Aoff staged through LDS).  A tile above
// the diagonal is written once, transposed, to each wave's LDS region, from
// which the sub-block leaves both as itself (transposing reads give each lane
// 8 consecutive columns of one row) and as its mirror (plain 16-byte reads of
// T's rows), in 16-byte stores.  A tile on the diagonal is built symmetric in
// LDS from its upper triangle and stored once.  The diagonal itself goes to
// the fp32 vector (its bf16 entry is 0).  Every wave passes the same
// barriers.
template <int MODE, int BM, int FM, int FN, bool F16>
__device__ __forceinline__ void epilogue(const NsGroup &args, float ca, float cb, float cc,
                                         f32x4 (&acc)[FM][FN], int batch, int m0, int n0, int R0,
                                         int C0, int wave, int lane, uint8_t *lds_all) {
    constexpr int SR = FM * 16, SC = FN * 16;      // sub-block rows, columns
    constexpr int RCH = SC / 8, TCH = SR / 8;      // chunks per row: row order, transposed
    static_assert(SC % 32 == 0, "row stores cover 32 columns");
    uint8_t *W = lds_all + wave * (SR * SC * 2);
    const uint32_t wb =
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)W);
    const bool below = R0 >= C0 + SC;
    const bool above = R0 + SR <= C0;
    const bool cross = !below && !above;
    const int64_t ldc = args.ldc;
    const bool of16 = args.out_f16 != 0;
    uint16_t *Cm = args.C + batch * args.c_stride;
    const float *dIn = args.dIn + batch * args.d_stride;
    float *dOut = args.dOut + batch * args.d_stride;
    const int col = lane & 15, quad = lane >> 4;
    if (MODE == kSyrkXXT && args.part != nullptr) {
        // one part of a split reduction: the raw fp32 sums (every workgroup
        // of the group takes this branch, so no barrier is skipped by some)
        float *Pm = args.part + batch * args.part_stride;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Pm[(int64_t)(R0 + i * 16 + quad * 4 + r) * ldc + C0 + j * 16 + col] = acc[i][j][r];
        return;
    }
    if (MODE == kSyrkXXT && args.xs != nullptr) {
        // first iteration: A = (s U)(s U)^T from the products of U
        const float s = args.xs[batch], s2 = s * s;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] *= s2;
    }
    // transposing read: lane 4q' + p of a 16-lane group addresses row +q',
    // columns 4p .. 4p+3 of a 4 x 16 block; lane i gets rows +0..+3 of column i
    const int tq = (lane >> 2) & 3, tp = lane & 3;
    auto tr_read = [](uint32_t addr) __attribute__((always_inline)) {
        u32x2 v;
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
        return v;
    };
    constexpr int TCHUNKS = SC * TCH;   // 16-byte chunks of the transposed image

    // 1. A A and L R: stage the input sub-block (Aoff / Loff, row order) and
    // complete the accumulators
    constexpr bool kIn = MODE == kSyrkAA || MODE == kSymLR;
    float da_c[FN], da_r[FM][4];
    // the wave's sub-block of a tile-shaped 16-bit matrix (base at this
    // matrix's element (0, 0)) into its region W, row order, chunk c of row i
    // at slot c ^ (i % RCH), with plain loads and LDS stores
    auto stage = [&](const uint16_t *src) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < SR * RCH / 64; ++k) {
            const int id = k * 64 + lane, i = id / RCH, c = id % RCH;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src + (int64_t)(R0 + i) * ldc + C0 + c * 8);
            *reinterpret_cast<u32x4 *>(W + i * (RCH * 16) + ((c ^ (i & (RCH - 1))) << 4)) = v;
        }
    };
    if (kIn && !below) {
        // (on 256 tiles the main loop's last stages have put the sub-block
        // there already)
        if (BM != 256) stage(args.E + batch * args.c_stride);
#pragma unroll
        for (int j = 0; j < FN; ++j) da_c[j] = dIn[C0 + j * 16 + col];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) da_r[i][r] = dIn[R0 + i * 16 + quad * 4 + r];
    }
    __syncthreads();
    // the staged input at the accumulators' positions: one transposing read
    // per 16 x 16 block gives each lane its 4 rows of one column; f(i, j, in4)
    // completes block (i, j)
    auto each_block = [&](auto f) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            u32x2 e[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                e[j] = tr_read(wb + swz<RCH>(i * 16 + quad * 4 + tq, j * 16 + 4 * tp));
            // the wait is tied to the registers, so no use moves above it
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e[0]));
#pragma unroll
            for (int j = 1; j < FN; ++j) asm volatile("" : "+v"(e[j]));
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const float in4[4] = {from_el<F16>(e[j].x & 0xFFFFu), from_el<F16>(e[j].x >> 16),
                                      from_el<F16>(e[j].y & 0xFFFFu), from_el<F16>(e[j].y >> 16)};
                f(i, j, in4);
            }
        }
    };
    if (MODE == kSyrkAA && !below) {
        // b Aoff + c (acc + (dA_i + dA_j) Aoff), diagonal a + b dA_i + c (acc + dA_i^2)
        each_block([&](int i, int j, const float(&in4)[4]) __attribute__((always_inline)) {
            const int gj = C0 + j * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gi = R0 + i * 16 + quad * 4 + r;
                const float in = in4[r], v = acc[i][j][r], da_i = da_r[i][r];
                float x = cb * in + cc * (v + (da_i + da_c[j]) * in);
                if (gi == gj) x = ca + (cb * da_i + cc * (v + da_i * da_i));
                acc[i][j][r] = x;
            }
        });
    }
    if (MODE == kSymLR && !below) {
        // L R of two symmetric matrices held as off-diagonal parts and
        // diagonals (acc = Loff Roff): acc + dL_i Roff_ij + Loff_ij dR_j,
        // diagonal acc + dL_i dR_i (both off-diagonal parts are 0 there).
        // Loff (staged above) with dR_j and the diagonal here; the main loop
        // has added dL_i Roff_ij.
        const float *dR = args.dIn2 + batch * args.d_stride;
#pragma unroll
        for (int j = 0; j < FN; ++j) da_c[j] = dR[C0 + j * 16 + col];
        each_block([&](int i, int j, const float(&in4)[4]) __attribute__((always_inline)) {
            const int gj = C0 + j * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gi = R0 + i * 16 + quad * 4 + r;
                const float v = acc[i][j][r];
                acc[i][j][r] = gi == gj ? v + da_r[i][r] * da_c[j] : v + in4[r] * da_c[j];
            }
        });
    }
    __syncthreads();

    if (m0 == n0) {
        // A tile on the diagonal is its own mirror: every wave puts each
        // value above the diagonal at both its places in a tile-wide image
        // (so the mirror of each value is that same bf16 value), 0 on the
        // diagonal, whose fp32 value goes to the vector; then the workgroup
        // stores the image once, in 16-byte chunks.
        constexpr int TB = BM / 8;  // 16-byte chunks per image row
        if (!below) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int lj = C0 - m0 + j * 16 + col;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int li = R0 - m0 + i * 16 + quad * 4 + r;
                        const float x = acc[i][j][r];
                        if (li < lj) {
                            const uint16_t h = (uint16_t)pack_el(x, 0.0f, of16);
                            *reinterpret_cast<uint16_t *>(lds_all + swz<TB>(li, lj)) = h;
                            *reinterpret_cast<uint16_t *>(lds_all + swz<TB>(lj, li)) = h;
                        } else if (li == lj) {
                            dOut[m0 + li] = x;
                            *reinterpret_cast<uint16_t *>(lds_all + swz<TB>(li, li)) = 0;
                        }
                    }
                }
        }
        __syncthreads();
        const int tid = wave * 64 + lane;
        constexpr int NT = BM * BM / (FM * 16 * FN * 16) * 64;  // threads of the workgroup
#pragma unroll 4
        for (int k = tid; k < BM * TB; k += NT) {
            const int i = k / TB, c = k % TB;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(lds_all + i * (TB * 16) + ((c ^ (i & (TB - 1))) << 4));
            *reinterpret_cast<u32x4 *>(Cm + (int64_t)(m0 + i) * ldc + m0 + c * 8) = v;
        }
        return;
    }
    // off the diagonal every sub-block lies above it
    const bool coalesced = !below && !cross;
    // 2. the sub-block transposed, T[lj][li], four consecutive rows per 8-byte
    // write; it serves both stores
    if (coalesced) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                *reinterpret_cast<u32x2 *>(W + swz<TCH>(j * 16 + col, i * 16 + quad * 4)) =
                    u32x2{pack_el(acc[i][j][0], acc[i][j][1], of16), pack_el(acc[i][j][2], acc[i][j][3], of16)};
    }
    __syncthreads();
    if (coalesced) {
        // the mirror: T's rows are its rows, 16-byte chunks
#pragma unroll 4
        for (int k = 0; k < TCHUNKS / 64; ++k) {
            const int id = k * 64 + lane, i = id / TCH, c = id % TCH;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(W + i * (TCH * 16) + ((c ^ (i & (TCH - 1))) << 4));
            *reinterpret_cast<u32x4 *>(Cm + (int64_t)(C0 + i) * ldc + R0 + c * 8) = v;
        }
        // the sub-block itself, from T by transposing reads: store s covers
        // rows 16 rb .. +15 and columns 32 ch .. +31; 16-lane group q reads
        // T rows 32 ch + 8q + {0..3} and + {4..7} at columns 16 rb .. +15, so
        // lane i holds 8 consecutive columns of row 16 rb + i
#pragma unroll 4
        for (int st = 0; st < (SR / 16) * (SC / 32); ++st) {
            const int rb = st / (SC / 32), ch = st % (SC / 32);
            const int t0 = ch * 32 + quad * 8 + tq, c0 = rb * 16 + 4 * tp;
            const u32x2 lo = tr_read(wb + swz<TCH>(t0, c0));
            const u32x2 hi = tr_read(wb + swz<TCH>(t0 + 4, c0));
            u32x4 v = u32x4{lo.x, lo.y, hi.x, hi.y};
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v));
            *reinterpret_cast<u32x4 *>(Cm + (int64_t)(R0 + rb * 16 + col) * ldc + C0 + ch * 32 +
                                       quad * 8) = v;
        }
    }
}


// Slot rel of a group -> its tile t (false: a padding slot).  Workgroups go
// to the 8 XCDs round-robin (tile0 and the grid are multiples of 8).  The
// tiles resident at one time (a round) are consecutive in the banded order, a
// compact block of the tile grid, and XCD x takes the x-th contiguous eighth
// of each round: its L2 then serves few operand panels, and the XCDs together
// stream the round's panels through the shared memory-side cache.
__device__ __forceinline__ bool round_tile(const NsGroup &G, int rel, int &t) {
    const int base = rel - rel % G.round_tiles;
    const int rem = G.padded - base < G.round_tiles ? G.padded - base : G.round_tiles;
    t = base + (rel & 7) * (rem >> 3) + ((rel - base) >> 3);
    return t < G.tiles;
}

// ----------------------------------------------------------------------------
// The main loop.  K advances in stages of 32 columns through kStages LDS
// buffers of 2 x BM rows x 64 bytes.  Operands go from global memory straight
// to LDS (buffer_load ... lds, 16 bytes per lane; one wave instruction fills
// one contiguous kilobyte = 16 rows of a stage); lane l fetches the chunk that
// the XOR swizzle (chunk c of row r at slot c ^ ((r >> 1) & 3)) puts at its
// LDS slot, which keeps the 16-byte fragment reads free of bank conflicts.
// Loads run kStages - 1 stages ahead.  Stages past the end of K read from a
// zero-size buffer descriptor, so they return zeros without touching memory
// and every iteration has the same shape (no branches, fixed wait counts).
//
// Iteration kt: wait until this wave's loads of stage kt+1 have landed ->
// barrier (everyone's have; everyone has finished reading stage kt) -> issue
// the loads of stage kt + kStages into stage kt's buffer -> read the
// fragments of stage kt+1, interleaved one by one with the MFMAs of stage kt
// (whose fragments were read in the previous iteration).
constexpr int kStages = 4;
constexpr int kBK = 32;
// s_waitcnt: vmcnt <= n and lgkmcnt = 0 (gfx9 field layout: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt high bits[15:14])
#define WAIT_VM_LGKM0(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4)))

template <int BM, int MODE, bool F16>
__global__ __launch_bounds__(Cfg<BM>::WR * Cfg<BM>::WC * 64)
__attribute__((amdgpu_waves_per_eu(Cfg<BM>::WPE))) void ns_gemm_kernel(NsLaunch L) {
    static_assert(MODE == kSyrkXXT || MODE == kSyrkAA || MODE == kSymLR, "B X has a kernel of its own");
    static_assert(!(F16 && MODE == kSyrkXXT), "X is bf16");
    constexpr int WR = Cfg<BM>::WR, WC = Cfg<BM>::WC, NW = WR * WC;
    constexpr int WTM = BM / WR, WTN = BM / WC, FM = WTM / 16, FN = WTN / 16;
    constexpr int ROW = 64, OPB = BM * ROW, STAGE = 2 * OPB;
    constexpr int LOADS = OPB / 1024 / NW, LPS = 2 * LOADS;
    constexpr int ND = FM + FN;  // LDS fragment reads per stage
    constexpr int NSTG = Cfg<BM>::SYM_STAGES;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == OPB, "tile");
    static_assert(NSTG * STAGE >= BM * BM * 2, "the epilogue regions fit in the stages");
    // L R: the tile's rows of dL, 1 KiB past the stage buffers
    constexpr bool kDiagR = MODE == kSymLR;
    constexpr int DLB = NSTG * STAGE;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTG * STAGE + (kDiagR ? 1024 : 0)];

    // group, matrix and tile of this workgroup
    const int bid = blockIdx.x;
    int gi = 0;
    while (gi + 1 < L.ngroups && bid >= L.g[gi + 1].tile0) ++gi;
    const NsGroup &G = L.g[gi];
    int t;
    if (!round_tile(G, bid - G.tile0, t)) return;
    const int batch = t / G.tiles_pm;
    t -= batch * G.tiles_pm;
    int ti, tj;
    tile_coords<MODE>(G, t, ti, tj);
    const int m0 = ti * BM, n0 = tj * BM;
    const int ld = G.ld, K = G.K;
    const uint16_t *Pb = G.P + batch * G.p_stride + (int64_t)m0 * ld;
    const uint16_t *Qb = G.Q + batch * G.q_stride + (int64_t)n0 * ld;
    const int panel_bytes = BM * ld * 2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WC, wc = wave % WC;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // loads: instruction q of this wave fills kilobyte k = q * NW + wave of
    // the operand's stage (rows 16k .. 16k+15); lane l takes row 16k + l / 4
    // and the chunk that the swizzle places at slot l % 4
    const int lrow = lane >> 2, lchunk = (lane & 3) ^ ((lrow >> 1) & 3);
    const int voff = (lrow * ld + lchunk * 8) * 2;
    // A A and L R on 256 tiles: the stages past the end of K (the last four
    // iterations' loads, into the four buffers as they free up) fetch the
    // input tile Aoff[m0.., n0..] (L R: Loff) that the epilogue needs, straight into the
    // per-wave regions it reads it from (wave w's 128 x 64 sub-block, rows of
    // 128 bytes, chunk c of row i at slot c ^ (i % 8), at w x 16 KiB: the
    // buffer of stage s holds the regions of waves 2s and 2s + 1).  Kilobyte k
    // of a region is its rows 8k .. 8k+7; lane l takes row l / 8 of it and the
    // chunk the swizzle puts at slot l % 8.
    constexpr bool kEpre = (MODE == kSyrkAA || MODE == kSymLR) && BM == 256;
    static_assert(!kEpre || (NSTG == 4 && NSTG * STAGE == BM * BM * 2), "four buffers hold the input tile");
    const uint16_t *Eb = kEpre ? G.E + batch * G.c_stride + (int64_t)m0 * G.ldc + n0 : nullptr;
    const int evoff = ((lane >> 3) * G.ldc + (((lane & 7) ^ (lane >> 3)) << 3)) * 2;
    auto gload = [&](int sbase, int k0) {
        const int bytes = k0 < K ? panel_bytes : 0;
        const __amdgpu_buffer_rsrc_t rp =
            __builtin_amdgcn_make_buffer_rsrc((void *)Pb, (short)0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rq =
            __builtin_amdgcn_make_buffer_rsrc((void *)Qb, (short)0, bytes, 0x00020000);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int k = q * NW + wave;
            const int soff = (16 * k * ld + k0) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, LDS_ADDR(&lds[sbase + k * 1024]), 16, voff,
                                                     soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, LDS_ADDR(&lds[sbase + OPB + k * 1024]), 16,
                                                     voff, soff, 0, 0);
        }
    };
    // the input tile's regions of waves 2B and 2B + 1 into stage buffer B
    auto egload = [&](auto B) __attribute__((always_inline)) {
        constexpr int ow = 2 * decltype(B)::value;
        const __amdgpu_buffer_rsrc_t re =
            __builtin_amdgcn_make_buffer_rsrc((void *)Eb, (short)0, BM * G.ldc * 2, 0x00020000);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int k = q * NW + wave;
            const int sp = (((ow / WC) * WTM + 8 * k) * G.ldc + (ow % WC) * WTN) * 2;
            const int sq = ((((ow + 1) / WC) * WTM + 8 * k) * G.ldc + ((ow + 1) % WC) * WTN) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                re, LDS_ADDR(&lds[decltype(B)::value * STAGE + k * 1024]), 16, evoff, sp, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                re, LDS_ADDR(&lds[decltype(B)::value * STAGE + OPB + k * 1024]), 16, evoff, sq, 0, 0);
        }
    };
    // MFMA 16x16x32 operand: lane l holds row l % 16, K-chunk l / 16 of the
    // stage (rowbase is a multiple of 16)
    const int fr = lane & 15, fh = lane >> 4;
    const int foff = fr * ROW + ((fh ^ ((fr >> 1) & 3)) << 4);
    bf16x8 fa[2][FM], fb[2][FN];
    auto read = [&](int buf, int sbase) {
        const uint8_t *pa = &lds[sbase + wr * WTM * ROW + foff];
        const uint8_t *pb = &lds[sbase + OPB + wc * WTN * ROW + foff];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[buf][i] = *reinterpret_cast<const bf16x8 *>(pa + i * 16 * ROW);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[buf][j] = *reinterpret_cast<const bf16x8 *>(pb + j * 16 * ROW);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                if constexpr (F16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(f16x8, fa[buf][i]), __builtin_bit_cast(f16x8, fb[buf][j]),
                        acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[buf][i], fb[buf][j],
                                                                        acc[i][j], 0, 0, 0);
    };

    // L R: dL_i Roff_ij in the main loop.  R is symmetric, so the Q stage of
    // a stage whose K range [32 s, 32 s + 32) lies inside the wave's rows
    // [R0w, R0w + WTM) holds R[n0 + c][32 s + kk] = Roff[32 s + kk][n0 + c]:
    // for the wave's row blocks 2q and 2q + 1 (32 s = R0w + 32 q), lane
    // (col, quad) reads its four rows of column j in one 8-byte read and adds
    // dL_row Roff to the accumulators.  dL of the tile's rows is in LDS (wave
    // 0 loads it first, so the prologue's wait covers it).
    const int R0w = m0 + wr * WTM;
    if constexpr (kDiagR) {
        if (wave == 0) {
            const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(G.dIn + batch * G.d_stride + m0), (short)0, BM * 4, 0x00020000);
            // (lanes past BM / 4 read zeros into the rest of the 1 KiB)
            const int lo16 = lane * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, LDS_ADDR(&lds[DLB]), 16, lo16, 0, 0, 0);
        }
    }
    // (one case per 32-row slice q, each with a marker of its own, so that
    // the cases are not merged into one with a run-time index into acc,
    // which would put acc in scratch memory)
    auto diagq = [&](auto Q, int k0, int sbase) __attribute__((always_inline)) {
        constexpr int q = decltype(Q)::value;
        if (k0 != q * kBK) return;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
            const int i = 2 * q + ii;
            const f32x4 dl = *reinterpret_cast<const f32x4 *>(&lds[DLB + (wr * WTM + i * 16 + fh * 4) * 4]);
            u32x2 qv[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wc * WTN + j * 16 + fr, ch = ii * 2 + (fh >> 1);
                qv[j] = *reinterpret_cast<const u32x2 *>(
                    &lds[sbase + OPB + row * ROW + ((ch ^ ((row >> 1) & 3)) << 4) + (fh & 1) * 8]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j][0] += dl[0] * from_el<F16>(qv[j].x & 0xFFFFu);
                acc[i][j][1] += dl[1] * from_el<F16>(qv[j].x >> 16);
                acc[i][j][2] += dl[2] * from_el<F16>(qv[j].y & 0xFFFFu);
                acc[i][j][3] += dl[3] * from_el<F16>(qv[j].y >> 16);
            }
        }
        asm volatile("; diag R slice %0" : : "n"(q));
    };
    auto diagR = [&](int s, int sbase) __attribute__((always_inline)) {
        const int k0 = s * kBK - R0w;
        static_assert(WTM / kBK >= 1 && WTM / kBK <= 4, "one to four 32-row slices per wave");
        diagq(std::integral_constant<int, 0>{}, k0, sbase);
        if constexpr (WTM / kBK > 1) diagq(std::integral_constant<int, 1>{}, k0, sbase);
        if constexpr (WTM / kBK > 2) diagq(std::integral_constant<int, 2>{}, k0, sbase);
        if constexpr (WTM / kBK > 3) diagq(std::integral_constant<int, 3>{}, k0, sbase);
    };
    // a wave whose sub-tile of a diagonal tile lies wholly below the diagonal
    // computes nothing the epilogue stores: it only loads and synchronises
    const bool dead = m0 == n0 && wr * WTM >= wc * WTN + WTN;

    const int KT = K / kBK;
#pragma unroll
    for (int s = 0; s < NSTG; ++s) gload(s * STAGE, s * kBK);
    __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM0((NSTG - 1) * LPS));
    __syncthreads();
    read(0, 0);
    if constexpr (kDiagR)
        if (!dead) diagR(0, 0);
    int cur = 0;  // buffer of stage kt
    // (TAIL >= 0: one of the last NSTG stages of a 256-tile A A, whose
    // buffer TAIL receives the input tile's regions instead of zeros)
    auto body = [&](int kt, auto PAR, auto LIVE, auto TAIL) __attribute__((always_inline)) {
        constexpr int par = decltype(PAR)::value;
        const int nxt = cur + 1 == NSTG ? 0 : cur + 1;
        __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM0((NSTG - 2) * LPS));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(TAIL)::value >= 0)
            egload(TAIL);
        else
            gload(cur * STAGE, (kt + NSTG) * kBK);
        if constexpr (decltype(LIVE)::value) {
        read(par ^ 1, nxt * STAGE);
        mma(par);
        }
#pragma unroll
        for (int x = 0; x < LPS; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
        }
#pragma unroll
        for (int x = 0; x < ND; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kDiagR && decltype(LIVE)::value) diagR(kt + 1, nxt * STAGE);
        cur = nxt;
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using NT = std::integral_constant<int, -1>;
    auto kloop = [&](auto LIVE) __attribute__((always_inline)) {
        int kt = 0;
        if constexpr (kEpre) {
            // K is a multiple of 256: the last four stages are stages 0 .. 3
            // of the buffers (cur = kt % 4)
#pragma clang loop unroll(disable)
            for (; kt + NSTG < KT; kt += 2) {
                body(kt, P0{}, LIVE, NT{});
                body(kt + 1, P1{}, LIVE, NT{});
            }
            body(kt, P0{}, LIVE, std::integral_constant<int, 0>{});
            body(kt + 1, P1{}, LIVE, std::integral_constant<int, 1>{});
            body(kt + 2, P0{}, LIVE, std::integral_constant<int, 2>{});
            body(kt + 3, P1{}, LIVE, std::integral_constant<int, 3>{});
        } else {
            // two stages per trip, so that the fragment buffer of each is static
#pragma clang loop unroll(disable)
            for (; kt + 2 <= KT; kt += 2) {
                body(kt, P0{}, LIVE, NT{});
                body(kt + 1, P1{}, LIVE, NT{});
            }
            if (kt < KT) body(kt, P0{}, LIVE, NT{});
        }
    };
    if (dead)
        kloop(std::false_type{});
    else
        kloop(std::true_type{});
    // the loads past the end still write (zeros) to LDS: drain them before
    // the epilogue reuses the buffers
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    epilogue<MODE, BM, FM, FN, F16>(G, L.a, L.b, L.c, acc, batch, m0, n0, m0 + wr * WTM, n0 + wc * WTN,
                               wave, lane, lds);
}

// ----------------------------------------------------------------------------
// X' = a X + B X: a persistent kernel.  The grid is one round of resident
// workgroups; workgroup w takes slots w, w + grid, w + 2 grid, ... (the
// slot -> tile map is the one above, so the tiles in flight at one time are
// still one compact round).  The stage pipeline runs on across tiles: when a
// tile's last stages are in flight the loads go on with the next tile's first
// ones, and the last stage's fragment reads are the next tile's first.  So
// the next tile's operands arrive while this one computes and stores, and no
// workgroup idles through a prologue (its stores, which vmcnt counts with the
// loads, are waited for at the next tile's first stage).
//
// P = B (its rows [m0, m0 + BM), K = m); Q = X, staged k-major: rows
// [k, k + 32) x columns [n0, n0 + BM) as they lie in memory (rows of QRB
// bytes; 32-byte unit u of row r at slot u ^ qsw(r)).  The MFMA B operand (8
// consecutive k of one column per lane) is two ds_read_b64_tr_b16 per 16 x 32
// fragment: lane 4q + p of a 16-lane group addresses row +q, columns
// 4p .. 4p+3 of a 4 x 16 block, and lane i receives rows +0..+3 of column i.
// A transposing read touches 16 rows x 32 bytes, and qsw spreads them over
// all eight 32-byte bank groups, two rows each (rows of 512 or 256 bytes
// start in the same banks; rows of 128 bytes alternate halves).
//
// The MFMA takes X's fragment as its first operand and B's as its second, so
// it accumulates the tile transposed: lane (c, q) = (l % 16, l / 16) of block
// (i, j) holds row 16i + c, columns 16j + 4q .. 16j + 4q + 3 of X'.  Four
// consecutive columns of one row pack into one 8-byte store, so the tile
// goes from registers straight to memory (no LDS staging, no barrier).
//
// (a + dB_i) X_ij: the Q stage of the stages whose K range [k1, k1 + 32)
// lies inside the wave's rows holds exactly X's rows of that range, so those
// stages add (a + dB_row) X[row][cols] to the two 16-row blocks there (one
// 8-byte read per block and lane), instead of reading X again in the
// epilogue.  dB for a tile's rows is copied into LDS (one of two buffers)
// while the tile before it runs.
//
// A launch whose groups all have K >= kStages * 32 runs the pipeline across
// tiles; otherwise each tile starts its own (the loads past its end read a
// zero-size buffer, as in the kernel above).
//
// (The LDS reads of X and dB are inline assembly: as ordinary LDS loads the
// compiler cannot tell them from the in-flight global->LDS copies into other
// buffers and would wait for those copies to finish.  Their results are tied
// to the next explicit wait.)
template <int BM>
__global__ __launch_bounds__(Cfg<BM>::WR * Cfg<BM>::WC * 64)
__attribute__((amdgpu_waves_per_eu(Cfg<BM>::WPE))) void ns_bx_kernel(NsLaunch L) {
    constexpr int WR = Cfg<BM>::WR, WC = Cfg<BM>::WC, NW = WR * WC;
    constexpr int WTM = BM / WR, WTN = BM / WC, FM = WTM / 16, FN = WTN / 16;
    constexpr int ROW = 64, OPB = BM * ROW, STAGE = 2 * OPB;
    constexpr int LOADS = OPB / 1024 / NW, LPS = 2 * LOADS;
    constexpr int QRB = 2 * BM, QCH = QRB / 16;
    constexpr int DLB = kStages * STAGE;  // two 1 KiB buffers of dB
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == OPB, "tile");
    static_assert(BM * 4 <= 1024, "dB rows fit a buffer");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * STAGE + 2048];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / WC, wc = wave % WC;
    const int grid = gridDim.x;
    const uint32_t lds_base =
        (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds);

    // The lane's index, computed afresh where it is used between tiles or
    // seldom, so that the values derived from it need no register across
    // the loops.
    auto lane_id = []() __attribute__((always_inline)) {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        return l;
    };
    struct Tile {
        int gi, batch, m0, n0;
    };
    // slot -> tile (false: a padding slot)
    auto locate = [&](int slot, Tile &T) __attribute__((always_inline)) -> bool {
        int gi = 0;
        while (gi + 1 < L.ngroups && slot >= L.g[gi + 1].tile0) ++gi;
        const NsGroup &G = L.g[gi];
        int t;
        if (!round_tile(G, slot - G.tile0, t)) return false;
        const int batch = t / G.tiles_pm;
        t -= batch * G.tiles_pm;
        int ti, tj;
        tile_coords<kGemmBX>(G, t, ti, tj);
        T = Tile{gi, batch, ti * BM, tj * BM};
        return true;
    };
    // this workgroup's first tile at or after `slot`; -1 if none
    auto seek = [&](int slot, Tile &T) __attribute__((always_inline)) -> int {
        for (; slot < L.total; slot += grid)
            if (locate(slot, T)) return slot;
        return -1;
    };

    // The load stream: stage ks (counted from the current tile's first)
    // comes from stage ks - sk of the stream's tile, or is zeros (!live).
    // Instruction q of this wave fills kilobyte k = q * NW + wave of each
    // operand's stage.  P: rows 16k .. 16k+15; lane l takes row 16k + l / 4
    // and the chunk that the swizzle (chunk c of row r at slot c ^ ((r >> 1)
    // & 3)) places at slot l % 4.  Q: kilobyte k holds stage rows
    // k * 1024 / QRB ...; lane l fills 16-byte slot l % QCH of row l / QCH.
    auto qsw = [](int r) __attribute__((always_inline)) {
        return BM >= 128 ? (r & 3) | (((r >> 3) & 1) << 2) : ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
    };
    const uint16_t *sP = nullptr, *sQ = nullptr;
    int sld = 0, sldq = 0, sk = 0;
    bool slive = false;
    int voff = 0, qv[LOADS];
    auto stream = [&](const Tile &T, int kbase, bool live) __attribute__((always_inline)) {
        const NsGroup &G = L.g[T.gi];
        sld = G.ld;
        sldq = G.ldq;
        sP = G.P + T.batch * G.p_stride + (int64_t)T.m0 * sld;
        sQ = G.Q + T.batch * G.q_stride + T.n0;
        sk = kbase;
        slive = live;
        const int ln = lane_id();
        const int lrow = ln >> 2, lchunk = (ln & 3) ^ ((lrow >> 1) & 3);
        voff = (lrow * sld + lchunk * 8) * 2;
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int r = (q * NW + wave) * (1024 / QRB) + ln / QCH, s16 = ln % QCH;
            qv[q] = (r * sldq + (((s16 >> 1) ^ qsw(r)) << 4) + ((s16 & 1) << 3)) * 2;
        }
    };
    auto gload = [&](int sbase, int ks) __attribute__((always_inline)) {
        const int k0 = (ks - sk) * kBK;
        const __amdgpu_buffer_rsrc_t rp =
            __builtin_amdgcn_make_buffer_rsrc((void *)sP, (short)0, slive ? BM * sld * 2 : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(sQ + (int64_t)k0 * sldq), (short)0, slive ? kBK * sldq * 2 : 0, 0x00020000);
#pragma unroll
        for (int q = 0; q < LOADS; ++q) {
            const int k = q * NW + wave;
            const int soff = (16 * k * sld + k0) * 2;
            const int qo = qv[q];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, LDS_ADDR(&lds[sbase + k * 1024]), 16, voff,
                                                     soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, LDS_ADDR(&lds[sbase + OPB + k * 1024]), 16,
                                                     qo, 0, 0, 0);
        }
    };
    // dB of tile T's rows into dB buffer `which` (wave 0, one instruction;
    // lanes past BM / 4 read zeros)
    auto load_db = [&](int which, const Tile &T) __attribute__((always_inline)) {
        if (wave == 0) {
            const NsGroup &G = L.g[T.gi];
            const float *src = G.dIn + T.batch * G.d_stride + T.m0;
            const __amdgpu_buffer_rsrc_t rd =
                __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, BM * 4, 0x00020000);
            // (a plain local as the offset operand: the host pass drops the
            // kernel's stub for some argument expressions)
            const int lo16 = lane_id() * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, LDS_ADDR(&lds[DLB + which * 1024]), 16,
                                                     lo16, 0, 0, 0);
        }
    };

    // MFMA 16x16x32 operand of B: lane l holds row l % 16, K-chunk l / 16
    const int fr = lane & 15, fh = lane >> 4;
    const int foff = fr * ROW + ((fh ^ ((fr >> 1) & 3)) << 4);
    bf16x8 fa[2][FM], fb[2][FN];
    // X's operand of column block j, K-chunk g = lane / 16: two transposing
    // reads of 4 x 16 blocks, rows 8g + {0..3} and 8g + {4..7} (qsw is the
    // same for both, so the second is the first plus 4 rows)
    auto unit = [&](int r, int j) __attribute__((always_inline)) {
        return r * QRB + ((((wc * WTN) / 16 + j) ^ qsw(r)) << 5);
    };
    int qro[FN];
    {
        const int tg = lane >> 4, tq = (lane >> 2) & 3, tp = lane & 3;
        const int tpo = ((tp >> 1) << 4) + ((tp & 1) << 3);
#pragma unroll
        for (int j = 0; j < FN; ++j) qro[j] = unit(8 * tg + tq, j) + tpo;
    }
    auto read_a = [&](int buf, int sbase, int i) __attribute__((always_inline)) {
        fa[buf][i] = *reinterpret_cast<const bf16x8 *>(&lds[sbase + wr * WTM * ROW + foff + i * 16 * ROW]);
    };
    auto read_b = [&](int buf, int sbase) __attribute__((always_inline)) {
        const uint32_t qb = lds_base + sbase;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            u32x2 lo, hi;
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(qb + qro[j]), "i"(OPB));
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(hi) : "v"(qb + qro[j]), "i"(OPB + 4 * QRB));
            fb[buf][j] = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
        }
    };
    auto read = [&](int buf, int sbase) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i) read_a(buf, sbase, i);
        read_b(buf, sbase);
    };
    f32x4 acc[FM][FN];
    auto mma = [&](int par) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[par][j], fa[par][i], acc[i][j],
                                                                    0, 0, 0);
    };
    // (a + dB_row) X[row][cols] for the stage at sbase, K range [k1, k1 + 32):
    // its rows are the wave's 16-row blocks I and I + 1.  Lane (c, q) reads
    // 8 bytes of stage row 16h + c (h = 0, 1) in 32-byte unit
    // (wc WTN / 16 + j) ^ qsw(c) = (wc WTN / 16) ^ qsw(c) ^ j (qsw(16 + c) =
    // qsw(c); the wave's first unit has no bits below j's), i.e. at
    // xb ^ (j << 5) + sbase, and dB of its row.  The addresses are formed in
    // the assembly, so that they take no registers between uses.
    const uint32_t xb = lds_base + OPB + fr * QRB + fh * 8 + ((((wc * WTN) / 16) ^ qsw(fr)) << 5);
    auto diag_pair = [&](auto I, int sbase, int dbuf) __attribute__((always_inline)) {
        constexpr int i0 = decltype(I)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float db;
            u32x2 xv[FN];
            const uint32_t da = lds_base + DLB + dbuf * 1024 + (wr * WTM + (lane_id() & 15)) * 4;
            asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(db) : "v"(da), "i"((i0 + h) * 64));
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                uint32_t t;
                asm volatile("v_xor_b32 %1, %2, %3\n\tv_add_u32 %1, %4, %1\n\tds_read_b64 %0, %1 offset:%5"
                             : "=v"(xv[j]), "=&v"(t)
                             : "i"(j << 5), "v"(xb), "s"(sbase), "i"(h * 16 * QRB));
            }
            // the wait is tied to the registers, so no use moves above it
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(db));
            const float d = db;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                asm volatile("" : "+v"(xv[j]));
                acc[i0 + h][j][0] += d * from_bf16(xv[j].x & 0xFFFFu);
                acc[i0 + h][j][1] += d * from_bf16(xv[j].x >> 16);
                acc[i0 + h][j][2] += d * from_bf16(xv[j].y & 0xFFFFu);
                acc[i0 + h][j][3] += d * from_bf16(xv[j].y >> 16);
            }
        }
        // (distinct per case, so that the cases' updates are not merged into
        // one through pointers, which would put acc in scratch memory)
        asm volatile("; diag %0" : : "n"(i0));
    };
    auto diag = [&](int sbase, int k1, const Tile &cu, int dbuf) __attribute__((always_inline)) {
        const int rel = k1 - (cu.m0 + wr * WTM);
        if (rel < 0 || rel >= WTM) return;
        switch (rel >> 5) {
            case 0: diag_pair(std::integral_constant<int, 0>{}, sbase, dbuf); break;
            case 1: if constexpr (FM > 2) diag_pair(std::integral_constant<int, 2>{}, sbase, dbuf); break;
            case 2: if constexpr (FM > 4) diag_pair(std::integral_constant<int, 4>{}, sbase, dbuf); break;
            case 3: if constexpr (FM > 6) diag_pair(std::integral_constant<int, 6>{}, sbase, dbuf); break;
        }
    };
    // the tile from registers: 8-byte row stores, and for X'^T (when wanted)
    // 2-byte stores down its columns; buffer stores off the wave's corner of
    // the tile, so a store needs one lane offset and a scalar one
    auto store = [&](const Tile &cu) __attribute__((always_inline)) {
        const NsGroup &G = L.g[cu.gi];
        const int R0 = cu.m0 + wr * WTM, C0 = cu.n0 + wc * WTN;
        const int ldc = G.ldc;
        const int ln = lane_id(), fr = ln & 15, fh = ln >> 4;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(G.C + cu.batch * G.c_stride + (int64_t)R0 * ldc + C0), (short)0, WTM * ldc * 2,
            0x00020000);
        const int vo = (fr * ldc + fh * 4) * 2;
        if (G.xs != nullptr) {
            // first iteration: X' = (a + dB) (s U) + Boff (s U) from the products of U
            const float s = G.xs[cu.batch];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] *= s;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{cvt_pk_bf16(acc[i][j][0], acc[i][j][1]), cvt_pk_bf16(acc[i][j][2], acc[i][j][3])},
                    rc, vo + j * 32, i * 32 * ldc, 0);
        if (G.CT != nullptr) {
            const int ldt = G.ldct;
            const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(G.CT + cu.batch * G.ct_stride + (int64_t)C0 * ldt + R0), (short)0,
                WTN * ldt * 2, 0x00020000);
            const int to = (fh * 4 * ldt + fr) * 2;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            (uint16_t)cvt_pk_bf16(acc[i][j][r], 0.0f), rt, to + i * 32,
                            (j * 16 + r) * ldt * 2, 0);
        }
    };

    Tile cu, nx{};
    int slot = seek(blockIdx.x, cu);
    if (slot < 0) return;
    int cur = 0;        // LDS buffer of the current stage
    int dbuf = 0;       // dB buffer of the current tile
    bool pref = false;  // the current tile's first stages are in flight
    load_db(0, cu);
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (;;) {
        const int KT = L.g[cu.gi].K / kBK;  // even: K is a multiple of the tile
        const int ksw = KT - kStages;       // from stage ksw on, loads fetch the next tile
        // the next tile, and its dB rows into the other buffer (everyone is
        // past the previous tile's last reads of that buffer)
        int nslot = -1;
        bool more = false, pf = false;
        auto find_next = [&]() __attribute__((always_inline)) {
            nslot = seek(slot + grid, nx);
            more = nslot >= 0;
            if (!more) nx = cu;
            pf = more && L.xpf != 0;
            if (more) load_db(dbuf ^ 1, nx);
        };
        find_next();
        if (!pref) {
            // this tile's own prologue (everyone is done with the buffers)
            __syncthreads();
            stream(cu, 0, true);
#pragma unroll
            for (int s = 0; s < kStages; ++s) {
                if (s == KT) stream(nx, KT, pf);
                gload(((cur + s) & (kStages - 1)) * STAGE, s);
            }
            __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM0((kStages - 1) * LPS));
            __syncthreads();
            read(0, cur * STAGE);
        }
        // (zeros made in place: a zero vector kept for this would be one
        // more register across the loops)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) asm volatile("v_mov_b32 %0, 0" : "=v"(acc[i][j][r]));
        // Stage kt: its (a + dB) X term, while its buffer still holds it ->
        // wait until this wave's loads of stage kt+1 have landed -> barrier
        // (everyone's have; everyone has finished reading stage kt) -> issue
        // the loads kStages stages ahead into stage kt's buffer -> read the
        // fragments of stage kt+1, interleaved with the MFMAs of stage kt
        // (read in the previous stage).
        // (the last stage reads the fragments of the stage after: the next
        // tile's first, or zeros)
        auto body = [&](int kt, auto PAR) __attribute__((always_inline)) {
            constexpr int par = decltype(PAR)::value;
            const int nxt = (cur + 1) & (kStages - 1);
            diag(cur * STAGE, kt * kBK, cu, dbuf);
            __builtin_amdgcn_s_waitcnt(WAIT_VM_LGKM0((kStages - 2) * LPS));
            // tie: the X operands read by inline assembly in the previous
            // stage are complete only after the wait above
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[par][j]));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            gload(cur * STAGE, kt + kStages);
            read(par ^ 1, nxt * STAGE);
            mma(par);
#pragma unroll
            for (int x = 0; x < LPS; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
            }
#pragma unroll
            for (int x = 0; x < FM + 2 * FN; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
        };
        // stages whose loads fetch this tile's own stages, then (from ksw on)
        // the next tile's first ones or zeros
        int kt = 0;
#pragma clang loop unroll(disable)
        for (; kt < ksw; kt += 2) {
            body(kt, P0{});
            body(kt + 1, P1{});
        }
        if (ksw >= 0) stream(nx, KT, pf);
#pragma clang loop unroll(disable)
        for (; kt < KT; kt += 2) {
            body(kt, P0{});
            body(kt + 1, P1{});
        }
        if (!pf) {
            // the loads past the end still write (zeros) to LDS: drain them
            // before the buffers are reused; the last stage's X operands
            // (zeros, never used) stay allocated until then, so their late
            // returns cannot land on other values
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" : : "v"(fb[0][j]));
        }
        store(cu);
        if (!more) break;
        sk -= KT;
        cu = nx;
        slot = nslot;
        dbuf = __builtin_amdgcn_readfirstlane(dbuf ^ 1);
        pref = pf;
    }
}

template <int T>
constexpr int kThreadsOf = Cfg<T>::WR * Cfg<T>::WC * 64;

// One launch's share of a group: its matrices [b0, b0 + nb), one product of
// a program step (pool slots in1, in2 -> out) in segment seg.
struct LaunchPart {
    int ref, b0, nb;
    int split = 0, nsplit = 1;  // X X^T: part `split` of the group's K split in nsplit
    int in1 = 0, in2 = 0, out = 0;
    int seg = 0;
    bool last = false;  // the step is in the group's last segment
    bool in_f16 = false, out_f16 = false;  // symmetric operands / output in fp16
};

// The operands of a part (X in the x buffer in even segments, in xt0 in odd
// ones; the other receives X').
NsGroup product_group(int mode, const NsGroupRef &r, const LaunchPart &p, int tile) {
    const MuonGeom &g = *r.geom;
    const MuonWorkspace &L = *r.layout;
    char *ws = r.base;
    const int b0 = p.b0;
    uint16_t *X = reinterpret_cast<uint16_t *>(ws + ((p.seg & 1) ? L.xt0 : L.x));
    uint16_t *Xn = reinterpret_cast<uint16_t *>(ws + ((p.seg & 1) ? L.x : L.xt0));
    uint16_t *XTout = reinterpret_cast<uint16_t *>(ws + L.xt1);
    auto sm = [&](int k) { return reinterpret_cast<uint16_t *>(ws + L.sm[k]); };
    auto sd = [&](int k) { return reinterpret_cast<float *>(ws + L.sd[k]); };
    const int64_t ds = (int64_t)(L.d_stride / 4);
    const int64_t xs = (int64_t)(L.x_stride / 2), as = (int64_t)(L.a_stride / 2);
    const int tm = g.mp / tile, tn = g.np / tile;
    NsGroup s{};
    s.d_stride = ds;
    s.tiles_m = tm;
    if (mode == kSyrkXXT) {
        s.P = X; s.Q = X; s.p_stride = xs; s.q_stride = xs; s.ld = g.np; s.K = g.np;
        s.tiles_n = tm; s.tiles_pm = tm * (tm + 1) / 2;
        s.C = sm(p.out); s.c_stride = as; s.ldc = g.mp;
        s.dIn = sd(p.out); s.dOut = sd(p.out);
    } else if (mode == kSyrkAA || mode == kSymLR) {
        s.P = sm(p.in1); s.Q = sm(mode == kSyrkAA ? p.in1 : p.in2);
        s.p_stride = as; s.q_stride = as; s.ld = g.mp; s.K = g.mp;
        s.tiles_n = tm; s.tiles_pm = tm * (tm + 1) / 2;
        s.C = sm(p.out); s.c_stride = as; s.ldc = g.mp;
        s.E = sm(p.in1);  // A A: Aoff; L R: Loff (the epilogue's staged input)
        s.dIn = sd(p.in1); s.dOut = sd(p.out);
        if (mode == kSymLR) s.dIn2 = sd(p.in2);
    } else {
        s.P = sm(p.in1); s.Q = X; s.p_stride = as; s.q_stride = xs; s.ld = g.mp; s.K = g.mp;
        s.ldq = g.np;
        s.tiles_n = tn; s.tiles_pm = tm * tn;
        s.C = Xn; s.c_stride = xs; s.ldc = g.np;
        s.CT = (p.last && g.transposed) ? XTout : nullptr; s.ct_stride = xs; s.ldct = g.mp;
        s.dIn = sd(p.in1); s.dOut = sd(p.in1);
    }
    if (p.seg == 0 && (mode == kSyrkXXT || mode == kGemmBX)) s.xs = muon_scale_ptr(ws, g, L) + b0;
    s.out_f16 = p.out_f16 ? 1 : 0;
    if (mode == kSyrkXXT && p.nsplit > 1) {
        // K range [split K / nsplit, (split + 1) K / nsplit) of X's columns;
        // s is applied by the fix-up, to the sum of the parts
        const int kp = g.np / p.nsplit;
        s.P += (int64_t)p.split * kp;
        s.Q += (int64_t)p.split * kp;
        s.K = kp;
        s.part_stride = (int64_t)g.mp * g.mp;
        s.part = reinterpret_cast<float *>(ws + L.part) +
                 (int64_t)p.split * g.batch * s.part_stride + b0 * s.part_stride;
        s.xs = nullptr;
    }
    // matrices from b0 on
    s.P += b0 * s.p_stride;
    s.Q += b0 * s.q_stride;
    s.C += b0 * s.c_stride;
    if (s.E) s.E += b0 * s.c_stride;
    if (s.CT) s.CT += b0 * s.ct_stride;
    s.dIn += b0 * s.d_stride;
    if (s.dIn2) s.dIn2 += b0 * s.d_stride;
    s.dOut += b0 * s.d_stride;
    return s;
}

// Workgroups of the T-tile kernel (B X, or the symmetric products) that the
// device holds at once.
template <int T>
int round_tiles_of(bool sym = false) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
        cus = 256;
    const int per_cu = (sym ? Cfg<T>::SYM_WPE : Cfg<T>::WPE) * 4 / (Cfg<T>::WR * Cfg<T>::WC);
    return (cus / 8) * per_cu * 8;
}

// Process-wide cap on the workgroups a persistent launch keeps resident (0:
// one full round of the device).
std::atomic<int> g_workgroup_limit{0};

template <int T>
int32_t bx_round_tiles() {
    int32_t r = round_tiles_of<T>();
    const int lim = g_workgroup_limit.load(std::memory_order_relaxed);
    return lim > 0 && lim < r ? lim : r;
}

template <int T, int MODE, bool F16>
hipError_t launch_product(const NsGroupRef *refs, const LaunchPart *parts, int n, float a,
                          float b, float c, hipStream_t stream) {
    const int32_t round_tiles = MODE == kGemmBX ? bx_round_tiles<T>() : round_tiles_of<T>(true);
    for (int first = 0; first < n; first += kMaxGroups) {
        const int cnt = n - first < kMaxGroups ? n - first : kMaxGroups;
        NsLaunch L{};
        L.a = a;
        L.b = b;
        L.c = c;
        L.ngroups = cnt;
        int64_t tiles = 0;
        for (int k = 0; k < cnt; ++k) {
            const LaunchPart &p = parts[first + k];
            NsGroup s = product_group(MODE, refs[p.ref], p, T);
            s.tiles = s.tiles_pm * p.nb;
            s.padded = (s.tiles + 7) / 8 * 8;
            s.round_tiles = round_tiles;
            s.tile0 = (int32_t)tiles;
            tiles += s.padded;
            L.g[k] = s;
        }
        if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
        L.total = (int32_t)tiles;
        if constexpr (MODE == kGemmBX) {
            L.xpf = 1;
            for (int k = 0; k < cnt; ++k) L.xpf &= L.g[k].K >= kStages * kBK ? 1 : 0;
            const int64_t grid = tiles < round_tiles ? tiles : round_tiles;
            hipLaunchKernelGGL((ns_bx_kernel<T>), dim3((uint32_t)grid), dim3(kThreadsOf<T>), 0, stream,
                               L);
        } else {
            hipLaunchKernelGGL((ns_gemm_kernel<T, MODE, F16>), dim3((uint32_t)tiles),
                               dim3(kThreadsOf<T>), 0, stream, L);
        }
    }
    return hipGetLastError();
}

// The parts whose tile size for the product is T, longest reduction first
// so that the short tiles fill the last rounds.
template <int T, int MODE>
int product_parts(const NsGroupRef *refs, const LaunchPart *all, int nall, LaunchPart *parts) {
    int n = 0;
    for (int i = 0; i < nall; ++i) {
        const MuonGeom &g = *refs[all[i].ref].geom;
        if ((MODE == kGemmBX ? g.tile_bx : g.tile) == T) parts[n++] = all[i];
    }
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0; --j) {
            const MuonGeom &p = *refs[parts[j - 1].ref].geom, &q = *refs[parts[j].ref].geom;
            const int kp = MODE == kSyrkXXT ? p.np / parts[j - 1].nsplit : p.mp,
                      kq = MODE == kSyrkXXT ? q.np / parts[j].nsplit : q.mp;
            if (kp >= kq) break;
            const LaunchPart t = parts[j - 1];
            parts[j - 1] = parts[j];
            parts[j] = t;
        }
    return n;
}

template <int MODE, bool F16 = false>
hipError_t run_mode(const NsGroupRef *refs, const LaunchPart *all, int nall, float a, float b,
                    float c, hipStream_t stream) {
    LaunchPart p256[2 * kMaxCallGroups], p128[2 * kMaxCallGroups + 1], p64[2 * kMaxCallGroups];
    int n256 = product_parts<256, MODE>(refs, all, nall, p256);
    int n128 = product_parts<128, MODE>(refs, all, nall, p128);
    const int n64 = product_parts<64, MODE>(refs, all, nall, p64);
    if (MODE == kGemmBX && n256 > 0) {
        // The 256-tile launch's last round: when only a few tiles are left for
        // it, the last group's trailing matrices go to the 128-tile launch
        // instead (the same arithmetic on smaller tiles: results are the same
        // bit for bit), if that saves a round of 256 tiles for at most one
        // round of 128 tiles, which take ~0.6 of the time.
        auto tiles = [&](const LaunchPart *p, int n, int t) {
            int64_t s = 0;
            for (int i = 0; i < n; ++i) {
                const MuonGeom &g = *refs[p[i].ref].geom;
                s += (int64_t)(g.mp / t) * (g.np / t) * p[i].nb;
            }
            return s;
        };
        const int64_t r256 = bx_round_tiles<256>(), r128 = bx_round_tiles<128>();
        const int64_t t256 = tiles(p256, n256, 256), t128 = tiles(p128, n128, 128);
        const int64_t rounds = (t256 + r256 - 1) / r256, rem = t256 - (rounds - 1) * r256;
        LaunchPart &lp = p256[n256 - 1];
        const MuonGeom &g = *refs[lp.ref].geom;
        const int64_t q = (int64_t)(g.mp / 256) * (g.np / 256);  // 256-tiles per matrix
        const int64_t m = (rem + q - 1) / q;                        // matrices to move
        const int64_t r128_before = (t128 + r128 - 1) / r128;
        const int64_t r128_after = (t128 + 4 * q * m + r128 - 1) / r128;
        if (rounds > 1 && rem * 4 <= r256 && m < lp.nb && r128_after - r128_before <= 1 &&
            n128 < 2 * kMaxCallGroups + 1) {
            LaunchPart mv = lp;
            mv.b0 = lp.b0 + lp.nb - (int)m;
            mv.nb = (int)m;
            p128[n128++] = mv;
            lp.nb -= (int)m;
        }
    }
    hipError_t e = hipSuccess;
    if (n256 > 0) e = launch_product<256, MODE, F16>(refs, p256, n256, a, b, c, stream);
    if (e == hipSuccess && n128 > 0)
        e = launch_product<128, MODE, F16>(refs, p128, n128, a, b, c, stream);
    if (e == hipSuccess && n64 > 0)
        e = launch_product<64, MODE, F16>(refs, p64, n64, a, b, c, stream);
    return e;
}

// X X^T of a group split along K: A from the ksplit fp32 parts, summed in
// part order, times s^2 in the first iteration -- the same values the
// unsplit epilogue forms from its accumulators -- with A's off-diagonal
// entries in bf16 on both sides of the diagonal, its diagonal 0 and the
// diagonal's fp32 values in dA.  One workgroup per 64 x 64 block on or above
// the diagonal (blockIdx.y: matrix); the mirror goes through LDS so that both
// stores are row runs.
__global__ __launch_bounds__(256) void ns_xxt_fixup_kernel(const float *__restrict__ part,
                                                           int64_t part_stride, int nsplit,
                                                           int mp, int batch,
                                                           const float *__restrict__ xs,
                                                           uint16_t *__restrict__ A,
                                                           int64_t a_stride, float *__restrict__ dA,
                                                           int64_t d_stride, int out_f16) {
    __shared__ uint16_t tt[64][64 + 2];
    const int nb = mp / 64;
    int t = blockIdx.x, bi = 0;
    while (t >= nb - bi) {
        t -= nb - bi;
        ++bi;
    }
    const int bj = bi + t;
    const int b = blockIdx.y;
    const float s = xs ? xs[b] : 1.0f, s2 = s * s;
    const int c = threadIdx.x & 63, rq = threadIdx.x >> 6;
    uint16_t *Am = A + b * a_stride;
    float *dm = dA + b * d_stride;
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
        const int r = rq * 16 + k;
        const int gi = bi * 64 + r, gj = bj * 64 + c;
        const int64_t o = (int64_t)b * part_stride + (int64_t)gi * mp + gj;
        float v = part[o];
        for (int p = 1; p < nsplit; ++p) v += part[o + (int64_t)p * batch * part_stride];
        if (xs) v *= s2;
        if (gi < gj) {
            const uint16_t h = (uint16_t)pack_el(v, 0.0f, out_f16 != 0);
            Am[(int64_t)gi * mp + gj] = h;
            tt[c][r] = h;
        } else if (gi == gj) {
            dm[gi] = v;
            Am[(int64_t)gi * mp + gi] = 0;
        }
    }
    __syncthreads();
    // the mirror: row gj of A, columns gi < gj of this block
    const int mr = threadIdx.x >> 2, c0 = (threadIdx.x & 3) * 16;
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
        const int gi = bi * 64 + c0 + k, gj = bj * 64 + mr;
        if (gi < gj) Am[(int64_t)gj * mp + gi] = tt[mr][c0 + k];
    }
}

hipError_t launch_xxt_fixups(const NsGroupRef *refs, const LaunchPart *all, int nall,
                             hipStream_t stream) {
    for (int i = 0; i < nall; ++i) {
        const LaunchPart &p = all[i];
        if (p.nsplit < 2 || p.split != 0) continue;
        const MuonGeom &g = *refs[p.ref].geom;
        const MuonWorkspace &L = *refs[p.ref].layout;
        char *ws = refs[p.ref].base;
        const int nb = g.mp / 64;
        const float *xs = p.seg == 0 ? muon_scale_ptr(ws, g, L) : nullptr;
        hipLaunchKernelGGL(ns_xxt_fixup_kernel, dim3(nb * (nb + 1) / 2, g.batch), dim3(256), 0,
                           stream, reinterpret_cast<const float *>(ws + L.part),
                           (int64_t)g.mp * g.mp, g.ksplit, g.mp, g.batch, xs,
                           reinterpret_cast<uint16_t *>(ws + L.sm[p.out]), (int64_t)(L.a_stride / 2),
                           reinterpret_cast<float *>(ws + L.sd[p.out]), (int64_t)(L.d_stride / 4),
                           p.out_f16 ? 1 : 0);
    }
    return hipGetLastError();
}

// The program of ns_steps steps in segments (ns_segments).  A segment of
// length L from X (= X_0 of the segment) [the Gram-matrix identities: with
// A_j = X_j X_j^T and P_j = a I + b A_j + c A_j^2, X_{j+1} = P_j X_j, so
// A_{j+1} = P_j A_j P_j = P_j^2 A_j (P_j is a polynomial in A_j) and
// X_L = P_{L-1} ... P_0 X_0]:
//   A_0 = X X^T
//   for j < L:  P_j = a I + b A_j + c A_j^2
//               Q_j = P_j Q_{j-1}            (Q_0 = P_0)
//               S_j = P_j P_j,  A_{j+1} = S_j A_j     (j < L - 1)
//   X' = Q_{L-1} X
// Every matrix on the way is a polynomial in A_0, so every product is of two
// commuting symmetric matrices and is itself symmetric.  With L = 1 this is
// the plain iteration (X X^T, P, P X).  Slots go lowest free first; five
// suffice for any L.  With f16 set the chain A_0 ... Q_{L-1} is held in fp16
// except Q_{L-1} (P_0 when L = 1), which X' = Q X reads beside the bf16 X;
// with f16 clear everything is bf16.
void build_program(bool gram, int ns_steps, bool f16, NsProgram &pr) {
    MuonGeom g{};
    g.gram = gram ? 1 : 0;
    int len[100];
    const int nseg = ns_segments(g, ns_steps, len);
    pr.len = 0;
    auto emit = [&](int kind, int seg, bool last) -> NsStep & {
        NsStep &st = pr.step[pr.len++];
        st = NsStep{};
        st.kind = (int8_t)kind;
        st.seg = (int16_t)seg;
        st.last_seg = last ? 1 : 0;
        return st;
    };
    bool h = false;  // this segment's chain in fp16
    auto add = [&](NsStep &st, int in1, int in2, int out, bool out16 = true) {
        st.in1[st.nprod] = (int8_t)in1;
        st.in2[st.nprod] = (int8_t)in2;
        st.out[st.nprod] = (int8_t)out;
        st.f16in = (st.kind == kSyrkAA || st.kind == kSymLR) && h ? 1 : 0;
        st.f16out[st.nprod] = st.kind != kGemmBX && h && out16 ? 1 : 0;
        ++st.nprod;
    };
    for (int sg = 0; sg < nseg; ++sg) {
        const bool last = sg + 1 == nseg;
        const int L = len[sg];
        h = f16;
        bool busy[kNsSlots] = {};
        auto alloc = [&]() {
            int k = 0;
            while (busy[k]) ++k;
            busy[k] = true;
            return k;
        };
        int A = alloc();
        add(emit(kSyrkXXT, sg, last), A, A, A);
        int Q = -1;
        for (int j = 0; j < L; ++j) {
            const int P = alloc();
            add(emit(kSyrkAA, sg, last), A, A, P, L > 1);  // P_0 = Q_0 in bf16 when L = 1
            int S = -1, Qn = -1;
            if (j > 0 || j + 1 < L) {
                NsStep &st = emit(kSymLR, sg, last);
                if (j > 0) {
                    Qn = alloc();
                    add(st, P, Q, Qn, j + 1 < L);  // Q_{L-1} in bf16
                }
                if (j + 1 < L) {
                    S = alloc();
                    add(st, P, P, S);
                }
            }
            if (j > 0) {
                busy[Q] = false;  // Q_{j-1} (P_0 for j = 1)
                busy[P] = false;
                Q = Qn;
            } else {
                Q = P;
            }
            if (j + 1 < L) {
                const int An = alloc();
                add(emit(kSymLR, sg, last), S, A, An);
                busy[S] = false;
                busy[A] = false;
                A = An;
            }
        }
        add(emit(kGemmBX, sg, last), Q, Q, Q);
    }
}

}  // namespace

void ns_set_workgroup_limit(int n) {
    g_workgroup_limit.store(n > 0 ? (n < 8 ? 8 : n / 8 * 8) : 0, std::memory_order_relaxed);
}

int ns_round_tiles(int tile) {
    switch (tile) {
        case 64: return round_tiles_of<64>();
        case 128: return round_tiles_of<128>();
        default: return round_tiles_of<256>();
    }
}

int ns_segments(const MuonGeom &g, int ns_steps, int *len) {
    if (ns_steps <= 0) return 0;
    const int per = g.gram ? kNsMaxSegment : 1;
    const int nseg = (ns_steps + per - 1) / per;
    if (len != nullptr) {
        const int base = ns_steps / nseg, extra = ns_steps % nseg;
        for (int i = 0; i < nseg; ++i) len[i] = base + (i < extra ? 1 : 0);
    }
    return nseg;
}

// fp16's largest finite value is 65504.  Every m x m matrix of a segment is a
// polynomial in its A_0 and symmetric, so no entry exceeds its largest
// |eigenvalue|: the polynomial's value on A_0's spectrum.  The first
// segment's X_0 has ||X_0||_F <= 1 (the pre-scale), so its singular values
// lie in [0, 1]; a step maps a singular value s to s p(s^2), a segment to
// s |q(s^2)| with q = p_{L-1} ... p_0 on the way.  The bound is the largest
// |value| of A_j, P_j, S_j = P_j^2, Q_j over a grid of s in [0, 1.05] (5% for
// rounding) carried through every segment; fp16 when twice it is below 2^14.
// (The last call's answer is kept: the check is a few thousand steps of
// scalar arithmetic per Newton-Schulz step.)
bool ns_gram_f16_safe(int ns_steps, float a, float b, float c) {
    static std::mutex mu;
    static int k_steps = -1;
    static float k_a = 0.0f, k_b = 0.0f, k_c = 0.0f;
    static bool k_ok = false;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (k_steps == ns_steps && k_a == a && k_b == b && k_c == c) return k_ok;
    }
    MuonGeom g{};
    g.gram = 1;
    int len[100];
    const int nseg = ns_segments(g, ns_steps, len);
    const double A = a, B = b, C = c;
    constexpr int kGrid = 2048;
    double worst = 0.0;
    for (int i = 0; i <= kGrid && std::isfinite(worst); ++i) {
        double sig = 1.05 * i / kGrid;
        for (int sg = 0; sg < nseg; ++sg) {
            double lam = sig * sig, q = 1.0;
            worst = std::max(worst, lam);
            for (int j = 0; j < len[sg]; ++j) {
                const double pv = A + B * lam + C * lam * lam;
                q *= pv;
                worst = std::max(worst, std::max(std::fabs(pv), std::fabs(q)));
                if (j + 1 < len[sg]) {
                    worst = std::max(worst, pv * pv);
                    lam *= pv * pv;
                    worst = std::max(worst, lam);
                }
            }
            sig *= std::fabs(q);
        }
    }
    const bool ok = std::isfinite(worst) && 2.0 * worst < 16384.0;
    std::lock_guard<std::mutex> lock(mu);
    k_steps = ns_steps;
    k_a = a;
    k_b = b;
    k_c = c;
    k_ok = ok;
    return ok;
}

void ns_schedule(const NsGroupRef *refs, int nrefs, int ns_steps, bool f16, NsSchedule &s) {
    s.used[0] = s.used[1] = 0;
    for (int i = 0; i < nrefs; ++i) s.used[refs[i].geom->gram ? 1 : 0] = 1;
    for (int p = 0; p < 2; ++p) {
        s.prog[p].len = 0;
        if (s.used[p] && ns_steps > 0) build_program(p == 1, ns_steps, f16, s.prog[p]);
    }
    const int n0 = s.prog[0].len, n1 = s.prog[1].len;
    const NsStep *a = s.prog[0].step, *b = s.prog[1].step;
    // longest common subsequence of the kinds of the two programs' suffixes
    std::vector<int16_t> d((size_t)(n0 + 1) * (n1 + 1), 0);
    auto D = [&](int i, int j) -> int16_t & { return d[(size_t)i * (n1 + 1) + j]; };
    for (int i = n0 - 1; i >= 0; --i)
        for (int j = n1 - 1; j >= 0; --j)
            D(i, j) = a[i].kind == b[j].kind ? (int16_t)(D(i + 1, j + 1) + 1)
                                              : std::max(D(i + 1, j), D(i, j + 1));
    int i = 0, j = 0, t = 0;
    while (i < n0 || j < n1) {
        if (i < n0 && j < n1 && a[i].kind == b[j].kind) {
            s.kind[t] = a[i].kind;
            s.idx[0][t] = (int16_t)i++;
            s.idx[1][t] = (int16_t)j++;
        } else if (j == n1 || (i < n0 && D(i + 1, j) >= D(i, j + 1))) {
            s.kind[t] = a[i].kind;
            s.idx[0][t] = (int16_t)i++;
            s.idx[1][t] = -1;
        } else {
            s.kind[t] = b[j].kind;
            s.idx[0][t] = -1;
            s.idx[1][t] = (int16_t)j++;
        }
        ++t;
    }
    s.nsteps = t;
}

hipError_t launch_ns_step(const NsGroupRef *refs, int nrefs, const NsSchedule &s, int t, float a,
                          float b, float c, hipStream_t stream) {
    if (nrefs < 1 || nrefs > kMaxCallGroups || t < 0 || t >= s.nsteps) return hipErrorInvalidValue;
    LaunchPart all[2 * kMaxCallGroups];
    int nall = 0;
    const int kind = s.kind[t];
    for (int i = 0; i < nrefs; ++i) {
        const MuonGeom &g = *refs[i].geom;
        for (const int tl : {g.tile, g.tile_bx})
            if ((tl != 64 && tl != 128 && tl != 256) || g.mp % tl != 0 || g.np % tl != 0)
                return hipErrorInvalidValue;
        const int p = g.gram ? 1 : 0;
        const int k = s.idx[p][t];
        if (k < 0) continue;
        const NsStep &st = s.prog[p].step[k];
        const int ns = kind == kSyrkXXT ? g.ksplit : 1;
        for (int q = 0; q < st.nprod; ++q)
            for (int sp = 0; sp < ns; ++sp) {
                if (nall == 2 * kMaxCallGroups) return hipErrorInvalidValue;
                LaunchPart lp{i, 0, g.batch, sp, ns};
                lp.in1 = st.in1[q];
                lp.in2 = st.in2[q];
                lp.out = st.out[q];
                lp.seg = st.seg;
                lp.last = st.last_seg != 0;
                // (a plain group whose m is past fp16's validated range keeps A in bf16)
                const bool f16ok = g.m <= kNsF16MaxM;
                lp.in_f16 = f16ok && st.f16in != 0;
                lp.out_f16 = f16ok && st.f16out[q] != 0;
                all[nall++] = lp;
            }
    }
    switch (kind) {
        case kSyrkXXT: {
            const hipError_t e = run_mode<kSyrkXXT>(refs, all, nall, a, b, c, stream);
            return e == hipSuccess ? launch_xxt_fixups(refs, all, nall, stream) : e;
        }
        case kSyrkAA:
        case kSymLR: {
            // one launch per operand type
            LaunchPart by[2][2 * kMaxCallGroups];
            int nby[2] = {0, 0};
            for (int i = 0; i < nall; ++i) by[all[i].in_f16 ? 1 : 0][nby[all[i].in_f16 ? 1 : 0]++] = all[i];
            hipError_t e = hipSuccess;
            if (nby[0] > 0)
                e = kind == kSyrkAA ? run_mode<kSyrkAA, false>(refs, by[0], nby[0], a, b, c, stream)
                                    : run_mode<kSymLR, false>(refs, by[0], nby[0], a, b, c, stream);
            if (e == hipSuccess && nby[1] > 0)
                e = kind == kSyrkAA ? run_mode<kSyrkAA, true>(refs, by[1], nby[1], a, b, c, stream)
                                    : run_mode<kSymLR, true>(refs, by[1], nby[1], a, b, c, stream);
            return e;
        }
        default: return run_mode<kGemmBX>(refs, all, nall, a, b, c, stream);
    }
}

}  // namespace zopt
