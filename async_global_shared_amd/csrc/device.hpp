// device.hpp -- gfx950 kernels of the pipelined FP32 GEMM and the tile copy.
//
// Structure (what each part restates from the pages):
//  * Layout / Operand: one K slice of A (BM x BK) or B (BK x BN) in LDS as
//    16-byte chunks. The pages' kernels move one float4 per thread per operand
//    per slice at the same addresses in both fills ("Day 74 -- Async copies
//    and pipelines", section "Two kernels, one arithmetic"); here each lane
//    owns a fixed list of chunks (4-byte pieces when alignment forbids 16-byte
//    loads) and both fills deliver exactly the same bytes to exactly the same
//    LDS positions.
//  * The asynchronous fill is gfx950's buffer_load ... lds: the wave issues it
//    and continues; the data goes from memory into LDS without a VGPR (the
//    role cp.async plays on the pages). Its LDS destination is M0 + lane*size,
//    so a wave instruction writes one contiguous run; bank-conflict-free reads
//    come from choosing which global chunk each lane fetches (an XOR swizzle
//    of the chunk index per row).
//  * Out-of-range elements are loaded through a buffer offset beyond the
//    descriptor's range, which reads zero, so ragged tiles hold +0.0 and never
//    stale data ("cp.async" TVM page, section "Predication is different from
//    zero fill").
//  * ValuTile / MfmaTile: the one computeTile both fills call
//    ("pipelined_gemm.cu", computeTile): VALU is an explicit fma chain per C
//    element with k ascending; MFMA uses v_mfma_f32_32x32x2_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ring.h"

namespace mgemm {

typedef __attribute__((address_space(3))) void lds_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLdsBytes = 160 * 1024; // LDS per CU (and per workgroup) on gfx950
constexpr int kWaves = 4;
constexpr int kBK = 16;
// Every buffer descriptor spans 2^31 bytes from its (per-block, per-slice)
// base; valid lanes use offsets below that, masked lanes use kMasked, which the
// range check turns into a zero read with no memory access.
constexpr unsigned kRecords = 0x80000000u;
constexpr unsigned kMasked = 0x80000000u;
constexpr int kDescWord3 = 0x00020000; // raw buffer, 32-bit data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)kRecords, kDescWord3);
}

// ---- LDS layouts ----------------------------------------------------------

struct SwzNone {
    MG_HD static constexpr int f(int) { return 0; }
};
// A tiles (row stride 64 B): XOR the 16-byte chunk index with row bits 2..3.
// Measured with SQ_LDS_BANK_CONFLICT on gfx950: for the ds_read_b128 patterns
// of both compute tiles (the VALU tile's 4 thread rows 4 apart, the MFMA
// tile's 32 consecutive rows per half-wave) this layout reads without bank
// conflicts, while the unswizzled layout costs 12 extra cycles per read.
// B tiles need no swizzle: their reads (contiguous runs per row) measured
// conflict-free as they are.
struct SwzA {
    MG_HD static constexpr int f(int r) { return (r >> 2) & 3; }
};

// Rows of 128 B (the 16-bit tiles' A slices, fp32 A slices of 32 k): 16
// consecutive rows on distinct 16-byte bank groups.
struct SwzA16 {
    MG_HD static constexpr int f(int r) { return (r >> 1) & 7; }
};
// Rows of 256 B (fp32 A slices of 64 k): 16 consecutive rows on distinct
// 16-byte bank groups.
struct SwzA256 {
    MG_HD static constexpr int f(int r) { return r & 15; }
};
// The A-slice swizzle for a row of KPS fp32 values.
template <int KPS>
using SwzRowsOf = typename std::conditional<KPS == 16, SwzA, typename std::conditional<KPS == 32, SwzA16, SwzA256>::type>::type;

// ROWS x COLS fp32 slice; chunk (r, c4) (4 floats) lives at chunk position
// r * CPR + (c4 ^ f(r)).
template <int ROWS, int COLS, class Swz>
struct Layout {
    static constexpr int kRows = ROWS, kCols = COLS;
    static constexpr int CPR = COLS / 4;
    static constexpr int CHUNKS = ROWS * CPR;
    static constexpr int BYTES = CHUNKS * 16;
    static_assert(COLS % 4 == 0, "whole 16-byte chunks per row");
    MG_HD static constexpr int pos(int r, int c4) { return r * CPR + (c4 ^ Swz::f(r)); }
    MG_HD static constexpr int row(int p) { return p / CPR; }
    MG_HD static constexpr int col4(int p) { return (p % CPR) ^ Swz::f(p / CPR); }
};

// ---- one operand's slice loader --------------------------------------------
//
// Unit i of wave w covers wave-instruction g = i*WAVES + w. With 16-byte
// loads lane l owns chunk position p = g*64 + l; with 4-byte loads it owns
// float q = g*64 + l of the slice (chunk q/4, element q%4). The LDS byte
// address is g*64*W + l*W in both cases, for the asynchronous and the
// register fill alike.
template <class L, int W, int WAVES = kWaves>
struct Operand {
    static constexpr int U = (W == 16) ? L::CHUNKS / (64 * WAVES) : (L::CHUNKS * 4) / (64 * WAVES);
    static_assert(W == 16 || W == 4, "load width");
    static_assert(L::CHUNKS % (64 * WAVES) == 0, "whole wave instructions per slice");
    // only the element offsets stay in registers; a unit's row and column are
    // recomputed (shifts and masks) where an edge slice needs them
    int off[U];
    int lane, wave;

    MG_HD void rc(int i, int &r, int &c) const {
        const int g = i * WAVES + wave;
        if constexpr (W == 16) {
            const int p = g * 64 + lane;
            r = L::row(p);
            c = 4 * L::col4(p);
        } else {
            const int q = g * 64 + lane;
            r = L::row(q >> 2);
            c = 4 * L::col4(q >> 2) + (q & 3);
        }
    }
    MG_HD void init(int lane_, int wave_, int ld) {
        lane = lane_;
        wave = wave_;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            int r, c;
            rc(i, r, c);
            off[i] = r * ld + c;
        }
    }
    // byte offset within the operand's region of a slot, for unit i of wave w
    MG_HD static constexpr int lds_off(int i, int wave) { return (i * WAVES + wave) * 64 * W; }

    __device__ unsigned voff(int i, int rowlim, int collim) const {
        int r, c;
        rc(i, r, c);
        return (r < rowlim && c < collim) ? (unsigned)off[i] * 4u : kMasked;
    }
    // the offset of a unit known to lie inside the operand (a full slice)
    __device__ unsigned voff_in(int i) const { return (unsigned)off[i] * 4u; }
};

// ---- compute tiles ----------------------------------------------------------

// VALU: 256 threads as 16 x 16; thread (tr, tc) owns rows 64h + 4tr + i and
// columns 64hn + 4tc + j (h < TM/4, hn < TN/4, i, j < 4).
template <int BM, int BN, int TM, int TN>
struct ValuTile {
    using LA = Layout<BM, kBK, SwzA>;
    using LB = Layout<kBK, BN, SwzNone>;
    // per K slice: A columns and B rows advanced (in 32-bit words / rows), k values
    static constexpr int A_STEP = kBK, B_STEP = kBK, KPS = kBK, EPW = 1, WAVES = kWaves;
    static constexpr int HM = TM / 4, HN = TN / 4;
    static_assert(BM == 64 * HM && BN == 64 * HN, "16 x 16 threads, 4-row groups 64 apart");
    float acc[TM][TN];
    int tr, tc;

    __device__ void init(int tid) {
        tr = tid >> 4;
        tc = tid & 15;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = 0.0f;
    }
    __device__ void poison() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_nanf("");
    }
    // An empty asm that reads and writes every accumulator: the slice's FMAs
    // are then issued before whatever follows in program order, instead of
    // being sunk below the next slice's (branchy) LDS stores, which would
    // keep all of the slice's LDS fragments live across them.
    __device__ void pin() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; j += 4)
                asm volatile("" : "+v"(acc[i][j]), "+v"(acc[i][j + 1]), "+v"(acc[i][j + 2]), "+v"(acc[i][j + 3]));
    }
    __device__ int row(int h, int i) const { return 64 * h + 4 * tr + i; }
    __device__ int col(int h) const { return 64 * h + 4 * tc; }

    // acc[i][j] = fma(A[row_i][k], B[k][col_j], acc[i][j]) for k = 0 .. BK-1
    __device__ void compute(const unsigned char *As, const unsigned char *Bs) {
#pragma unroll
        for (int kc = 0; kc < kBK / 4; ++kc) {
            f32x4 a[TM];
#pragma unroll
            for (int h = 0; h < HM; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[4 * h + i] = *(const f32x4 *)(As + LA::pos(row(h, i), kc) * 16);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                f32x4 b[HN];
#pragma unroll
                for (int h = 0; h < HN; ++h)
                    b[h] = *(const f32x4 *)(Bs + LB::pos(4 * kc + kk, col(h) >> 2) * 16);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int h = 0; h < HN; ++h)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][4 * h + j] = __builtin_fmaf(a[i][kk], b[h][j], acc[i][4 * h + j]);
            }
        }
    }

    __device__ void store(float *C, int ldc, int m0, int n0, int M, int N, bool vec) const {
#pragma unroll
        for (int h = 0; h < HM; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = m0 + row(h, i);
                if (r >= M)
                    continue;
#pragma unroll
                for (int hn = 0; hn < HN; ++hn) {
                    const int c = n0 + col(hn);
                    float *p = C + (size_t)r * ldc + c;
                    const float *v = &acc[4 * h + i][4 * hn];
                    if (vec && c + 3 < N) {
                        *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (c + j < N)
                                p[j] = v[j];
                    }
                }
            }
    }
};

// MFMA: 4 waves as 2 x 2; each wave owns WTM x WTN tiles of 32 x 32, computed
// with v_mfma_f32_32x32x2_f32. Lane l supplies A[m0 + l%32][k_l] and
// B[k_l][n0 + l%32] with k_l = 8kb + 4(l/32) + s in MFMA step s, so the four
// steps of an 8-k group cover its eight k values. A K slice holds KPS_ k
// values (16, 32 or 64): the MFMA sequence of each accumulator depends on the
// absolute k only, not on how the slices cut it.
template <int WTM, int WTN, int KPS_ = kBK>
struct MfmaTile {
    static constexpr int BM = 64 * WTM, BN = 64 * WTN;
    static constexpr int A_STEP = KPS_, B_STEP = KPS_, KPS = KPS_, EPW = 1, WAVES = kWaves;
    static_assert(KPS == 16 || KPS == 32 || KPS == 64, "K slice");
    using LA = Layout<BM, KPS, SwzRowsOf<KPS>>;
    using LB = Layout<KPS, BN, SwzNone>;
    f32x16 acc[WTM][WTN];
    int wm, wn, lane;

    __device__ void init(int tid) {
        lane = tid & 63;
        const int w = tid >> 6;
        wm = w >> 1;
        wn = w & 1;
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[a][b][i] = 0.0f;
    }

    __device__ void pin() {} // MFMA results stay where the MFMAs are issued
    __device__ void poison() {
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[a][b][i] = __builtin_nanf("");
    }

    __device__ void compute(const unsigned char *As, const unsigned char *Bs) {
        const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int kb = 0; kb < KPS / 8; ++kb) {
            f32x4 a[WTM];
#pragma unroll
            for (int ta = 0; ta < WTM; ++ta) {
                const int m = 32 * WTM * wm + 32 * ta + l32;
                a[ta] = *(const f32x4 *)(As + LA::pos(m, 2 * kb + h) * 16);
            }
            float b[WTN][4];
#pragma unroll
            for (int tb = 0; tb < WTN; ++tb)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int k = 8 * kb + 4 * h + s;
                    const int n = 32 * WTN * wn + 32 * tb + l32;
                    b[tb][s] = *(const float *)(Bs + LB::pos(k, n >> 2) * 16 + (n & 3) * 4);
                }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ta = 0; ta < WTM; ++ta)
#pragma unroll
                    for (int tb = 0; tb < WTN; ++tb)
                        acc[ta][tb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[ta][s], b[tb][s], acc[ta][tb], 0, 0, 0);
        }
    }

    __device__ void store(float *C, int ldc, int m0, int n0, int M, int N, bool) const {
        const int h = lane >> 5, l32 = lane & 31;
        if (m0 + BM <= M && n0 + BN <= N) { // interior tile: no bounds per element
            float *base = C + (size_t)(m0 + 32 * WTM * wm + h * 4) * ldc + n0 + 32 * WTN * wn + l32;
#pragma unroll
            for (int ta = 0; ta < WTM; ++ta)
#pragma unroll
                for (int tb = 0; tb < WTN; ++tb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        base[(size_t)(32 * ta + (i >> 2) * 8 + (i & 3)) * ldc + 32 * tb] = acc[ta][tb][i];
            return;
        }
#pragma unroll
        for (int ta = 0; ta < WTM; ++ta)
#pragma unroll
            for (int tb = 0; tb < WTN; ++tb) {
                const int c = n0 + 32 * WTN * wn + 32 * tb + l32;
                if (c >= N)
                    continue;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = m0 + 32 * WTM * wm + 32 * ta + (i >> 2) * 8 + h * 4 + (i & 3);
                    if (r < M)
                        C[(size_t)r * ldc + c] = acc[ta][tb][i];
                }
            }
    }
};

// 16-bit inputs (bfloat16 or binary16), fp32 accumulation: per wave WTM x WTN
// tiles of 32 x 32 with v_mfma_f32_32x32x16_{bf16,f16}; a K slice is 64
// elements. A is stored as in the fp32 tiles (rows of the slice, k
// contiguous): lane l reads its 8 k values A[m][16ks + 8(l/32) + 0..7] as one
// 16-byte chunk. B stays row-major (k rows, n contiguous) as the fill wrote
// it; gfx950's transposing LDS read ds_read_b64_tr_b16 turns it into the
// operand: within each 16-lane group, lane i receives element i%4 of the
// 8-byte pieces that lanes i/4, 4+i/4, 8+i/4 and 12+i/4 address. If lane q
// addresses row k0 + q/4, columns nb + 4(q%4) .. +3, lane i receives
// B[k0 .. k0+3][nb + i], so two such reads give B[16ks + 8(l/32) + 0..7][n],
// the same k values its A operand holds.
#ifndef MGEMM_SWZB16
#define MGEMM_SWZB16 2
#endif
struct SwzB16 { // the 4 rows of one transposing read on distinct 64-byte bank groups
    MG_HD static constexpr int f(int r) { return (r & 3) << MGEMM_SWZB16; }
};
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// K elements per slice of the 16-bit tiles: 64 (rows of 128 B) or 32 (rows
// of 64 B, the fp32 tiles' row size, half the LDS per stage)
#ifndef MGEMM_K16
#define MGEMM_K16 64
#endif
constexpr int kK16 = MGEMM_K16;
static_assert(kK16 == 32 || kK16 == 64, "16-bit K slice");

// WGM x WGN waves, each WTM x WTN tiles of 32 x 32.
template <int WTM, int WTN, int WGM, int WGN, bool BF16, int KPS_ = kK16>
struct Mfma16Tile {
    static constexpr int BM = 32 * WTM * WGM, BN = 32 * WTN * WGN, WAVES = WGM * WGN;
    static constexpr int KPS = KPS_, EPW = 2, A_STEP = KPS / EPW, B_STEP = KPS;
    using LA = Layout<BM, A_STEP, typename std::conditional<KPS == 64, SwzA16, SwzA>::type>; // BM rows x KPS/2 words
    using LB = Layout<KPS, BN / EPW, SwzB16>;                                                 // KPS k rows x BN/2 words
    f32x16 acc[WTM][WTN];
    int wm, wn, lane;

    __device__ void init(int tid) {
        lane = tid & 63;
        const int w = tid >> 6;
        wm = w / WGN;
        wn = w % WGN;
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[a][b][i] = 0.0f;
    }
    __device__ void pin() {} // MFMA results stay where the MFMAs are issued
    __device__ void poison() {
#pragma unroll
        for (int a = 0; a < WTM; ++a)
#pragma unroll
            for (int b = 0; b < WTN; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    acc[a][b][i] = __builtin_nanf("");
    }

    // The LDS reads are issued from inline asm, and a separate asm wait
    // lists their destinations as outputs: the compiler's wait pass does not
    // model ds_read_b64_tr_b16 against in-flight LDS-DMA fills and would
    // drain the whole prefetch (vmcnt(0)) before it, although the ring's own
    // wait and barrier already made this slot's slice visible. Outputs are
    // early-clobber where one asm block issues several reads: a read may land
    // while later reads of the block still need their address registers.
    //
    // One k step's operands: WTM A rows (16 bytes each) and two transposing
    // B reads per column tile.
    struct Frag {
        u32x4 a[WTM];
        i16x4 b[WTN][2];
    };
    // Issue one k step's LDS reads without waiting for them. `aa` addresses
    // A row 32 WTM wm + l32 at this k step (row tiles ta are 32 rows, an
    // immediate, apart: the swizzle repeats every 32 rows); ab[tb] address
    // the B pieces; the k step's rows are immediates on top.
    template <int KS>
    __device__ static void issue_reads(unsigned aa, const unsigned *ab, Frag &f) {
        constexpr int TA = 32 * LA::CPR * 16;
        constexpr int B0 = (16 * KS) * LB::CPR * 16, B1 = (16 * KS + 4) * LB::CPR * 16;
        if constexpr (WTM == 4)
            asm volatile("ds_read_b128 %0, %4\n\t"
                         "ds_read_b128 %1, %4 offset:%5\n\t"
                         "ds_read_b128 %2, %4 offset:%6\n\t"
                         "ds_read_b128 %3, %4 offset:%7"
                         : "=&v"(f.a[0]), "=&v"(f.a[1]), "=&v"(f.a[2]), "=&v"(f.a[3])
                         : "v"(aa), "i"(TA), "i"(2 * TA), "i"(3 * TA));
        else
            asm volatile("ds_read_b128 %0, %2\n\t"
                         "ds_read_b128 %1, %2 offset:%3"
                         : "=&v"(f.a[0]), "=&v"(f.a[1])
                         : "v"(aa), "i"(TA));
        // two transposing reads (row quads 0 and 1) per column tile
#pragma unroll
        for (int tb = 0; tb < WTN; ++tb)
            asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\t"
                         "ds_read_b64_tr_b16 %1, %2 offset:%4"
                         : "=&v"(f.b[tb][0]), "=&v"(f.b[tb][1])
                         : "v"(ab[tb]), "i"(B0), "i"(B1));
    }
    // Read R of one k step alone: R < WTM is A row tile R, the rest are the
    // B pieces (column tile (R - WTM) / 2, row quad (R - WTM) % 2).
    template <int KS, int R>
    __device__ static void issue_read(unsigned aa, const unsigned *ab, Frag &f) {
        constexpr int TA = 32 * LA::CPR * 16;
        constexpr int B0 = (16 * KS) * LB::CPR * 16, B1 = (16 * KS + 4) * LB::CPR * 16;
        if constexpr (R < WTM) {
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f.a[R]) : "v"(aa), "i"(R * TA));
        } else {
            constexpr int q = R - WTM, tb = q / 2;
            asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                         : "=v"(f.b[tb][q % 2])
                         : "v"(ab[tb]), "i"(q % 2 ? B1 : B0));
        }
    }
    // Wait for every LDS read of this wave; the fragment's registers are
    // outputs of the wait, so nothing reads them before it.
    __device__ static void wait_reads(Frag &f) {
        if constexpr (WTM == 4 && WTN == 4)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0][0]), "+v"(f.b[0][1]),
                           "+v"(f.b[1][0]), "+v"(f.b[1][1]), "+v"(f.b[2][0]), "+v"(f.b[2][1]), "+v"(f.b[3][0]),
                           "+v"(f.b[3][1]));
        else if constexpr (WTM == 4)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.b[0][0]), "+v"(f.b[0][1]),
                           "+v"(f.b[1][0]), "+v"(f.b[1][1]));
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.b[0][0]), "+v"(f.b[0][1]), "+v"(f.b[1][0]),
                           "+v"(f.b[1][1]));
    }
    template <int ta, int tb>
    __device__ void mfma_one(const Frag &f) {
        const i16x4 lo = f.b[tb][0], hi = f.b[tb][1];
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (BF16)
            acc[ta][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, f.a[ta]), __builtin_bit_cast(bf16x8, bv), acc[ta][tb], 0, 0, 0);
        else
            acc[ta][tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, f.a[ta]), __builtin_bit_cast(f16x8, bv), acc[ta][tb], 0, 0, 0);
    }
    __device__ void mfma(const Frag &f) {
        static_for<0, WTM * WTN>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            mfma_one<j / WTN, j % WTN>(f);
        });
    }

    static constexpr bool kSplit = true;
    __device__ void lane_addrs(const unsigned char *As, const unsigned char *Bs, unsigned &as, unsigned *ab) const {
        const int h = lane >> 5, q = lane & 15, g16 = (lane >> 4) & 1;
        as = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)As;
        const unsigned bs = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)Bs;
#pragma unroll
        for (int tb = 0; tb < WTN; ++tb) {
            const int k = 8 * h + (q >> 2);
            const int n = 32 * WTN * wn + 32 * tb + 16 * g16 + 4 * (q & 3);
            ab[tb] = bs + LB::pos(k, n >> 3) * 16 + (n & 7) * 2;
        }
    }
    // The k steps of a slice are software-pipelined: step ks+1's reads are
    // in flight while step ks's MFMAs run (scheduling barriers keep the
    // MFMAs between the issue and the wait). head, body and tail split one
    // slice's compute at its ends (the split ring interleaves them across
    // slices); compute runs the three in a row.
    static constexpr int NKS = KPS / 16;
    static_assert(NKS % 2 == 0, "the last k step's fragment set differs from the first's");
    // Within a k step of the body, the next step's LDS reads go one after
    // each MFMA rather than as one burst before them, so they issue while the
    // matrix pipe is busy (measured +1-2 % on the 256-row tiles). Only where
    // the MFMAs outnumber the reads: the 128 x 128 tile's 4 MFMAs and 6 reads
    // were measured 1-3 % slower this way.
    static constexpr int NR = WTM + 2 * WTN, NM = WTM * WTN;
    static constexpr bool kInterleave = NM >= NR;
    Frag fr[2];
    __device__ void head(const unsigned char *As, const unsigned char *Bs) {
        static_assert((WTN == 2 && (WTM == 2 || WTM == 4)) || (WTN == 4 && WTM == 4), "wait_reads covers these wave tiles");
        const int h = lane >> 5, m = 32 * WTM * wm + (lane & 31);
        unsigned as, ab[WTN];
        lane_addrs(As, Bs, as, ab);
        issue_reads<0>(as + LA::pos(m, h) * 16, ab, fr[0]);
        __builtin_amdgcn_sched_barrier(0);
    }
    __device__ void body(const unsigned char *As, const unsigned char *Bs) {
        const int h = lane >> 5, m = 32 * WTM * wm + (lane & 31);
        unsigned as, ab[WTN];
        lane_addrs(As, Bs, as, ab);
        __builtin_amdgcn_sched_barrier(0);
        wait_reads(fr[0]);
        static_for<0, NKS - 1>([&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            const unsigned aa = as + LA::pos(m, 2 * (ks + 1) + h) * 16;
            if constexpr (kInterleave) {
                static_for<0, NM>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if constexpr (j < NR) {
                        issue_read<ks + 1, j>(aa, ab, fr[(ks + 1) & 1]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    mfma_one<j / WTN, j % WTN>(fr[ks & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                });
            } else {
                issue_reads<ks + 1>(aa, ab, fr[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mfma(fr[ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_reads(fr[(ks + 1) & 1]);
        });
    }
    __device__ void tail() {
        __builtin_amdgcn_sched_barrier(0);
        mfma(fr[(NKS - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // The same MFMAs with f(Int<j>) placed after the j-th of them (the ring
    // spreads a slice's fill instructions there, so no wave stalls on a
    // burst of them while the matrix pipe runs dry).
    static constexpr int TAIL_OPS = WTM * WTN;
    // Spread the ring's refill over the tail: measured faster for the 8-wave
    // tile (two waves per SIMD stall together on a burst of fills); the
    // 4-wave tiles hold twice the fill units per wave, and keeping their
    // offsets live across the tail costs them occupancy.
    static constexpr bool kSpreadFill = WAVES == 8;
    // Waves that issue the asynchronous ring's fills: with 8 waves only
    // waves 0-3 (one per SIMD under the dispatcher's round-robin placement),
    // each issuing twice the units, so the other wave of each SIMD never
    // stalls behind fill instructions (measured +2-3 % at 4096^3 and 8192^3).
    // The register-staged ring keeps all waves loading.
    static constexpr int FILL_WAVES = WAVES == 8 ? 4 : WAVES;
    template <class F>
    __device__ void tail_with(F &&f) {
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, TAIL_OPS>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            mfma_one<j / WTN, j % WTN>(fr[(NKS - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            f(jc);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    __device__ void compute(const unsigned char *As, const unsigned char *Bs) {
        head(As, Bs);
        body(As, Bs);
        tail();
    }

    __device__ void store(float *C, int ldc, int m0, int n0, int M, int N, bool) const {
        const int h = lane >> 5, l32 = lane & 31;
        if (m0 + BM <= M && n0 + BN <= N) { // interior tile: no bounds per element
            float *base = C + (size_t)(m0 + 32 * WTM * wm + h * 4) * ldc + n0 + 32 * WTN * wn + l32;
#pragma unroll
            for (int ta = 0; ta < WTM; ++ta)
#pragma unroll
                for (int tb = 0; tb < WTN; ++tb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        base[(size_t)(32 * ta + (i >> 2) * 8 + (i & 3)) * ldc + 32 * tb] = acc[ta][tb][i];
            return;
        }
#pragma unroll
        for (int ta = 0; ta < WTM; ++ta)
#pragma unroll
            for (int tb = 0; tb < WTN; ++tb) {
                const int c = n0 + 32 * WTN * wn + 32 * tb + l32;
                if (c >= N)
                    continue;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = m0 + 32 * WTM * wm + 32 * ta + (i >> 2) * 8 + h * 4 + (i & 3);
                    if (r < M)
                        C[(size_t)r * ldc + c] = acc[ta][tb][i];
                }
            }
    }
};

// Tile configurations (block tile, compute tile).
struct CfgValu64 {
    using Tile = ValuTile<64, 64, 4, 4>;
    static constexpr int BM = 64, BN = 64;
};
struct CfgValu128 {
    using Tile = ValuTile<128, 128, 8, 8>;
    static constexpr int BM = 128, BN = 128;
};
// 64 x 64 MFMA tile with a K slice of 32 or 64: one wave per 32 x 32 tile
// issues only 4 MFMAs per 8 k, so the slice's fixed costs (barrier, fill
// issue, first LDS reads) are spread over more of them; the planner takes
// 64 where each CU holds one block, 32 where several blocks share it (the
// longer slot would cut their residency).
template <int KPS>
struct CfgMfma64K {
    using Tile = MfmaTile<1, 1, KPS>;
    static constexpr int BM = 64, BN = 64;
};
struct CfgMfma128 {
    using Tile = MfmaTile<2, 2>;
    static constexpr int BM = 128, BN = 128;
};
struct CfgMfma256x128 {
    using Tile = MfmaTile<4, 2>;
    static constexpr int BM = 256, BN = 128;
};
template <bool BF16>
struct CfgH128 {
    using Tile = Mfma16Tile<2, 2, 2, 2, BF16>;
    static constexpr int BM = 128, BN = 128;
};
template <bool BF16>
struct CfgH256x128 {
    using Tile = Mfma16Tile<4, 2, 2, 2, BF16>;
    static constexpr int BM = 256, BN = 128;
};
template <bool BF16>
struct CfgH256x256 { // 8 waves (2 per SIMD), each 128 x 64 as in the 256 x 128 tile
    using Tile = Mfma16Tile<4, 2, 2, 4, BF16>;
    static constexpr int BM = 256, BN = 256;
};

// ---- block -> C tile ----------------------------------------------------------
#ifndef MGEMM_GROUP_ROWS
#define MGEMM_GROUP_ROWS 4 // tile-rows walked before moving one tile right (fewest L2 misses measured)
#endif
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b on XCD
// b % 8), each with its own L2. Give each XCD a contiguous range of logical
// tiles, then walk the logical order a few tile-rows down before moving right, so
// the blocks resident on one XCD share A and B panels in its L2.
__device__ inline int xcd_linear(int bid, int nb) {
    const int x = bid & 7, i = bid >> 3;
    const int q = nb >> 3, r = nb & 7;
    return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}
__device__ inline void block_tile(int bid, int gm, int gn, int &tm, int &tn) {
    const int lin = xcd_linear(bid, gm * gn);
    constexpr int G = MGEMM_GROUP_ROWS;
    const int per_group = G * gn;
    const int grp = lin / per_group;
    const int first = grp * G;
    const int rows = min(G, gm - first);
    const int in = lin - grp * per_group;
    tm = first + in % rows;
    tn = in / rows;
}

// ---- waits and barriers --------------------------------------------------------

// s_waitcnt vmcnt(N). The counter field is 6 bits: a request above 63 waits
// for 63, i.e. for more completions than asked, which stays correct.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0, "vmcnt");
    constexpr int n = N < 63 ? N : 63;
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
// Block barrier after this wave's LDS reads and writes have completed.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One asynchronous global -> LDS fill instruction of W bytes per lane. (The
// width is spelled as a literal: clang checks this builtin's size argument
// before a function template is instantiated.)
template <int W>
__device__ inline void lds_dma(__amdgpu_buffer_rsrc_t r, unsigned char *lds, unsigned off) {
    if constexpr (W == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t *)lds, 16, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t *)lds, 4, off, 0, 0, 0);
}

// The full-slice branch of the fills is hinted as the likely one for 16-byte
// loads (the common layout; measured faster on the 4096^3 three-stage ring).
// The 4-byte loaders of the big 16-bit tiles get no hint: with it, their
// register allocation spills.
template <int W>
__device__ inline bool likely_full(bool full) {
    if constexpr (W == 16)
        return __builtin_expect(full, 1);
    else
        return full;
}

// A and B are addressed as 32-bit words (fp32 elements, or pairs of 16-bit
// elements); lda and ldb are in words, a_cols is the row extent of A in words.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int M, N, K;
    int lda, ldb, ldc;
    int gm, gn;
    int vec_store;
    int a_cols;
};

template <int W>
struct RegOf {
    using type = u32x4;
};
template <>
struct RegOf<4> {
    using type = unsigned;
};

// Waves of a tile that issue the asynchronous fills (all, unless the tile
// says otherwise).
template <class T, class = void>
struct FillWaves : std::integral_constant<int, T::WAVES> {};
template <class T>
struct FillWaves<T, std::void_t<decltype(T::FILL_WAVES)>> : std::integral_constant<int, T::FILL_WAVES> {};

// Tiles whose compute splits into head / body / tail run the split ring
// (with 16-byte loads).
template <class T, class = void>
struct SplitTile : std::false_type {};
template <class T>
struct SplitTile<T, std::void_t<decltype(T::kSplit)>> : std::integral_constant<bool, T::kSplit> {};

// State one block of the GEMM shares between its ring operations. FWv waves
// load each slice (the operands' units are split among them).
template <class Tile, int W, int FWv = Tile::WAVES>
struct GemmCtx {
    using LA = typename Tile::LA;
    using LB = typename Tile::LB;
    static constexpr int FW = FWv;
    using OA = Operand<LA, W, FW>;
    using OB = Operand<LB, W, FW>;
    static constexpr int SLOT = LA::BYTES + LB::BYTES;

    OA oa;
    OB ob;
    Tile tile;
    unsigned char *smem;
    int wave, lane;
    const float *Ablk; // A + m0 * lda
    const float *Bblk; // B + n0 (in words)
    int ldb, K, a_cols, a_rows, b_cols;

    // slice s covers A[m0.., s*A_STEP..] and B[s*B_STEP.., n0..] (words / rows);
    // the limits are relative to the slice
    __device__ const float *a_ptr(int s) const { return Ablk + s * Tile::A_STEP; }
    __device__ const float *b_ptr(int s) const { return Bblk + (size_t)s * Tile::B_STEP * ldb; }
    __device__ int a_klim(int s) const { return a_cols - s * Tile::A_STEP; }
    __device__ int b_klim(int s) const { return K - s * Tile::B_STEP; }
    // every unit of this slice lies inside A and B (the block's rows and
    // columns and the slice's k range): the loads need no masks (a
    // block-uniform test, so a scalar branch)
    __device__ bool full(int ka, int kb) const {
        return ka >= LA::kCols && kb >= LB::kRows && a_rows >= LA::kRows && b_cols >= LB::kCols;
    }
    __device__ void barrier() { lds_barrier(); }
    __device__ void compute(int, int slot) {
        const unsigned char *base = smem + slot * SLOT;
        tile.compute(base, base + LA::BYTES);
    }
    // the split ring's three parts (tiles with head / body / tail)
    __device__ void head(int, int slot) {
        const unsigned char *base = smem + slot * SLOT;
        tile.head(base, base + LA::BYTES);
    }
    __device__ void body(int, int slot) {
        const unsigned char *base = smem + slot * SLOT;
        tile.body(base, base + LA::BYTES);
    }
    __device__ void tail(int) { tile.tail(); }
};

// Asynchronous fill: buffer_load ... lds straight into the ring slot.
// (4-byte loaders keep every wave filling: four times the units per wave
// would not fit the registers)
template <class Tile, int W>
constexpr int kPipedFillWaves = W == 16 ? FillWaves<Tile>::value : Tile::WAVES;

template <class Tile, int W>
struct PipedOps : GemmCtx<Tile, W, kPipedFillWaves<Tile, W>> {
    using C = GemmCtx<Tile, W, kPipedFillWaves<Tile, W>>;
    // wave w issues fills (block-uniform per wave: a scalar test)
    MG_HD static constexpr bool fills_wave(int w) { return C::FW == Tile::WAVES || w < C::FW; }
    __device__ bool fills() const { return fills_wave(this->wave); }
    static constexpr int UNITS = C::OA::U + C::OB::U;
    // Slice s's fill instructions one unit at a time (units 0 .. OA::U-1 are
    // A's, the rest B's; FULL: the slice lies inside A and B). The buffer
    // resources are sizeless, so they travel as arguments, not in a struct.
    template <int u, bool FULL>
    __device__ void unit(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, unsigned char *base, int ka, int kb) {
        if constexpr (u < C::OA::U) {
            const unsigned off = FULL ? this->oa.voff_in(u) : this->oa.voff(u, this->a_rows, ka);
            lds_dma<W>(ra, base + C::OA::lds_off(u, this->wave), off);
        } else {
            constexpr int i = u - C::OA::U;
            const unsigned off = FULL ? this->ob.voff_in(i) : this->ob.voff(i, kb, this->b_cols);
            lds_dma<W>(rb, base + C::LA::BYTES + C::OB::lds_off(i, this->wave), off);
        }
    }
    template <int B, int E, bool FULL>
    __device__ void units(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, unsigned char *base, int ka, int kb) {
        static_for<B, E>([&](auto uc) { this->template unit<decltype(uc)::value, FULL>(ra, rb, base, ka, kb); });
    }
    __device__ void issue(int s, int slot) {
        if (!fills())
            return;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(this->a_ptr(s)), rb = make_rsrc(this->b_ptr(s));
        const int ka = this->a_klim(s), kb = this->b_klim(s);
        unsigned char *base = this->smem + slot * C::SLOT;
        if (likely_full<W>(this->full(ka, kb)))
            units<0, UNITS, true>(ra, rb, base, ka, kb);
        else
            units<0, UNITS, false>(ra, rb, base, ka, kb);
    }
    // tail(slice - 1) of the split ring with issue(s, slot) spread over its
    // MFMAs: the j-th MFMA is followed by units [j U / J, (j + 1) U / J).
    // Only the offsets depend on the full-slice test; the MFMAs stay out of
    // that branch, or each side would get its own accumulator registers.
    // Without `refill` (the last S-1 slices) only the tail runs; the test is
    // block-uniform and guards the fill instructions alone. (16-byte loaders
    // only: the 4-byte ones, with four times the units, keep the plain ring.)
    // Tiles without kSpreadFill issue the slice before the tail instead:
    // the offsets held across the tail would cost them occupancy.
    __device__ void tail_issue(int tprev, int s, int slot, bool refill) {
        static_assert(W == 16, "the split ring runs with 16-byte loads");
        if constexpr (!Tile::kSpreadFill) {
            if (refill)
                issue(s, slot);
            this->tail(tprev);
        } else {
            refill = refill && fills();
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(this->a_ptr(s)), rb = make_rsrc(this->b_ptr(s));
            const int ka = this->a_klim(s), kb = this->b_klim(s);
            unsigned char *base = this->smem + slot * C::SLOT;
            unsigned voff[UNITS];
            if (!refill) {
#pragma unroll
                for (int u = 0; u < UNITS; ++u)
                    voff[u] = 0;
            } else if (likely_full<W>(this->full(ka, kb))) {
#pragma unroll
                for (int i = 0; i < C::OA::U; ++i)
                    voff[i] = this->oa.voff_in(i);
#pragma unroll
                for (int i = 0; i < C::OB::U; ++i)
                    voff[C::OA::U + i] = this->ob.voff_in(i);
            } else {
#pragma unroll
                for (int i = 0; i < C::OA::U; ++i)
                    voff[i] = this->oa.voff(i, this->a_rows, ka);
#pragma unroll
                for (int i = 0; i < C::OB::U; ++i)
                    voff[C::OA::U + i] = this->ob.voff(i, kb, this->b_cols);
            }
            constexpr int J = Tile::TAIL_OPS;
            this->tile.tail_with([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if (refill)
                    static_for<j * UNITS / J, (j + 1) * UNITS / J>([&](auto uc) {
                        constexpr int u = decltype(uc)::value;
                        if constexpr (u < C::OA::U)
                            lds_dma<W>(ra, base + C::OA::lds_off(u, this->wave), voff[u]);
                        else
                            lds_dma<W>(rb, base + C::LA::BYTES + C::OB::lds_off(u - C::OA::U, this->wave), voff[u]);
                    });
            });
        }
    }
    // each slice is OA::U + OB::U fill instructions of a filling wave (a
    // wave that fills nothing has none in flight: its waits pass at once)
    template <int P>
    __device__ void wait() {
        wait_vm<P *(C::OA::U + C::OB::U)>();
    }
};

// Synchronous fill: global -> register set -> LDS.
template <class Tile, int W, int NSET>
struct SyncOps : GemmCtx<Tile, W> {
    using C = GemmCtx<Tile, W>;
    using R = typename RegOf<W>::type;
    R va[NSET][C::OA::U];
    R vb[NSET][C::OB::U];

    __device__ static R ld(__amdgpu_buffer_rsrc_t r, unsigned off) {
        if constexpr (W == 16)
            return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    // A slice past the last one (kb <= 0) masks every lane; its descriptors
    // are built on slice 0's addresses so that none points past the operands.
    // With two register sets or more, 16-byte loads take one form only
    // (masked offsets) and stay ahead of the compute: alternative load
    // blocks made the compiler's wait counts drain the newest slice before
    // each store, and loads in the compute's block were sunk below it.
    // 4-byte loads keep the full-slice fast path: with four times the units,
    // a selected offset per unit costs more registers than exact waits gain
    // (VALU 128x128, S=3: 267 -> 182 VGPRs, 37 -> 63 TFLOP/s at 4099x3001x1537).
    template <int SET>
    __device__ void load(int s) {
        const int ka = this->a_klim(s), kb = this->b_klim(s);
        const int sp = kb > 0 ? s : 0;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(this->a_ptr(sp));
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(this->b_ptr(sp));
        if ((NSET == 1 || W == 4) && likely_full<W>(this->full(ka, kb))) {
#pragma unroll
            for (int i = 0; i < C::OA::U; ++i)
                va[SET][i] = ld(ra, this->oa.voff_in(i));
#pragma unroll
            for (int i = 0; i < C::OB::U; ++i)
                vb[SET][i] = ld(rb, this->ob.voff_in(i));
            return;
        }
#pragma unroll
        for (int i = 0; i < C::OA::U; ++i)
            va[SET][i] = ld(ra, this->oa.voff(i, this->a_rows, ka));
#pragma unroll
        for (int i = 0; i < C::OB::U; ++i)
            vb[SET][i] = ld(rb, this->ob.voff(i, kb, this->b_cols));
        if constexpr (NSET > 1)
            __builtin_amdgcn_sched_barrier(0);
    }
    __device__ void compute(int t, int slot) {
        C::compute(t, slot);
        this->tile.pin();
    }
    template <int SET>
    __device__ void store(int slot) {
        unsigned char *base = this->smem + slot * C::SLOT;
#pragma unroll
        for (int i = 0; i < C::OA::U; ++i)
            *(R *)(base + C::OA::lds_off(i, this->wave) + this->lane * W) = va[SET][i];
#pragma unroll
        for (int i = 0; i < C::OB::U; ++i)
            *(R *)(base + C::LA::BYTES + C::OB::lds_off(i, this->wave) + this->lane * W) = vb[SET][i];
    }
};

template <class Cfg, int S, bool PIPED, int W>
__global__ void __launch_bounds__(64 * Cfg::Tile::WAVES) sgemm_kernel(GemmArgs g) {
    using Tile = typename Cfg::Tile;
    using Ctx = GemmCtx<Tile, W>;
    // a ring deeper than the CU's LDS is never planned; its kernel is empty
    constexpr bool kFits = S * Ctx::SLOT <= kLdsBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kFits ? S * Ctx::SLOT : 1024];
    if constexpr (!kFits)
        return;

    int tm, tn;
    block_tile(blockIdx.x, g.gm, g.gn, tm, tn);
    const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
    const int tid = threadIdx.x;
    const int T = (g.K + Tile::KPS - 1) / Tile::KPS;

    using Ops = typename std::conditional<PIPED, PipedOps<Tile, W>, SyncOps<Tile, W, (S > 1 ? S - 1 : 1)>>::type;
    Ops ops;
    ops.smem = smem;
    ops.lane = tid & 63;
    ops.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    ops.Ablk = g.A + (size_t)m0 * g.lda;
    ops.Bblk = g.B + n0 / Tile::EPW;
    ops.ldb = g.ldb;
    ops.K = g.K;
    ops.a_cols = g.a_cols;
    ops.a_rows = g.M - m0;
    ops.b_cols = (g.N - n0) / Tile::EPW;
    // (waves past the fill waves hold offsets they never use)
    ops.oa.init(ops.lane, ops.wave % Ops::FW, g.lda);
    ops.ob.init(ops.lane, ops.wave % Ops::FW, g.ldb);
    ops.tile.init(tid);
    if constexpr (PIPED && SplitTile<Tile>::value && W == 16)
        piped_schedule_split<S>(T, ops);
    else if constexpr (PIPED)
        piped_schedule<S>(T, ops);
    else
        sync_schedule<S>(T, ops);
    ops.tile.store(g.C, g.ldc, m0, n0, g.M, g.N, g.vec_store != 0);
}

// ---- warp-specialised ring ------------------------------------------------------
//
// The producer/consumer form of the pipeline ("A study on CUDA async memcpy",
// sections "block-scoped pipeline" and the warp-specialisation remark after
// the real-world example): some waves only fill, the others only compute, and
// a pair of per-stage events, "produced" and "consumed", replaces the block
// barrier. gfx950 has no mbarrier, so each event is a cumulative LDS counter:
//   ready[slot]    += 1 by each filling wave once its own fills of the slice
//                  in that slot have landed (its vmcnt counts nothing else);
//   consumed[slot] += 1 by each computing wave once its LDS reads of that
//                  slice have completed (lgkmcnt(0)).
// Slice t uses slot t % S for the (t / S)-th time, so it is ready when
// ready[slot] >= kWsFill * (t / S + 1), and its slot may be refilled with slice
// t + S once consumed[slot] >= kWsCompute * (t / S + 1). Waves of one block are
// co-resident, so every wait is eventually satisfied; a bounded spin still
// guards each wait: on timeout the block marks itself broken, every wave
// leaves its loop and the computing waves write NaN, so a protocol error
// shows up as a wrong result rather than a hang.
constexpr int kWsCompute = 4;          // computing waves (the 2 x 2 compute tile)
constexpr int kWsFill = 4;             // filling waves (same unit split as the 4-wave ring)
constexpr int kWsThreads = 64 * (kWsCompute + kWsFill);
constexpr unsigned kWsSpinLimit = 1u << 22;

struct WsCounters {
    int ready[kMaxPipedStages];
    int consumed[kMaxPipedStages];
    int broken;
};

__device__ inline int lds_load_relaxed(int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Spin until *p >= target. Returns false when the block is (or becomes) broken.
__device__ inline bool ws_wait_ge(int *p, int target, int *broken) {
    for (unsigned i = 0; i < kWsSpinLimit; ++i) {
        if (lds_load_relaxed(p) >= target) {
            asm volatile("" ::: "memory"); // later LDS reads stay after the observed event
            return true;
        }
        if (lds_load_relaxed(broken))
            return false;
        __builtin_amdgcn_s_sleep(1);
    }
    __hip_atomic_store(broken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return false;
}

__device__ inline void ws_arrive(int *p, int lane) {
    if (lane == 0)
        __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <class Cfg, int S, int W>
__global__ void __launch_bounds__(kWsThreads) sgemm_ws_kernel(GemmArgs g) {
    using Tile = typename Cfg::Tile;
    using Ops = PipedOps<Tile, W>;
    static_assert(S >= 1 && S <= kMaxPipedStages, "stages");
    // a ring deeper than the CU's LDS is never planned; its kernel is empty
    constexpr bool kFits = S * Ops::SLOT + (int)sizeof(WsCounters) <= kLdsBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kFits ? S * Ops::SLOT : 1024];
    __shared__ WsCounters ctr;
    if constexpr (!kFits)
        return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid < 2 * kMaxPipedStages + 1)
        ((int *)&ctr)[tid] = 0;
    __syncthreads();

    int tm, tn;
    block_tile(blockIdx.x, g.gm, g.gn, tm, tn);
    const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
    const int T = (g.K + Tile::KPS - 1) / Tile::KPS;

    Ops ops;
    ops.smem = smem;
    ops.lane = lane;
    ops.Ablk = g.A + (size_t)m0 * g.lda;
    ops.Bblk = g.B + n0 / Tile::EPW;
    ops.ldb = g.ldb;
    ops.K = g.K;
    ops.a_cols = g.a_cols;
    ops.a_rows = g.M - m0;
    ops.b_cols = (g.N - n0) / Tile::EPW;

    if (wave >= kWsCompute) {
        // filling wave f: the fills of unit split f of every slice
        ops.wave = wave - kWsCompute;
        ops.oa.init(lane, ops.wave, g.lda);
        ops.ob.init(lane, ops.wave, g.ldb);
        constexpr int L = Ops::OA::U + Ops::OB::U; // fill instructions per slice
        constexpr int D = S >= 2 ? S - 2 : 0;      // slices left in flight when one is signalled
        int signalled = 0;
        for (int t = 0; t < T; ++t) {
            const int slot = t % S;
            if (t >= S && !ws_wait_ge(&ctr.consumed[slot], kWsCompute * (t / S), &ctr.broken)) {
                wait_vm<0>(); // no fill of this wave outlives it
                return;
            }
            ops.issue(t, slot);
            if (t >= D) {
                wait_vm<D * L>();
                ws_arrive(&ctr.ready[signalled % S], lane);
                ++signalled;
            }
        }
        wait_vm<0>();
        for (; signalled < T; ++signalled)
            ws_arrive(&ctr.ready[signalled % S], lane);
        return;
    }

    // computing waves 0..3: the same compute tile as the barrier ring
    ops.tile.init(tid);
    bool ok = true;
    for (int t = 0; t < T && ok; ++t) {
        const int slot = t % S;
        ok = ws_wait_ge(&ctr.ready[slot], kWsFill * (t / S + 1), &ctr.broken);
        if (ok) {
            ops.compute(t, slot);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); // this wave's reads of the slot are done
            ws_arrive(&ctr.consumed[slot], lane);
        }
    }
    if (!ok)
        ops.tile.poison();
    ops.tile.store(g.C, g.ldc, m0, n0, g.M, g.N, g.vec_store != 0);
}

// C[0:M, 0:N] = +0 (the empty sum, K == 0).
__global__ void __launch_bounds__(kThreads) zero_kernel(float *C, int M, int N, int ldc) {
    const int64_t n = (int64_t)M * N;
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        C[(i / N) * (int64_t)ldc + (i % N)] = 0.0f;
}

// ---- pipelined tile copy -----------------------------------------------------------
//
// dst = src through an S-slot ring of 64 x 64 fp32 LDS tiles. Of the block's
// WAVES waves (8 or 16), the first half only fill (asynchronous global -> LDS,
// non-temporal: the data is used once) and the second half only drain (LDS
// -> VGPR -> global, non-temporal stores). Keeping stores out of the filling
// waves keeps their vmcnt a pure count of their own fills, so the ring's
// waits are exact. Block b copies runs b, b + G, b + 2G, ... (G = grid size)
// of R consecutive tiles; the launch makes G the number of runs (one run per
// block), so the blocks in flight, dispatched in order, sweep one window of
// memory.
constexpr int kCopyWavesMax = 16;
constexpr int kAuxNonTemporal = 2; // buffer load cache-policy bit: streaming

struct CopyArgs {
    const float *src;
    float *dst;
    int rows, cols, lds, ldd;
    int tcols;  // tiles per tile-row
    int ntiles;
    int run_log2; // blocks take runs of 2^run_log2 consecutive tiles
};

using CopyLayout = Layout<64, 64, SwzNone>;

template <int W, bool VST, int WAVES>
struct CopyOps {
    static_assert(WAVES == 8 || WAVES == 16, "copy block");
    static constexpr int SLOT = CopyLayout::BYTES;
    static constexpr int PW = WAVES / 2;
    using OP = Operand<CopyLayout, W, PW>;
    CopyArgs a;
    OP op;
    unsigned char *smem;
    int wave, lane, G;
    bool producer;

    // The t-th tile of this block: runs of R = 2^run_log2 consecutive tiles,
    // run j of the block being run blockIdx.x + j G. Ids past the last tile
    // (in a final partial run) land beyond the last row: their loads are
    // masked and their stores skipped.
    __device__ void coords(int t, int &r0, int &c0) const {
        const int R = 1 << a.run_log2;
        const int id = (((int)blockIdx.x + (t >> a.run_log2) * G) << a.run_log2) + (t & (R - 1));
        r0 = (id / a.tcols) * 64;
        c0 = (id % a.tcols) * 64;
    }
    __device__ void issue(int t, int slot) {
        if (!producer)
            return;
        int r0, c0;
        coords(t, r0, c0);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.src + (size_t)r0 * a.lds + c0);
        unsigned char *base = smem + slot * SLOT;
#pragma unroll
        for (int i = 0; i < OP::U; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_t *)(base + OP::lds_off(i, wave)), W,
                                                      op.voff(i, a.rows - r0, a.cols - c0), 0, 0, kAuxNonTemporal);
    }
    template <int P>
    __device__ void wait() {
        if (producer)
            wait_vm<P * OP::U>();
    }
    __device__ void barrier() { lds_barrier(); }
    __device__ void compute(int t, int slot) {
        if (producer)
            return;
        int r0, c0;
        coords(t, r0, c0);
        const unsigned char *base = smem + slot * SLOT;
        constexpr int CW = WAVES - PW;
        static_assert(CopyLayout::CHUNKS % (64 * CW) == 0, "whole chunks per draining wave");
        constexpr int PER = CopyLayout::CHUNKS / (64 * CW);
        const int cw = wave - PW; // drains chunk positions [cw*PER*64, (cw+1)*PER*64)
        f32x4 v[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j)
            v[j] = *(const f32x4 *)(base + ((cw * PER + j) * 64 + lane) * 16);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int p = (cw * PER + j) * 64 + lane;
            const int r = r0 + CopyLayout::row(p);
            const int c = c0 + 4 * CopyLayout::col4(p);
            if (r >= a.rows)
                continue;
            float *d = a.dst + (size_t)r * a.ldd + c;
            if constexpr (VST) {
                if (c < a.cols)
                    __builtin_nontemporal_store(v[j], (f32x4 *)d);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c + e < a.cols)
                        d[e] = v[j][e];
            }
        }
    }
};

template <int S, int W, bool VST, int WAVES>
__global__ void __launch_bounds__(64 * WAVES) tile_copy_kernel(CopyArgs a) {
    using Ops = CopyOps<W, VST, WAVES>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[S * Ops::SLOT];
    Ops ops;
    ops.a = a;
    ops.smem = smem;
    ops.lane = threadIdx.x & 63;
    ops.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    ops.producer = ops.wave < Ops::PW;
    ops.G = gridDim.x;
    ops.op.init(ops.lane, ops.producer ? ops.wave : 0, a.lds);
    const int nruns = (a.ntiles + (1 << a.run_log2) - 1) >> a.run_log2;
    const int T = ((nruns - (int)blockIdx.x + ops.G - 1) / ops.G) << a.run_log2;
    piped_schedule<S>(T, ops);
}

// ---- plain copy (the ceiling the tile copy is read against) -------------------------
//
// dst = src with no LDS and no ring: each lane moves one 16-byte chunk (or
// one 4-byte element where alignment forbids 16) with a non-temporal load
// into a register and a non-temporal store, and the grid holds one lane per
// chunk, dispatched in order. It is the practical HBM copy rate of the
// device, measured the same way as the tile copy.
constexpr int kPlainThreads = 256;

struct PlainCopyArgs {
    const float *src;
    float *dst;
    long long lds, ldd, rows, cpr; // cpr: units (chunks or elements) per row
};

template <int W>
__global__ void __launch_bounds__(kPlainThreads) plain_copy_kernel(PlainCopyArgs a) {
    const long long u = (long long)blockIdx.x * kPlainThreads + threadIdx.x;
    if (u >= a.rows * a.cpr)
        return;
    const long long r = u / a.cpr, c = u - r * a.cpr;
    if constexpr (W == 16) {
        const f32x4 v = __builtin_nontemporal_load((const f32x4 *)(a.src + r * a.lds) + c);
        __builtin_nontemporal_store(v, (f32x4 *)(a.dst + r * a.ldd) + c);
    } else {
        __builtin_nontemporal_store(__builtin_nontemporal_load(a.src + r * a.lds + c), a.dst + r * a.ldd + c);
    }
}

} // namespace mgemm
