// attention.hpp -- scaled dot-product attention forward on the asynchronous
// K/V ring, for gfx950 (CDNA4).
//
// The async copy article ("from cp.async to memcpy_async"), section 6.2,
// "FlashAttention's tile pipeline":
// a block keeps its Q tile for the whole loop, the K/V tiles stream through
// the LDS ring (the next one in flight while the current one is scored), and
// each step rescales and accumulates the running result (the online
// softmax). The ring, its loaders and its waits are the GEMM's; only the
// per-slice step differs.
//
// Per block 8 waves x 32 queries of one (batch, head); per slice 64 keys.
// Each wave works in the transposed form so that a lane owns one query:
//   S^T (64 keys x 32 queries) = K (from LDS) . Q^T (registers, loaded once)
//   O^T (D x 32 queries)      += V^T (transposing LDS reads) . P^T
// where P^T comes straight out of the S^T accumulators: the 16 scores a lane
// holds for its query in a 32 x 32 tile (keys 8(i/4) + 4(l/32) + i%4) are,
// 8 at a time, exactly the k values of one MFMA B operand, and the V reads
// deliver V rows in the same k order. Scores live in the log2 domain
// (x = scale * log2(e) * s) so that v_exp_f32 (2^x) serves for exp.
#pragma once

#include "device.hpp"

namespace mgemm {

constexpr int kAttnBK = 64;                 // keys per ring slice
constexpr int kAttnWaves = 8;               // waves per block (2 per SIMD), 32 queries each
constexpr float kLazyRescale = 8.0f;        // log2 headroom before the running maximum moves
constexpr int kAttnBQ = 32 * kAttnWaves;    // queries per block
constexpr int kAttnThreads = 64 * kAttnWaves;

// K slice rows (D/2 words): the 32 consecutive rows of one ds_read_b128 land
// on distinct 16-byte bank groups.
template <int CPR>
struct SwzKeys;
template <>
struct SwzKeys<16> { // 256-byte rows (D = 128)
    MG_HD static constexpr int f(int r) { return r & 15; }
};
template <>
struct SwzKeys<8> { // 128-byte rows (D = 64)
    MG_HD static constexpr int f(int r) { return (r >> 1) & 7; }
};
// V slice rows: the 4 rows x 64 bytes of one half-wave's transposing read
// land on distinct bank groups.
template <int CPR>
struct SwzVals;
template <>
struct SwzVals<16> {
    MG_HD static constexpr int f(int r) { return (r & 3) << 2; }
};
template <>
struct SwzVals<8> {
    MG_HD static constexpr int f(int r) { return ((r >> 1) & 1) << 2; }
};

// Q, K and V are addressed as 32-bit words (pairs of 16-bit elements); their
// strides are in words, O's in floats.
struct AttnArgs {
    const float *Q, *K, *V;
    float *O;
    long long q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;
    int q_ld, k_ld, v_ld, o_ld;
    int heads, seq_q, seq_k, nqb, nblocks;
    float c; // scale * log2(e)
    int vec_store;
};

__device__ inline unsigned lds_addr(const unsigned char *p) {
    return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

// max / sum of a value over the two lanes (l, l ^ 32) that hold one query
__device__ inline float pair_max(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float pair_sum(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <int D, bool BF16>
struct AttnTile {
    static constexpr int BK = kAttnBK, CPR = D / 8, NDS = D / 16, NDT = D / 32, NKT = BK / 32, NKK = BK / 16;
    static constexpr int WAVES = kAttnWaves;
    static_assert(D == 64 || D == 128, "head dimension");
    using LK = Layout<BK, D / 2, SwzKeys<CPR>>;
    using LV = Layout<BK, D / 2, SwzVals<CPR>>;
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x8 __attribute__((ext_vector_type(8)));

    u32x4 qf[NDS]; // this lane's query: elements 16 ds + 8 (l/32) .. +7
    f32x16 o[NDT]; // O^T tiles (dv tile dt, this wave's 32 queries)
    float mrow, lrow, c;
    int lane;

    // ---- LDS reads from inline asm (see the 16-bit GEMM tile: the compiler's
    // wait pass would otherwise drain the in-flight fills before them) ----
    template <int O1>
    __device__ static void read_k(unsigned a, u32x4 &k0, u32x4 &k1) {
        asm volatile("ds_read_b128 %0, %2\n\t"
                     "ds_read_b128 %1, %2 offset:%3"
                     : "=&v"(k0), "=&v"(k1)
                     : "v"(a), "i"(O1));
    }
    __device__ static void wait_k(u32x4 &k0, u32x4 &k1) {
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k0), "+v"(k1));
    }
    // V^T fragments of one 16-key step for every dv tile: two transposing
    // reads (rows k0 .. k0+3 and k0+8 .. k0+11) per tile
    template <int OA, int OB>
    __device__ static void read_v(const unsigned *a, i16x4 (&v)[NDT][2]) {
        if constexpr (NDT == 4)
            asm volatile("ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
                         "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
                         "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
                         "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
                         "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
                         "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
                         "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
                         "ds_read_b64_tr_b16 %7, %11 offset:%13"
                         : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1]), "=&v"(v[2][0]),
                           "=&v"(v[2][1]), "=&v"(v[3][0]), "=&v"(v[3][1])
                         : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OA), "i"(OB));
        else
            asm volatile("ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
                         "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
                         "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
                         "ds_read_b64_tr_b16 %3, %5 offset:%7"
                         : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[1][0]), "=&v"(v[1][1])
                         : "v"(a[0]), "v"(a[1]), "i"(OA), "i"(OB));
    }
    __device__ static void wait_v(i16x4 (&v)[NDT][2]) {
        if constexpr (NDT == 4)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[2][0]), "+v"(v[2][1]),
                           "+v"(v[3][0]), "+v"(v[3][1]));
        else
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]), "+v"(v[1][1]));
    }

    __device__ static f32x16 mma(u32x4 a, u32x4 b, f32x16 acc) {
        if constexpr (BF16)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                           acc, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                          acc, 0, 0, 0);
    }
    __device__ static u32x4 pack(f32x8 p) {
        if constexpr (BF16)
            return __builtin_bit_cast(u32x4, __builtin_convertvector(p, bf16x8));
        else
            return __builtin_bit_cast(u32x4, __builtin_convertvector(p, f16x8));
    }

    // Load this lane's query row (zero beyond seq_q) and clear the state. A
    // negative scale is folded into the sign of Q (every 16-bit element's
    // sign bit flipped: the MFMA then forms exactly -s, as its products and
    // round-to-nearest sums are sign-symmetric), so that c >= 0.
    template <int W>
    __device__ void init(int tid, const float *Qh, int q_ld, int row, int seq_q, float c_) {
        lane = tid & 63;
        c = c_ < 0.0f ? -c_ : c_;
        mrow = -__builtin_inff();
        lrow = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                o[dt][i] = 0.0f;
        const __amdgpu_buffer_rsrc_t r = make_rsrc(Qh);
        const int h = lane >> 5;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            const unsigned off = (unsigned)(row * q_ld + 8 * ds + 4 * h) * 4u;
            const unsigned voff = row < seq_q ? off : kMasked;
            if constexpr (W == 16) {
                qf[ds] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    qf[ds][j] = __builtin_amdgcn_raw_buffer_load_b32(r, row < seq_q ? off + 4 * j : kMasked, 0, 0);
            }
        }
        if (c_ < 0.0f) { // block-uniform
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds)
                qf[ds] ^= 0x80008000u;
        }
    }

    static constexpr int KT1 = 32 * CPR * 16; // the second 32-key tile, 32 rows on (the swizzle repeats)

    // Online softmax over one slice's scores s (replaced by the
    // probabilities). x = c s with c = scale log2(e) >= 0 (init() folds a
    // negative scale into the sign of Q); p = 2^(x - m) is formed as one fma,
    // 2^(fma(s, c, -m)), with m a running reference at most kLazyRescale
    // below the maximum of x so far (c times the raw maximum). Keys >= seq_k
    // (FULL false: the last slice) get p = 0. O is rescaled unless every
    // lane's reference stayed put (alpha == 1 exactly: x * 1 == x, so
    // skipping changes no bit).
    template <bool FULL>
    __device__ void softmax(f32x16 (&s)[NKT], int key0, int seq_k) {
        const int h = lane >> 5;
        auto valid = [&](int kt, int i) { return key0 + 32 * kt + 8 * (i >> 2) + 4 * h + (i & 3) < seq_k; };
        float ext = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                ext = fmaxf(ext, FULL || valid(kt, i) ? s[kt][i] : -__builtin_inff());
        // the running maximum moves only when the slice's exceeds it by more
        // than kLazyRescale (log2 units); otherwise the probabilities of this
        // slice may reach 2^kLazyRescale, which fp32 sums and the 16-bit P
        // hold with the same relative rounding. Softmax does not depend on
        // the shift, so O = sum p v / sum p is unchanged, and most slices
        // then skip the rescale of O below.
        const float mcand = fmaxf(mrow, c * pair_max(ext)); // finite: key0 < seq_k
        const float mnew = mcand > mrow + kLazyRescale ? mcand : mrow;
        const float alpha = __builtin_amdgcn_exp2f(mrow - mnew);
        float rs = 0.0f;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], c, -mnew));
                if constexpr (!FULL)
                    p = valid(kt, i) ? p : 0.0f;
                s[kt][i] = p;
                rs += p;
            }
        lrow = lrow * alpha + pair_sum(rs);
        mrow = mnew;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    o[dt][i] *= alpha;
        }
    }

    // One ring slice: keys key0 .. key0 + 63 of this head (those >= seq_k are
    // masked out; their K and V rows arrive as zeros).
    __device__ void step(const unsigned char *Ks, const unsigned char *Vs, int key0, int seq_k) {
        const int h = lane >> 5, l32 = lane & 31, q = lane & 15, g16 = (lane >> 4) & 1;
        const unsigned ks = lds_addr(Ks), vs = lds_addr(Vs);

        // ---- S^T = K Q^T, d steps pipelined one ahead ----
        f32x16 s[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s[kt][i] = 0.0f;
        u32x4 kf[2][NKT];
        read_k<KT1>(ks + LK::pos(l32, h) * 16, kf[0][0], kf[0][1]);
        wait_k(kf[0][0], kf[0][1]);
        static_for<0, NDS>([&](auto dsc) {
            constexpr int ds = decltype(dsc)::value;
            if constexpr (ds + 1 < NDS)
                read_k<KT1>(ks + LK::pos(l32, 2 * (ds + 1) + h) * 16, kf[(ds + 1) & 1][0], kf[(ds + 1) & 1][1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                s[kt] = mma(kf[ds & 1][kt], qf[ds], s[kt]);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ds + 1 < NDS)
                wait_k(kf[(ds + 1) & 1][0], kf[(ds + 1) & 1][1]);
        });

        // ---- online softmax (log2 domain) ----
        // only the last slice can hold keys >= seq_k (a block-uniform test);
        // at head dim 64 one masked copy keeps the registers for 4 waves per SIMD
        if (D == 128 && key0 + BK <= seq_k)
            softmax<true>(s, key0, seq_k);
        else
            softmax<false>(s, key0, seq_k);

        // ---- O^T += V^T P^T, 16-key steps pipelined one ahead ----
        u32x4 pf[NKK];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            f32x8 p8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                p8[j] = s[kk >> 1][8 * (kk & 1) + j];
            pf[kk] = pack(p8);
        }
        // lane part of the V read address: row 4h + q/4 of the 16-key step,
        // columns 32 dt + 16 g16 + 4 (q % 4) .. +3
        unsigned av[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int n = 32 * dt + 16 * g16 + 4 * (q & 3);
            av[dt] = vs + LV::pos(4 * h + (q >> 2), n >> 3) * 16 + (n & 7) * 2;
        }
        constexpr int ROW = CPR * 16; // bytes per V row
        i16x4 vf[2][NDT][2];
        read_v<0, 8 * ROW>(av, vf[0]);
        wait_v(vf[0]);
        static_for<0, NKK>([&](auto kkc) {
            constexpr int kk = decltype(kkc)::value;
            if constexpr (kk + 1 < NKK)
                read_v<16 * (kk + 1) * ROW, (16 * (kk + 1) + 8) * ROW>(av, vf[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const i16x4 lo = vf[kk & 1][dt][0], hi = vf[kk & 1][dt][1];
                const i16x8 v8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[dt] = mma(__builtin_bit_cast(u32x4, v8), pf[kk], o[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (kk + 1 < NKK)
                wait_v(vf[(kk + 1) & 1]);
        });
    }

    // O[row][32 dt + 8 (i/4) + 4 (l/32) + i%4] = o[dt][i] / l
    __device__ void store(float *Oh, int o_ld, int row, int seq_q, bool vec) const {
        if (row >= seq_q)
            return;
        const int h = lane >> 5;
        const float inv = 1.0f / lrow;
        float *out = Oh + (size_t)row * o_ld;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * dt + 8 * g + 4 * h;
                if (vec) {
                    float4 v;
                    v.x = o[dt][4 * g] * inv;
                    v.y = o[dt][4 * g + 1] * inv;
                    v.z = o[dt][4 * g + 2] * inv;
                    v.w = o[dt][4 * g + 3] * inv;
                    *(float4 *)(out + col) = v;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        out[col + j] = o[dt][4 * g + j] * inv;
                }
            }
    }
};

// State one block shares between its ring operations.
template <class Tile, int W>
struct AttnCtx {
    using LK = typename Tile::LK;
    using LV = typename Tile::LV;
    using OK = Operand<LK, W, Tile::WAVES>;
    using OV = Operand<LV, W, Tile::WAVES>;
    static constexpr int SLOT = LK::BYTES + LV::BYTES;
    static constexpr int COLS = LK::kCols; // words per K / V row

    OK ok;
    OV ov;
    Tile tile;
    unsigned char *smem;
    int wave, lane;
    const float *Kh, *Vh; // this head's K and V
    int k_ld, v_ld, seq_k;

    __device__ const float *k_ptr(int s) const { return Kh + (size_t)s * kAttnBK * k_ld; }
    __device__ const float *v_ptr(int s) const { return Vh + (size_t)s * kAttnBK * v_ld; }
    __device__ int rows(int s) const { return seq_k - s * kAttnBK; }
    __device__ void barrier() { lds_barrier(); }
    __device__ void compute(int s, int slot) {
        const unsigned char *base = smem + slot * SLOT;
        tile.step(base, base + LK::BYTES, s * kAttnBK, seq_k);
    }
};

template <class Tile, int W>
struct AttnPipedOps : AttnCtx<Tile, W> {
    using C = AttnCtx<Tile, W>;
    __device__ void issue(int s, int slot) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(this->k_ptr(s));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(this->v_ptr(s));
        const int rows = this->rows(s);
        unsigned char *base = this->smem + slot * C::SLOT;
        if (__builtin_expect(rows >= kAttnBK, 1)) { // a full slice: no masks (a block-uniform branch)
#pragma unroll
            for (int i = 0; i < C::OK::U; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_t *)(base + C::OK::lds_off(i, this->wave)), W,
                                                          this->ok.voff_in(i), 0, 0, 0);
#pragma unroll
            for (int i = 0; i < C::OV::U; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (lds_t *)(base + C::LK::BYTES + C::OV::lds_off(i, this->wave)), W, this->ov.voff_in(i), 0, 0,
                    0);
            return;
        }
#pragma unroll
        for (int i = 0; i < C::OK::U; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_t *)(base + C::OK::lds_off(i, this->wave)), W,
                                                      this->ok.voff(i, rows, C::COLS), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::OV::U; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_t *)(base + C::LK::BYTES + C::OV::lds_off(i, this->wave)),
                                                      W, this->ov.voff(i, rows, C::COLS), 0, 0, 0);
    }
    template <int P>
    __device__ void wait() {
        wait_vm<P *(C::OK::U + C::OV::U)>();
    }
};

template <class Tile, int W, int NSET>
struct AttnSyncOps : AttnCtx<Tile, W> {
    using C = AttnCtx<Tile, W>;
    using R = typename RegOf<W>::type;
    R vk[NSET][C::OK::U];
    R vv[NSET][C::OV::U];

    __device__ static R ld(__amdgpu_buffer_rsrc_t r, unsigned off) {
        if constexpr (W == 16)
            return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        else
            return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    // A slice past the last one (rows <= 0) masks every lane; its descriptors
    // are built on slice 0's addresses so that none points past K or V.
    template <int SET>
    __device__ void load(int s) {
        const int rows = this->rows(s);
        const int sp = rows > 0 ? s : 0;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(this->k_ptr(sp));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(this->v_ptr(sp));
        // two register sets or more: one load form, kept ahead of the compute
        // (as in the GEMM's register-staged ring; with the full-slice fast
        // path as well, S=3 measured 668 -> 608 TFLOP/s at D = 64)
        if (NSET == 1 && __builtin_expect(rows >= kAttnBK, 1)) {
#pragma unroll
            for (int i = 0; i < C::OK::U; ++i)
                vk[SET][i] = ld(rk, this->ok.voff_in(i));
#pragma unroll
            for (int i = 0; i < C::OV::U; ++i)
                vv[SET][i] = ld(rv, this->ov.voff_in(i));
            return;
        }
#pragma unroll
        for (int i = 0; i < C::OK::U; ++i)
            vk[SET][i] = ld(rk, this->ok.voff(i, rows, C::COLS));
#pragma unroll
        for (int i = 0; i < C::OV::U; ++i)
            vv[SET][i] = ld(rv, this->ov.voff(i, rows, C::COLS));
        if constexpr (NSET > 1)
            __builtin_amdgcn_sched_barrier(0);
    }
    template <int SET>
    __device__ void store(int slot) {
        unsigned char *base = this->smem + slot * C::SLOT;
#pragma unroll
        for (int i = 0; i < C::OK::U; ++i)
            *(R *)(base + C::OK::lds_off(i, this->wave) + this->lane * W) = vk[SET][i];
#pragma unroll
        for (int i = 0; i < C::OV::U; ++i)
            *(R *)(base + C::LK::BYTES + C::OV::lds_off(i, this->wave) + this->lane * W) = vv[SET][i];
    }
};

// Two waves per SIMD at least: one wave's softmax overlaps the other's MFMAs.
template <int D>
constexpr int kAttnWavesPerEu = 2;

template <int D, bool BF16, int S, bool PIPED, int W>
__global__ void __launch_bounds__(kAttnThreads)
    __attribute__((amdgpu_waves_per_eu(kAttnWavesPerEu<D>))) attention_kernel(AttnArgs a) {
    using Tile = AttnTile<D, BF16>;
    using Ctx = AttnCtx<Tile, W>;
    constexpr bool kFits = S * Ctx::SLOT <= kLdsBytes;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kFits ? S * Ctx::SLOT : 1024];
    if constexpr (!kFits)
        return;

    // (batch, head, query block) of this workgroup; the query blocks of one
    // head stay on one XCD, whose L2 then serves its K and V to all of them
    const int lin = xcd_linear(blockIdx.x, a.nblocks);
    const int bh = lin / a.nqb, qb = lin - bh * a.nqb;
    const int b = bh / a.heads, hd = bh - b * a.heads;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q0 = qb * kAttnBQ + 32 * wave;

    using Ops = typename std::conditional<PIPED, AttnPipedOps<Tile, W>, AttnSyncOps<Tile, W, (S > 1 ? S - 1 : 1)>>::type;
    Ops ops;
    ops.smem = smem;
    ops.lane = tid & 63;
    ops.wave = wave;
    ops.Kh = a.K + b * a.k_sb + hd * a.k_sh;
    ops.Vh = a.V + b * a.v_sb + hd * a.v_sh;
    ops.k_ld = a.k_ld;
    ops.v_ld = a.v_ld;
    ops.seq_k = a.seq_k;
    ops.ok.init(ops.lane, wave, a.k_ld);
    ops.ov.init(ops.lane, wave, a.v_ld);
    const float *Qh = a.Q + b * a.q_sb + hd * a.q_sh + (size_t)q0 * a.q_ld;
    ops.tile.template init<W>(tid, Qh, a.q_ld, tid & 31, a.seq_q - q0, a.c);
    const int T = (a.seq_k + kAttnBK - 1) / kAttnBK;
    if constexpr (PIPED)
        piped_schedule<S>(T, ops);
    else
        sync_schedule<S>(T, ops);
    float *Oh = a.O + b * a.o_sb + hd * a.o_sh + (size_t)q0 * a.o_ld;
    ops.tile.store(Oh, a.o_ld, tid & 31, a.seq_q - q0, a.vec_store != 0);
}

} // namespace mgemm
