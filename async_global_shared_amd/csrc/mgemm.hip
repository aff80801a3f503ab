// mgemm.hip -- the C ABI (include/mgemm.h): argument validation, the launch
// plan, the gfx950 gate and kernel dispatch for the pipelined FP32 GEMM and
// tile copy of device.hpp.
//
// The pages' program refuses a device without the asynchronous copy before
// allocating anything ("pipelined_gemm.cu", main: capability gate) and
// rejects shapes and stage counts its kernels cannot run at compile time
// (static_asserts beside the tile constants). A library cannot exit, so the
// same refusals become status codes returned before any work is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "attention.hpp"
#include "device.hpp"
#include "mgemm.h"

using namespace mgemm;

namespace {

constexpr int64_t kMaxLd = int64_t(1) << 21;     // 256 rows x 2^21 words x 4 B: in-block byte offsets stay below 2^31
constexpr int64_t kMaxExtent = int64_t(1) << 31; // rows * ld per operand, in elements
constexpr int kMaxStages16 = 4;                  // asynchronous ring depth of the 16-bit GEMM
constexpr int64_t kCUs = 256;                    // MI355X compute units, for the planner's wave model

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [lo, hi) byte range of a rows x cols row-major block with leading dimension ld
struct Range {
    uintptr_t lo = 0, hi = 0;
};
Range span(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    Range r;
    if (rows > 0 && cols > 0) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * 4);
    }
    return r;
}
bool overlap(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

int check_matrix(const void *p, int64_t rows, int64_t cols, int64_t ld) {
    if (rows < 0 || cols < 0 || ld < 0)
        return MGEMM_ERR_ARG;
    if (rows > 0 && cols > 0) {
        if (p == nullptr || ld < cols)
            return MGEMM_ERR_ARG;
        if (ld >= kMaxLd || rows * ld >= kMaxExtent)
            return MGEMM_ERR_UNSUPPORTED;
    }
    return MGEMM_OK;
}

int plan_gemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
              const float *C, int64_t ldc, int stages, int fill, int compute, int tile, int loader,
              mgemm_plan_t *pl) {
    if (M < 0 || N < 0 || K < 0)
        return MGEMM_ERR_ARG;
    if (stages < 1 || stages > kMaxPipedStages ||
        (fill != MGEMM_FILL_SYNC && fill != MGEMM_FILL_PIPED && fill != MGEMM_FILL_PIPED_WS) ||
        (fill == MGEMM_FILL_SYNC && stages > kMaxSyncStages) ||
        (compute != MGEMM_COMPUTE_VALU && compute != MGEMM_COMPUTE_MFMA) || tile < MGEMM_TILE_AUTO ||
        tile > MGEMM_TILE_256x128 || loader < MGEMM_LOADER_AUTO || loader > MGEMM_LOADER_B32 ||
        (tile == MGEMM_TILE_256x128 && compute != MGEMM_COMPUTE_MFMA))
        return MGEMM_ERR_ARG;
    int st;
    if ((st = check_matrix(A, M, K, lda)) != MGEMM_OK || (st = check_matrix(B, K, N, ldb)) != MGEMM_OK ||
        (st = check_matrix(C, M, N, ldc)) != MGEMM_OK)
        return st;
    if (M >= kMaxExtent || N >= kMaxExtent || K >= kMaxExtent)
        return MGEMM_ERR_UNSUPPORTED;
    const Range rc = span(C, M, N, ldc);
    if (overlap(rc, span(A, M, K, lda)) || overlap(rc, span(B, K, N, ldb)))
        return MGEMM_ERR_ALIAS;

    // 16-byte lanes need every chunk wholly inside or outside its operand:
    // aligned bases, ld multiple of 4 and contiguous extent multiple of 4.
    const bool b128_ok = aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0 && K % 4 == 0 && N % 4 == 0;
    int W;
    if (loader == MGEMM_LOADER_B128) {
        if (!b128_ok)
            return MGEMM_ERR_ARG;
        W = 16;
    } else if (loader == MGEMM_LOADER_B32) {
        W = 4;
    } else {
        W = b128_ok ? 16 : 4;
    }

    if (tile == MGEMM_TILE_AUTO) {
        // 64x64 or 128x128, whichever has the least estimated time: each of
        // the 256 CUs works through ceil(blocks / 256) tiles, each costing
        // its area over the tile's relative throughput (8192^3, piped S=2:
        // 64x64 runs at 0.90 (VALU) / 0.91 (MFMA) of 128x128), slowed where
        // few blocks share a CU: one wave issues a dependence-free FMA only
        // every few cycles, so the VALU tile needs several waves per SIMD
        // (measured 1.80x slower with one, 1.13x with two, 1.05x with three);
        // the MFMA tile 1.1x with one. Resident blocks are capped by the
        // ring's LDS and by the kernel's registers. Ties keep 128x128.
        const bool valu = compute == MGEMM_COMPUTE_VALU;
        struct Cand {
            int tile, bm, bn, cap;
            double eff;
        };
        const Cand cands[] = {{MGEMM_TILE_128x128, 128, 128, valu ? 4 : 5, 1.0},
                              {MGEMM_TILE_64x64, 64, 64, 8, valu ? 0.90 : 0.91}};
        double best = 0.0;
        for (const Cand &c : cands) {
            const int64_t blocks = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
            const int64_t per_cu = (blocks + 255) / 256;
            const int slot = (c.bm + c.bn) * kBK * 4;
            const int64_t lds_cap = std::max<int64_t>(1, kLdsBytes / (std::max(stages, 1) * slot));
            const int64_t resident = std::min<int64_t>({per_cu, (int64_t)c.cap, lds_cap});
            const double slow = valu ? (resident <= 1 ? 1.80 : resident == 2 ? 1.13 : resident == 3 ? 1.05 : 1.0)
                                     : (resident <= 1 ? 1.10 : 1.0);
            const double t = (double)per_cu * c.bm * c.bn / c.eff * slow;
            if (tile == MGEMM_TILE_AUTO || t < best) {
                tile = c.tile;
                best = t;
            }
        }
        // Where 128x128 wins with MFMA on the asynchronous ring of 2 or 3
        // stages, the 256x128 tile (two resident per CU) takes over when
        // every CU gets an even number of its tiles: it then runs at the
        // 128x128 rate or above and fetches about a third of the HBM bytes
        // (8192^3: 3.6 against 9.5 GB). With an odd or uneven count its last
        // block runs alone on the CU, one wave per SIMD (measured, N = K =
        // 8192, TFLOP/s, 256x128 S=2 / 128x128 S=2: 2, 4, 6, 8, 10, 12 tiles
        // per CU 147.3 / 146.2, 147.9 / 147.7, 148.2 / 147.4, 148.2 / 148.0,
        // 148.1 / 147.9, 148.0 / 148.0; 3, 5, 7, 9, 11 tiles 110 / 146, 125 /
        // 147, 135 / 147, 143 / 147, 146 / 146; S=3 148.3-148.8 against
        // 145.0-146.6 for 128x128 S=3 at 6-12). Every MFMA tile gives the
        // same bits (each accumulator sees the k values in the same order).
        if (tile == MGEMM_TILE_128x128 && !valu && fill == MGEMM_FILL_PIPED && (stages == 2 || stages == 3)) {
            const int64_t big = ((M + 255) / 256) * ((N + 127) / 128);
            if (big >= 512 && big % 512 == 0)
                tile = MGEMM_TILE_256x128;
        }
    }
    const int bm = tile == MGEMM_TILE_256x128 ? 256 : tile == MGEMM_TILE_128x128 ? 128 : 64;
    const int bn = tile == MGEMM_TILE_64x64 ? 64 : 128;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    // the 64x64 MFMA tile's K slice, from the shape alone (so that every
    // fill and depth of one shape runs the same MFMA sequence): 64 k where
    // each of the 256 CUs gets one block at most, else 32 (measured,
    // piped, TFLOP/s: 16384x64x4096 16/32/64 k: 79/97/106; 4099x3001x1537:
    // 117/117/111)
    const int bk = (compute == MGEMM_COMPUTE_MFMA && tile == MGEMM_TILE_64x64) ? (tiles <= kCUs ? 64 : 32) : kBK;
    mgemm_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.compute = compute;
    p.tile = tile;
    p.bm = bm;
    p.bn = bn;
    p.bk = bk;
    p.threads = fill == MGEMM_FILL_PIPED_WS ? kWsThreads : kThreads;
    p.blocks = (int)(((M + bm - 1) / bm) * ((N + bn - 1) / bn));
    p.load_bytes = W;
    p.slices = (int)((K + bk - 1) / bk);
    p.stages = stages;
    p.fill_mode = fill;
    p.lds_bytes = stages * (bm * bk + bk * bn) * 4 + (fill == MGEMM_FILL_PIPED_WS ? (int)sizeof(WsCounters) : 0);
    // one 64-lane instruction moves 64*W bytes; a slice of both operands is
    // (bm+bn)*bk*4 bytes, shared by the 4 waves
    p.loads_per_slice = ((bm + bn) * bk * 4) / (64 * W) / kWaves;
    p.max_vmcnt = fill != MGEMM_FILL_SYNC ? std::min(63, std::max(0, stages - 2) * p.loads_per_slice) : 0;
    if (p.lds_bytes > kLdsBytes) // a ring deeper than the CU's LDS
        return MGEMM_ERR_UNSUPPORTED;
    if (pl)
        *pl = p;
    return MGEMM_OK;
}

// ---- device gate --------------------------------------------------------------

std::atomic<int> g_arch[64]; // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[64];

int current_device(int *dev) {
    if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= 64)
        return MGEMM_ERR_ARCH;
    int a = g_arch[*dev].load(std::memory_order_relaxed);
    if (a == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, *dev) != hipSuccess)
            return MGEMM_ERR_ARCH;
        a = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_cus[*dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        g_arch[*dev].store(a, std::memory_order_relaxed);
    }
    return a == 1 ? MGEMM_OK : MGEMM_ERR_ARCH;
}

// ---- kernel tables ----------------------------------------------------------------

} // namespace

// Every kernel is instantiated explicitly: referencing the templates only
// through the dispatch functions below left some host-side launch stubs
// undefined with this compiler.
#define MG_GEMM_INST(CFG, S, W)                                                                          \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, S, true, W>(mgemm::GemmArgs);               \
    template __global__ void mgemm::sgemm_ws_kernel<mgemm::CFG, S, W>(mgemm::GemmArgs);
#define MG_GEMM_SYNC_INST(CFG, S, W)                                                                     \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, S, false, W>(mgemm::GemmArgs);
#define MG_GEMM_CFG(CFG)                                                                                 \
    MG_GEMM_INST(CFG, 1, 16) MG_GEMM_INST(CFG, 2, 16) MG_GEMM_INST(CFG, 3, 16) MG_GEMM_INST(CFG, 4, 16)  \
    MG_GEMM_INST(CFG, 5, 16) MG_GEMM_INST(CFG, 6, 16) MG_GEMM_INST(CFG, 1, 4) MG_GEMM_INST(CFG, 2, 4)    \
    MG_GEMM_INST(CFG, 3, 4) MG_GEMM_INST(CFG, 4, 4) MG_GEMM_INST(CFG, 5, 4) MG_GEMM_INST(CFG, 6, 4)      \
    MG_GEMM_SYNC_INST(CFG, 1, 16) MG_GEMM_SYNC_INST(CFG, 2, 16) MG_GEMM_SYNC_INST(CFG, 3, 16)            \
    MG_GEMM_SYNC_INST(CFG, 1, 4) MG_GEMM_SYNC_INST(CFG, 2, 4) MG_GEMM_SYNC_INST(CFG, 3, 4)
MG_GEMM_CFG(CfgValu64)
MG_GEMM_CFG(CfgValu128)
MG_GEMM_CFG(CfgMfma64K<32>)
MG_GEMM_CFG(CfgMfma64K<64>)
MG_GEMM_CFG(CfgMfma128)
MG_GEMM_CFG(CfgMfma256x128)
#define MG_GEMM16_INST(CFG, S, W)                                                                        \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, S, true, W>(mgemm::GemmArgs);               \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, S, false, W>(mgemm::GemmArgs);
#define MG_GEMM16_CFG(CFG)                                                                               \
    MG_GEMM16_INST(CFG, 1, 16) MG_GEMM16_INST(CFG, 2, 16) MG_GEMM16_INST(CFG, 3, 16)                     \
    MG_GEMM16_INST(CFG, 1, 4) MG_GEMM16_INST(CFG, 2, 4) MG_GEMM16_INST(CFG, 3, 4)                        \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, 4, true, 16>(mgemm::GemmArgs);              \
    template __global__ void mgemm::sgemm_kernel<mgemm::CFG, 4, true, 4>(mgemm::GemmArgs);
MG_GEMM16_CFG(CfgH128<true>)
MG_GEMM16_CFG(CfgH128<false>)
MG_GEMM16_CFG(CfgH256x128<true>)
MG_GEMM16_CFG(CfgH256x128<false>)
MG_GEMM16_CFG(CfgH256x256<true>)
MG_GEMM16_CFG(CfgH256x256<false>)
#define MG_COPY_INST(S)                                                                                  \
    template __global__ void mgemm::tile_copy_kernel<S, 16, true, 8>(mgemm::CopyArgs);                   \
    template __global__ void mgemm::tile_copy_kernel<S, 16, false, 8>(mgemm::CopyArgs);                  \
    template __global__ void mgemm::tile_copy_kernel<S, 4, true, 8>(mgemm::CopyArgs);                    \
    template __global__ void mgemm::tile_copy_kernel<S, 4, false, 8>(mgemm::CopyArgs);                   \
    template __global__ void mgemm::tile_copy_kernel<S, 16, true, 16>(mgemm::CopyArgs);                  \
    template __global__ void mgemm::tile_copy_kernel<S, 16, false, 16>(mgemm::CopyArgs);                 \
    template __global__ void mgemm::tile_copy_kernel<S, 4, true, 16>(mgemm::CopyArgs);                   \
    template __global__ void mgemm::tile_copy_kernel<S, 4, false, 16>(mgemm::CopyArgs);
template __global__ void mgemm::plain_copy_kernel<16>(mgemm::PlainCopyArgs);
template __global__ void mgemm::plain_copy_kernel<4>(mgemm::PlainCopyArgs);
MG_COPY_INST(1)
MG_COPY_INST(2)
MG_COPY_INST(3)
MG_COPY_INST(4)
MG_COPY_INST(5)
MG_COPY_INST(6)
#define MG_ATTN_INST(D, BF, S, W)                                                                        \
    template __global__ void mgemm::attention_kernel<D, BF, S, true, W>(mgemm::AttnArgs);                \
    template __global__ void mgemm::attention_kernel<D, BF, S, false, W>(mgemm::AttnArgs);
#define MG_ATTN_CFG(D, BF)                                                                               \
    MG_ATTN_INST(D, BF, 1, 16) MG_ATTN_INST(D, BF, 2, 16) MG_ATTN_INST(D, BF, 3, 16)                     \
    MG_ATTN_INST(D, BF, 1, 4) MG_ATTN_INST(D, BF, 2, 4) MG_ATTN_INST(D, BF, 3, 4)                        \
    template __global__ void mgemm::attention_kernel<D, BF, 4, true, 16>(mgemm::AttnArgs);               \
    template __global__ void mgemm::attention_kernel<D, BF, 4, true, 4>(mgemm::AttnArgs);
MG_ATTN_CFG(64, true)
MG_ATTN_CFG(64, false)
MG_ATTN_CFG(128, true)
MG_ATTN_CFG(128, false)

namespace {

template <class Cfg, int S, int W>
const void *gk(int fill) {
    if constexpr (S <= kMaxSyncStages)
        if (fill == MGEMM_FILL_SYNC)
            return (const void *)&sgemm_kernel<Cfg, S, false, W>;
    if (fill == MGEMM_FILL_PIPED_WS)
        return (const void *)&sgemm_ws_kernel<Cfg, S, W>;
    return (const void *)&sgemm_kernel<Cfg, S, true, W>;
}
template <class Cfg, int W>
const void *gemm_kernel_w(int S, int fill) {
    switch (S) {
    case 1: return gk<Cfg, 1, W>(fill);
    case 2: return gk<Cfg, 2, W>(fill);
    case 3: return gk<Cfg, 3, W>(fill);
    case 4: return gk<Cfg, 4, W>(fill);
    case 5: return gk<Cfg, 5, W>(fill);
    default: return gk<Cfg, 6, W>(fill);
    }
}
template <class Cfg>
const void *gemm_kernel(int S, int fill, int W) {
    return W == 16 ? gemm_kernel_w<Cfg, 16>(S, fill) : gemm_kernel_w<Cfg, 4>(S, fill);
}

template <int S, int WAVES>
const void *ck(int W, bool vst) {
    if (W == 16)
        return vst ? (const void *)&tile_copy_kernel<S, 16, true, WAVES>
                   : (const void *)&tile_copy_kernel<S, 16, false, WAVES>;
    return vst ? (const void *)&tile_copy_kernel<S, 4, true, WAVES> : (const void *)&tile_copy_kernel<S, 4, false, WAVES>;
}
template <int WAVES>
const void *copy_kernel_w(int S, int W, bool vst) {
    switch (S) {
    case 1: return ck<1, WAVES>(W, vst);
    case 2: return ck<2, WAVES>(W, vst);
    case 3: return ck<3, WAVES>(W, vst);
    case 4: return ck<4, WAVES>(W, vst);
    case 5: return ck<5, WAVES>(W, vst);
    default: return ck<6, WAVES>(W, vst);
    }
}
const void *copy_kernel(int S, int W, bool vst, int waves) {
    return waves == 16 ? copy_kernel_w<16>(S, W, vst) : copy_kernel_w<8>(S, W, vst);
}

const void *select_gemm(const mgemm_plan_t &p) {
    const int piped = p.fill_mode;
    if (p.compute == MGEMM_COMPUTE_VALU)
        return p.tile == MGEMM_TILE_128x128 ? gemm_kernel<CfgValu128>(p.stages, piped, p.load_bytes)
                                            : gemm_kernel<CfgValu64>(p.stages, piped, p.load_bytes);
    if (p.tile == MGEMM_TILE_256x128)
        return gemm_kernel<CfgMfma256x128>(p.stages, piped, p.load_bytes);
    if (p.tile == MGEMM_TILE_128x128)
        return gemm_kernel<CfgMfma128>(p.stages, piped, p.load_bytes);
    return p.bk == 64 ? gemm_kernel<CfgMfma64K<64>>(p.stages, piped, p.load_bytes)
                      : gemm_kernel<CfgMfma64K<32>>(p.stages, piped, p.load_bytes);
}

int launch(const void *fn, int blocks, void *arg, hipStream_t stream, int threads = kThreads, int dyn_lds = 0) {
    void *args[] = {arg};
    const hipError_t e = hipLaunchKernel(fn, dim3(blocks), dim3(threads), args, dyn_lds, stream);
    return e == hipSuccess ? MGEMM_OK : MGEMM_ERR_LAUNCH;
}

// Resident blocks per CU of a kernel with `dyn` bytes of dynamic LDS per
// block, as the runtime computes them (cached; 0 if the query fails).
int occupancy(const void *fn, int threads, int dyn) {
    static std::mutex mu;
    static std::map<std::pair<const void *, int>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(fn, dyn);
    const auto it = cache.find(key);
    if (it != cache.end())
        return it->second;
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads, dyn) != hipSuccess)
        occ = 0;
    cache[key] = occ;
    return occ;
}

// Residency cap of the fp32 GEMM. When each CU must take exactly one block
// more than it holds (n = b + 1 blocks per CU with b = 3 or 4 resident), the
// blocks of a round run in lockstep and the extra one then runs alone;
// holding ceil(n/2) blocks instead splits the CU's tiles into two even
// rounds. Measured (MFMA 128x128, N = K = 4096, TFLOP/s): piped S=3 with
// 896 / 960 / 1024 tiles 111 / 110 / 116 -> 121 / 134 / 142; sync S=2 with
// 1152 / 1280 tiles 107 / 117 -> 126 / 119; capping any other case (n = b,
// n = b + 2) measured slower. The cap is imposed as unused dynamic LDS and
// applied only if the runtime then reports exactly that residency. Returns
// the dynamic LDS bytes per block (0: no cap) and the resulting residency.
// Not for the 64x64 VALU tile: one wave issues a dependence-free FMA only
// every few cycles, so that small tile needs its resident waves (capped at
// S=6, N=2048 it ran 5 % slower); the 128x128 VALU tile gained 3-5 %.
bool residency_cap_applies(const mgemm_plan_t &p) {
    return !(p.compute == MGEMM_COMPUTE_VALU && p.tile == MGEMM_TILE_64x64);
}

int residency_pad(const void *fn, int threads, int64_t blocks, int cus, int static_lds, int *resident) {
    const int b = occupancy(fn, threads, 0);
    *resident = b;
    if (cus <= 0 || (b != 3 && b != 4))
        return 0;
    const int64_t n = (blocks + cus - 1) / cus;
    if (n != b + 1)
        return 0;
    const int r = (int)((n + 1) / 2);
    const int per_block = (kLdsBytes / r) / 2048 * 2048;
    const int pad = per_block - static_lds;
    if (pad <= 0 || pad > 65536 || occupancy(fn, threads, pad) != r)
        return 0;
    *resident = r;
    return pad;
}

// ---- 16-bit GEMM -------------------------------------------------------------------

int plan_gemm16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                const float *C, int64_t ldc, int dtype, int stages, int fill, int tile, mgemm_plan_t *pl) {
    if (M < 0 || N < 0 || K < 0 || (dtype != MGEMM_DTYPE_BF16 && dtype != MGEMM_DTYPE_F16) || stages < 1 ||
        stages > (fill == MGEMM_FILL_PIPED ? kMaxStages16 : kMaxSyncStages) ||
        (fill != MGEMM_FILL_SYNC && fill != MGEMM_FILL_PIPED) ||
        (tile != MGEMM_TILE_AUTO && tile != MGEMM_TILE_128x128 && tile != MGEMM_TILE_256x128 &&
         tile != MGEMM_TILE_256x256))
        return MGEMM_ERR_ARG;
    // the loaders move 32-bit words: pairs of 16-bit elements along k (A) and n (B)
    // (an empty operand is never read: its base and leading dimension are free)
    const bool a_used = M > 0 && K > 0, b_used = K > 0 && N > 0;
    if (K % 2 || N % 2 || (a_used && (lda % 2 || (reinterpret_cast<uintptr_t>(A) & 3))) ||
        (b_used && (ldb % 2 || (reinterpret_cast<uintptr_t>(B) & 3))))
        return MGEMM_ERR_ARG;
    int st;
    if ((st = check_matrix(A, M, K / 2, lda / 2)) != MGEMM_OK || (st = check_matrix(B, K, N / 2, ldb / 2)) != MGEMM_OK ||
        (st = check_matrix(C, M, N, ldc)) != MGEMM_OK)
        return st;
    if (M > 0 && K > 0 && lda < K)
        return MGEMM_ERR_ARG;
    if (M >= kMaxExtent || N >= kMaxExtent || K >= kMaxExtent)
        return MGEMM_ERR_UNSUPPORTED;
    const Range rc = span(C, M, N, ldc);
    if (overlap(rc, span(A, M, K / 2, lda / 2)) || overlap(rc, span(B, K, N / 2, ldb / 2)))
        return MGEMM_ERR_ALIAS;
    const bool b128_ok = aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0 && K % 8 == 0 && N % 8 == 0;
    const int W = b128_ok ? 16 : 4;
    if (tile == MGEMM_TILE_AUTO) {
        // The tile with the least estimated time: each of the 256 CUs works
        // through ceil(blocks / 256) tiles, each costing its area over the
        // tile's relative throughput (bf16 8192^3, piped S=2: 256x256 1.0,
        // 256x128 0.92, 128x128 0.80). Fewer, larger tiles win while they
        // still fill the CUs' rounds; with 4-byte loads the 8-wave tile would
        // spill (every wave holds 256 VGPRs at most), so it is not a candidate.
        struct Cand {
            int tile, bm, bn;
            double eff;
        };
        const Cand cands[] = {{MGEMM_TILE_256x256, 256, 256, 1.0},
                              {MGEMM_TILE_256x128, 256, 128, 0.92},
                              {MGEMM_TILE_128x128, 128, 128, 0.80}};
        double best = 0.0;
        for (const Cand &c : cands) {
            if (c.tile == MGEMM_TILE_256x256 && W != 16)
                continue;
            const int64_t blocks = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
            const double t = (double)((blocks + 255) / 256) * c.bm * c.bn / c.eff;
            if (tile == MGEMM_TILE_AUTO || t < best) {
                tile = c.tile;
                best = t;
            }
        }
    }
    const int bm = tile == MGEMM_TILE_128x128 ? 128 : 256, bn = tile == MGEMM_TILE_256x256 ? 256 : 128;
    const int waves = tile == MGEMM_TILE_256x256 ? 8 : kWaves;
    constexpr int kps = kK16;
    mgemm_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.compute = MGEMM_COMPUTE_MFMA;
    p.tile = tile;
    p.bm = bm;
    p.bn = bn;
    p.bk = kps;
    p.threads = 64 * waves;
    p.blocks = (int)(((M + bm - 1) / bm) * ((N + bn - 1) / bn));
    p.load_bytes = W;
    p.slices = (int)((K + kps - 1) / kps);
    p.stages = stages;
    p.fill_mode = fill;
    const int slice_bytes = (bm * kps + kps * bn) * 2;
    p.lds_bytes = stages * slice_bytes;
    // per filling wave: with 16-byte loads the 8-wave tile's asynchronous
    // ring fills from 4 waves only
    const int fill_waves = (waves == 8 && fill == MGEMM_FILL_PIPED && W == 16) ? 4 : waves;
    p.loads_per_slice = slice_bytes / (64 * W) / fill_waves;
    p.max_vmcnt = fill == MGEMM_FILL_PIPED ? std::min(63, std::max(0, stages - 2) * p.loads_per_slice) : 0;
    if (p.lds_bytes > kLdsBytes)
        return MGEMM_ERR_UNSUPPORTED;
    if (pl)
        *pl = p;
    return MGEMM_OK;
}

template <class Cfg, int S, int W>
const void *gk16(int fill) {
    return fill == MGEMM_FILL_SYNC ? (const void *)&sgemm_kernel<Cfg, S, false, W>
                                   : (const void *)&sgemm_kernel<Cfg, S, true, W>;
}
template <class Cfg, int W>
const void *gemm16_kernel_w(int S, int fill) {
    switch (S) {
    case 1: return gk16<Cfg, 1, W>(fill);
    case 2: return gk16<Cfg, 2, W>(fill);
    case 3: return gk16<Cfg, 3, W>(fill);
    default: return (const void *)&sgemm_kernel<Cfg, 4, true, W>; // piped only
    }
}
template <class Cfg>
const void *gemm16_kernel(const mgemm_plan_t &p) {
    return p.load_bytes == 16 ? gemm16_kernel_w<Cfg, 16>(p.stages, p.fill_mode)
                              : gemm16_kernel_w<Cfg, 4>(p.stages, p.fill_mode);
}
const void *select_gemm16(const mgemm_plan_t &p, int dtype) {
    const bool big = p.tile == MGEMM_TILE_256x128, w16 = p.load_bytes == 16;
    if (p.tile == MGEMM_TILE_256x256)
        return dtype == MGEMM_DTYPE_BF16 ? gemm16_kernel<CfgH256x256<true>>(p) : gemm16_kernel<CfgH256x256<false>>(p);
    if (dtype == MGEMM_DTYPE_BF16) {
        if (big)
            return w16 ? gemm16_kernel_w<CfgH256x128<true>, 16>(p.stages, p.fill_mode)
                       : gemm16_kernel_w<CfgH256x128<true>, 4>(p.stages, p.fill_mode);
        return w16 ? gemm16_kernel_w<CfgH128<true>, 16>(p.stages, p.fill_mode)
                   : gemm16_kernel_w<CfgH128<true>, 4>(p.stages, p.fill_mode);
    }
    if (big)
        return w16 ? gemm16_kernel_w<CfgH256x128<false>, 16>(p.stages, p.fill_mode)
                   : gemm16_kernel_w<CfgH256x128<false>, 4>(p.stages, p.fill_mode);
    return w16 ? gemm16_kernel_w<CfgH128<false>, 16>(p.stages, p.fill_mode)
               : gemm16_kernel_w<CfgH128<false>, 4>(p.stages, p.fill_mode);
}

// ---- host recorder for mgemm_ring_trace ----------------------------------------------

struct Recorder {
    int *ev;
    int cap, n;
    void put(int op, int a, int b) {
        if (n < cap) {
            ev[3 * n] = op;
            ev[3 * n + 1] = a;
            ev[3 * n + 2] = b;
        }
        ++n;
    }
    void issue(int s, int slot) { put(1, s, slot); }
    template <int P>
    void wait() { put(2, P, 0); }
    void barrier() { put(3, 0, 0); }
    void compute(int s, int slot) { put(4, s, slot); }
    void head(int s, int slot) { put(7, s, slot); }
    void body(int s, int slot) { put(4, s, slot); }
    void tail(int s) { put(8, s, 0); }
    void tail_issue(int tprev, int s, int slot, bool refill) {
        if (refill)
            issue(s, slot);
        tail(tprev);
    }
    template <int SET>
    void store(int slot) { put(5, SET, slot); }
    template <int SET>
    void load(int s) { put(6, s, SET); }
};


// ---- attention ----------------------------------------------------------------------

// [lo, hi) byte range of a (batch, heads, rows, cols) view of `esize`-byte elements
Range span4(const void *p, int64_t batch, int64_t heads, int64_t rows, int64_t cols, int64_t sb, int64_t sh,
            int64_t ld, int esize) {
    Range r;
    if (batch > 0 && heads > 0 && rows > 0 && cols > 0) {
        r.lo = reinterpret_cast<uintptr_t>(p);
        r.hi = r.lo + (uintptr_t)(((batch - 1) * sb + (heads - 1) * sh + (rows - 1) * ld + cols) * esize);
    }
    return r;
}

// Every element of a strided view has its own address: with the
// dimensions of extent > 1 taken in order of stride, each stride exceeds the
// furthest offset the smaller ones reach. (A sufficient test; it accepts
// every permuted dense layout, e.g. (batch, seq, head, dim) storage.)
bool disjoint_view(int n, const int64_t *size, const int64_t *stride) {
    std::pair<int64_t, int64_t> dims[8]; // (stride, extent) of the dimensions with extent > 1
    int k = 0;
    for (int i = 0; i < n && i < 8; ++i)
        if (size[i] > 1)
            dims[k++] = {stride[i], size[i]};
    std::sort(dims, dims + k);
    int64_t reach = 0; // furthest offset the dimensions taken so far reach
    for (int i = 0; i < k; ++i) {
        if (dims[i].first <= reach)
            return false;
        reach += dims[i].first * (dims[i].second - 1);
    }
    return true;
}

struct AttnView {
    const void *p;
    int64_t sb, sh, ld;
};

int check_view16(const AttnView &v, int64_t rows, int64_t D) {
    if (v.p == nullptr || v.sb < 0 || v.sh < 0 || v.ld < D)
        return MGEMM_ERR_ARG;
    // pairs of 16-bit elements are moved as 32-bit words
    if ((reinterpret_cast<uintptr_t>(v.p) & 3) || v.sb % 2 || v.sh % 2 || v.ld % 2)
        return MGEMM_ERR_ARG;
    if (v.ld / 2 >= kMaxLd || rows >= kMaxExtent)
        return MGEMM_ERR_UNSUPPORTED;
    return MGEMM_OK;
}
bool view16_b128(const AttnView &v) { return aligned16(v.p) && v.sb % 8 == 0 && v.sh % 8 == 0 && v.ld % 8 == 0; }

int plan_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t D, const AttnView &q,
                   const AttnView &k, const AttnView &v, const AttnView &o, int dtype, int stages, int fill,
                   mgemm_plan_t *pl) {
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || (D != 64 && D != 128) ||
        (dtype != MGEMM_DTYPE_BF16 && dtype != MGEMM_DTYPE_F16) || stages < 1 ||
        stages > (fill == MGEMM_FILL_PIPED ? kMaxStages16 : kMaxSyncStages) ||
        (fill != MGEMM_FILL_SYNC && fill != MGEMM_FILL_PIPED))
        return MGEMM_ERR_ARG;
    const bool work = batch > 0 && heads > 0 && seq_q > 0;
    mgemm_plan_t p;
    std::memset(&p, 0, sizeof p);
    p.compute = MGEMM_COMPUTE_MFMA;
    p.bm = kAttnBQ;
    p.bn = (int)D;
    p.bk = kAttnBK;
    p.threads = kAttnThreads;
    p.stages = stages;
    p.fill_mode = fill;
    if (work) {
        if (seq_k == 0) // softmax over no keys is undefined
            return MGEMM_ERR_ARG;
        int st;
        if ((st = check_view16(q, seq_q, D)) != MGEMM_OK || (st = check_view16(k, seq_k, D)) != MGEMM_OK ||
            (st = check_view16(v, seq_k, D)) != MGEMM_OK)
            return st;
        if (o.p == nullptr || o.sb < 0 || o.sh < 0 || o.ld < D || (reinterpret_cast<uintptr_t>(o.p) & 3))
            return MGEMM_ERR_ARG;
        if (o.ld >= kMaxLd)
            return MGEMM_ERR_UNSUPPORTED;
        // distinct (batch, head, query, column) outputs need distinct addresses
        const int64_t osize[4] = {batch, heads, seq_q, D}, ostride[4] = {o.sb, o.sh, o.ld, 1};
        if (!disjoint_view(4, osize, ostride))
            return MGEMM_ERR_ALIAS;
        const int64_t nqb = (seq_q + kAttnBQ - 1) / kAttnBQ;
        if (seq_q >= kMaxExtent || seq_k >= kMaxExtent || batch * heads >= kMaxExtent ||
            batch * heads * nqb >= kMaxExtent)
            return MGEMM_ERR_UNSUPPORTED;
        const Range ro = span4(o.p, batch, heads, seq_q, D, o.sb, o.sh, o.ld, 4);
        if (overlap(ro, span4(q.p, batch, heads, seq_q, D, q.sb, q.sh, q.ld, 2)) ||
            overlap(ro, span4(k.p, batch, heads, seq_k, D, k.sb, k.sh, k.ld, 2)) ||
            overlap(ro, span4(v.p, batch, heads, seq_k, D, v.sb, v.sh, v.ld, 2)))
            return MGEMM_ERR_ALIAS;
        p.blocks = (int)(batch * heads * nqb);
        p.slices = (int)((seq_k + kAttnBK - 1) / kAttnBK);
    }
    const int W = (view16_b128(q) && view16_b128(k) && view16_b128(v)) ? 16 : 4;
    p.load_bytes = W;
    const int slice_bytes = 2 * kAttnBK * (int)D * 2; // a K and a V tile
    p.lds_bytes = stages * slice_bytes;
    p.loads_per_slice = slice_bytes / (64 * W) / kAttnWaves;
    p.max_vmcnt = fill == MGEMM_FILL_PIPED ? std::min(63, std::max(0, stages - 2) * p.loads_per_slice) : 0;
    if (p.lds_bytes > kLdsBytes)
        return MGEMM_ERR_UNSUPPORTED;
    if (pl)
        *pl = p;
    return MGEMM_OK;
}

template <int D, bool BF, int W>
const void *attention_kernel_w(int S, int fill) {
    const bool piped = fill == MGEMM_FILL_PIPED;
    switch (S) {
    case 1: return piped ? (const void *)&attention_kernel<D, BF, 1, true, W> : (const void *)&attention_kernel<D, BF, 1, false, W>;
    case 2: return piped ? (const void *)&attention_kernel<D, BF, 2, true, W> : (const void *)&attention_kernel<D, BF, 2, false, W>;
    case 3: return piped ? (const void *)&attention_kernel<D, BF, 3, true, W> : (const void *)&attention_kernel<D, BF, 3, false, W>;
    default: return (const void *)&attention_kernel<D, BF, 4, true, W>; // piped only
    }
}
template <int D, bool BF>
const void *attention_kernel_d(const mgemm_plan_t &p) {
    return p.load_bytes == 16 ? attention_kernel_w<D, BF, 16>(p.stages, p.fill_mode)
                              : attention_kernel_w<D, BF, 4>(p.stages, p.fill_mode);
}
const void *select_attention(const mgemm_plan_t &p, int dtype) {
    const bool bf = dtype == MGEMM_DTYPE_BF16;
    if (p.bn == 64)
        return bf ? attention_kernel_d<64, true>(p) : attention_kernel_d<64, false>(p);
    return bf ? attention_kernel_d<128, true>(p) : attention_kernel_d<128, false>(p);
}

} // namespace

// ---- host-side fill map for mgemm_fill_trace ------------------------------------------
// One slice's fill instructions, enumerated with the operand types and fill
// wave rules the kernels instantiate.

struct FillRecorder {
    int *ev;
    int cap, n;
    void put(int a, int b, int c, int d, int e, int f) {
        if (n < cap) {
            int *p = ev + 6 * n;
            p[0] = a, p[1] = b, p[2] = c, p[3] = d, p[4] = e, p[5] = f;
        }
        ++n;
    }
};

// operand `which` of a slot: its loader type O (units split among the waves
// that fill it), its layout L, byte offset `base` in the slot; wave w fills
// when `fills(w)`
template <class O, class L, int W, class F>
void trace_operand(FillRecorder &rec, int which, int base, int waves, int fw, F fills) {
    for (int w = 0; w < waves; ++w) {
        if (!fills(w))
            continue;
        for (int lane = 0; lane < 64; ++lane) {
            O o;
            o.init(lane, w % fw, 0);
            for (int u = 0; u < O::U; ++u) {
                int r, c;
                o.rc(u, r, c);
                rec.put(which, w, base + O::lds_off(u, w) + lane * W, r, c, base + L::pos(r, c >> 2) * 16 + (c & 3) * 4);
            }
        }
    }
}

template <class Cfg, int W, bool PIPED>
void trace_gemm_fill(FillRecorder &rec) {
    using Tile = typename Cfg::Tile;
    using C = typename std::conditional<PIPED, typename PipedOps<Tile, W>::C, typename SyncOps<Tile, W, 1>::C>::type;
    auto fills = [](int w) { return !PIPED || PipedOps<Tile, W>::fills_wave(w); };
    rec.put(-1, C::SLOT, C::LA::kRows, C::LA::kCols, C::LB::kRows, C::LB::kCols);
    trace_operand<typename C::OA, typename C::LA, W>(rec, 0, 0, Tile::WAVES, C::FW, fills);
    trace_operand<typename C::OB, typename C::LB, W>(rec, 1, C::LA::BYTES, Tile::WAVES, C::FW, fills);
}

template <int D, int W>
void trace_attention_fill(FillRecorder &rec) {
    using Tile = AttnTile<D, true>;
    using C = AttnCtx<Tile, W>;
    auto all = [](int) { return true; };
    rec.put(-1, C::SLOT, C::LK::kRows, C::LK::kCols, C::LV::kRows, C::LV::kCols);
    trace_operand<typename C::OK, typename C::LK, W>(rec, 0, 0, Tile::WAVES, Tile::WAVES, all);
    trace_operand<typename C::OV, typename C::LV, W>(rec, 1, C::LK::BYTES, Tile::WAVES, Tile::WAVES, all);
}

template <int W, int WAVES>
void trace_copy_fill(FillRecorder &rec) {
    using Ops = CopyOps<W, true, WAVES>;
    auto producer = [](int w) { return w < Ops::PW; };
    rec.put(-1, Ops::SLOT, CopyLayout::kRows, CopyLayout::kCols, 0, 0);
    trace_operand<typename Ops::OP, CopyLayout, W>(rec, 0, 0, WAVES, Ops::PW, producer);
}

template <int W, bool PIPED>
bool fill_trace_kind(int kind, FillRecorder &rec) {
    switch (kind) {
    case 0: trace_gemm_fill<CfgValu64, W, PIPED>(rec); return true;
    case 1: trace_gemm_fill<CfgValu128, W, PIPED>(rec); return true;
    case 2: trace_gemm_fill<CfgMfma64K<32>, W, PIPED>(rec); return true;
    case 3: trace_gemm_fill<CfgMfma128, W, PIPED>(rec); return true;
    case 4: trace_gemm_fill<CfgMfma256x128, W, PIPED>(rec); return true;
    case 5: trace_gemm_fill<CfgH128<true>, W, PIPED>(rec); return true;
    case 6: trace_gemm_fill<CfgH256x128<true>, W, PIPED>(rec); return true;
    case 7: trace_gemm_fill<CfgH256x256<true>, W, PIPED>(rec); return true;
    case 8: trace_attention_fill<64, W>(rec); return true;
    case 9: trace_attention_fill<128, W>(rec); return true;
    case 10:
        if (!PIPED)
            return false;
        trace_copy_fill<W, 8>(rec);
        return true;
    case 11: trace_gemm_fill<CfgMfma64K<64>, W, PIPED>(rec); return true;
    case 12:
        if (!PIPED)
            return false;
        trace_copy_fill<W, 16>(rec);
        return true;
    default: return false;
    }
}

extern "C" {

const char *mgemm_status_string(int s) {
    switch (s) {
    case MGEMM_OK: return "ok";
    case MGEMM_ERR_ARG: return "invalid argument";
    case MGEMM_ERR_ALIAS: return "output overlaps an input";
    case MGEMM_ERR_ARCH: return "current device is not gfx950 (or no device)";
    case MGEMM_ERR_LAUNCH: return "kernel launch failed";
    case MGEMM_ERR_UNSUPPORTED: return "extent beyond the supported addressing range";
    default: return "unknown status";
    }
}

int mgemm_version(void) { return MGEMM_VERSION; }

int mgemm_plan_sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                     const float *C, int64_t ldc, int stages, int fill_mode, int compute, int tile, int loader,
                     mgemm_plan_t *plan) {
    return plan_gemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader, plan);
}

int mgemm_sgemm_ex(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                   float *C, int64_t ldc, int stages, int fill_mode, int compute, int tile, int loader,
                   void *stream) {
    mgemm_plan_t p;
    int st = plan_gemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader, &p);
    if (st != MGEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return MGEMM_OK;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t n = M * N;
        const int blocks = (int)std::min<int64_t>((n + kThreads - 1) / kThreads, 4096);
        int m = (int)M, nn = (int)N, l = (int)ldc;
        void *args[] = {&C, &m, &nn, &l};
        const hipError_t e = hipLaunchKernel((const void *)&zero_kernel, dim3(blocks), dim3(kThreads), args, 0, s);
        return e == hipSuccess ? MGEMM_OK : MGEMM_ERR_LAUNCH;
    }
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.lda = (int)lda;
    g.ldb = (int)ldb;
    g.ldc = (int)ldc;
    g.gm = (int)((M + p.bm - 1) / p.bm);
    g.gn = (int)((N + p.bn - 1) / p.bn);
    g.vec_store = aligned16(C) && ldc % 4 == 0;
    g.a_cols = (int)K;
    const void *fn = select_gemm(p);
    int resident;
    const int pad = residency_cap_applies(p)
                        ? residency_pad(fn, p.threads, p.blocks, g_cus[dev].load(std::memory_order_relaxed),
                                        (int)p.lds_bytes, &resident)
                        : 0;
    return launch(fn, p.blocks, &g, s, p.threads, pad);
}

int mgemm_sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                float *C, int64_t ldc, int stages, int fill_mode, void *stream) {
    return mgemm_sgemm_ex(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, MGEMM_COMPUTE_VALU, MGEMM_TILE_AUTO,
                          MGEMM_LOADER_AUTO, stream);
}

int mgemm_plan_gemm16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const float *C, int64_t ldc, int dtype, int stages, int fill_mode, int tile,
                      mgemm_plan_t *plan) {
    return plan_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile, plan);
}

int mgemm_gemm16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb, float *C,
                 int64_t ldc, int dtype, int stages, int fill_mode, int tile, void *stream) {
    mgemm_plan_t p;
    int st = plan_gemm16(M, N, K, A, lda, B, ldb, C, ldc, dtype, stages, fill_mode, tile, &p);
    if (st != MGEMM_OK)
        return st;
    if (M == 0 || N == 0)
        return MGEMM_OK;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (K == 0) {
        const int64_t n = M * N;
        const int blocks = (int)std::min<int64_t>((n + kThreads - 1) / kThreads, 4096);
        int m = (int)M, nn = (int)N, l = (int)ldc;
        void *args[] = {&C, &m, &nn, &l};
        const hipError_t e = hipLaunchKernel((const void *)&zero_kernel, dim3(blocks), dim3(kThreads), args, 0, s);
        return e == hipSuccess ? MGEMM_OK : MGEMM_ERR_LAUNCH;
    }
    GemmArgs g;
    g.A = static_cast<const float *>(A);
    g.B = static_cast<const float *>(B);
    g.C = C;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.lda = (int)(lda / 2);
    g.ldb = (int)(ldb / 2);
    g.ldc = (int)ldc;
    g.gm = (int)((M + p.bm - 1) / p.bm);
    g.gn = (int)((N + p.bn - 1) / p.bn);
    g.vec_store = 0;
    g.a_cols = (int)(K / 2);
    return launch(select_gemm16(p, dtype), p.blocks, &g, s, p.threads);
}

int mgemm_tile_copy(int64_t rows, int64_t cols, const float *src, int64_t lds, float *dst, int64_t ldd, int stages,
                    void *stream) {
    if (stages < 1 || stages > kMaxPipedStages)
        return MGEMM_ERR_ARG;
    int st;
    if ((st = check_matrix(src, rows, cols, lds)) != MGEMM_OK || (st = check_matrix(dst, rows, cols, ldd)) != MGEMM_OK)
        return st;
    if (overlap(span(src, rows, cols, lds), span(dst, rows, cols, ldd)))
        return MGEMM_ERR_ALIAS;
    if (rows == 0 || cols == 0)
        return MGEMM_OK;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    const int W = (aligned16(src) && lds % 4 == 0 && cols % 4 == 0) ? 16 : 4;
    const bool vst = aligned16(dst) && ldd % 4 == 0 && cols % 4 == 0;
    CopyArgs a;
    a.src = src;
    a.dst = dst;
    a.rows = (int)rows;
    a.cols = (int)cols;
    a.lds = (int)lds;
    a.ldd = (int)ldd;
    a.tcols = (int)((cols + 63) / 64);
    const int64_t ntiles = ((rows + 63) / 64) * a.tcols;
    if (ntiles > kMaxExtent - 4) // tile ids of a final partial run stay below 2^31
        return MGEMM_ERR_UNSUPPORTED;
    a.ntiles = (int)ntiles;
    // One block per run of 2 adjacent tiles (1 tile without a ring to
    // pipeline through), the whole grid in one launch: blocks are dispatched
    // in order as others retire, so the blocks in flight cover one sliding
    // window of memory. Measured on the 1 GiB copy, S=3 (TB/s, 16384-wide /
    // 64-wide views): this grid 6.10 / 6.09; a persistent grid taking every
    // G-th run of 4 (resp. 1) tiles 5.78 / 5.89; runs of 4 in this grid
    // 5.98 / 5.87.
    a.run_log2 = stages >= 2 ? 1 : 0;
    // Blocks of 16 waves (8 filling, 8 draining) or 8 (4 + 4). Measured on
    // the 1 GiB copy (TB/s, 8 / 16 waves): S=2 faster with 16 at every tile-row
    // width from 1 to 1024 tiles (16384-wide 5.96 / 6.34, 64-wide 6.14 /
    // 6.30); S=3 faster with 16 from 4 tiles per tile-row up (16384-wide
    // 6.09 / 6.40, 1024-wide 6.19 / 6.53), slower with one or two (64-wide
    // 6.12 / 5.62, 128-wide 6.15 / 5.63); S=1 (one tile per block) faster
    // with 8 on contiguous tiles (64-wide 6.34 / 6.00).
    const int waves = (stages == 2 || (stages >= 3 && a.tcols > 2)) ? 16 : 8;
    const void *fn = copy_kernel(stages, W, vst, waves);
    const int64_t runs = (ntiles + (1 << a.run_log2) - 1) >> a.run_log2;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return launch(fn, (int)runs, &a, s, 64 * waves);
}

int mgemm_plain_copy(int64_t rows, int64_t cols, const float *src, int64_t lds, float *dst, int64_t ldd,
                     void *stream) {
    int st;
    if ((st = check_matrix(src, rows, cols, lds)) != MGEMM_OK || (st = check_matrix(dst, rows, cols, ldd)) != MGEMM_OK)
        return st;
    if (overlap(span(src, rows, cols, lds), span(dst, rows, cols, ldd)))
        return MGEMM_ERR_ALIAS;
    if (rows == 0 || cols == 0)
        return MGEMM_OK;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    const bool w16 = aligned16(src) && aligned16(dst) && lds % 4 == 0 && ldd % 4 == 0 && cols % 4 == 0;
    PlainCopyArgs a;
    a.src = src;
    a.dst = dst;
    a.lds = lds;
    a.ldd = ldd;
    a.rows = rows;
    a.cpr = w16 ? cols / 4 : cols;
    const int64_t units = rows * a.cpr;
    const int64_t blocks = (units + kPlainThreads - 1) / kPlainThreads;
    return launch(w16 ? (const void *)&plain_copy_kernel<16> : (const void *)&plain_copy_kernel<4>, (int)blocks, &a,
                  reinterpret_cast<hipStream_t>(stream), kPlainThreads);
}

int mgemm_blocks_per_cu(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                        const float *C, int64_t ldc, int stages, int fill_mode, int compute, int tile, int loader,
                        int *blocks_per_cu) {
    mgemm_plan_t p;
    int st = plan_gemm(M, N, K, A, lda, B, ldb, C, ldc, stages, fill_mode, compute, tile, loader, &p);
    if (st != MGEMM_OK)
        return st;
    if (blocks_per_cu == nullptr)
        return MGEMM_ERR_ARG;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    const void *fn = select_gemm(p);
    int resident = occupancy(fn, p.threads, 0);
    if (resident < 1)
        return MGEMM_ERR_LAUNCH;
    if (residency_cap_applies(p))
        residency_pad(fn, p.threads, p.blocks, g_cus[dev].load(std::memory_order_relaxed), (int)p.lds_bytes,
                      &resident);
    *blocks_per_cu = resident;
    return MGEMM_OK;
}

int mgemm_fill_trace(int kind, int load_bytes, int fill_mode, int *events, int cap) {
    if ((load_bytes != 16 && load_bytes != 4) || (fill_mode != MGEMM_FILL_SYNC && fill_mode != MGEMM_FILL_PIPED) ||
        cap < 0 || (cap > 0 && events == nullptr))
        return MGEMM_ERR_ARG;
    FillRecorder rec{events, cap, 0};
    const bool piped = fill_mode == MGEMM_FILL_PIPED;
    const bool ok = load_bytes == 16 ? (piped ? fill_trace_kind<16, true>(kind, rec) : fill_trace_kind<16, false>(kind, rec))
                                     : (piped ? fill_trace_kind<4, true>(kind, rec) : fill_trace_kind<4, false>(kind, rec));
    return ok ? rec.n : MGEMM_ERR_ARG;
}

int mgemm_ring_trace(int kind, int stages, int fill_mode, int slices, int *events, int cap) {
    if (stages < 1 || slices < 0 || cap < 0 || (cap > 0 && events == nullptr) || kind < 0 || kind > 2 ||
        (fill_mode != MGEMM_FILL_SYNC && fill_mode != MGEMM_FILL_PIPED) ||
        (kind != 0 && fill_mode != MGEMM_FILL_PIPED) ||
        stages > (fill_mode == MGEMM_FILL_PIPED ? kMaxPipedStages : kMaxSyncStages))
        return MGEMM_ERR_ARG;
    Recorder r{events, cap, 0};
    if (kind == 2) {
        switch (stages) {
        case 1: piped_schedule_split<1>(slices, r); break;
        case 2: piped_schedule_split<2>(slices, r); break;
        case 3: piped_schedule_split<3>(slices, r); break;
        case 4: piped_schedule_split<4>(slices, r); break;
        case 5: piped_schedule_split<5>(slices, r); break;
        default: piped_schedule_split<6>(slices, r); break;
        }
    } else if (fill_mode == MGEMM_FILL_PIPED) {
        switch (stages) {
        case 1: piped_schedule<1>(slices, r); break;
        case 2: piped_schedule<2>(slices, r); break;
        case 3: piped_schedule<3>(slices, r); break;
        case 4: piped_schedule<4>(slices, r); break;
        case 5: piped_schedule<5>(slices, r); break;
        default: piped_schedule<6>(slices, r); break;
        }
    } else {
        switch (stages) {
        case 1: sync_schedule<1>(slices, r); break;
        case 2: sync_schedule<2>(slices, r); break;
        default: sync_schedule<3>(slices, r); break;
        }
    }
    return r.n;
}

int mgemm_plan_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                         const void *Q, int64_t q_sb, int64_t q_sh, int64_t q_ld, const void *K, int64_t k_sb,
                         int64_t k_sh, int64_t k_ld, const void *V, int64_t v_sb, int64_t v_sh, int64_t v_ld,
                         const float *O, int64_t o_sb, int64_t o_sh, int64_t o_ld, int dtype, int stages,
                         int fill_mode, mgemm_plan_t *plan) {
    return plan_attention(batch, heads, seq_q, seq_k, head_dim, {Q, q_sb, q_sh, q_ld}, {K, k_sb, k_sh, k_ld},
                          {V, v_sb, v_sh, v_ld}, {O, o_sb, o_sh, o_ld}, dtype, stages, fill_mode, plan);
}

int mgemm_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim, const void *Q,
                    int64_t q_sb, int64_t q_sh, int64_t q_ld, const void *K, int64_t k_sb, int64_t k_sh,
                    int64_t k_ld, const void *V, int64_t v_sb, int64_t v_sh, int64_t v_ld, float *O, int64_t o_sb,
                    int64_t o_sh, int64_t o_ld, float scale, int dtype, int stages, int fill_mode, void *stream) {
    mgemm_plan_t p;
    int st = plan_attention(batch, heads, seq_q, seq_k, head_dim, {Q, q_sb, q_sh, q_ld}, {K, k_sb, k_sh, k_ld},
                            {V, v_sb, v_sh, v_ld}, {O, o_sb, o_sh, o_ld}, dtype, stages, fill_mode, &p);
    if (st != MGEMM_OK)
        return st;
    if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
        return MGEMM_ERR_ARG;
    if (batch == 0 || heads == 0 || seq_q == 0)
        return MGEMM_OK;
    int dev;
    if ((st = current_device(&dev)) != MGEMM_OK)
        return st;
    AttnArgs a;
    a.Q = static_cast<const float *>(Q);
    a.K = static_cast<const float *>(K);
    a.V = static_cast<const float *>(V);
    a.O = O;
    a.q_sb = q_sb / 2;
    a.q_sh = q_sh / 2;
    a.k_sb = k_sb / 2;
    a.k_sh = k_sh / 2;
    a.v_sb = v_sb / 2;
    a.v_sh = v_sh / 2;
    a.o_sb = o_sb;
    a.o_sh = o_sh;
    a.q_ld = (int)(q_ld / 2);
    a.k_ld = (int)(k_ld / 2);
    a.v_ld = (int)(v_ld / 2);
    a.o_ld = (int)o_ld;
    a.heads = (int)heads;
    a.seq_q = (int)seq_q;
    a.seq_k = (int)seq_k;
    a.nqb = (int)((seq_q + kAttnBQ - 1) / kAttnBQ);
    a.nblocks = p.blocks;
    a.c = (float)((double)scale * 1.4426950408889634); // log2(e)
    a.vec_store = aligned16(O) && o_sb % 4 == 0 && o_sh % 4 == 0 && o_ld % 4 == 0;
    return launch(select_attention(p, dtype), p.blocks, &a, reinterpret_cast<hipStream_t>(stream), p.threads);
}

} // extern "C"
