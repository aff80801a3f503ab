/*
 * mgemm.h -- C ABI of the MI355X (gfx950) pipelined FP32 GEMM and tile copy.
 *
 * What the library computes is defined on these pages:
 *  - "Day 74 -- Async copies and pipelines" (sections "A copy that skips the
 *    registers", "Two kernels, one arithmetic", "Exercise"): a register-tiled
 *    FP32 GEMM whose shared-memory tiles are filled either synchronously
 *    (global -> register -> shared, then a barrier) or asynchronously through
 *    a multi-stage pipeline, so that the fetch of the next K slice overlaps the
 *    compute on the current one; both fills feed one shared computeTile and
 *    must give bit-identical results.
 *  - "pipelined_gemm.cu" (kernels matmulTileSync and matmulTilePiped, and
 *    matmulCpu): the tile shapes, the per-thread float4 fill, the lookahead
 *    loop that keeps up to kStages fetches in flight, and the reference.
 *  - "A study on CUDA async memcpy" (section "async-group based approach"):
 *    a wait that returns once no more than N of the thread's newest copy
 *    groups are still outstanding; this library realises it per wave with
 *    s_waitcnt vmcnt(N) and per block with s_barrier.
 *  - "cp.async" (TVM TIRx, section "Predication is different from zero fill"):
 *    out-of-range parts of a tile are filled with zeros, never left unwritten.
 *
 * Conventions for every entry point:
 *  - Matrices are row-major fp32 in device memory; ld* is the row stride in
 *    elements. A is M x K (lda >= K), B is K x N (ldb >= N), C is M x N
 *    (ldc >= N). The caller owns all buffers; the library never allocates,
 *    never frees and never synchronises the host.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously on it; a returned MGEMM_OK means "launched".
 *  - Arguments are validated before any HIP call; a non-OK status means
 *    nothing was enqueued. No entry point exits the process.
 *  - C must not overlap A or B (the pages' kernels take __restrict__ inputs).
 *  - Each operand extent (rows x ld) must stay below 2^31 32-bit words and
 *    every ld below 2^21 words (2^22 elements of a 16-bit operand), so that
 *    every byte offset inside a 256-row block tile fits the buffer loads'
 *    31-bit range; larger problems return MGEMM_ERR_UNSUPPORTED.
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct mgemm_plan; /* defined below (mgemm_plan_t) */

#define MGEMM_VERSION 100 /* 1.0.0 */

/* fill_mode: how LDS tiles are filled ("Two kernels, one arithmetic"). */
#define MGEMM_FILL_SYNC 0  /* global -> VGPR -> LDS; stages>=2 stage slices in registers */
#define MGEMM_FILL_PIPED 1 /* asynchronous global -> LDS (buffer_load ... lds) ring */
#define MGEMM_FILL_PIPED_WS 2 /* the same asynchronous fill issued by dedicated filling waves;
                                 per-slot LDS counters replace the block barrier (512 threads) */

/* compute: the inner product on the LDS tiles. */
#define MGEMM_COMPUTE_VALU 0 /* per element fma chain, k ascending (the pages' computeTile) */
#define MGEMM_COMPUTE_MFMA 1 /* v_mfma_f32_32x32x2_f32 wave tiles */

/* tile: block tile of C (BM x BN, K slice 16 unless noted, 256 threads). */
#define MGEMM_TILE_AUTO 0      /* 64x64 or 128x128, whichever a wave model of the CUs estimates faster;
                                  with MFMA on the asynchronous ring of 2 or 3 stages, 256x128 in place
                                  of 128x128 when every CU gets an even number of its tiles (same rate,
                                  fewer HBM bytes). Every tile of one compute kind gives the same bits,
                                  so the choice never changes C. */
#define MGEMM_TILE_64x64 1   /* VALU: 4x4 micro-tile per thread (the pages' shape); MFMA: one 32x32
                                tile per wave, K slice 64 where the grid gives each of 256 CUs one
                                block at most, else 32 (chosen from the shape alone) */
#define MGEMM_TILE_128x128 2 /* VALU: 8x8 micro-tile; MFMA: 2x2 32x32 tiles per wave */
#define MGEMM_TILE_256x128 3 /* MFMA only: 4x2 32x32 tiles per wave (BM 256, BN 128) */
#define MGEMM_TILE_256x256 4 /* 16-bit only: 8 waves of 4x2 32x32 tiles (BM 256, BN 256) */

/* loader: width of each lane's global load (results never depend on it). */
#define MGEMM_LOADER_AUTO 0 /* 16 B when bases, ld and extents allow, else 4 B */
#define MGEMM_LOADER_B128 1 /* 16 B; refused (MGEMM_ERR_ARG) when alignment forbids it */
#define MGEMM_LOADER_B32 2  /* 4 B, any alignment */

/* status codes */
#define MGEMM_OK 0
#define MGEMM_ERR_ARG (-1)         /* negative size, ld too small, NULL with nonzero extent, bad enum */
#define MGEMM_ERR_ALIAS (-2)       /* C overlaps A or B (or dst overlaps src) */
#define MGEMM_ERR_ARCH (-3)        /* current device is not gfx950, or no device */
#define MGEMM_ERR_LAUNCH (-4)      /* the kernel launch failed; hipGetLastError has the cause */
#define MGEMM_ERR_UNSUPPORTED (-5) /* extent beyond the 32-bit buffer addressing limits above */

/*
 * C[0:M, 0:N] = A[0:M, 0:K] * B[0:K, 0:N]  (fp32, "Two kernels, one arithmetic").
 * stages: LDS ring depth, 1 .. 6 for MGEMM_FILL_PIPED (the pages' exercise
 * sweeps the depth; 1 = fetch, wait, compute, no overlap) and for
 * MGEMM_FILL_PIPED_WS, 1 .. 3 for MGEMM_FILL_SYNC (stages-1 register sets);
 * piped keeps stages-1 slices in flight during compute. fill_mode is
 * MGEMM_FILL_SYNC, MGEMM_FILL_PIPED or MGEMM_FILL_PIPED_WS ("A study on CUDA
 * async memcpy", producer/consumer pipeline). Uses the VALU compute tile and the
 * automatic tile and loader choice. For a fixed (shape, compute), every
 * (tile, stages, fill_mode, loader) gives bit-identical C. M == 0 or N == 0: no-op.
 * K == 0: C[0:M, 0:N] = +0. Cells of C outside M x N are never written.
 * MGEMM_FILL_PIPED_WS guards each of its LDS-counter waits with a bounded
 * spin (about 2^22 polls); a block whose wait runs out, which a correct
 * protocol never lets happen, stops and writes NaN to its whole C tile.
 * That is the only report: the call has already returned MGEMM_OK, so a
 * caller that must tell such a failure from NaN in the data checks C.
 */
int mgemm_sgemm(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc,
                int stages, int fill_mode, void *stream);

/* As mgemm_sgemm with the compute variant, block tile and loader width chosen
 * by the caller (MGEMM_COMPUTE_*, MGEMM_TILE_*, MGEMM_LOADER_*). */
int mgemm_sgemm_ex(int64_t M, int64_t N, int64_t K,
                   const float *A, int64_t lda,
                   const float *B, int64_t ldb,
                   float *C, int64_t ldc,
                   int stages, int fill_mode, int compute, int tile, int loader,
                   void *stream);

/* element formats of mgemm_gemm16 */
#define MGEMM_DTYPE_BF16 1 /* bfloat16: the upper half of a binary32 */
#define MGEMM_DTYPE_F16 2  /* IEEE 754 binary16 */

/*
 * C[0:M, 0:N] = A[0:M, 0:K] * B[0:K, 0:N] for 16-bit A and B (dtype
 * MGEMM_DTYPE_BF16 or MGEMM_DTYPE_F16, the same format for both) and fp32 C:
 * the tensor-core GEMM that the day-74 lesson names as the next user of its
 * pipeline, here v_mfma_f32_32x32x16_{bf16,f16} on the same asynchronous LDS
 * ring (64-element K slices). Products and sums are
 * fp32 inside the MFMA. lda and ldb count 16-bit elements, ldc fp32
 * elements. Requirements (else MGEMM_ERR_ARG): K, N, lda and ldb even; A and
 * B 4-byte aligned. stages 1 .. 4 (piped) or 1 .. 3 (sync); fill_mode MGEMM_FILL_SYNC or
 * MGEMM_FILL_PIPED (bit-identical results); tile MGEMM_TILE_AUTO,
 * MGEMM_TILE_128x128, MGEMM_TILE_256x128 or MGEMM_TILE_256x256 (512 threads); a
 * ring deeper than the CU's 160 KiB of LDS gives MGEMM_ERR_UNSUPPORTED.
 * Other conventions as mgemm_sgemm.
 */
int mgemm_gemm16(int64_t M, int64_t N, int64_t K,
                 const void *A, int64_t lda,
                 const void *B, int64_t ldb,
                 float *C, int64_t ldc,
                 int dtype, int stages, int fill_mode, int tile, void *stream);

/* The launch mgemm_gemm16 would make (no device access); as mgemm_plan_sgemm. */
int mgemm_plan_gemm16(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb,
                      const float *C, int64_t ldc,
                      int dtype, int stages, int fill_mode, int tile,
                      struct mgemm_plan *plan);

/*
 * Scaled dot-product attention forward (the async copy article, "from
 * cp.async to memcpy_async", section 6.2 "FlashAttention's tile pipeline":
 * the Q tile stays put, K/V tiles
 * stream through the asynchronous LDS ring while the current one is scored,
 * and each step rescales and accumulates the running output):
 *   O[b,h,i,:] = sum_j w_ij V[b,h,j,:],
 *   w_ij = exp(scale * Q[b,h,i,:].K[b,h,j,:]) / sum_t exp(scale * Q[b,h,i,:].K[b,h,t,:])
 * for b < batch, h < heads, i < seq_q, j < seq_k. Q, K and V hold 16-bit
 * elements of format dtype (MGEMM_DTYPE_BF16 / _F16), O is fp32; element
 * (b, h, i, d) of X is at X + b*x_sb + h*x_sh + i*x_ld + d (element
 * strides), d < head_dim, head_dim 64 or 128 (the value dimension equals
 * it). Scores and the P.V product accumulate in fp32 on
 * v_mfma_f32_32x32x16_{bf16,f16}; the probabilities enter that product
 * rounded to the input format. Caller-owned device buffers, asynchronous on
 * `stream`, no allocation. Requirements (else MGEMM_ERR_ARG): Q, K, V 4-byte
 * aligned with even strides, every ld >= head_dim, O 4-byte aligned,
 * seq_k >= 1 whenever there is a query (softmax over no keys is undefined),
 * finite scale, stages 1 .. 4 (piped) or 1 .. 3 (sync), fill_mode
 * MGEMM_FILL_SYNC or MGEMM_FILL_PIPED (bit-identical results). O must not
 * overlap Q, K or V, and distinct (b, h, i, d) outputs must have distinct
 * addresses (else MGEMM_ERR_ALIAS; any permuted dense layout qualifies).
 * batch, heads or seq_q == 0 is a no-op.
 */
int mgemm_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                    const void *Q, int64_t q_sb, int64_t q_sh, int64_t q_ld,
                    const void *K, int64_t k_sb, int64_t k_sh, int64_t k_ld,
                    const void *V, int64_t v_sb, int64_t v_sh, int64_t v_ld,
                    float *O, int64_t o_sb, int64_t o_sh, int64_t o_ld,
                    float scale, int dtype, int stages, int fill_mode, void *stream);

/* The launch mgemm_attention would make (no device access): bm = queries
 * per block, bn = head_dim, bk = keys per ring slice; as mgemm_plan_sgemm. */
int mgemm_plan_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k, int64_t head_dim,
                         const void *Q, int64_t q_sb, int64_t q_sh, int64_t q_ld,
                         const void *K, int64_t k_sb, int64_t k_sh, int64_t k_ld,
                         const void *V, int64_t v_sb, int64_t v_sh, int64_t v_ld,
                         const float *O, int64_t o_sb, int64_t o_sh, int64_t o_ld,
                         int dtype, int stages, int fill_mode, struct mgemm_plan *plan);

/*
 * dst[0:rows, 0:cols] = src[0:rows, 0:cols], streamed global -> LDS -> global
 * in 64 x 64 tiles through a `stages`-slot LDS ring filled asynchronously
 * (stages 1 .. 6; 1 = no overlap). The bytes of dst equal those of src;
 * padding columns of dst are not written. Isolates the fill bandwidth of the
 * GEMM's loader ("cp.async", section "Example: four 16-byte copies per
 * thread", which copies global -> shared -> global and checks equality).
 */
int mgemm_tile_copy(int64_t rows, int64_t cols, const float *src, int64_t lds,
                    float *dst, int64_t ldd, int stages, void *stream);

/*
 * dst[0:rows, 0:cols] = src[0:rows, 0:cols] with no LDS and no ring: each
 * lane moves one 16-byte chunk (4-byte element where bases, ld or cols
 * forbid 16) through a register, with non-temporal loads and stores, over a
 * grid of one lane per chunk. This is the practical HBM copy rate of the
 * device, the ceiling the tile copy's fill bandwidth is read against. It is
 * not a row of the method itself. Validation and ownership as
 * mgemm_tile_copy.
 */
int mgemm_plain_copy(int64_t rows, int64_t cols, const float *src, int64_t lds,
                     float *dst, int64_t ldd, void *stream);

/* Static description of a status code (never NULL). */
const char *mgemm_status_string(int status);

/* MGEMM_VERSION of the loaded library. */
int mgemm_version(void);

/*
 * The launch the library would make for these arguments, without touching
 * the device (no HIP call). Returns the status mgemm_sgemm_ex would return
 * from validation; on MGEMM_OK fills *plan.
 */
typedef struct mgemm_plan {
    int compute;       /* MGEMM_COMPUTE_* */
    int tile;          /* MGEMM_TILE_64x64, _128x128 or _256x128 */
    int bm, bn, bk;    /* block tile and K slice */
    int threads;       /* per block */
    int blocks;        /* 1-D grid */
    int load_bytes;    /* 16 or 4: per-lane width of each global load */
    int slices;        /* ceil(K / bk) */
    int stages;
    int fill_mode;
    int lds_bytes;     /* LDS per block: stages * (bm*bk + bk*bn) * 4 */
    int loads_per_slice; /* vector-memory instructions per filling wave per K slice (the 16-bit
                            256x256 tile fills its asynchronous ring from 4 of its 8 waves) */
    int max_vmcnt;     /* largest s_waitcnt vmcnt immediate the schedule uses */
} mgemm_plan_t;

int mgemm_plan_sgemm(int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     const float *C, int64_t ldc,
                     int stages, int fill_mode, int compute, int tile, int loader,
                     mgemm_plan_t *plan);

/*
 * Resident blocks per compute unit of the kernel mgemm_sgemm_ex would launch
 * for these arguments (registers, LDS and wave limits together), for the
 * stage-depth study of "Day 74 -- Async copies and pipelines" (section
 * "Exercise": a deeper ring costs LDS per block and so resident blocks).
 * This includes the launch's residency cap: where every CU would take exactly
 * one block more than the 3 or 4 it holds (any tile but the 64x64 VALU one,
 * which needs its resident waves for FMA issue), mgemm_sgemm_ex requests unused
 * dynamic LDS so that each CU holds half its blocks, rounded up (two even
 * rounds instead of a lockstep round and a lone block). Results do not depend on it.
 * Validates like mgemm_plan_sgemm, then queries the current device:
 * MGEMM_ERR_ARCH without a gfx950 device.
 */
int mgemm_blocks_per_cu(int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda,
                        const float *B, int64_t ldb,
                        const float *C, int64_t ldc,
                        int stages, int fill_mode, int compute, int tile, int loader,
                        int *blocks_per_cu);

/*
 * Record the stage schedule that a kernel's ring executes for `slices` K
 * slices (fill_mode, stages as above; kind 0 = fp32 GEMM, 1 = tile copy,
 * 2 = the 16-bit GEMM's asynchronous ring, whose computes are split so that
 * one slice's last k step overlaps the next slice's first LDS reads), as
 * produced by the very template the kernels instantiate. Each event is 3 ints
 * {op, a, b} written to events[0 .. 3*cap): op 1 = issue(slice a -> slot b),
 * 2 = wait(at most a slices of this wave in flight), 3 = barrier,
 * 4 = compute(slice a from slot b; for kind 2 every k step but the last),
 * 5 = store register set a -> slot b (sync fill), 6 = load slice a into
 * register set b (sync fill; a >= slices is a load with every lane masked,
 * whose set is never stored), 7 = head(issue the first k step's LDS reads of
 * slice a from slot b; kind 2), 8 = tail(the last k step of slice a, from
 * registers; kind 2). Kinds 1 and 2 exist for MGEMM_FILL_PIPED only.
 * Returns the number of events (which may exceed cap; only cap are written),
 * or MGEMM_ERR_ARG (also for MGEMM_FILL_PIPED_WS, whose waves follow
 * separate filling and computing loops). Host only; no device needed.
 */
int mgemm_ring_trace(int kind, int stages, int fill_mode, int slices, int *events, int cap);

/*
 * Record where one K slice's fill instructions put each element: the
 * loader map of a kernel's ring, enumerated with the operand types and the
 * filling-wave rules the kernels instantiate (the tile loader and zero-fill
 * row of the method: coalesced 16-byte or 4-byte lanes, each lane's
 * destination in the LDS slot). kind: 0 fp32 VALU 64x64, 1 VALU 128x128,
 * 2 fp32 MFMA 64x64 with a 32-k slice, 3 MFMA 128x128, 4 MFMA 256x128,
 * 5 16-bit 128x128, 6 16-bit 256x128, 7 16-bit 256x256, 8 attention head
 * dim 64, 9 head dim 128, 10 tile copy in blocks of 8 waves (MGEMM_FILL_PIPED
 * only), 11 fp32 MFMA 64x64 with a 64-k slice, 12 tile copy in blocks of 16
 * waves (MGEMM_FILL_PIPED only); load_bytes 16 or 4;
 * fill_mode MGEMM_FILL_SYNC (register-staged) or MGEMM_FILL_PIPED.
 * Events are 6 ints written to events[0 .. 6*cap). The first is a header
 * {-1, slot bytes, rows and 32-bit columns of operand 0, rows and columns of
 * operand 1}. Each other event is one lane's load of one unit:
 * {operand (0: A / K / the copy tile, 1: B / V), wave, LDS byte offset of
 * the written data in the slot, row, first 32-bit column, LDS byte offset
 * at which the compute side's layout reads that element}. Returns the
 * number of events (may exceed cap; only cap are written) or MGEMM_ERR_ARG.
 * Host only; no device needed.
 */
int mgemm_fill_trace(int kind, int load_bytes, int fill_mode, int *events, int cap);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H */
