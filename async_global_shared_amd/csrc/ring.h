// ring.h -- stage schedules of the LDS ring, shared by the kernels and the
// host-side trace (mgemm_ring_trace), so the schedule that is tested on the
// CPU is the one the GPU executes.
//
// The pages' pipelined kernel ("pipelined_gemm.cu", matmulTilePiped) keeps a
// fetch counter at most kStages slices ahead of the compute counter; each
// iteration tops up the fetches, waits for the oldest stage, computes on it
// and releases it ("Day 74 -- Async copies and pipelines", section "Two
// kernels, one arithmetic"). The pipeline object is a FIFO of stages whose
// consumer_wait waits on the oldest stage only ("A study on CUDA async
// memcpy", section "cuda::pipeline").
//
// On gfx950 there is no pipeline object. Completion of a wave's own
// asynchronous global->LDS loads is counted by its vmcnt (in order), and the
// block-wide "stage ready" and "stage released" events are one s_barrier: a
// barrier orders threads but does not complete copies ("Day 74", section
// "Pitfalls"), so every wave waits on its own count first, then barriers.
#pragma once

#if defined(__HIPCC__)
#define MG_HD __host__ __device__
#else
#define MG_HD
#endif

namespace mgemm {

constexpr int kMaxPipedStages = 6; // asynchronous ring depth
constexpr int kMaxSyncStages = 3;  // register-staged ring depth (S-1 register sets)

template <int I>
struct Int {
    static constexpr int value = I;
};

template <int B, int E, class F>
MG_HD inline void static_for(F &&f) {
    if constexpr (B < E) {
        f(Int<B>{});
        static_for<B + 1, E>(f);
    }
}

// Asynchronous ring, `S` LDS slots. Ops provides:
//   issue(slice, slot)   start the global->LDS fill of `slice` into `slot`
//   wait<P>()            this wave: at most P of its issued slices in flight
//   barrier()            block barrier after the wave's LDS reads completed
//   compute(slice, slot) consume `slot`, which holds `slice`
// S == 1 has no lookahead (fetch, wait, compute, release). For S >= 2 the
// prologue issues S-1 slices; iteration t waits for slice t (leaving the
// slices issued after it in flight: S-2 in the steady state, fewer in the
// last S-2 iterations), barriers (slice t visible to all waves; slot
// (t-1) % S released by all waves), refills that released slot with slice
// t+S-1, then computes slice t.
template <int S, class Ops>
MG_HD inline void piped_schedule(int T, Ops &ops) {
    static_assert(S >= 1 && S <= kMaxPipedStages, "stages must be 1 .. 6");
    if constexpr (S == 1) {
        for (int t = 0; t < T; ++t) {
            ops.issue(t, 0);
            ops.template wait<0>();
            ops.barrier();
            ops.compute(t, 0);
            ops.barrier();
        }
    } else {
        for (int s = 0; s < S - 1 && s < T; ++s)
            ops.issue(s, s);
        for (int t = 0; t < T; ++t) {
            // slices issued after slice t so far: t+1 .. min(t+S-2, T-1)
            const int pending = (t + S - 2 < T ? t + S - 2 : T - 1) - t;
            static_for<0, S - 1>([&](auto p) {
                if (pending == p.value)
                    ops.template wait<p.value>();
            });
            ops.barrier();
            if (t + S - 1 < T)
                ops.issue(t + S - 1, (t + S - 1) % S);
            ops.compute(t, t % S);
        }
    }
}

// Asynchronous ring with each compute split in three: head(slice, slot)
// issues the LDS reads of the slice's first k step, body(slice, slot)
// runs every k step but the last, whose reads it completes, and tail(slice)
// runs the last k step from registers alone. Slice t-1's tail is placed
// after slice t's head, so its matrix instructions cover the latency of
// those reads instead of every wave waiting on them after the barrier, and
// the refill of the slot just released is spread over those instructions
// (tail_issue): issued as one burst, every wave's fills queue at the CU's
// address unit and each wave stalls, in order, with the matrix pipe idle.
// Each accumulator still sees the k steps in the same order, so results equal
// piped_schedule's. The barrier of iteration t follows body(t-1), after
// which the wave reads nothing more from slice t-1's slot: releasing it
// there is safe although tail(t-1) has not run yet.
template <int S, class Ops>
MG_HD inline void piped_schedule_split(int T, Ops &ops) {
    static_assert(S >= 1 && S <= kMaxPipedStages, "stages must be 1 .. 6");
    if constexpr (S == 1) {
        for (int t = 0; t < T; ++t) {
            ops.issue(t, 0);
            ops.template wait<0>();
            ops.barrier();
            ops.head(t, 0);
            if (t > 0)
                ops.tail(t - 1);
            ops.body(t, 0);
            ops.barrier();
        }
    } else {
        // iteration 0 is peeled (it has no tail), so in the loop the tail
        // is on the straight path: a tail in two branches, one of them with
        // the refill spread over it, would give the accumulators two register
        // assignments to reconcile
        for (int s = 0; s < S - 1 && s < T; ++s)
            ops.issue(s, s);
        const auto wait_for = [&](int t) {
            // slices issued after slice t so far: t+1 .. min(t+S-2, T-1)
            const int pending = (t + S - 2 < T ? t + S - 2 : T - 1) - t;
            static_for<0, S - 1>([&](auto p) {
                if (pending == p.value)
                    ops.template wait<p.value>();
            });
        };
        if (T > 0) {
            wait_for(0);
            ops.barrier();
            ops.head(0, 0);
            if (S - 1 < T)
                ops.issue(S - 1, S - 1);
            ops.body(0, 0);
        }
        for (int t = 1; t < T; ++t) {
            wait_for(t);
            ops.barrier();
            ops.head(t, t % S);
            // tail(t-1), with the refill of the slot just released spread
            // over its matrix instructions (none in the last S-1 iterations)
            ops.tail_issue(t - 1, t + S - 1, (t + S - 1) % S, t + S - 1 < T);
            ops.body(t, t % S);
        }
    }
    if (T > 0)
        ops.tail(T - 1);
}

// Synchronous ring: global -> registers -> LDS. Ops provides:
//   load<SET>(slice)      issue global->register loads of `slice` into set SET;
//                         a slice >= T must issue the same loads with every
//                         lane masked (zeros, no memory access)
//   store<SET>(slot)      write register set SET to LDS `slot` (waits on loads)
//   barrier(), compute(slice, slot) as above
// S == 1 is the pages' matmulTileSync: load, store, barrier, compute, barrier.
// For S >= 2 (a double buffer built from synchronous loads, as in the
// "async copy pipeline" article's benchmark), S-1 register sets keep S-1
// slices in flight: iteration t issues slice t+S-1, computes slice t, then
// stores slice t+1 into its slot and barriers.
// With two sets or more the loop runs whole groups of S-1 iterations,
// stopping before the last slice, so that register-set indices are
// compile-time constants and every load, compute and store in its body is
// unconditional (a load past the last slice is the masked one, and its set
// is never stored). Conditional loads or stores there made the compiler's
// wait counts assume the worst path and drain the slice issued last before
// each store; a set index chosen at run time made it copy the sets between
// branches; computes under a branch each made it keep a second copy of the
// accumulators. The last 1 .. S-1 slices run after the loop.
template <int S, class Ops>
MG_HD inline void sync_schedule(int T, Ops &ops) {
    static_assert(S >= 1 && S <= kMaxSyncStages, "stages must be 1, 2 or 3");
    if constexpr (S == 1) {
        for (int t = 0; t < T; ++t) {
            ops.template load<0>(t);
            ops.template store<0>(0);
            ops.barrier();
            ops.compute(t, 0);
            ops.barrier();
        }
    } else {
        constexpr int R = S - 1;
        static_for<0, R>([&](auto s) {
            if (s.value < T)
                ops.template load<s.value>(s.value);
        });
        if (T > 0) {
            ops.template store<0>(0);
            ops.barrier();
        }
        if constexpr (R == 1) {
            // one register set: its store waits for the newest loads, so
            // conditional loads cost no wait precision
            for (int t = 0; t < T; ++t) {
                if (t + 1 < T)
                    ops.template load<0>(t + 1);
                ops.compute(t, t % S);
                if (t + 1 < T)
                    ops.template store<0>((t + 1) % S);
                ops.barrier();
            }
            return;
        }
        const int Tm = T > 0 ? (T - 1) / R * R : 0;
        for (int t0 = 0; t0 < Tm; t0 += R)
            static_for<0, R>([&](auto u) {
                const int t = t0 + u.value;
                ops.template load<u.value>(t + R);
                ops.compute(t, t % S);
                ops.template store<(u.value + 1) % R>((t + 1) % S);
                ops.barrier();
            });
        static_for<0, R>([&](auto u) {
            const int t = Tm + u.value;
            if (t < T) {
                ops.compute(t, t % S);
                if (t + 1 < T)
                    ops.template store<(u.value + 1) % R>((t + 1) % S);
                ops.barrier();
            }
        });
    }
}

} // namespace mgemm
