/*
 * fa_micro.h -- C ABI of the machine microbenchmarks (libfa355_micro.so).
 *
 * These kernels measure the gfx950 units the attention kernels are bound by, under load
 * on every compute unit: the bf16 matrix-core (MFMA) rate, the v_exp_f32 rate, LDS read
 * bandwidth and fp32 global atomic-add throughput.  They compute nothing of attention;
 * the bench reports them beside the data-sheet peaks so that a kernel's fraction of peak
 * can also be read against what the chip sustains at its running clock.
 *
 * Conventions
 *  - `out` / `buf` are DEVICE pointers to float32 arrays owned by the caller.
 *  - `blocks` is the grid size in workgroups of 256 threads; fa_micro_grid_blocks()
 *    returns the size that puts two workgroups on every compute unit (or -1 if the
 *    device cannot be queried).
 *  - Every call only enqueues one kernel on `stream` (0 = the null stream) and returns;
 *    it never allocates or synchronises.  Time it with events on the same stream.
 *  - Return value: 0 on success, -1 for a NULL pointer or a count below 1 (nothing is
 *    enqueued), -6 when the launch fails.
 */
#ifndef FA355_FA_MICRO_H
#define FA355_FA_MICRO_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fa_stream_t; /* identical to hipStream_t */

/* Workgroups that put two 256-thread workgroups on every compute unit, or -1. */
int fa_micro_grid_blocks(void);

/* bf16 MFMA rate: every wave runs 8 independent accumulation chains of `iters`
 * v_mfma_f32_32x32x16_bf16 products (32768 FLOP each), so one call performs
 * blocks * 4 * 8 * iters * 32768 FLOP.  `out` holds blocks * 256 floats (one sum of
 * accumulators per thread, written so the work is not removed). */
int fa_micro_mfma_bf16(float* out, int blocks, int iters, fa_stream_t stream);

/* v_exp_f32 rate: every thread runs 16 independent chains of `iters` exponentials
 * (blocks * 256 * 16 * iters in total).  `out` holds blocks * 256 floats. */
int fa_micro_exp(float* out, int blocks, int iters, fa_stream_t stream);

/* LDS read bandwidth: every wave issues 8 * iters 128-bit reads of 1 KiB contiguous
 * (bank-conflict free) from a 40 KiB tile, blocks * 4 * 8 * iters KiB in total.
 * `out` holds blocks * 256 floats. */
int fa_micro_lds_read(float* out, int blocks, int iters, fa_stream_t stream);

/* fp32 global atomic-add throughput on whole 64 x 128 tiles (32 KiB): workgroup w adds
 * 1.0 to every element of the `tiles` tiles at positions (w + t) % ntiles of `buf`, which
 * holds ntiles * 8192 floats; blocks * tiles * 8192 atomic adds in total. */
int fa_micro_atomic_tiles(float* buf, int ntiles, int blocks, int tiles, fa_stream_t stream);

/* MFMA / VALU co-execution on one SIMD: workgroups of 512 threads (8 waves, one workgroup
 * per compute unit; waves w and w + 4 share a SIMD).  mode 1: waves 0-3 run `mfma_iters`
 * iterations of 8 independent v_mfma_f32_32x32x16_bf16 chains (as fa_micro_mfma_bf16);
 * mode 2: waves 4-7 run `valu_iters` iterations of 16 independent per-lane chains,
 * x <- exp2(-x) on v_exp_f32 (valu_kind 0) or x <- fma(x, 0.999, 1e-4) on v_fma_f32
 * (valu_kind 1), from x0 = 0.25 + 0.03 k + 1e-6 (thread % 256); mode 3: both at once.
 * `out` holds blocks * 512 floats: the MFMA waves' accumulator sums (0 when idle) and
 * the VALU waves' chain sums (0 when idle).
 * valu_kind 2 (transcendental beside FMA on one SIMD): waves 0-3 run the exp2 chains for
 * `mfma_iters` iterations (mode bit 0) and waves 4-7 the FMA chains for `valu_iters`
 * (bit 1); out: the exp chains' sums, then the FMA chains' sums.
 * valu_kind 3 (both in one wave): waves 0-3 run the exp2 chains (`mfma_iters`, bit 0)
 * and the FMA chains (`valu_iters`, bit 1) interleaved in one instruction stream, waves
 * 4-7 idle; out[t] = exp chain sum of thread t < 256, out[256 + t] = its FMA chain sum
 * (0 for a stream not run).
 * Returns -1 for a NULL pointer, a count below 1 or a mode / valu_kind out of range. */
int fa_micro_coexec(float* out, int blocks, int mode, int valu_kind, int mfma_iters, int valu_iters,
                    fa_stream_t stream);

/* Issue rate of bf16 products in a given order: one 256-thread workgroup per compute unit
 * (96 KiB of LDS each), one wave per SIMD.  A operands are bf16 2^-10; accumulation
 * chain k takes B = bf16 2^-10 (1 + k/128) (o[0..3]: k = 0..3, the score accumulators
 * k = 4..), so each product adds 2^-16 (1 + k/128) to every element of its accumulator.
 * Each wave runs `iters` blocks of 32 v_mfma_f32_32x32x16_bf16 and its lane 0 writes the
 * s_memtime difference (shader-clock ticks) to ticks[block * 4 + wave]; 32 products take
 * at least 32 * 32 = 1024 ticks.  variant 0: 8 independent chains (4 products each per
 * block); 1: the attention forward's MFMA operation -- 16 P.V products over 4
 * accumulators, then 16 score products over 2 accumulators, the first from C = 0;
 * 2: as 1 with the scores over 4 accumulators (the first two from C = 0); 3: as 1 with
 * every A operand read from LDS four products ahead.  sink[block * 256 + t] receives
 * thread t's total: the per-block score sums (element 0 of each score accumulator) plus
 * every accumulator element at the end (variants 1 and 3 compute the same values).
 * ticks: blocks * 4 entries, sink: blocks * 256 floats, device pointers.  Returns -1 for
 * a NULL pointer, blocks or iters below 1 or a variant outside 0..3. */
int fa_micro_mfma_order(unsigned long long* ticks, float* sink, int blocks, int variant, int iters,
                        fa_stream_t stream);

/* Accumulation precision of the fp8 matrix product: one v_mfma_scale_f32_32x32x64_f8f6f4
 * (OCP E4M3 codes for both operands, unit scales) on one wave, C = A B^T + C0.  a and b
 * hold 32 x 64 E4M3 codes row-major (row i of b is column i of B), c0 and c 32 x 32
 * floats row-major; all four are device pointers.  One 64-thread workgroup. */
int fa_micro_mfma_fp8_tile(const void* a, const void* b, const float* c0, float* c, fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA355_FA_MICRO_H */
