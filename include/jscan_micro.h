/*
 * jscan_micro.h - microbenchmarks of the MI355X (gfx950) resources the selective scan is
 * bound by: vector-ALU issue (fused multiply-add, the base-2 exponential, their mix, DPP and
 * permlane forms), matrix cores running beside the vector ALU, LDS reads, and HBM streams.
 *
 * They fix the rates behind the scan's roofline: a state element of the S6 recurrence (notes
 * page "Jamba: A Hybrid Transformer-Mamba Language Model", section "Mamba layer") costs one
 * exponential and four multiply or multiply-add operations, and whether that work, not HBM,
 * bounds the prefill depends on how fast this chip issues them.
 *
 * These entry points are measurement tools, not part of the scan.  Conventions:
 *   - every pointer argument is a DEVICE pointer owned by the caller, except ms_out and the
 *     small host result arrays named as such;
 *   - each call launches on `stream` (a hipStream_t; NULL = the default stream), times its
 *     own launches with HIP events recorded on that stream, synchronises the stream, and
 *     writes the elapsed milliseconds of the timed launches to *ms_out;
 *   - `sink` receives per-thread results so that the compiler keeps the work (at least
 *     blocks * threads floats), plus a clock record (see jscan_micro_valu);
 *   - the return value is 0, or -1 for arguments outside the documented ranges (nothing is
 *     launched then), or the hipError_t of a failed launch or event call (a positive int).
 */
#ifndef JSCAN_MICRO_H
#define JSCAN_MICRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Vector-ALU issue rate.  kind selects the loop body; every thread runs `iters` trips of it,
 * each trip 16 instructions on 16 registers, written in inline assembly so
 * that the instruction count per trip is exact:
 *   0  v_fmac_f32 x16                      (fused multiply-add)
 *   1  v_exp_f32 x16                       (base-2 exponential)
 *   2  v_exp_f32 x8 + v_fmac_f32 x8        (the two interleaved, independent)
 *   3  v_exp_f32 x4 + v_fmac_f32 x12
 *   4  v_mul_f32 with a DPP row broadcast (row_newbcast) x16
 *   5  v_permlane32_swap x8 + v_max_f32 x8
 *   6  v_permlane16_swap x8 + v_max_f32 x8
 *   7  v_mul_f32 x8 + v_exp_f32 x8 on dependent pairs (the decay's product and exponential)
 *   8  4 tokens of the scan for a lane holding two states, B and C as scalar (SGPR) operands:
 *      per token 2 exponent products, 2 exponentials, 2 input products, 2 state FMAs and the
 *      2-term output partial (10 instructions), plus 2 register moves (12 per token counted)
 *   9  the same with B and C broadcast by DPP (row_newbcast) inside the multiplies
 *  10  v_fmac_f32 x16, independent, with three distinct source registers each
 *  11  an inclusive scan of 8 independent (a, b) chains over the wave's 64 lanes: 6 levels
 *      (row_shr 1, 2, 4, 8, then row_bcast 15 and 31), each a v_fmac_f32_dpp (b) and a
 *      v_mul_f32_dpp (a) per chain: 96 instructions per trip
 * sink: blocks * threads floats, then 4 more: (shader clocks, 100 MHz real-time ticks) of
 * block 0's first wave over its loop, as two pairs of floats (low, high 32 bits); kinds 0-7
 * and 10 then store each wave's HW_ID and XCC_ID registers (2 floats per wave, as raw bits),
 * so sink must hold blocks * threads + 4 + 2 * blocks * threads / 64 floats.
 * blocks in [1, 65536], threads in {64, 128, 256, 512, 1024}, iters in [1, 2^24]. */
int jscan_micro_valu(int kind, int64_t iters, int blocks, int threads, float *sink, void *stream, float *ms_out);

/* Matrix cores beside the vector ALU.  Each wave runs `iters` trips; a trip holds 4
 * independent v_mfma_f32_16x16x4_f32 (each 1024 multiply-adds) and/or 32 v_fmac_f32:
 *   mode 0  the MFMAs only;  mode 1  the FMAs only;  mode 2  both, interleaved;
 *   mode 3  v_mfma_f32_16x16x32_bf16 in place of the fp32 MFMA, alone;  mode 4  that, with the FMAs.
 * If the matrix core runs beside the vector ALU, mode 2 takes about the longer of modes 0
 * and 1, not their sum.  With threads = 64 and 4 blocks per CU each SIMD runs one wave, which
 * shows whether one wave's vector instructions issue while its own MFMAs execute.
 * blocks in [1, 65536], threads in {64, 128, 256, 512}, iters in [1, 2^24]. */
int jscan_micro_mfma_valu(int mode, int64_t iters, int blocks, int threads, float *sink, void *stream,
                          float *ms_out);

/* One wave, one fp32 MFMA against the vector ALU's fused multiply-adds on the same operands.
 * variant 0: v_mfma_f32_4x4x1_16b_f32, 16 blocks of 4x4 outer products with K = 1: lane l holds
 *            A[l/4][l%4] (block l/4, row l%4) in a[l], B of block l/4, column l%4 in b[l], and
 *            rows 0..3 of column l%4 of block l/4 in c/d[4l .. 4l+3]; d_fma[4l+i] =
 *            fmaf(a[4(l/4)+i], b[l], c[4l+i]).
 * variant 1: v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16] in a[l], B[l/16][l%16] in b[l],
 *            and rows 4(l/16)..4(l/16)+3 of column l%16 in c/d[4l .. 4l+3]; d_fma is the chain
 *            fmaf over k = 0..3 from c.  With one nonzero product per output this checks that
 *            the matrix core rounds a*b + c exactly like the FMA.
 * Also checks the operand layouts stated here: a wrong layout shows as large differences.
 * a, b: 64 floats; c, d_mfma, d_fma: 256 floats. */
int jscan_micro_mfma_rounding(int variant, const float *a, const float *b, const float *c, float *d_mfma,
                              float *d_fma, void *stream);

/* LDS read bandwidth: every thread reads 16 bytes (ds_read_b128) per instruction, 8 per trip.
 * Lane l reads at (l % unique) * 16 bytes from the start of each KiB: unique = 64 gives every
 * lane its own address (a contiguous KiB per instruction); 16 or 32 make 4 or 2 groups of lanes
 * read the same addresses (one 16-lane row's worth, broadcast).  unique in {16, 32, 64},
 * blocks in [1, 65536], threads in {64, 128, 256, 512, 1024}, iters in [1, 2^24]. */
int jscan_micro_lds(int64_t iters, int unique, int blocks, int threads, float *sink, void *stream, float *ms_out);

/* HBM streams over `bytes` (a multiple of 16 KiB, at most 2^36): kind 0 reads src (summing
 * it into sink), 1 writes dst, 2 copies src to dst.  nontemporal != 0 uses non-temporal
 * loads and stores.  Grid-stride over 16-byte vectors with `blocks` work-groups of 256
 * threads (blocks in [1, 65536]).  `reps` launches are timed back to back (reps in [1, 1000]).
 * src and dst must be 16-byte aligned; sink holds blocks * 256 floats. */
int jscan_micro_hbm(int kind, int nontemporal, const void *src, void *dst, int64_t bytes, int blocks, int reps,
                    float *sink, void *stream, float *ms_out);

#ifdef __cplusplus
}
#endif

#endif /* JSCAN_MICRO_H */
