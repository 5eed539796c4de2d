// micro.hip - libjscan_micro: the microbenchmarks declared in include/jscan_micro.h.
//
// Each loop body is written in inline assembly so that the number and kind of instructions
// per trip is exactly what the name says; the compiler only supplies registers.  Results go
// to a sink buffer so that nothing is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jscan_micro.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void clock_mark(uint64_t &t, uint64_t &rt) {
    t = __builtin_amdgcn_s_memtime();
    rt = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void store_clock(float *sink, int n, uint64_t t0, uint64_t t1, uint64_t r0, uint64_t r1) {
    const uint64_t dt = t1 - t0, dr = r1 - r0;
    sink[n + 0] = __uint_as_float((uint32_t)dt);
    sink[n + 1] = __uint_as_float((uint32_t)(dt >> 32));
    sink[n + 2] = __uint_as_float((uint32_t)dr);
    sink[n + 3] = __uint_as_float((uint32_t)(dr >> 32));
}

#define R16 "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]), \
            "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]), "+v"(r[14]), "+v"(r[15])

template <int KIND>
__device__ __forceinline__ void valu_trip(float (&r)[16], float a, float b) {
    if constexpr (KIND == 0) {
        asm volatile(
            "v_fmac_f32 %0, %16, %17\n\tv_fmac_f32 %1, %16, %17\n\tv_fmac_f32 %2, %16, %17\n\tv_fmac_f32 %3, %16, %17\n\t"
            "v_fmac_f32 %4, %16, %17\n\tv_fmac_f32 %5, %16, %17\n\tv_fmac_f32 %6, %16, %17\n\tv_fmac_f32 %7, %16, %17\n\t"
            "v_fmac_f32 %8, %16, %17\n\tv_fmac_f32 %9, %16, %17\n\tv_fmac_f32 %10, %16, %17\n\tv_fmac_f32 %11, %16, %17\n\t"
            "v_fmac_f32 %12, %16, %17\n\tv_fmac_f32 %13, %16, %17\n\tv_fmac_f32 %14, %16, %17\n\tv_fmac_f32 %15, %16, %17"
            : R16 : "v"(a), "v"(b));
    } else if constexpr (KIND == 1) {
        asm volatile(
            "v_exp_f32_e64 %0, -%0\n\tv_exp_f32_e64 %1, -%1\n\tv_exp_f32_e64 %2, -%2\n\tv_exp_f32_e64 %3, -%3\n\t"
            "v_exp_f32_e64 %4, -%4\n\tv_exp_f32_e64 %5, -%5\n\tv_exp_f32_e64 %6, -%6\n\tv_exp_f32_e64 %7, -%7\n\t"
            "v_exp_f32_e64 %8, -%8\n\tv_exp_f32_e64 %9, -%9\n\tv_exp_f32_e64 %10, -%10\n\tv_exp_f32_e64 %11, -%11\n\t"
            "v_exp_f32_e64 %12, -%12\n\tv_exp_f32_e64 %13, -%13\n\tv_exp_f32_e64 %14, -%14\n\tv_exp_f32_e64 %15, -%15"
            : R16);
    } else if constexpr (KIND == 2) {
        asm volatile(
            "v_exp_f32_e64 %0, -%0\n\tv_fmac_f32 %1, %16, %17\n\tv_exp_f32_e64 %2, -%2\n\tv_fmac_f32 %3, %16, %17\n\t"
            "v_exp_f32_e64 %4, -%4\n\tv_fmac_f32 %5, %16, %17\n\tv_exp_f32_e64 %6, -%6\n\tv_fmac_f32 %7, %16, %17\n\t"
            "v_exp_f32_e64 %8, -%8\n\tv_fmac_f32 %9, %16, %17\n\tv_exp_f32_e64 %10, -%10\n\tv_fmac_f32 %11, %16, %17\n\t"
            "v_exp_f32_e64 %12, -%12\n\tv_fmac_f32 %13, %16, %17\n\tv_exp_f32_e64 %14, -%14\n\tv_fmac_f32 %15, %16, %17"
            : R16 : "v"(a), "v"(b));
    } else if constexpr (KIND == 3) {
        asm volatile(
            "v_exp_f32_e64 %0, -%0\n\tv_fmac_f32 %1, %16, %17\n\tv_fmac_f32 %2, %16, %17\n\tv_fmac_f32 %3, %16, %17\n\t"
            "v_exp_f32_e64 %4, -%4\n\tv_fmac_f32 %5, %16, %17\n\tv_fmac_f32 %6, %16, %17\n\tv_fmac_f32 %7, %16, %17\n\t"
            "v_exp_f32_e64 %8, -%8\n\tv_fmac_f32 %9, %16, %17\n\tv_fmac_f32 %10, %16, %17\n\tv_fmac_f32 %11, %16, %17\n\t"
            "v_exp_f32_e64 %12, -%12\n\tv_fmac_f32 %13, %16, %17\n\tv_fmac_f32 %14, %16, %17\n\tv_fmac_f32 %15, %16, %17"
            : R16 : "v"(a), "v"(b));
    } else if constexpr (KIND == 4) {
        // a is never written by a vector instruction, so its DPP read needs no wait state
        asm volatile(
            "v_mul_f32_dpp %0, %16, %0 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %1, %16, %1 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %2, %16, %2 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %3, %16, %3 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %4, %16, %4 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %5, %16, %5 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %6, %16, %6 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %7, %16, %7 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %8, %16, %8 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %9, %16, %9 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %10, %16, %10 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %11, %16, %11 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %12, %16, %12 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %13, %16, %13 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %14, %16, %14 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %15, %16, %15 row_newbcast:0 row_mask:0xf bank_mask:0xf"
            : R16 : "v"(a));
    } else if constexpr (KIND == 5 || KIND == 6) {
#define JSCAN_PL(op)                                                                                              \
    asm volatile(op " %0, %1\n\t" op " %2, %3\n\t" op " %4, %5\n\t" op " %6, %7\n\t" op " %8, %9\n\t" op       \
                    " %10, %11\n\t" op " %12, %13\n\t" op " %14, %15\n\t"                                          \
                    "v_max_f32 %0, %0, %1\n\tv_max_f32 %2, %2, %3\n\tv_max_f32 %4, %4, %5\n\tv_max_f32 %6, %6, %7\n\t" \
                    "v_max_f32 %8, %8, %9\n\tv_max_f32 %10, %10, %11\n\tv_max_f32 %12, %12, %13\n\t"                \
                    "v_max_f32 %14, %14, %15"                                                                        \
                    : R16)
        if constexpr (KIND == 5)
            JSCAN_PL("v_permlane32_swap_b32");
        else
            JSCAN_PL("v_permlane16_swap_b32");
#undef JSCAN_PL
    } else if constexpr (KIND == 10) {
        // 16 independent FMAs whose three operands all differ (no register-bank pile-up):
        // r[i] += r[(i + 5) % 16] * r[(i + 11) % 16] reads registers written a trip earlier
        asm volatile(
            "v_fmac_f32 %0, %5, %11\n\tv_fmac_f32 %1, %6, %12\n\tv_fmac_f32 %2, %7, %13\n\tv_fmac_f32 %3, %8, %14\n\t"
            "v_fmac_f32 %4, %9, %15\n\tv_fmac_f32 %5, %10, %0\n\tv_fmac_f32 %6, %11, %1\n\tv_fmac_f32 %7, %12, %2\n\t"
            "v_fmac_f32 %8, %13, %3\n\tv_fmac_f32 %9, %14, %4\n\tv_fmac_f32 %10, %15, %5\n\tv_fmac_f32 %11, %0, %6\n\t"
            "v_fmac_f32 %12, %1, %7\n\tv_fmac_f32 %13, %2, %8\n\tv_fmac_f32 %14, %3, %9\n\tv_fmac_f32 %15, %4, %10"
            : R16);
    } else if constexpr (KIND == 11) {
        // one inclusive scan of 8 independent (a, b) chains over the 64 lanes, by DPP: the
        // composition (a, b) of lanes i-k and i is (a_{i-k} a_i, a_i b_{i-k} + b_i), k = 1, 2, 4, 8
        // inside each 16-lane row (row_shr; lanes with no source lane keep their pair), then across
        // rows (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).  r[j] holds a of
        // chain j, r[8 + j] its b; b is updated before a so that it uses the old a.
#define JSCAN_LVL(ctl)                                                                                    \
    "v_fmac_f32_dpp %8, %8, %0 " ctl "\n\tv_fmac_f32_dpp %9, %9, %1 " ctl "\n\t"                          \
    "v_fmac_f32_dpp %10, %10, %2 " ctl "\n\tv_fmac_f32_dpp %11, %11, %3 " ctl "\n\t"                       \
    "v_fmac_f32_dpp %12, %12, %4 " ctl "\n\tv_fmac_f32_dpp %13, %13, %5 " ctl "\n\t"                       \
    "v_fmac_f32_dpp %14, %14, %6 " ctl "\n\tv_fmac_f32_dpp %15, %15, %7 " ctl "\n\t"                       \
    "v_mul_f32_dpp %0, %0, %0 " ctl "\n\tv_mul_f32_dpp %1, %1, %1 " ctl "\n\t"                             \
    "v_mul_f32_dpp %2, %2, %2 " ctl "\n\tv_mul_f32_dpp %3, %3, %3 " ctl "\n\t"                             \
    "v_mul_f32_dpp %4, %4, %4 " ctl "\n\tv_mul_f32_dpp %5, %5, %5 " ctl "\n\t"                             \
    "v_mul_f32_dpp %6, %6, %6 " ctl "\n\tv_mul_f32_dpp %7, %7, %7 " ctl "\n\t"
        asm volatile(JSCAN_LVL("row_shr:1 row_mask:0xf bank_mask:0xf")
                     JSCAN_LVL("row_shr:2 row_mask:0xf bank_mask:0xf")
                     JSCAN_LVL("row_shr:4 row_mask:0xf bank_mask:0xf")
                     JSCAN_LVL("row_shr:8 row_mask:0xf bank_mask:0xf")
                     JSCAN_LVL("row_bcast:15 row_mask:0xa bank_mask:0xf")
                     JSCAN_LVL("row_bcast:31 row_mask:0xc bank_mask:0xf")
                     : R16);
#undef JSCAN_LVL
    } else if constexpr (KIND == 7) {
        // 8 (product, exponential) pairs: the decay 2^(delta * A2) of 8 state elements;
        // r[8 + i] holds the product, r[i] the exponential
        asm volatile(
            "v_mul_f32 %8, %0, %16\n\tv_mul_f32 %9, %1, %16\n\tv_mul_f32 %10, %2, %16\n\tv_mul_f32 %11, %3, %16\n\t"
            "v_mul_f32 %12, %4, %16\n\tv_mul_f32 %13, %5, %16\n\tv_mul_f32 %14, %6, %16\n\tv_mul_f32 %15, %7, %16\n\t"
            "v_exp_f32_e64 %0, -%8\n\tv_exp_f32_e64 %1, -%9\n\tv_exp_f32_e64 %2, -%10\n\tv_exp_f32_e64 %3, -%11\n\t"
            "v_exp_f32_e64 %4, -%12\n\tv_exp_f32_e64 %5, -%13\n\tv_exp_f32_e64 %6, -%14\n\tv_exp_f32_e64 %7, -%15"
            : R16 : "v"(a));
    }
}
#undef R16

// One token of the scan for a lane holding two states, as the two operand deliveries of B and C:
//   SGPR: B and C wave-uniform scalar operands (a wave holds one state pair for all its lanes);
//   DPP:  B and C broadcast from lane k of each 16-lane row inside the multiply (row_newbcast).
// Per token 10 vector instructions: 2 exponent products, 2 exponentials, 2 input products, 2
// state FMAs and the 2-term output partial.  h0/h1 carry the states across tokens.
struct ScanRegs {
    float h0, h1, p0, p1, p2, p3, e0, e1, b0, b1;
};
template <bool kDpp, int TAU>
__device__ __forceinline__ void scan_token(ScanRegs &g, float dlt, float u, float a0, float a1, float sb0, float sb1,
                                           float sc0, float sc1, float &p) {
    if constexpr (!kDpp) {
        asm volatile(
            "v_mul_f32 %2, %6, %8\n\tv_mul_f32 %3, %6, %9\n\t"
            "v_exp_f32_e32 %2, %2\n\tv_exp_f32_e32 %3, %3\n\t"
            "v_mul_f32 %4, %10, %7\n\tv_mul_f32 %5, %11, %7\n\t"
            "v_fmac_f32 %4, %2, %0\n\tv_fmac_f32 %5, %3, %1\n\t"
            "v_mov_b32 %0, %4\n\tv_mov_b32 %1, %5"
            : "+v"(g.h0), "+v"(g.h1), "=&v"(g.e0), "=&v"(g.e1), "=&v"(g.b0), "=&v"(g.b1)
            : "v"(dlt), "v"(u), "v"(a0), "v"(a1), "s"(sb0), "s"(sb1));
        asm volatile("v_mul_f32 %0, %3, %1\n\tv_fmac_f32 %0, %4, %2" : "=&v"(p) : "v"(g.h0), "v"(g.h1), "s"(sc0),
                     "s"(sc1));
    } else {
        asm volatile(
            "v_mul_f32 %2, %6, %8\n\tv_mul_f32 %3, %6, %9\n\t"
            "v_exp_f32_e32 %2, %2\n\tv_exp_f32_e32 %3, %3\n\t"
            "v_mul_f32_dpp %4, %10, %7 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
            "v_mul_f32_dpp %5, %11, %7 row_newbcast:%12 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32 %4, %2, %0\n\tv_fmac_f32 %5, %3, %1\n\t"
            "v_mov_b32 %0, %4\n\tv_mov_b32 %1, %5"
            : "+v"(g.h0), "+v"(g.h1), "=&v"(g.e0), "=&v"(g.e1), "=&v"(g.b0), "=&v"(g.b1)
            : "v"(dlt), "v"(u), "v"(a0), "v"(a1), "v"(sb0), "v"(sb1), "i"(TAU));
        asm volatile(
            "v_mul_f32_dpp %0, %3, %1 row_newbcast:%5 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %0, %4, %2 row_newbcast:%5 row_mask:0xf bank_mask:0xf"
            : "=&v"(p) : "v"(g.h0), "v"(g.h1), "v"(sc0), "v"(sc1), "i"(TAU));
    }
}

// kind 8 (SGPR operands) or 9 (DPP broadcasts): 4 tokens per trip, 40 vector instructions
// (the two v_mov_b32 per token that rename the state registers are counted separately).
template <bool kDpp>
__global__ void scan_body_kernel(int64_t iters, float *sink) {
    ScanRegs g;
    g.h0 = 0.1f * (threadIdx.x & 63);
    g.h1 = -g.h0;
    const float a0 = -1.44f - 1e-3f * (threadIdx.x & 15), a1 = -2.88f;
    float acc = 0.0f;
    float sb0 = 0.5f, sb1 = -0.25f, sc0 = 0.75f, sc1 = 1.5f;
    if constexpr (!kDpp) {
        sb0 = __builtin_amdgcn_readfirstlane(sb0 + 1e-3f * threadIdx.x);
        sc0 = __builtin_amdgcn_readfirstlane(sc0 + 1e-3f * threadIdx.x);
    }
    const float dl[4] = {0.1f, 0.2f, 0.15f, 0.3f}, uu[4] = {0.5f, -0.3f, 0.2f, 0.1f};
    uint64_t t0 = 0, r0 = 0, t1 = 0, r1 = 0;
    const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
    if (rec) clock_mark(t0, r0);
    for (int64_t k = 0; k < iters; ++k) {
        float p0, p1, p2, p3;
        scan_token<kDpp, 0>(g, dl[0], uu[0], a0, a1, sb0, sb1, sc0, sc1, p0);
        scan_token<kDpp, 1>(g, dl[1], uu[1], a0, a1, sb0, sb1, sc0, sc1, p1);
        scan_token<kDpp, 2>(g, dl[2], uu[2], a0, a1, sb0, sb1, sc0, sc1, p2);
        scan_token<kDpp, 3>(g, dl[3], uu[3], a0, a1, sb0, sb1, sc0, sc1, p3);
        acc += (p0 + p1) + (p2 + p3);
    }
    if (rec) clock_mark(t1, r1);
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc + g.h0 + g.h1;
    if (rec) store_clock(sink, (int)gridDim.x * (int)blockDim.x, t0, t1, r0, r1);
}

template <int KIND>
__global__ void valu_kernel(int64_t iters, float *sink) {
    float r[16];
    const float seed = 0.5f + 1e-3f * (threadIdx.x & 63);
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = seed + 0.01f * i;
    const float a = KIND == 4 ? 1.0f : KIND == 7 ? 1.0f : 0.999f, b = 1e-3f;
    uint64_t t0 = 0, r0 = 0, t1 = 0, r1 = 0;
    const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
    if (rec) clock_mark(t0, r0);
    for (int64_t k = 0; k < iters; ++k) valu_trip<KIND>(r, a, b);
    if (rec) clock_mark(t1, r1);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += r[i];
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    sink[g] = s;
    const int n = (int)gridDim.x * (int)blockDim.x;
    if (rec) store_clock(sink, n, t0, t1, r0, r1);
    if ((threadIdx.x & 63) == 0) {
        // where the wave ran: HW_ID (wave slot, SIMD, CU, shader array, engine) and XCC_ID
        const int wv = (int)(g >> 6);
        sink[n + 4 + 2 * wv] = __uint_as_float(__builtin_amdgcn_s_getreg((31 << 11) | 4));
        sink[n + 4 + 2 * wv + 1] = __uint_as_float(__builtin_amdgcn_s_getreg((31 << 11) | 20));
    }
}

// A trip: 4 independent 16x16x4 fp32 MFMAs and/or 32 v_fmac_f32 (8 between consecutive MFMAs).
template <int MODE>
__global__ void mfma_valu_kernel(int64_t iters, float *sink) {
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0.5f + 0.01f * i;
    const float a = 1e-3f + 1e-6f * (threadIdx.x & 63), b = 0.999f;
    // bf16 operands: 8 values of about 1e-2 (bf16 0x3c24) in four registers
    typedef short bf16x8 __attribute__((ext_vector_type(8)));
    const bf16x8 bq = (bf16x8)(short)0x3c24;
    for (int64_t k = 0; k < iters; ++k) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (MODE == 0 || MODE == 2)
                asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+v"(acc[m]) : "v"(a), "v"(b));
            if constexpr (MODE == 3 || MODE == 4)
                asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[m]) : "v"(bq), "v"(bq));
            if constexpr (MODE == 1 || MODE == 2 || MODE == 4)
                asm volatile(
                    "v_fmac_f32 %0, %8, %9\n\tv_fmac_f32 %1, %8, %9\n\tv_fmac_f32 %2, %8, %9\n\tv_fmac_f32 %3, %8, %9\n\t"
                    "v_fmac_f32 %4, %8, %9\n\tv_fmac_f32 %5, %8, %9\n\tv_fmac_f32 %6, %8, %9\n\tv_fmac_f32 %7, %8, %9"
                    : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7])
                    : "v"(a), "v"(b));
        }
    }
    // the compiler cannot see the MFMAs' latency inside the asm: wait them out before reading
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += r[i];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int VARIANT>
__global__ void mfma_rounding_kernel(const float *a, const float *b, const float *c, float *d_mfma, float *d_fma) {
    const int l = threadIdx.x;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(c + 4 * l);
    const float av = a[l], bv = b[l];
    // one tied operand: the destination quad is the addend's quad exactly (the compiler's
    // intrinsic may place them partly overlapping); the s_nops cover the operand-read and
    // result-read hazards that the compiler cannot see inside the asm
    if constexpr (VARIANT == 0)
        asm volatile("s_nop 4\n\tv_mfma_f32_4x4x1_16b_f32 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 15"
                     : "+v"(acc) : "v"(av), "v"(bv));
    else
        asm volatile("s_nop 4\n\tv_mfma_f32_16x16x4_f32 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15"
                     : "+v"(acc) : "v"(av), "v"(bv));
    *reinterpret_cast<f32x4 *>(d_mfma + 4 * l) = acc;
    if constexpr (VARIANT == 0) {
        // lane l = 4 * blk + j holds rows i = 0..3 of column j of block blk
        const int blk = l >> 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) d_fma[4 * l + i] = __builtin_fmaf(a[4 * blk + i], bv, c[4 * l + i]);
    } else {
        // lane l holds rows 4 (l / 16) + v of column l % 16; A[i][k] is at lane i + 16 k, B[k][j] at j + 16 k
        const int j = l & 15;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 4 * (l >> 4) + v;
            float r = c[4 * l + v];
#pragma unroll
            for (int k = 0; k < 4; ++k) r = __builtin_fmaf(a[i + 16 * k], b[j + 16 * k], r);
            d_fma[4 * l + v] = r;
        }
    }
}

__global__ void lds_kernel(int64_t iters, int unique, float *sink) {
    __shared__ __attribute__((aligned(16))) float buf[2048 + 256];
    for (int i = threadIdx.x; i < 2048 + 256; i += blockDim.x) buf[i] = 1e-3f * (float)(i & 255);
    __syncthreads();
    // lane l of a wave reads 16 bytes at (l % unique) * 16 + k * 1024: with unique = 64 each
    // instruction reads a contiguous KiB; with 16 the four 16-lane rows read the same 256 bytes
    const uint32_t base = (uint32_t)(uintptr_t)buf + ((threadIdx.x & 63) % unique) * 16;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t k = 0; k < iters; ++k) {
        f32x4 v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\tds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\tds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
            : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
            : "v"(base) : "memory");
        s = __builtin_elementwise_max(s, __builtin_elementwise_max(__builtin_elementwise_max(v0, v1),
                                                                   __builtin_elementwise_max(v2, v3)));
        s = __builtin_elementwise_max(s, __builtin_elementwise_max(__builtin_elementwise_max(v4, v5),
                                                                   __builtin_elementwise_max(v6, v7)));
    }
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

template <int KIND, bool NT>
__global__ __launch_bounds__(256) void hbm_kernel(const f32x4 *__restrict__ src, f32x4 *__restrict__ dst, int64_t n,
                                                  float *sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 w = f32x4{1.f, 2.f, 3.f, 4.f};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        if constexpr (KIND == 0) {
            acc += NT ? __builtin_nontemporal_load(src + i) : src[i];
        } else if constexpr (KIND == 1) {
            if constexpr (NT)
                __builtin_nontemporal_store(w, dst + i);
            else
                dst[i] = w;
        } else {
            if constexpr (NT)
                __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
            else
                dst[i] = src[i];
        }
    }
    if constexpr (KIND == 0) sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

bool threads_ok(int t, int maxt) { return t == 64 || t == 128 || t == 256 || t == 512 || (t == 1024 && maxt >= 1024); }

// Launches `launch` once untimed, then `reps` times between two events on `stream`.
template <typename F>
int timed(hipStream_t stream, int reps, float *ms_out, F launch) {
    launch();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    hipEvent_t a, b;
    if ((e = hipEventCreate(&a)) != hipSuccess) return (int)e;
    if ((e = hipEventCreate(&b)) != hipSuccess) {
        (void)hipEventDestroy(a);
        return (int)e;
    }
    (void)hipEventRecord(a, stream);
    for (int i = 0; i < reps; ++i) launch();
    e = hipGetLastError();
    (void)hipEventRecord(b, stream);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (e != hipSuccess) return (int)e;
    if (ms_out) *ms_out = ms;
    return 0;
}

}  // namespace

extern "C" {

int jscan_micro_valu(int kind, int64_t iters, int blocks, int threads, float *sink, void *stream, float *ms_out) {
    if (kind < 0 || kind > 11 || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > 65536 ||
        !threads_ok(threads, 1024) || !sink || !ms_out)
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto go = [&](auto k) {
        constexpr int K = decltype(k)::value;
        return timed(s, 1, ms_out, [&] {
            hipLaunchKernelGGL(valu_kernel<K>, dim3(blocks), dim3(threads), 0, s, iters, sink);
        });
    };
    if (kind == 8 || kind == 9)
        return timed(s, 1, ms_out, [&] {
            if (kind == 8)
                hipLaunchKernelGGL(scan_body_kernel<false>, dim3(blocks), dim3(threads), 0, s, iters, sink);
            else
                hipLaunchKernelGGL(scan_body_kernel<true>, dim3(blocks), dim3(threads), 0, s, iters, sink);
        });
    switch (kind) {
    case 0: return go(std::integral_constant<int, 0>{});
    case 1: return go(std::integral_constant<int, 1>{});
    case 2: return go(std::integral_constant<int, 2>{});
    case 3: return go(std::integral_constant<int, 3>{});
    case 4: return go(std::integral_constant<int, 4>{});
    case 5: return go(std::integral_constant<int, 5>{});
    case 6: return go(std::integral_constant<int, 6>{});
    case 7: return go(std::integral_constant<int, 7>{});
    case 11: return go(std::integral_constant<int, 11>{});
    default: return go(std::integral_constant<int, 10>{});
    }
}

int jscan_micro_mfma_valu(int mode, int64_t iters, int blocks, int threads, float *sink, void *stream,
                          float *ms_out) {
    if (mode < 0 || mode > 4 || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > 65536 ||
        !threads_ok(threads, 512) || !sink || !ms_out)
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto go = [&](auto k) {
        constexpr int M = decltype(k)::value;
        return timed(s, 1, ms_out, [&] {
            hipLaunchKernelGGL(mfma_valu_kernel<M>, dim3(blocks), dim3(threads), 0, s, iters, sink);
        });
    };
    if (mode == 0) return go(std::integral_constant<int, 0>{});
    if (mode == 1) return go(std::integral_constant<int, 1>{});
    if (mode == 2) return go(std::integral_constant<int, 2>{});
    if (mode == 3) return go(std::integral_constant<int, 3>{});
    return go(std::integral_constant<int, 4>{});
}

int jscan_micro_mfma_rounding(int variant, const float *a, const float *b, const float *c, float *d_mfma,
                              float *d_fma, void *stream) {
    if ((variant != 0 && variant != 1) || !a || !b || !c || !d_mfma || !d_fma) return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (variant == 0)
        hipLaunchKernelGGL(mfma_rounding_kernel<0>, dim3(1), dim3(64), 0, s, a, b, c, d_mfma, d_fma);
    else
        hipLaunchKernelGGL(mfma_rounding_kernel<1>, dim3(1), dim3(64), 0, s, a, b, c, d_mfma, d_fma);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return (int)e;
}

int jscan_micro_lds(int64_t iters, int unique, int blocks, int threads, float *sink, void *stream, float *ms_out) {
    if (iters < 1 || iters > (1 << 24) || (unique != 16 && unique != 32 && unique != 64) || blocks < 1 ||
        blocks > 65536 || !threads_ok(threads, 1024) || !sink || !ms_out)
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return timed(s, 1, ms_out,
                 [&] { hipLaunchKernelGGL(lds_kernel, dim3(blocks), dim3(threads), 0, s, iters, unique, sink); });
}

int jscan_micro_hbm(int kind, int nontemporal, const void *src, void *dst, int64_t bytes, int blocks, int reps,
                    float *sink, void *stream, float *ms_out) {
    if (kind < 0 || kind > 2 || bytes <= 0 || bytes % 16384 != 0 || bytes > ((int64_t)1 << 36) || blocks < 1 ||
        blocks > 65536 || reps < 1 || reps > 1000 || !sink || !ms_out)
        return -1;
    if ((kind != 1 && (!src || (reinterpret_cast<uintptr_t>(src) & 15))) ||
        (kind != 0 && (!dst || (reinterpret_cast<uintptr_t>(dst) & 15))))
        return -1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const f32x4 *sv = static_cast<const f32x4 *>(src);
    f32x4 *dv = static_cast<f32x4 *>(dst);
    const int64_t n = bytes / 16;
    auto go = [&](auto k, auto nt) {
        constexpr int K = decltype(k)::value;
        constexpr bool NT = decltype(nt)::value;
        return timed(s, reps, ms_out,
                     [&] { hipLaunchKernelGGL((hbm_kernel<K, NT>), dim3(blocks), dim3(256), 0, s, sv, dv, n, sink); });
    };
    using T = std::true_type;
    using F = std::false_type;
    if (kind == 0) return nontemporal ? go(std::integral_constant<int, 0>{}, T{}) : go(std::integral_constant<int, 0>{}, F{});
    if (kind == 1) return nontemporal ? go(std::integral_constant<int, 1>{}, T{}) : go(std::integral_constant<int, 1>{}, F{});
    return nontemporal ? go(std::integral_constant<int, 2>{}, T{}) : go(std::integral_constant<int, 2>{}, F{});
}

}  // extern "C"
