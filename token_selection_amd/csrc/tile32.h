// Matrix-core building blocks of the saliency kernels (bf16 Q and K, fp32
// logits): 32x32x16 MFMA tiles, the operand layout they share, and the
// per-row (reference, sum of exp2) partials of the first softmax pass.
//
// Operand layout (v_mfma_f32_32x32x16_bf16): lane l supplies row/column
// (l % 32) and the 8 consecutive k-slots of lane half (l / 32). At k-step ks
// the slot (half, v) carries head-dim element ks*16 + half*8 + v, for K and Q
// alike (any order works as long as both operands use the same one). A 32x32
// result tile leaves lane l with column (l % 32) and rows
// 8*(v/4) + 4*(l/32) + (v%4), v = 0..15.
//
// Softmax arithmetic is in the log2 domain: with c = scale * log2(e) a logit x
// contributes exp2(c*x - ref), and a row's LSE2 is ref + log2(sum).
#pragma once

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kvsel {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegBig = -1.0e30f;
constexpr float kOverflow = 0x1p64f;  // a partial sum this large means the reference was too low

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int v = 0; v < 16; ++v) z[v] = 0.f;
    return z;
}

// Key offset, within a 32-key block, of result register v of lane half hf.
__device__ __forceinline__ int tile_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

__device__ __forceinline__ void merge(float& m, float& z, float mo, float zo) {
    const float mn = fmaxf(m, mo);
    z = z * fexp2(m - mn) + zo * fexp2(mo - mn);
    m = mn;
}

// Logits of one 32-key block against one 32-row block: key-major (K as the A
// operand: lane = query row, registers = keys) or row-major (Q as A: lane =
// key, registers = query rows).
template <int KS>
__device__ __forceinline__ f32x16 logits(const bf16x8 (&a)[KS], const bf16x8 (&b)[KS]) {
    f32x16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mma(a[ks], b[ks], acc);
    return acc;
}

// Pass 1, common case: the reference is the lane's running one (`run`), or
// its first logit while it has none (run == kNegBig). Any value is a valid
// reference as far as the final LSE goes (partials are merged by rescaling to
// a common one); it only has to keep exp2 in range, and a sum of kOverflow or
// more (or inf) sends the block to pass1_max. Keys far below the reference
// add exp2 terms that underflow to zero next to a sum of at least 1 (the
// reference logit's own term, or the row maximum's). The exponentials of
// block kb run while block kb+1 is in the matrix core.
template <int D, int KB>
__device__ __forceinline__ float pass1_fast(const bf16x8 (&kf)[KB][D / 16], const bf16x8 (&qf)[D / 16], float c,
                                            float run, float& ref) {
    constexpr int KS = D / 16;
    f32x16 cur = logits<KS>(kf[0], qf);
    ref = run > kNegBig ? run : cur[0] * c;
    float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        f32x16 nxt;
        if (kb + 1 < KB) nxt = logits<KS>(kf[kb + 1], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v) zs[v & 3] += fexp2(cur[v] * c - ref);
        if (kb + 1 < KB) cur = nxt;
    }
    return (zs[0] + zs[1]) + (zs[2] + zs[3]);
}

// Pass 1 with the row maximum as the reference: blocks that reach the causal
// window (keys past lim are masked) and the rare blocks whose first logit was
// too low a reference. The logits are computed twice (maximum, then sum).
template <int D, int KB, bool MASK>
__device__ __forceinline__ float pass1_max(const bf16x8 (&kf)[KB][D / 16], const bf16x8 (&qf)[D / 16], float c,
                                        int kfirst, int hf, int lim, float& ref) {
    constexpr int KS = D / 16;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const f32x16 acc = logits<KS>(kf[kb], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (!MASK || kfirst + kb * 32 + tile_row(v, hf) <= lim) mx = fmaxf(mx, acc[v]);
    }
    ref = fmaxf(kNegBig, mx * c);
    float zs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const f32x16 acc = logits<KS>(kf[kb], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (!MASK || kfirst + kb * 32 + tile_row(v, hf) <= lim) zs[v & 3] += fexp2(acc[v] * c - ref);
    }
    return (zs[0] + zs[1]) + (zs[2] + zs[3]);
}

// Pivot statistics ride on pass 1: next to the sum z of exp2(c*x - ref) a row
// carries s = sum of exp2(c*x - ref) * x and q = sum of exp2(c*x - ref)^2 on the
// same reference, so that sum p*x = s / z and sum p^2 = q / z^2 once the
// reference is final. With them the fast path needs a tighter overflow bound:
// z < 2^40 keeps q <= z^2 finite.
constexpr float kOverflowSt = 0x1p40f;

struct Moments {
    float s, q;
};

__device__ __forceinline__ void merge_st(float& m, float& z, Moments& a, float mo, float zo, Moments b) {
    const float mn = fmaxf(m, mo);
    const float f = fexp2(m - mn);
    const float g = fexp2(mo - mn);
    z = z * f + zo * g;
    a.s = a.s * f + b.s * g;
    a.q = a.q * (f * f) + b.q * (g * g);
    m = mn;
}

template <int D, int KB>
__device__ __forceinline__ float pass1_fast_st(const bf16x8 (&kf)[KB][D / 16], const bf16x8 (&qf)[D / 16], float c,
                                               float& ref, Moments& mo) {
    constexpr int KS = D / 16;
    f32x16 cur = logits<KS>(kf[0], qf);
    ref = cur[0] * c;
    float zs[2] = {0.f, 0.f}, ss[2] = {0.f, 0.f}, qs[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        f32x16 nxt;
        if (kb + 1 < KB) nxt = logits<KS>(kf[kb + 1], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float e = fexp2(cur[v] * c - ref);
            zs[v & 1] += e;
            ss[v & 1] += e * cur[v];
            qs[v & 1] += e * e;
        }
        if (kb + 1 < KB) cur = nxt;
    }
    mo.s = ss[0] + ss[1];
    mo.q = qs[0] + qs[1];
    return zs[0] + zs[1];
}

template <int D, int KB, bool MASK>
__device__ __forceinline__ float pass1_max_st(const bf16x8 (&kf)[KB][D / 16], const bf16x8 (&qf)[D / 16], float c,
                                              int kfirst, int hf, int lim, float& ref, Moments& mo) {
    constexpr int KS = D / 16;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const f32x16 acc = logits<KS>(kf[kb], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (!MASK || kfirst + kb * 32 + tile_row(v, hf) <= lim) mx = fmaxf(mx, acc[v]);
    }
    ref = fmaxf(kNegBig, mx * c);
    float zs[2] = {0.f, 0.f}, ss[2] = {0.f, 0.f}, qs[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const f32x16 acc = logits<KS>(kf[kb], qf);
#pragma unroll
        for (int v = 0; v < 16; ++v)
            if (!MASK || kfirst + kb * 32 + tile_row(v, hf) <= lim) {
                const float e = fexp2(acc[v] * c - ref);
                zs[v & 1] += e;
                ss[v & 1] += e * acc[v];
                qs[v & 1] += e * e;
            }
    }
    mo.s = ss[0] + ss[1];
    mo.q = qs[0] + qs[1];
    return zs[0] + zs[1];
}

}  // namespace tile
}  // namespace kvsel
