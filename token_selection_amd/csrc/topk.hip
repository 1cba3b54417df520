// Exact per-row top-k of the prefix scores plus the recent window.
//
// FastKV (page section 2A) keeps the most salient tokens plus a window of the
// newest; the budgets for the propagated token set and for the stored KV
// entries are separate calls (FastKV section 2B, StructKV section 3).
//
// Selection is exact and deterministic: the k-th largest score is found by a
// most-significant-digit-first radix select over the order-preserving
// integer image of the fp32 score bits (four 8-bit digits, histograms in
// LDS), which yields the threshold T and how many of the elements equal to T
// are taken. A block-wide scan then writes, in ascending position, every
// element above T and the lowest-positioned elements equal to T - which is
// exactly the order "score descending, then position ascending". The window
// positions follow.

#include <stdint.h>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkPerThread = 4;
constexpr int kTopkTile = kTopkThreads * kTopkPerThread;

// Monotone map from fp32 bits to uint32: a < b (as floats) <=> key(a) < key(b);
// -0 ranks equal to +0.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int64_t Np, int32_t w,
                                                               int32_t budget) {
    const int64_t row = blockIdx.x;
    const uint32_t* x = reinterpret_cast<const uint32_t*>(scores) + row * Np;
    int32_t* out = idx + row * (int64_t)budget;
    const int32_t kk = budget - w;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[2];
    __shared__ uint32_t wsum[kTopkThreads / 64];

    if (kk > 0) {
        uint32_t prefix = 0u, mask = 0u, remaining = (uint32_t)kk;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            if (tid < 256) hist[tid] = 0u;
            __syncthreads();
            for (int64_t i = tid; i < Np; i += kTopkThreads) {
                const uint32_t u = order_key(x[i]);
                if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 0xFFu], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                // walk digits from the top until the running count reaches
                // the number still to be selected
                uint32_t cum = 0u;
                int dgt = 255;
                for (; dgt > 0; --dgt) {
                    const uint32_t c = hist[dgt];
                    if (cum + c >= remaining) break;
                    cum += c;
                }
                sh[0] = prefix | ((uint32_t)dgt << shift);
                sh[1] = remaining - cum;
            }
            __syncthreads();
            prefix = sh[0];
            remaining = sh[1];
            mask |= 0xFFu << shift;
            __syncthreads();
        }
        const uint32_t T = prefix;         // key of the kk-th largest score
        const uint32_t take_eq = remaining;  // how many elements equal to T are kept
        uint32_t base_gt = 0u, base_eq = 0u;
        for (int64_t t0 = 0; t0 < Np; t0 += kTopkTile) {
            uint32_t flags = 0u, cgt = 0u, ceq = 0u;
#pragma unroll
            for (int e = 0; e < kTopkPerThread; ++e) {
                const int64_t i = t0 + (int64_t)tid * kTopkPerThread + e;
                if (i < Np) {
                    const uint32_t u = order_key(x[i]);
                    if (u > T) {
                        flags |= 1u << e;
                        ++cgt;
                    } else if (u == T) {
                        flags |= 16u << e;
                        ++ceq;
                    }
                }
            }
            // block exclusive scan of (gt count, eq count) packed 16:16; a
            // tile holds at most 4096 elements so neither half overflows
            const uint32_t v = (cgt << 16) | ceq;
            const uint32_t incl = wave_inclusive_scan(v, lane);
            if (lane == 63) wsum[wave] = incl;
            __syncthreads();
            uint32_t before = 0u, total = 0u;
#pragma unroll
            for (int w2 = 0; w2 < kTopkThreads / 64; ++w2) {
                const uint32_t s = wsum[w2];
                if (w2 < wave) before += s;
                total += s;
            }
            const uint32_t excl = before + incl - v;
            uint32_t gt_before = base_gt + (excl >> 16);
            uint32_t eq_before = base_eq + (excl & 0xFFFFu);
#pragma unroll
            for (int e = 0; e < kTopkPerThread; ++e) {
                const int32_t i = (int32_t)(t0 + (int64_t)tid * kTopkPerThread + e);
                if (flags & (1u << e)) {
                    out[gt_before + min(eq_before, take_eq)] = i;
                    ++gt_before;
                } else if (flags & (16u << e)) {
                    if (eq_before < take_eq) out[gt_before + eq_before] = i;
                    ++eq_before;
                }
            }
            base_gt += total >> 16;
            base_eq += total & 0xFFFFu;
            __syncthreads();
        }
    }
    for (int32_t m = tid; m < w; m += kTopkThreads) out[kk + m] = (int32_t)Np + m;
}

}  // namespace

hipError_t launch_topk(int32_t rows, int64_t n_keys, int32_t window, int32_t budget, const float* scores,
                       int32_t* idx, hipStream_t st) {
    const int64_t Np = n_keys - window;
    hipLaunchKernelGGL(topk_row_kernel, dim3(rows), dim3(kTopkThreads), 0, st, scores, idx, Np, window, budget);
    return hipGetLastError();
}

}  // namespace kvsel
