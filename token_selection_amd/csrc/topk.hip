// Exact per-row top-k of the prefix scores plus the recent window.
//
// FastKV (page section 2A) keeps the most salient tokens plus a window of the
// newest; the budgets for the propagated token set and for the stored KV
// entries are separate calls (FastKV section 2B, StructKV section 3).
//
// Selection is exact and deterministic. Scores map to an order-preserving
// 32-bit key; the k-th largest key T is found by a most-significant-digit
// radix select (digits of 11, 11 and 10 bits), which also yields how many
// keys equal to T are kept. Writing, in ascending position, every key above
// T and the lowest-positioned keys equal to T gives exactly the order "score
// descending, then position ascending"; the window positions follow.
//
// Every row is split into chunks handled by separate work-groups so that a
// handful of rows still fills the chip. Kernel boundaries order the steps:
//   hist(p)   per chunk: LDS histogram of digit p over keys matching the
//             prefix chosen so far, added bin by bin (integer atomics, so the
//             total is exact and order-independent) into hist[row][p][bins]
//   select(p) suffix-scan the bins of pass p, pick the digit holding the
//             k-th key, update (prefix, remaining): run by every work-group
//             of the next kernel (hist(p+1), or count after the last pass) on
//             the merged histogram, the row's first chunk also recording the
//             result in state[row][p]
//   count     per chunk: keys above T and equal to T
//   write     per chunk: exclusive offsets from the earlier chunks' counts,
//             then an in-order block scan that writes kept positions.

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "kvsel_internal.h"

// Scratch of kvsel_topk_noalloc: the histograms, per-pass states and chunk
// counts of one call, in a static device array (one copy per GPU, held until
// the process ends). Host code must not pass `scratch` itself to a kernel: its
// name is a host-side stand-in, so the device address is looked up once per
// device with hipGetSymbolAddress (topk_scratch below) and that is what the
// kernels get.
static __device__ __align__(256) unsigned char scratch[kvsel::kTopkScratchBytes];

namespace kvsel {
namespace {

constexpr int kThreads = 256;
constexpr int kBins = 2048;  // 11-bit digits
constexpr int kPasses = 3;
__host__ __device__ constexpr int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__host__ __device__ constexpr uint32_t digit_mask(int p) { return p == 2 ? 0x3FFu : 0x7FFu; }
// key bits already decided before pass p
__host__ __device__ constexpr uint32_t prefix_mask(int p) {
    return p == 0 ? 0u : (p == 1 ? 0xFFE00000u : 0xFFFFFC00u);
}

// Monotone map from fp32 bits to uint32: a < b (as floats) <=> key(a) < key(b);
// -0 ranks equal to +0.
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rank key of prefix position i of a row: protected sink positions take the
// largest key (above +inf's), so the select keeps them and orders them by
// position like any other tie.
__device__ __forceinline__ uint32_t rank_key(const uint32_t* x, int64_t i, int32_t n_sink) {
    return i < n_sink ? 0xFFFFFFFFu : order_key(x[i]);
}

struct TopkGeom {
    const uint32_t* x;  // scores as bits [rows][Np]
    int32_t* idx;       // [rows][budget]
    int64_t Np;
    int32_t w, budget, kk;
    int32_t n_sink;     // positions 0 .. n_sink-1 rank above every score (always kept)
    int32_t chunks;     // chunks per row
    int64_t chunk_len;  // elements per chunk (the last one may be shorter)
    uint32_t* hist;     // [rows][kPasses][kBins], zeroed by the window kernel
    uint32_t* state;    // [rows][kPasses][2]: prefix, remaining after each pass
    uint32_t* counts;   // [rows][chunks][2]: keys above T, keys equal to T
};

__device__ __forceinline__ void chunk_range(const TopkGeom& g, int chunk, int64_t& b, int64_t& e) {
    b = (int64_t)chunk * g.chunk_len;
    e = b + g.chunk_len;
    if (e > g.Np) e = g.Np;
    if (b > g.Np) b = g.Np;
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    return v;
}

// select(p) by the whole block: scan the merged histogram of pass p and choose
// the digit that holds the k-th largest key among those still matching; every
// thread gets the new (prefix, remaining). The row's first chunk records them
// in state[row][p] for the kernels after the next one.
__device__ void block_select(const TopkGeom& g, int64_t row, int pass, int chunk, uint32_t& prefix,
                             uint32_t& remaining) {
    constexpr int PER = kBins / kThreads;  // 8 consecutive digits per thread, highest first
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ uint32_t res[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t c[PER];
    uint32_t tot = 0u;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = kBins - 1 - (tid * PER + k);
        c[k] = g.hist[(row * kPasses + pass) * kBins + d];
        tot += c[k];
    }
    const uint32_t incl = wave_inclusive_scan(tot, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t above = incl - tot;  // keys in digits above this thread's first digit
    for (int w2 = 0; w2 < wave; ++w2) above += wsum[w2];
    // exactly one digit holds the k-th key (remaining <= the keys still matching)
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int d = kBins - 1 - (tid * PER + k);
        if (above < remaining && above + c[k] >= remaining) {
            res[0] = prefix | ((uint32_t)d << digit_shift(pass));
            res[1] = remaining - above;
        }
        above += c[k];
    }
    __syncthreads();
    prefix = res[0];
    remaining = res[1];
    if (chunk == 0 && tid == 0) {
        g.state[(row * kPasses + pass) * 2] = prefix;
        g.state[(row * kPasses + pass) * 2 + 1] = remaining;
    }
}

// (prefix, remaining) after pass p - 1 = select(p - 1) on the state after
// pass p - 2 (the initial one for pass 0: no prefix, kk to find).
__device__ __forceinline__ void state_after(const TopkGeom& g, int64_t row, int p1, int chunk, uint32_t& prefix,
                                            uint32_t& remaining) {
    prefix = p1 == 0 ? 0u : g.state[(row * kPasses + p1 - 1) * 2];
    remaining = p1 == 0 ? (uint32_t)g.kk : g.state[(row * kPasses + p1 - 1) * 2 + 1];
    block_select(g, row, p1, chunk, prefix, remaining);
}

__global__ __launch_bounds__(kThreads) void topk_hist_kernel(TopkGeom g, int pass) {
    __shared__ uint32_t h[kBins];
    const int chunk = blockIdx.x;
    const int64_t row = blockIdx.y;
    for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
    uint32_t prefix = 0u, remaining = (uint32_t)g.kk;
    if (pass > 0) state_after(g, row, pass - 1, chunk, prefix, remaining);
    const uint32_t pm = prefix_mask(pass);
    const int shift = digit_shift(pass);
    const uint32_t dm = digit_mask(pass);
    __syncthreads();
    int64_t b, e;
    chunk_range(g, chunk, b, e);
    const uint32_t* x = g.x + row * g.Np;
    for (int64_t i0 = b; i0 < e; i0 += kThreads * 8) {
        uint32_t u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = i0 + threadIdx.x + (int64_t)k * kThreads;
            u[k] = i < e ? rank_key(x, i, g.n_sink) : 0u;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = i0 + threadIdx.x + (int64_t)k * kThreads;
            if (i < e && (u[k] & pm) == prefix) atomicAdd(&h[(u[k] >> shift) & dm], 1u);
        }
    }
    __syncthreads();
    uint32_t* out = g.hist + (row * kPasses + pass) * kBins;
    for (int i = threadIdx.x; i < kBins; i += kThreads)
        if (h[i]) atomicAdd(&out[i], h[i]);
}

__global__ __launch_bounds__(kThreads) void topk_count_kernel(TopkGeom g) {
    __shared__ uint32_t red[2][kThreads / 64];
    const int chunk = blockIdx.x;
    const int64_t row = blockIdx.y;
    uint32_t T, take_eq;
    state_after(g, row, kPasses - 1, chunk, T, take_eq);
    int64_t b, e;
    chunk_range(g, chunk, b, e);
    const uint32_t* x = g.x + row * g.Np;
    uint32_t gt = 0u, eq = 0u;
    for (int64_t i0 = b; i0 < e; i0 += kThreads * 8) {
        uint32_t u[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = i0 + threadIdx.x + (int64_t)k * kThreads;
            u[k] = i < e ? rank_key(x, i, g.n_sink) : 0u;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t i = i0 + threadIdx.x + (int64_t)k * kThreads;
            gt += (i < e && u[k] > T) ? 1u : 0u;
            eq += (i < e && u[k] == T) ? 1u : 0u;
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        gt += __shfl_xor(gt, off);
        eq += __shfl_xor(eq, off);
    }
    if (lane == 0) {
        red[0][wave] = gt;
        red[1][wave] = eq;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t sg = 0u, se = 0u;
        for (int w2 = 0; w2 < kThreads / 64; ++w2) {
            sg += red[0][w2];
            se += red[1][w2];
        }
        g.counts[(row * g.chunks + chunk) * 2] = sg;
        g.counts[(row * g.chunks + chunk) * 2 + 1] = se;
    }
}

// Write this chunk's kept positions in ascending order: a key above T is
// kept; a key equal to T is kept while fewer than take_eq equal keys precede
// it in the row. The output slot is (#keys above T before it) +
// min(#equal keys before it, take_eq).
__global__ __launch_bounds__(kThreads) void topk_write_kernel(TopkGeom g) {
    constexpr int PER = 16;  // consecutive elements per thread per tile
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ uint32_t wsum2[kThreads / 64];
    __shared__ uint32_t base_sh[2];
    const int chunk = blockIdx.x;
    const int64_t row = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t T = g.state[(row * kPasses + kPasses - 1) * 2];
    const uint32_t take_eq = g.state[(row * kPasses + kPasses - 1) * 2 + 1];
    int32_t* out = g.idx + row * (int64_t)g.budget;
    {
        // counts of the chunks before this one, summed by the whole block
        uint32_t sg = 0u, se = 0u;
        for (int ch = tid; ch < chunk; ch += kThreads) {
            sg += g.counts[(row * g.chunks + ch) * 2];
            se += g.counts[(row * g.chunks + ch) * 2 + 1];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sg += __shfl_xor(sg, off);
            se += __shfl_xor(se, off);
        }
        if (lane == 0) {
            wsum[wave] = sg;
            wsum2[wave] = se;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t a0 = 0u, a1 = 0u;
            for (int w2 = 0; w2 < kThreads / 64; ++w2) {
                a0 += wsum[w2];
                a1 += wsum2[w2];
            }
            base_sh[0] = a0;
            base_sh[1] = a1;
        }
    }
    __syncthreads();
    uint32_t base_gt = base_sh[0], base_eq = base_sh[1];
    int64_t b, e;
    chunk_range(g, chunk, b, e);
    const uint32_t* x = g.x + row * g.Np;
    for (int64_t t0 = b; t0 < e; t0 += (int64_t)kThreads * PER) {
        uint32_t u[PER];
        const int64_t first = t0 + (int64_t)tid * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) u[k] = first + k < e ? rank_key(x, first + k, g.n_sink) : 0u;
        uint32_t cgt = 0u, ceq = 0u;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const bool in = first + k < e;
            cgt += (in && u[k] > T) ? 1u : 0u;
            ceq += (in && u[k] == T) ? 1u : 0u;
        }
        // packed 16:16 block scan; a tile holds 4096 elements
        const uint32_t v = (cgt << 16) | ceq;
        const uint32_t incl = wave_inclusive_scan(v, lane);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint32_t before = 0u, total = 0u;
#pragma unroll
        for (int w2 = 0; w2 < kThreads / 64; ++w2) {
            const uint32_t s2 = wsum[w2];
            if (w2 < wave) before += s2;
            total += s2;
        }
        const uint32_t excl = before + incl - v;
        uint32_t gt_before = base_gt + (excl >> 16);
        uint32_t eq_before = base_eq + (excl & 0xFFFFu);
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            if (first + k < e) {
                const int32_t i = (int32_t)(first + k);
                if (u[k] > T) {
                    out[gt_before + min(eq_before, take_eq)] = i;
                    ++gt_before;
                } else if (u[k] == T) {
                    if (eq_before < take_eq) out[gt_before + eq_before] = i;
                    ++eq_before;
                }
            }
        }
        base_gt += total >> 16;
        base_eq += total & 0xFFFFu;
        __syncthreads();
    }
}

// Rows of at most kRowMax prefix keys (the short rows of small problems,
// where six launches would cost more than the work) take one work-group of
// kRowThreads threads per row and a single launch: thread t holds the rank keys of the
// row's positions [t*kRowPer, t*kRowPer + kRowPer) in registers, each wave
// counts digits into its own LDS histogram (conflicts stay inside a wave), the
// histograms are summed per digit and scanned from the highest digit down to
// pick the digit of the k-th key, three times (11, 11, 10 bits); then each
// thread counts its keys above T and equal to T, one block scan turns the
// counts into output slots, and every thread writes its kept positions in
// ascending order.
constexpr int kRowThreads = 256;
constexpr int kRowPer = 16;
constexpr int kRowMax = kRowThreads * kRowPer;  // 4096
constexpr int kRowWaves = kRowThreads / 64;

// Exclusive scan of v over the block (kRowThreads threads); *total gets the sum.
__device__ __forceinline__ uint32_t row_block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t incl = wave_inclusive_scan(v, lane);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0u, all = 0u;
#pragma unroll
    for (int w2 = 0; w2 < kRowWaves; ++w2) {
        const uint32_t t = wsum[w2];
        before += w2 < wave ? t : 0u;
        all += t;
    }
    __syncthreads();  // wsum is reused by the next scan
    *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const uint32_t* __restrict__ scores, int32_t* idx,
                                                               int64_t Np, int32_t w, int32_t budget, int32_t kk,
                                                               int32_t n_sink) {
    __shared__ uint32_t hist[kRowWaves][kBins];
    __shared__ uint32_t wsum[kRowWaves];
    __shared__ uint32_t res[2];
    const int tid = threadIdx.x, wave = tid >> 6;
    const int64_t row = blockIdx.x;
    int32_t* out = idx + row * (int64_t)budget;
    for (int m = tid; m < w; m += kRowThreads) out[kk + m] = (int32_t)(Np + m);
    if (kk == 0) return;
    const uint32_t* x = scores + row * Np;
    const int64_t first = (int64_t)tid * kRowPer;
    uint32_t u[kRowPer];
#pragma unroll
    for (int k = 0; k < kRowPer; ++k) u[k] = first + k < Np ? rank_key(x, first + k, n_sink) : 0u;
    uint32_t prefix = 0u, remaining = (uint32_t)kk;
#pragma unroll 1
    for (int pass = 0; pass < kPasses; ++pass) {
        for (int i = tid; i < kRowWaves * kBins; i += kRowThreads) (&hist[0][0])[i] = 0u;
        __syncthreads();
        const uint32_t pm = prefix_mask(pass);
        const int shift = digit_shift(pass);
        const uint32_t dm = digit_mask(pass);
#pragma unroll
        for (int k = 0; k < kRowPer; ++k)
            if (first + k < Np && (u[k] & pm) == prefix) atomicAdd(&hist[wave][(u[k] >> shift) & dm], 1u);
        __syncthreads();
        // thread t owns the kDig digits 2047 - kDig*t ... (highest first)
        constexpr int kDig = kBins / kRowThreads;
        uint32_t c[kDig];
        uint32_t mine = 0u;
#pragma unroll
        for (int k = 0; k < kDig; ++k) {
            const int d = kBins - 1 - (kDig * tid + k);
            uint32_t sum = 0u;
#pragma unroll
            for (int w2 = 0; w2 < kRowWaves; ++w2) sum += hist[w2][d];
            c[k] = sum;
            mine += sum;
        }
        uint32_t tot;
        uint32_t above = row_block_scan(mine, wsum, &tot);
#pragma unroll
        for (int k = 0; k < kDig; ++k) {
            const int d = kBins - 1 - (kDig * tid + k);
            if (above < remaining && above + c[k] >= remaining) {
                res[0] = prefix | ((uint32_t)d << shift);
                res[1] = remaining - above;
            }
            above += c[k];
        }
        __syncthreads();
        prefix = res[0];
        remaining = res[1];
        __syncthreads();  // res and hist are rewritten by the next pass
    }
    // prefix is now the k-th key T; remaining is how many keys equal to T are kept
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int k = 0; k < kRowPer; ++k) {
        const bool in = first + k < Np;
        gt += (in && u[k] > prefix) ? 1u : 0u;
        eq += (in && u[k] == prefix) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t excl = row_block_scan((gt << 16) | eq, wsum, &tot);
    uint32_t gt_before = excl >> 16, eq_before = excl & 0xFFFFu;
#pragma unroll
    for (int k = 0; k < kRowPer; ++k) {
        if (first + k >= Np) break;
        if (u[k] > prefix) {
            out[gt_before + min(eq_before, remaining)] = (int32_t)(first + k);
            ++gt_before;
        } else if (u[k] == prefix) {
            if (eq_before < remaining) out[gt_before + eq_before] = (int32_t)(first + k);
            ++eq_before;
        }
    }
}

// Writes the window positions and zeroes the digit histograms (it runs first).
__global__ __launch_bounds__(kThreads) void topk_window_kernel(int32_t* idx, int32_t rows, int64_t Np, int32_t w,
                                                               int32_t budget, uint32_t* hist) {
    if (hist) {
        const int64_t nh = (int64_t)rows * kPasses * kBins;
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nh; i += (int64_t)gridDim.x * kThreads)
            hist[i] = 0u;
    }
    const int64_t total = (int64_t)rows * w;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
        const int64_t row = i / w;
        const int32_t m = (int32_t)(i - row * w);
        idx[row * budget + (budget - w) + m] = (int32_t)Np + m;
    }
}

void plan_chunks(int32_t rows, int64_t Np, int32_t& chunks, int64_t& chunk_len) {
    // about 512 work-groups in all, each with at least 2048 elements
    int64_t c = (512 + rows - 1) / rows;
    const int64_t max_c = (Np + 2047) / 2048;
    if (c > max_c) c = max_c;
    if (c < 1) c = 1;
    chunk_len = (Np + c - 1) / c;
    chunk_len = (chunk_len + 255) & ~(int64_t)255;
    if (chunk_len < 256) chunk_len = 256;
    chunks = (int32_t)((Np + chunk_len - 1) / chunk_len);
    if (chunks < 1) chunks = 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t topk_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            // this device's copy of the array (the current device's address)
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

size_t topk_workspace_bytes(int32_t rows, int64_t Np) {
    int32_t chunks;
    int64_t chunk_len;
    plan_chunks(rows, Np > 0 ? Np : 1, chunks, chunk_len);
    return align256((size_t)rows * kPasses * kBins * sizeof(uint32_t)) +
           align256((size_t)rows * kPasses * 2 * sizeof(uint32_t)) +
           align256((size_t)rows * chunks * 2 * sizeof(uint32_t));
}

hipError_t launch_topk(int32_t rows, int64_t n_keys, int32_t window, int32_t budget, int32_t n_sink,
                       const float* scores, int32_t* idx, void* ws, hipStream_t st) {
    const int64_t Np = n_keys - window;
    if (Np <= kRowMax) {
        // short rows: one work-group per row, one launch (longer rows need
        // the chunked kernels' parallelism)
        hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, st,
                           reinterpret_cast<const uint32_t*>(scores), idx, Np, window, budget, budget - window,
                           n_sink);
        return hipGetLastError();
    }
    TopkGeom g;
    g.n_sink = n_sink;
    g.x = reinterpret_cast<const uint32_t*>(scores);
    g.idx = idx;
    g.Np = Np;
    g.w = window;
    g.budget = budget;
    g.kk = budget - window;
    g.hist = nullptr;
    if (g.kk > 0) {
        plan_chunks(rows, Np, g.chunks, g.chunk_len);
        char* p = static_cast<char*>(ws);
        g.hist = reinterpret_cast<uint32_t*>(p);
        p += align256((size_t)rows * kPasses * kBins * sizeof(uint32_t));
        g.state = reinterpret_cast<uint32_t*>(p);
        p += align256((size_t)rows * kPasses * 2 * sizeof(uint32_t));
        g.counts = reinterpret_cast<uint32_t*>(p);
    }
    int64_t work = (int64_t)rows * window;
    if (g.hist && (int64_t)rows * kPasses * kBins > work) work = (int64_t)rows * kPasses * kBins;
    int64_t blocks = (work + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(topk_window_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, st, idx, rows, Np, window, budget,
                       g.hist);
    if (g.kk > 0) {
        const dim3 grid((unsigned)g.chunks, (unsigned)rows);
        for (int pass = 0; pass < kPasses; ++pass)
            hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kThreads), 0, st, g, pass);
        hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kThreads), 0, st, g);
        hipLaunchKernelGGL(topk_write_kernel, grid, dim3(kThreads), 0, st, g);
    }
    return hipGetLastError();
}

}  // namespace kvsel
