// Row gather (cache compaction) and score accumulation.
//
// Gather: FastKV (page section 2A) passes only the kept tokens on, and both
// FastKV section 2B and StructKV section 3 store only the kept KV entries;
// the copy is bit for bit. Accumulation: StructKV section 1 adds a token's
// scores over layers; the head mean gives FastKV's single token set per
// sequence.

#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {
namespace {

struct GatherGeom {
    const char* src;
    int64_t s0, s1, s2, s3;  // byte strides over (layer, b, head, row)
    const int32_t* idx;
    int32_t B, H, idx_heads, budget;
    int64_t n_src;
    int64_t cpr;    // copy units per row
    int64_t total;  // copy units in the whole output
};

__device__ __forceinline__ const char* gather_src_row(const GatherGeom& g, int64_t row, bool& valid) {
    const int64_t t = row % g.budget;
    int64_t rest = row / g.budget;
    const int64_t h = rest % g.H;
    rest /= g.H;
    const int64_t b = rest % g.B;
    const int64_t l = rest / g.B;
    const int32_t j = g.idx[(b * g.idx_heads + (g.idx_heads == 1 ? 0 : h)) * g.budget + t];
    valid = j >= 0 && (int64_t)j < g.n_src;
    return g.src + l * g.s0 + b * g.s1 + h * g.s2 + (valid ? (int64_t)j : 0) * g.s3;
}

// 16-byte units: consecutive threads copy consecutive units of a row, so a
// 256-byte K row is one fully used 256-byte burst per 16 threads.
__global__ __launch_bounds__(256) void gather16_kernel(GatherGeom g, uint4* __restrict__ dst) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < g.total;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = c / g.cpr;
        const int64_t off = c - row * g.cpr;
        bool valid;
        const char* s = gather_src_row(g, row, valid);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (valid) v = reinterpret_cast<const uint4*>(s)[off];
        dst[c] = v;
    }
}

// Slab form of the 16-byte gather, for rows whose unit count is a power of
// two times U: grid row y is one (layer, b, head) slab, so the source base and
// index row are set once per work-group, and each work item is one
// (kept row, lane slot) pair copying U units, slot q taking units q, q + ipr, ...
// (ipr = units per row / U). A row's ipr lanes thus read and write contiguous
// 16*ipr-byte pieces per load, and no work item divides by a run-time size.
struct GatherSlab {
    const char* src;
    int64_t s0, s1, s2, s3;  // byte strides over (layer, b, head, row)
    const int32_t* idx;
    int32_t B, H, idx_heads, budget;
    int64_t n_src;
    int32_t cpr;        // units per row
    int32_t ipr_shift;  // log2(units per row / U)
    int32_t items;      // budget << ipr_shift
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void gather16_slab_kernel(GatherSlab g, uint4* __restrict__ dst) {
    const int slab = blockIdx.y;  // (l*B + b)*H + h
    const int h = slab % g.H;
    const int lb = slab / g.H;
    const int b = lb % g.B;
    const int l = lb / g.B;
    const int32_t* idx = g.idx + (int64_t)(b * g.idx_heads + (g.idx_heads == 1 ? 0 : h)) * g.budget;
    const char* src = g.src + l * g.s0 + b * g.s1 + h * g.s2;
    uint4* out = dst + (int64_t)slab * g.budget * g.cpr;
    const int ipr = 1 << g.ipr_shift;
    for (int it = blockIdx.x * 256 + threadIdx.x; it < g.items; it += gridDim.x * 256) {
        const int t = it >> g.ipr_shift;
        const int q = it & (ipr - 1);
        const int32_t j = idx[t];
        const bool valid = j >= 0 && (int64_t)j < g.n_src;
        const uint4* s = reinterpret_cast<const uint4*>(src + (valid ? (int64_t)j : 0) * g.s3) + q;
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = valid ? s[u * ipr] : make_uint4(0u, 0u, 0u, 0u);
        // non-temporal stores: the output is not read again soon; kept out of
        // the caches, it no longer delays the reads of the copy that follows
        u32x4* o = reinterpret_cast<u32x4*>(out + (int64_t)t * g.cpr + q);
#pragma unroll
        for (int u = 0; u < U; ++u) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v[u]), o + u * ipr);
    }
}

__global__ __launch_bounds__(256) void gather1_kernel(GatherGeom g, char* __restrict__ dst) {
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < g.total;
         c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = c / g.cpr;
        const int64_t off = c - row * g.cpr;
        bool valid;
        const char* s = gather_src_row(g, row, valid);
        dst[c] = valid ? s[off] : (char)0;
    }
}

__global__ __launch_bounds__(256) void acc_add_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] += src[i];
}

__global__ __launch_bounds__(256) void acc_head_mean_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                            int32_t B, int32_t H, int64_t n) {
    const int64_t total = (int64_t)B * n;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / n;
        const int64_t j = i - b * n;
        float sum = 0.f;
        for (int32_t h = 0; h < H; ++h) sum += src[((int64_t)b * H + h) * n + j];
        dst[i] = sum / (float)H;
    }
}

unsigned grid_for(int64_t work) {
    int64_t blocks = (work + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    return (unsigned)blocks;
}

}  // namespace

hipError_t launch_gather(int32_t L, int32_t B, int32_t H, int32_t idx_heads, int32_t budget, int64_t n_src_rows,
                         int64_t row_bytes, const void* src, const int64_t s[4], const int32_t* idx, void* dst,
                         hipStream_t st) {
    GatherGeom g;
    g.src = static_cast<const char*>(src);
    g.s0 = s[0];
    g.s1 = s[1];
    g.s2 = s[2];
    g.s3 = s[3];
    g.idx = idx;
    g.B = B;
    g.H = H;
    g.idx_heads = idx_heads;
    g.budget = budget;
    g.n_src = n_src_rows;
    const int64_t rows = (int64_t)L * B * H * budget;
    bool vec = (row_bytes % 16 == 0) && (((uintptr_t)src | (uintptr_t)dst) % 16 == 0);
    for (int i = 0; i < 4; ++i) vec = vec && (s[i] % 16 == 0);
    if (vec) {
        // the slab form: whole powers of two of 4 units (64 bytes) per row, or
        // rows of 1 or 2 units, with the grid rows and work items in range
        const int64_t cpr = row_bytes / 16;
        const int u = cpr % 4 == 0 ? 4 : 1;
        const int64_t ipr = cpr / u;
        const int64_t slabs = (int64_t)L * B * H;
        if ((ipr & (ipr - 1)) == 0 && slabs <= 65535 && (int64_t)budget * ipr < ((int64_t)1 << 31)) {
            GatherSlab gs;
            gs.src = g.src;
            gs.s0 = s[0];
            gs.s1 = s[1];
            gs.s2 = s[2];
            gs.s3 = s[3];
            gs.idx = idx;
            gs.B = B;
            gs.H = H;
            gs.idx_heads = idx_heads;
            gs.budget = budget;
            gs.n_src = n_src_rows;
            gs.cpr = (int32_t)cpr;
            gs.ipr_shift = 0;
            while (((int64_t)1 << gs.ipr_shift) < ipr) ++gs.ipr_shift;
            gs.items = (int32_t)((int64_t)budget * ipr);
            int64_t bx = ((int64_t)gs.items + 255) / 256;
            if (bx > 4096) bx = 4096;
            const dim3 grid((unsigned)bx, (unsigned)slabs);
            if (u == 4)
                hipLaunchKernelGGL(gather16_slab_kernel<4>, grid, dim3(256), 0, st, gs, static_cast<uint4*>(dst));
            else
                hipLaunchKernelGGL(gather16_slab_kernel<1>, grid, dim3(256), 0, st, gs, static_cast<uint4*>(dst));
            return hipGetLastError();
        }
        g.cpr = row_bytes / 16;
        g.total = rows * g.cpr;
        hipLaunchKernelGGL(gather16_kernel, dim3(grid_for(g.total)), dim3(256), 0, st, g, static_cast<uint4*>(dst));
    } else {
        g.cpr = row_bytes;
        g.total = rows * g.cpr;
        hipLaunchKernelGGL(gather1_kernel, dim3(grid_for(g.total)), dim3(256), 0, st, g, static_cast<char*>(dst));
    }
    return hipGetLastError();
}

hipError_t launch_accumulate(int32_t B, int32_t H, int64_t n, const float* src, float* dst, int mode,
                             hipStream_t st) {
    if (n == 0) return hipSuccess;
    if (mode == KVSEL_ACC_ADD) {
        const int64_t total = (int64_t)B * H * n;
        hipLaunchKernelGGL(acc_add_kernel, dim3(grid_for(total)), dim3(256), 0, st, src, dst, total);
    } else {
        hipLaunchKernelGGL(acc_head_mean_kernel, dim3(grid_for((int64_t)B * n)), dim3(256), 0, st, src, dst, B, H, n);
    }
    return hipGetLastError();
}

}  // namespace kvsel
