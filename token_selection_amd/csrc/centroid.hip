// CentroidKV chunked soft matching (CSM), one clustering round on the GPU
// (page "Technische Samenvatting: CentroidKV", section "Methodologie":
// part 2 keeps attention sinks and recent tokens out of the partition, part 3
// chunks the rest, splits every chunk alternately into sets A and B, matches
// each A token to its most similar B token and merges only the best-ranked
// matches, part 4 turns each cluster into a degree-weighted centroid).
//
// Slab layout: S slabs (layer, sequence, KV head) of n tokens, keys and
// values contiguous [S][n][d] bf16; degrees [S][n] int32 (all 1 when absent).
// The middle [n_sink, n - n_recent) is cut into chunks of C tokens (C even,
// <= 64); in a chunk offsets 0, 2, ... are A and 1, 3, ... are B. The A
// tokens of a slab are numbered in position order: A index c*C/2 + i for the
// i-th A token of chunk c.
//
//   csm_match_kernel   one wave per chunk: the A x B cosine similarities of
//                      the chunk as one 32x32 tile of 32x32x16 MFMAs (A keys
//                      as the B operand, so a lane is an A token and its
//                      registers are B tokens), the best B of each A (ties to
//                      the lower position) -> score, match, and the A token's
//                      flag cleared.
//   (kvsel top-k)      the n_merge best scores of each slab, ties to the lower
//                      A index (the selection kernels with no window).
//   csm_flag_kernel    marks the chosen A tokens.
//   csm_offsets_kernel survivors before each chunk (exclusive scan per slab).
//   csm_merge_kernel   one work-group per span of chunks: survivors in
//                      position order; a B token that received merges becomes
//                      the degree-weighted
//                      mean of its cluster (fp32 sum of (degree_i / W) * x_i,
//                      rounded to bf16 to nearest even), every other survivor
//                      is copied bit for bit.
//   csm_edges_kernel   copies the sinks and the recent tokens.

#include <math.h>
#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"
#include "tile32.h"

namespace kvsel {
namespace {

using namespace tile;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kCsmWaves = 4;  // chunks per work-group

struct CsmGeom {
    int32_t S, d;
    int64_t n, n_out;
    int32_t C, n_sink, n_recent;
    int64_t M;         // middle tokens
    int32_t n_chunks;  // per slab
    int64_t n_a;       // A tokens per slab
    int32_t n_merge;
};

__device__ __forceinline__ void chunk_range(const CsmGeom& g, int c, int64_t& start, int& len) {
    start = g.n_sink + (int64_t)c * g.C;
    const int64_t end = g.n_sink + g.M;
    len = (int)min((int64_t)g.C, end - start);
}

template <int D>
__global__ void __launch_bounds__(256) csm_match_kernel(CsmGeom g, const uint16_t* __restrict__ k, float* score,
                                                        int32_t* match, uint8_t* flags) {
    constexpr int KS = D / 16;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int c = blockIdx.x * kCsmWaves + wave;
    const int slab = blockIdx.y;
    if (c >= g.n_chunks) return;
    int64_t start;
    int len;
    chunk_range(g, c, start, len);
    const int na = (len + 1) >> 1;
    const int nb = len >> 1;
    const uint16_t* ks = k + (int64_t)slab * g.n * D;
    // Each load instruction reads 32 consecutive rows of the chunk, 32 bytes
    // of each (a faster pattern than every other row): lane col < 16 takes
    // row 2*col (A token col), lane col >= 16 row 2*(col-16) + 1 (B token
    // col-16), in the first 32 rows (x) and the next 32 (y); rows past the
    // chunk read its last row (those tokens are masked). Swapping x's lanes
    // 16-31 with y's lanes 0-15 (and 48-63 with 32-47) leaves A tokens 0-31
    // in x and B tokens 0-31 in y: lane (col, hf) holds A token col and B
    // token col, head-dim elements s*16 + hf*8 .. +7.
    const int r0 = col < 16 ? 2 * col : 2 * (col - 16) + 1;
    const int64_t px = start + min(r0, len - 1);
    const int64_t py = start + min(32 + r0, len - 1);
    bf16x8 fa[KS], fb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint4 x = *reinterpret_cast<const uint4*>(ks + px * D + s * 16 + hf * 8);
        const uint4 y = *reinterpret_cast<const uint4*>(ks + py * D + s * 16 + hf * 8);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
        uint32_t as[4], bs[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const auto r = __builtin_amdgcn_permlane16_swap(xs[h], ys[h], false, false);
            as[h] = r[0];
            bs[h] = r[1];
        }
        fa[s] = __builtin_bit_cast(bf16x8, make_uint4(as[0], as[1], as[2], as[3]));
        fb[s] = __builtin_bit_cast(bf16x8, make_uint4(bs[0], bs[1], bs[2], bs[3]));
    }
    // |k|^2 of A token col and of B token col: bf16 pairs squared and summed in fp32 (v_dot2)
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const uint4 ua = __builtin_bit_cast(uint4, fa[s]);
        const uint4 ub = __builtin_bit_cast(uint4, fb[s]);
        const uint32_t wa[4] = {ua.x, ua.y, ua.z, ua.w};
        const uint32_t wb[4] = {ub.x, ub.y, ub.z, ub.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const bf16x2 xa = __builtin_bit_cast(bf16x2, wa[h]);
            const bf16x2 xb = __builtin_bit_cast(bf16x2, wb[h]);
            sa = __builtin_amdgcn_fdot2_f32_bf16(xa, xa, sa, false);
            sb = __builtin_amdgcn_fdot2_f32_bf16(xb, xb, sb, false);
        }
    }
    sa += __shfl_xor(sa, 32);
    sb += __shfl_xor(sb, 32);
    // 1/|k| (0 for a zero key, whose cosine with anything is taken as 0)
    const float inv_a = sa > 0.f ? __builtin_amdgcn_rsqf(sa) : 0.f;
    const float inv_b = sb > 0.f ? __builtin_amdgcn_rsqf(sb) : 0.f;
    // dot[A col][B tile_row(v, hf)]: B keys as the A operand (rows), A keys as the B operand (lanes)
    const f32x16 dot = logits<KS>(fb, fa);
    float best = -INFINITY;
    int best_j = -1;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int j = tile_row(v, hf);  // ascending in v for a fixed half
        const float sim = dot[v] * (inv_a * __shfl(inv_b, j));
        if (j < nb && sim > best) {
            best = sim;
            best_j = j;
        }
    }
    const float ob = __shfl_xor(best, 32);
    const int oj = __shfl_xor(best_j, 32);
    if (ob > best || (ob == best && oj >= 0 && (best_j < 0 || oj < best_j))) {
        best = ob;
        best_j = oj;
    }
    if (hf == 0 && col < na) {
        const int64_t ai = (int64_t)slab * g.n_a + (int64_t)c * (g.C >> 1) + col;
        score[ai] = best;
        match[ai] = best_j >= 0 ? (int32_t)(start + 2 * best_j + 1) : -1;
        flags[ai] = 0;  // every A slot is written here: the chosen ones are flagged after the ranking
    }
}

// flags[S][n_a] = 1 for the chosen A tokens (the match kernel zeroed them all).
__global__ void csm_flag_kernel(CsmGeom g, const int32_t* chosen, uint8_t* flags) {
    const int64_t total = (int64_t)g.S * g.n_merge;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t slab = i / g.n_merge;
        flags[slab * g.n_a + chosen[i]] = 1;
    }
}

// offsets[S][n_chunks]: survivors of the slab's earlier chunks. One
// work-group per slab walks its chunks 256 at a time: a thread per chunk
// counts the chunk's survivors (its length less its chosen A tokens, flag
// bytes read four at a time where the chunks' flag runs are 4-byte aligned)
// and a block scan turns the counts into offsets.
__global__ void __launch_bounds__(256) csm_offsets_kernel(CsmGeom g, const uint8_t* flags, int32_t* offsets) {
    __shared__ int32_t wsum[4];
    const int slab = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = g.C >> 1;
    const bool words = half % 4 == 0 && g.n_a % 4 == 0;
    int32_t carry = 0;
    for (int c0 = 0; c0 < g.n_chunks; c0 += 256) {
        const int c = c0 + threadIdx.x;
        int32_t surv = 0;
        if (c < g.n_chunks) {
            int64_t start;
            int len;
            chunk_range(g, c, start, len);
            const int na = (len + 1) >> 1;
            const uint8_t* f = flags + (int64_t)slab * g.n_a + (int64_t)c * half;
            int removed = 0, i = 0;
            if (words) {
                const uint32_t* fw = reinterpret_cast<const uint32_t*>(f);
                for (; i + 4 <= na; i += 4) removed += (int)((fw[i >> 2] * 0x01010101u) >> 24);  // bytes are 0 or 1
            }
            for (; i < na; ++i) removed += f[i];
            surv = len - removed;
        }
        int32_t incl = surv;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const int32_t t = wsum[w2];
            if (w2 < wave) before += t;
            total += t;
        }
        if (c < g.n_chunks) offsets[(int64_t)slab * g.n_chunks + c] = carry + before + incl - surv;
        carry += total;
        __syncthreads();  // wsum is rewritten by the next tile
    }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);  // finite inputs
}

// acc (=|+=) w * x for N consecutive bf16 elements at p (16-byte loads).
template <int N>
__device__ __forceinline__ void add_scaled(float (&acc)[N], const uint16_t* p, float w, bool first) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int u = 0; u < N / 8; ++u) {
        const uint4 x = q[u];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float lo = w * __uint_as_float(xs[h] << 16);
            const float hi = w * __uint_as_float(xs[h] & 0xFFFF0000u);
            acc[8 * u + 2 * h] = first ? lo : acc[8 * u + 2 * h] + lo;
            acc[8 * u + 2 * h + 1] = first ? hi : acc[8 * u + 2 * h + 1] + hi;
        }
    }
}

// N fp32 values to bf16 (nearest even), 16-byte stores.
template <int N>
__device__ __forceinline__ void store_bf16(uint16_t* p, const float (&x)[N]) {
    uint4* q = reinterpret_cast<uint4*>(p);
#pragma unroll
    for (int u = 0; u < N / 8; ++u) {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h)
            w[h] = (uint32_t)bf16_rne(x[8 * u + 2 * h]) | ((uint32_t)bf16_rne(x[8 * u + 2 * h + 1]) << 16);
        q[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// One work-group per span of whole chunks (64 / C chunks, at most 64
// positions). Wave 0 does the bookkeeping with lane t = span position t:
// which tokens survive, each survivor's output row (the chunk's offset plus
// its rank among the chunk's survivors), and for each B token the mask of
// chosen A tokens that merge into it. Then every thread moves an eighth of a
// row: eight threads per position, all rows in flight at once.
constexpr int kMergeThreads = 512;

template <int D>
__global__ void __launch_bounds__(kMergeThreads) csm_merge_kernel(CsmGeom g, const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, const int32_t* degree,
                                                        const int32_t* match, const uint8_t* flags,
                                                        const int32_t* offsets, uint16_t* k_out, uint16_t* v_out,
                                                        int32_t* degree_out) {
    constexpr int Q = D / 8;  // elements per thread (an eighth of a row)
    __shared__ unsigned long long mem_s[64];
    __shared__ long long dst_s[64];
    const int tid = threadIdx.x;
    const int slab = blockIdx.y;
    const int cpw = max(1, 64 / g.C);         // chunks per work-group
    const int c0 = blockIdx.x * cpw;          // first chunk of the span
    const int64_t span0 = g.n_sink + (int64_t)c0 * g.C;
    if (tid < 64) {
        mem_s[tid] = 0ull;
        const int t = tid;
        const int ci = t / g.C;
        const int o = t - ci * g.C;
        const int c = c0 + ci;
        bool in = false;
        int64_t start = 0;
        int len = 0;
        if (ci < cpw && c < g.n_chunks) {
            chunk_range(g, c, start, len);
            in = o < len;
        }
        const int64_t ai = (int64_t)slab * g.n_a + (int64_t)c * (g.C >> 1) + (o >> 1);
        const bool chosen = in && (o & 1) == 0 && flags[ai] != 0;
        const uint64_t surv = __ballot(in && !chosen);
        // merges: a chosen A token marks its partner (same chunk, so inside the
        // span). A chosen token without a partner (match -1: only with
        // non-finite keys, whose similarities are NaN) is dropped unmerged.
        __builtin_amdgcn_wave_barrier();
        if (chosen) {
            const int64_t off = (int64_t)match[ai] - span0;
            if (off >= 0 && off < 64) atomicOr(&mem_s[off], 1ull << t);
        }
        long long dst = -1;
        if (in && !chosen) {
            const uint64_t chunk_bits = (ci * g.C + g.C >= 64) ? ~0ull << (ci * g.C) : ((1ull << (ci * g.C + g.C)) - 1) & (~0ull << (ci * g.C));
            const uint64_t below = t == 0 ? 0ull : (~0ull >> (64 - t));
            const int rank = __popcll(surv & chunk_bits & below);
            dst = (long long)slab * g.n_out + g.n_sink + offsets[(int64_t)slab * g.n_chunks + c] + rank;
        }
        dst_s[t] = dst;
    }
    __syncthreads();
    const int t = tid >> 3;   // span position
    const int qt = tid & 7;   // eighth of the row
    const long long dst = dst_s[t];
    if (dst < 0) return;
    const int64_t src = (int64_t)slab * g.n + span0 + t;
    uint64_t mem = mem_s[t];
    const int32_t dt = degree ? degree[src] : 1;
    if (mem == 0) {
        const uint4* ks = reinterpret_cast<const uint4*>(k + src * D + qt * Q);
        const uint4* vs = reinterpret_cast<const uint4*>(v + src * D + qt * Q);
        uint4* kd = reinterpret_cast<uint4*>(k_out + dst * D + qt * Q);
        uint4* vd = reinterpret_cast<uint4*>(v_out + dst * D + qt * Q);
        uint4 a[Q / 8], b[Q / 8];
#pragma unroll
        for (int u = 0; u < Q / 8; ++u) {
            a[u] = ks[u];
            b[u] = vs[u];
        }
#pragma unroll
        for (int u = 0; u < Q / 8; ++u) {
            kd[u] = a[u];
            vd[u] = b[u];
        }
        if (qt == 0) degree_out[dst] = dt;
        return;
    }
    // cluster weight first, then sum w_i / W * x_i (each weight <= 1, so no
    // partial sum of finite inputs can overflow)
    int64_t wsum = dt;
    for (uint64_t mm = mem; mm; mm &= mm - 1) {
        const int64_t ms = (int64_t)slab * g.n + span0 + __builtin_ctzll(mm);
        wsum += degree ? degree[ms] : 1;
    }
    const float inv = 1.0f / (float)wsum;
    float ak[Q], av[Q];
    add_scaled<Q>(ak, k + src * D + qt * Q, (float)dt * inv, true);
    add_scaled<Q>(av, v + src * D + qt * Q, (float)dt * inv, true);
    while (mem) {
        const int64_t ms = (int64_t)slab * g.n + span0 + __builtin_ctzll(mem);
        mem &= mem - 1;
        const float wm = (float)(degree ? degree[ms] : 1) * inv;
        add_scaled<Q>(ak, k + ms * D + qt * Q, wm, false);
        add_scaled<Q>(av, v + ms * D + qt * Q, wm, false);
    }
    store_bf16<Q>(k_out + dst * D + qt * Q, ak);
    store_bf16<Q>(v_out + dst * D + qt * Q, av);
    if (qt == 0) degree_out[dst] = (int32_t)wsum;
}

// Sinks [0, n_sink) and recent tokens [n - n_recent, n) keep their rows.
template <int D>
__global__ void csm_edges_kernel(CsmGeom g, const uint16_t* k, const uint16_t* v, const int32_t* degree,
                                 uint16_t* k_out, uint16_t* v_out, int32_t* degree_out) {
    const int slab = blockIdx.y;
    const int edge = g.n_sink + g.n_recent;
    for (int r = blockIdx.x; r < edge; r += gridDim.x) {
        const int64_t src = (int64_t)slab * g.n + (r < g.n_sink ? r : g.n - edge + r);
        const int64_t dst = (int64_t)slab * g.n_out + (r < g.n_sink ? r : g.n_out - edge + r);
        for (int e = threadIdx.x; e < D; e += blockDim.x) {
            k_out[dst * D + e] = k[src * D + e];
            v_out[dst * D + e] = v[src * D + e];
        }
        if (threadIdx.x == 0) degree_out[dst] = degree ? degree[src] : 1;
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Grid of a 256-thread grid-stride loop over `work` items.
unsigned blocks_for(int64_t work) {
    int64_t b = (work + 255) / 256;
    if (b > 4096) b = 4096;
    if (b < 1) b = 1;
    return (unsigned)b;
}

CsmGeom make_geom(int32_t S, int64_t n, int32_t d, int32_t C, int32_t n_sink, int32_t n_recent, int32_t n_merge) {
    CsmGeom g;
    g.S = S;
    g.d = d;
    g.n = n;
    g.C = C;
    g.n_sink = n_sink;
    g.n_recent = n_recent;
    g.M = n - n_sink - n_recent;
    g.n_chunks = (int32_t)((g.M + C - 1) / C);
    const int64_t last = g.M - (int64_t)(g.n_chunks > 0 ? g.n_chunks - 1 : 0) * C;
    g.n_a = g.n_chunks > 0 ? (int64_t)(g.n_chunks - 1) * (C / 2) + (last + 1) / 2 : 0;
    g.n_merge = n_merge;
    g.n_out = n - n_merge;
    return g;
}

struct CsmWs {
    size_t score_off, match_off, chosen_off, flags_off, offsets_off, topk_off, total;
};

CsmWs csm_ws(const CsmGeom& g) {
    CsmWs w;
    w.score_off = 0;
    w.match_off = align256(w.score_off + (size_t)g.S * g.n_a * sizeof(float));
    w.chosen_off = align256(w.match_off + (size_t)g.S * g.n_a * sizeof(int32_t));
    w.flags_off = align256(w.chosen_off + (size_t)g.S * g.n_merge * sizeof(int32_t));
    w.offsets_off = align256(w.flags_off + (size_t)g.S * g.n_a);
    w.topk_off = align256(w.offsets_off + (size_t)g.S * g.n_chunks * sizeof(int32_t));
    w.total = w.topk_off + align256(topk_workspace_bytes(g.S, g.n_a > 0 ? g.n_a : 1));
    return w;
}

}  // namespace

int64_t csm_candidates(int64_t n, int32_t C, int32_t n_sink, int32_t n_recent) {
    const int64_t M = n - n_sink - n_recent;
    if (M <= 0) return 0;
    const int64_t full = M / C, last = M % C;
    return full * (C / 2) + (last >= 2 ? (last + 1) / 2 : 0);
}

size_t csm_workspace_bytes(int32_t S, int64_t n, int32_t C, int32_t n_sink, int32_t n_recent, int32_t n_merge) {
    return csm_ws(make_geom(S, n, 128, C, n_sink, n_recent, n_merge)).total;
}

hipError_t launch_csm(int32_t S, int64_t n, int32_t d, int32_t C, int32_t n_sink, int32_t n_recent, int32_t n_merge,
                      const uint16_t* k, const uint16_t* v, const int32_t* degree, uint16_t* k_out, uint16_t* v_out,
                      int32_t* degree_out, float* score_out, int32_t* match_out, int32_t* chosen_out, void* workspace,
                      hipStream_t st) {
    const CsmGeom g = make_geom(S, n, d, C, n_sink, n_recent, n_merge);
    const CsmWs w = csm_ws(g);
    char* ws = static_cast<char*>(workspace);
    float* score = score_out ? score_out : reinterpret_cast<float*>(ws + w.score_off);
    int32_t* match = match_out ? match_out : reinterpret_cast<int32_t*>(ws + w.match_off);
    int32_t* chosen = chosen_out ? chosen_out : reinterpret_cast<int32_t*>(ws + w.chosen_off);
    uint8_t* flags = reinterpret_cast<uint8_t*>(ws + w.flags_off);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + w.offsets_off);
    const dim3 cgrid((unsigned)((g.n_chunks + kCsmWaves - 1) / kCsmWaves), (unsigned)S);
    if (g.n_chunks > 0) {
        if (d == 128)
            hipLaunchKernelGGL(csm_match_kernel<128>, cgrid, dim3(256), 0, st, g, k, score, match, flags);
        else
            hipLaunchKernelGGL(csm_match_kernel<64>, cgrid, dim3(256), 0, st, g, k, score, match, flags);
        if (n_merge > 0) {
            const hipError_t e =
                launch_topk(S, g.n_a, 0, n_merge, 0, score, chosen, ws + w.topk_off, st);
            if (e != hipSuccess) return e;
            const int64_t nc = (int64_t)S * n_merge;
            hipLaunchKernelGGL(csm_flag_kernel, dim3(blocks_for(nc)), dim3(256), 0, st,
                               g, chosen, flags);
        }
        hipLaunchKernelGGL(csm_offsets_kernel, dim3((unsigned)S), dim3(256), 0, st, g, flags, offsets);
        const int cpw = 64 / C > 1 ? 64 / C : 1;
        const dim3 mgrid((unsigned)((g.n_chunks + cpw - 1) / cpw), (unsigned)S);
        if (d == 128)
            hipLaunchKernelGGL(csm_merge_kernel<128>, mgrid, dim3(kMergeThreads), 0, st, g, k, v, degree, match, flags,
                               offsets, k_out, v_out, degree_out);
        else
            hipLaunchKernelGGL(csm_merge_kernel<64>, mgrid, dim3(kMergeThreads), 0, st, g, k, v, degree, match, flags,
                               offsets, k_out, v_out, degree_out);
    }
    if (n_sink + n_recent > 0) {
        const dim3 egrid((unsigned)min(n_sink + n_recent, 1024), (unsigned)S);
        if (d == 128)
            hipLaunchKernelGGL(csm_edges_kernel<128>, egrid, dim3(128), 0, st, g, k, v, degree, k_out, v_out,
                               degree_out);
        else
            hipLaunchKernelGGL(csm_edges_kernel<64>, egrid, dim3(128), 0, st, g, k, v, degree, k_out, v_out,
                               degree_out);
    }
    return hipGetLastError();
}

}  // namespace kvsel
