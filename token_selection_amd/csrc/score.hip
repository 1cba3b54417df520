// Window-attention saliency scores on gfx950 matrix cores.
//
// Computes, per (layer, sequence, KV head) "slab", the score each prefix key
// receives from the observation window: the window queries' softmax
// probabilities summed over the window and averaged over the GQA group, then
// an average pool along the sequence, summed over the layers of the call
// (saliency: FastKV page, section 2A; layer sum: StructKV page, section 1).
//
// Two passes over K, because a key's probability needs its row's final
// log-sum-exp, which depends on every key:
//   pass 1  lse_partial_kernel: per key chunk, the online (max, sum) of every
//           window row in the log2 domain; lse_combine_kernel merges chunks.
//   pass 2  raw_score_kernel: recompute the logits, exp2(x - LSE2) and sum
//           them per key over all G*w rows of the KV head.
//   then    pool_acc_kernel: the average pool, summed over layers (or
//           pool_max_acc_kernel: the max pool of each layer, summed).
//
// Logits come from v_mfma_f32_16x16x32_bf16 (bf16 inputs) or
// v_mfma_f32_16x16x4_f32 (fp32 inputs) with fp32 accumulation. The window
// rows of one KV head (G*w of them) are processed in groups of RB*16 rows
// whose query fragments stay in registers for the whole key chunk; each wave
// streams 16-key blocks of K straight from global memory into MFMA operand
// registers.
//
// Matrix-core operand layout (16x16xK): lane l supplies row/column (l % 16)
// and k-slots of lane group (l / 16). The head-dim elements are assigned so
// that lane group q of any row owns the contiguous elements
// [q*D/4, (q+1)*D/4): each lane reads D/4 contiguous elements of its row
// with 16-byte loads. Both operands use the same assignment, so the
// contraction still runs over every head-dim element. The 16x16 result puts
// column (l % 16) and rows 4*(l/16) .. +3 in lane l.

#include <math.h>
#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T, int D>
struct Frag;

// bf16 operands: 8 elements (16 bytes) per lane per k-step, D/32 k-steps.
template <int D>
struct Frag<uint16_t, D> {
    static constexpr int KS = D / 32;
    typedef bf16x8 type;
    __device__ static __forceinline__ void load(const uint16_t* row, int lg, type (&f)[KS]) {
        const uint4* p = reinterpret_cast<const uint4*>(row + lg * (D / 4));
#pragma unroll
        for (int s = 0; s < KS; ++s) f[s] = __builtin_bit_cast(bf16x8, p[s]);
    }
    __device__ static __forceinline__ void zero(type (&f)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s) f[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
    __device__ static __forceinline__ f32x4 mma(type a, type b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// fp32 operands: one element per lane per k-step, D/4 k-steps.
template <int D>
struct Frag<float, D> {
    static constexpr int KS = D / 4;
    typedef float type;
    __device__ static __forceinline__ void load(const float* row, int lg, type (&f)[KS]) {
        const float4* p = reinterpret_cast<const float4*>(row + lg * (D / 4));
#pragma unroll
        for (int s = 0; s < KS / 4; ++s) {
            const float4 v = p[s];
            f[4 * s + 0] = v.x;
            f[4 * s + 1] = v.y;
            f[4 * s + 2] = v.z;
            f[4 * s + 3] = v.w;
        }
    }
    __device__ static __forceinline__ void zero(type (&f)[KS]) {
#pragma unroll
        for (int s = 0; s < KS; ++s) f[s] = 0.f;
    }
    __device__ static __forceinline__ f32x4 mma(type a, type b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

struct SlabId {
    int l, b, kvh;
};

__device__ __forceinline__ SlabId slab_id(const ScoreGeom& g, int s) {
    SlabId id;
    id.kvh = s % g.Hkv;
    id.b = (s / g.Hkv) % g.B;
    id.l = s / (g.Hkv * g.B);
    return id;
}

// Load this lane's query fragments for row group rg (rows as the 16-wide
// operand index). Rows past G*w are zero.
template <typename T, int D, int RB>
__device__ __forceinline__ void load_queries(const ScoreGeom& g, const T* qbase, int kvh, int rg, int col, int lg,
                                             typename Frag<T, D>::type (&qf)[RB][Frag<T, D>::KS], int (&lim)[RB]) {
    using F = Frag<T, D>;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r = (rg * RB + rb) * 16 + col;
        if (r < g.R) {
            const int h = kvh * g.G + r / g.w;
            const int i = r % g.w;
            F::load(qbase + h * g.qs[2] + i * g.qs[3], lg, qf[rb]);
            lim[rb] = (int)g.Np + i;  // last key this window row may see
        } else {
            F::zero(qf[rb]);
            lim[rb] = -1;
        }
    }
}

// Pass 1: per (key chunk, slab), the online (max, sum of exp2) of every
// window row over the chunk's visible keys, in the log2 domain.
template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void lse_partial_kernel(ScoreGeom g) {
    using F = Frag<T, D>;
    const int chunk = blockIdx.x;
    const int s = blockIdx.y;
    const SlabId id = slab_id(g, s);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int lg = lane >> 4;
    const T* kslab = static_cast<const T*>(g.k) + id.l * g.ks[0] + id.b * g.ks[1] + id.kvh * g.ks[2];
    const T* qbase = static_cast<const T*>(g.q) + id.l * g.qs[0] + id.b * g.qs[1];
    const int j0 = chunk * g.chunk;
    const int j1 = (int)min<int64_t>(g.N, (int64_t)j0 + g.chunk);
    const int Np = (int)g.Np;
    __shared__ float2 red[4][RB * 16];

    for (int rg = 0; rg < g.n_groups; ++rg) {
        typename F::type qf[RB][F::KS];
        int lim[RB];
        load_queries<T, D, RB>(g, qbase, id.kvh, rg, col, lg, qf, lim);
        float m[RB], z[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m[rb] = kNegBig;
            z[rb] = 0.f;
        }
        for (int kb = j0 + wave * 16; kb < j1; kb += 64) {
            // operand A = 16 keys (rows of the product), B = 16 window rows
            const int jload = min(kb + col, (int)g.N - 1);
            typename F::type kf[F::KS];
            F::load(kslab + (int64_t)jload * g.ks[3], lg, kf);
            const bool edge = kb + 16 > Np;  // reaches the window (causal) or the end of K
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < F::KS; ++ks) acc = F::mma(kf[ks], qf[rb][ks], acc);
                float x[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) x[v] = acc[v] * g.c;
                if (edge) {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (kb + lg * 4 + v > lim[rb]) x[v] = -INFINITY;
                }
                const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                const float mn = fmaxf(m[rb], mx);
                float acc_z = z[rb] * fast_exp2(m[rb] - mn);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc_z += fast_exp2(x[v] - mn);
                z[rb] = acc_z;
                m[rb] = mn;
            }
        }
        // the 4 lane groups of a column hold the same row: merge them
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float mo = __shfl_xor(m[rb], off);
                const float zo = __shfl_xor(z[rb], off);
                const float mn = fmaxf(m[rb], mo);
                z[rb] = z[rb] * fast_exp2(m[rb] - mn) + zo * fast_exp2(mo - mn);
                m[rb] = mn;
            }
            if (lg == 0) red[wave][rb * 16 + col] = make_float2(m[rb], z[rb]);
        }
        __syncthreads();
        const int t = threadIdx.x;
        if (t < RB * 16) {
            float2 a = red[0][t];
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) {
                const float2 o = red[w2][t];
                const float mn = fmaxf(a.x, o.x);
                a.y = a.y * fast_exp2(a.x - mn) + o.y * fast_exp2(o.x - mn);
                a.x = mn;
            }
            g.part[((int64_t)s * g.n_chunks1 + chunk) * g.Rpad + rg * RB * 16 + t] = a;
        }
        __syncthreads();
    }
}

// Merge the chunk partials of each row into its LSE (log2 domain); padded
// rows get +inf so that pass 2 gives them probability 0.
// A block takes kCombRows rows; each row's chunks are spread over
// kCombSubs threads (thread t: row t % kCombRows, every kCombSubs-th chunk
// from t / kCombRows on, so a wave reads consecutive rows of a chunk), whose
// running (max, sum) states then merge through LDS.
constexpr int kCombRows = 16;
constexpr int kCombSubs = 256 / kCombRows;

__global__ __launch_bounds__(256) void lse_combine_kernel(ScoreGeom g) {
    __shared__ float2 red[kCombSubs][kCombRows];
    const int s = blockIdx.y;
    const int rl = threadIdx.x % kCombRows, sub = threadIdx.x / kCombRows;
    const int r = blockIdx.x * kCombRows + rl;
    float M = kNegBig, Z = 0.f;
    if (r < g.Rpad) {
        const float2* p = g.part + (int64_t)s * g.n_chunks1 * g.Rpad + r;
        for (int c = sub; c < g.n_chunks1; c += kCombSubs) {
            const float2 v = p[(int64_t)c * g.Rpad];
            const float mn = fmaxf(M, v.x);
            Z = Z * exp2f(M - mn) + v.y * exp2f(v.x - mn);
            M = mn;
        }
    }
    red[sub][rl] = make_float2(M, Z);
    __syncthreads();
    if (sub != 0 || r >= g.Rpad) return;
    for (int s2 = 1; s2 < kCombSubs; ++s2) {
        const float2 o = red[s2][rl];
        const float mn = fmaxf(M, o.x);
        Z = Z * exp2f(M - mn) + o.y * exp2f(o.x - mn);
        M = mn;
    }
    if (r < g.R) {
        const float l2 = M + log2f(Z);
        g.lse2[(int64_t)s * g.Rpad + r] = l2;
        if (g.lse_out) {
            const SlabId id = slab_id(g, s);
            const int h = id.kvh * g.G + r / g.w;
            const int i = r % g.w;
            g.lse_out[(((int64_t)id.l * g.B + id.b) * g.Hq + h) * g.w + i] = l2 * 0.69314718055994530942f;
        }
    } else {
        g.lse2[(int64_t)s * g.Rpad + r] = INFINITY;
    }
}

// Pass 2: per (prefix key chunk, slab), sum over all G*w rows of
// exp2(x - LSE2) for every key, times 1/G.
template <typename T, int D, int RB>
__global__ __launch_bounds__(256) void raw_score_kernel(ScoreGeom g) {
    using F = Frag<T, D>;
    constexpr int NKB = kScoreChunk / 64;  // 16-key blocks per wave in the largest chunk
    const int chunk = blockIdx.x;
    const int s = blockIdx.y;
    const SlabId id = slab_id(g, s);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int lg = lane >> 4;
    const T* kslab = static_cast<const T*>(g.k) + id.l * g.ks[0] + id.b * g.ks[1] + id.kvh * g.ks[2];
    const T* qbase = static_cast<const T*>(g.q) + id.l * g.qs[0] + id.b * g.qs[1];
    const int j0 = chunk * g.chunk;
    const int j1 = (int)min<int64_t>(g.Np, (int64_t)j0 + g.chunk);
    const float* lse2 = g.lse2 + (int64_t)s * g.Rpad;

    float cs[NKB];
#pragma unroll
    for (int t = 0; t < NKB; ++t) cs[t] = 0.f;

    for (int rg = 0; rg < g.n_groups; ++rg) {
        typename F::type qf[RB][F::KS];
        int lim[RB];
        load_queries<T, D, RB>(g, qbase, id.kvh, rg, col, lg, qf, lim);
        float lr[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int v = 0; v < 4; ++v) lr[rb][v] = lse2[(rg * RB + rb) * 16 + lg * 4 + v];
#pragma unroll
        for (int t = 0; t < NKB; ++t) {
            const int kb = j0 + wave * 16 + t * 64;
            if (kb < j1) {
                // operand A = 16 window rows, B = 16 keys (columns of the product)
                const int jload = min(kb + col, (int)g.N - 1);
                typename F::type kf[F::KS];
                F::load(kslab + (int64_t)jload * g.ks[3], lg, kf);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < F::KS; ++ks) acc = F::mma(qf[rb][ks], kf[ks], acc);
#pragma unroll
                    for (int v = 0; v < 4; ++v) cs[t] += fast_exp2(acc[v] * g.c - lr[rb][v]);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NKB; ++t) {
        float v = cs[t];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        const int j = j0 + wave * 16 + t * 64 + col;
        if (lg == 0 && j < j1) g.raw[(int64_t)s * g.Np + j] = v * g.invG;
    }
}

// Average pool (zero padded, divisor = kernel) of the raw scores summed over
// the layers of the call, added to scores when accumulating. Pooling is
// linear, so the layers are summed first and pooled once: each work-group
// sums a tile of kPoolTile positions plus a halo of r positions on each side
// into LDS, every thread its kPoolSlots positions (one per 256) with their
// loads of four layers issued together, then pools from LDS. The layers add
// in order, so the result does not depend on the tiling.
constexpr int kPoolTile = 1024;
constexpr int kPoolMaxR = 127;
constexpr int kPoolSlots = (kPoolTile + 2 * kPoolMaxR + 255) / 256;  // 5
__global__ __launch_bounds__(256) void pool_acc_kernel(const float* __restrict__ raw, float* __restrict__ scores,
                                                       int L, int64_t BH, int64_t Np, int kern, int accumulate) {
    __shared__ float tile[kPoolTile + 2 * kPoolMaxR];
    const int64_t bh = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kPoolTile;
    const int r = (kern - 1) / 2;
    const int span = kPoolTile + 2 * r;
    const float* p = raw + bh * Np;
    const int64_t lstride = BH * Np;
    bool in[kPoolSlots];
    float sum[kPoolSlots];
#pragma unroll
    for (int u = 0; u < kPoolSlots; ++u) {
        const int t = threadIdx.x + u * 256;
        const int64_t j = j0 - r + t;
        in[u] = t < span && j >= 0 && j < Np;
        sum[u] = 0.f;
    }
    // four layers' loads (20 per thread) in flight before their adds, which
    // keep the layers' order
    for (int l = 0; l < L; l += 4) {
        float v[4][kPoolSlots];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool lq = l + q < L;
            const float* pl = p + (int64_t)(l + q) * lstride + j0 - r + threadIdx.x;
#pragma unroll
            for (int u = 0; u < kPoolSlots; ++u) v[q][u] = (lq && in[u]) ? pl[u * 256] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int u = 0; u < kPoolSlots; ++u) sum[u] += v[q][u];
    }
#pragma unroll
    for (int u = 0; u < kPoolSlots; ++u) {
        const int t = threadIdx.x + u * 256;
        if (t < span) tile[t] = sum[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPoolTile / 256; ++u) {
        const int t0 = threadIdx.x + u * 256;
        const int64_t j = j0 + t0;
        if (j >= Np) break;
        float pooled = 0.f;
        for (int t = 0; t < kern; ++t) pooled += tile[t0 + t];
        const float val = pooled / (float)kern;
        const int64_t o = bh * Np + j;
        scores[o] = accumulate ? scores[o] + val : val;
    }
}

// Max pool variant: s[j] = max over t = -r..r of raw[j + t], positions outside
// [0, Np) left out (scores are >= 0, so this equals zero padding). A max does
// not commute with the sum over layers, so each layer is pooled on its own and
// the pooled layers are added up (in layer order). Tiles as in the average
// pool: each thread loads its kPoolSlots positions of four layers into
// registers together, then per layer they pass through LDS for the window max.
__global__ __launch_bounds__(256) void pool_max_acc_kernel(const float* __restrict__ raw, float* __restrict__ scores,
                                                           int L, int64_t BH, int64_t Np, int kern, int accumulate) {
    __shared__ float tile[kPoolTile + 2 * kPoolMaxR];
    const int64_t bh = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kPoolTile;
    const int r = (kern - 1) / 2;
    const int span = kPoolTile + 2 * r;
    const float* p = raw + bh * Np;
    const int64_t lstride = BH * Np;
    bool in[kPoolSlots];
#pragma unroll
    for (int u = 0; u < kPoolSlots; ++u) {
        const int t = threadIdx.x + u * 256;
        const int64_t j = j0 - r + t;
        in[u] = t < span && j >= 0 && j < Np;
    }
    float acc[kPoolTile / 256];
#pragma unroll
    for (int k = 0; k < kPoolTile / 256; ++k) acc[k] = 0.f;
    for (int l = 0; l < L; l += 4) {
        float v[4][kPoolSlots];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool lq = l + q < L;
            const float* pl = p + (int64_t)(l + q) * lstride + j0 - r + threadIdx.x;
#pragma unroll
            for (int u = 0; u < kPoolSlots; ++u) v[q][u] = (lq && in[u]) ? pl[u * 256] : -INFINITY;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (l + q >= L) break;
            __syncthreads();  // the previous layer's tile has been read
#pragma unroll
            for (int u = 0; u < kPoolSlots; ++u) {
                const int t = threadIdx.x + u * 256;
                if (t < span) tile[t] = v[q][u];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < kPoolTile / 256; ++k) {
                const int t0 = threadIdx.x + k * 256;
                float m = -INFINITY;
                for (int t = 0; t < kern; ++t) m = fmaxf(m, tile[t0 + t]);
                acc[k] += m;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kPoolTile / 256; ++k) {
        const int64_t j = j0 + threadIdx.x + k * 256;
        if (j >= Np) break;
        const int64_t o = bh * Np + j;
        scores[o] = accumulate ? scores[o] + acc[k] : acc[k];
    }
}

// Row LSE2 of every slab from a handed-in natural-log LSE (prefill attention
// already has it): lse2[s][r] = LSE[l][b][g*G + r/w][r%w] * log2(e) for r < R,
// +inf (probability 0) on padded rows.
__global__ void lse_from_input_kernel(const float* lse_in, float* lse2, int S, int stride, int R, int w, int B,
                                      int Hq, int Hkv, int G, int S0, int Gs) {
    const int s = blockIdx.y;
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= S || r >= stride) return;
    const int t = s / S0, s0 = s - t * S0;  // head group, (layer, b, kv head) slab
    const int rows = min(Gs, G - t * Gs) * w;
    float v = INFINITY;
    if (r < rows && r < R) {
        const int kvh = s0 % Hkv;
        const int b = (s0 / Hkv) % B;
        const int l = s0 / (Hkv * B);
        const int h = kvh * G + t * Gs + r / w;
        const int i = r % w;
        v = lse_in[(((int64_t)l * B + b) * Hq + h) * w + i] * 1.44269504088896340736f;
    }
    lse2[(int64_t)s * stride + r] = v;
}

template <typename T, int D, int RB>
void launch_passes(const ScoreGeom& g, hipStream_t st) {
    if (g.lse_in) {
        hipLaunchKernelGGL(lse_from_input_kernel, dim3((g.Rpad + 255) / 256, g.S), dim3(256), 0, st, g.lse_in, g.lse2,
                           g.S, g.Rpad, g.R, g.w, g.B, g.Hq, g.Hkv, g.G, g.S, g.G);
    } else {
        hipLaunchKernelGGL((lse_partial_kernel<T, D, RB>), dim3(g.n_chunks1, g.S), dim3(256), 0, st, g);
        hipLaunchKernelGGL(lse_combine_kernel, dim3((g.Rpad + kCombRows - 1) / kCombRows, g.S), dim3(256), 0, st, g);
    }
    if (g.Np > 0)
        hipLaunchKernelGGL((raw_score_kernel<T, D, RB>), dim3(g.n_chunks2, g.S), dim3(256), 0, st, g);
}

template <typename T, int D>
bool dispatch_rb(const ScoreGeom& g, int RB, hipStream_t st) {
    switch (RB) {
        case 1: launch_passes<T, D, 1>(g, st); return true;
        case 2: launch_passes<T, D, 2>(g, st); return true;
        case 3: launch_passes<T, D, 3>(g, st); return true;
        case 4: launch_passes<T, D, 4>(g, st); return true;
        case 5: launch_passes<T, D, 5>(g, st); return true;
        case 6: launch_passes<T, D, 6>(g, st); return true;
        case 7: launch_passes<T, D, 7>(g, st); return true;
        case 8: launch_passes<T, D, 8>(g, st); return true;
        default: return false;
    }
}

template <>
bool dispatch_rb<float, 128>(const ScoreGeom& g, int RB, hipStream_t st) {
    switch (RB) {
        case 1: launch_passes<float, 128, 1>(g, st); return true;
        case 2: launch_passes<float, 128, 2>(g, st); return true;
        case 3: launch_passes<float, 128, 3>(g, st); return true;
        case 4: launch_passes<float, 128, 4>(g, st); return true;
        default: return false;
    }
}

}  // namespace

int score_row_blocks(int dtype, int head_dim, int R) {
    // Query fragments of one row block cost 16 registers (bf16, d=128),
    // 8 (bf16, d=64), 16 (fp32, d=64) or 32 (fp32, d=128) per lane; a group
    // keeps them all in registers, so groups are capped at 128 registers.
    const int cap = (dtype == KVSEL_DTYPE_F32 && head_dim == 128) ? 4 : 8;
    const int nb = (R + 15) / 16;
    const int groups = (nb + cap - 1) / cap;
    return (nb + groups - 1) / groups;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ScoreWs score_workspace_layout(int64_t S, int64_t n_chunks1, int64_t Rpad, int64_t Np) {
    ScoreWs w;
    w.part_off = 0;
    w.lse2_off = align256(w.part_off + (size_t)S * n_chunks1 * Rpad * sizeof(float2));
    w.raw_off = align256(w.lse2_off + (size_t)S * Rpad * sizeof(float));
    w.total = align256(w.raw_off + (size_t)S * Np * sizeof(float));
    return w;
}

hipError_t launch_score_passes(const ScoreGeom& g, int dtype, int head_dim, int RB, hipStream_t st) {
    bool ok = false;
    if (dtype == KVSEL_DTYPE_BF16) {
        ok = head_dim == 128 ? dispatch_rb<uint16_t, 128>(g, RB, st) : dispatch_rb<uint16_t, 64>(g, RB, st);
    } else {
        ok = head_dim == 128 ? dispatch_rb<float, 128>(g, RB, st) : dispatch_rb<float, 64>(g, RB, st);
    }
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_lse_from_input(const float* lse_in, float* lse2, int S, int stride, int R, int w, int B, int Hq,
                                 int Hkv, int G, int S0, int Gs, hipStream_t st) {
    if (S < 1 || S > 65535 || stride < 1 || S0 < 1 || Gs < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(lse_from_input_kernel, dim3((unsigned)((stride + 255) / 256), (unsigned)S), dim3(256), 0, st,
                       lse_in, lse2, S, stride, R, w, B, Hq, Hkv, G, S0, Gs);
    return hipGetLastError();
}

hipError_t launch_pool(const float* raw, float* scores, int L, int64_t BH, int64_t Np, int pool_kernel,
                       int pool_type, int accumulate, hipStream_t st) {
    if (Np <= 0) return hipSuccess;
    if ((pool_kernel - 1) / 2 > kPoolMaxR || BH > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((Np + kPoolTile - 1) / kPoolTile), (unsigned)BH);
    if (pool_type == KVSEL_POOL_MAX)
        hipLaunchKernelGGL(pool_max_acc_kernel, grid, dim3(256), 0, st, raw, scores, L, BH, Np, pool_kernel,
                           accumulate);
    else
        hipLaunchKernelGGL(pool_acc_kernel, grid, dim3(256), 0, st, raw, scores, L, BH, Np, pool_kernel, accumulate);
    return hipGetLastError();
}

}  // namespace kvsel
