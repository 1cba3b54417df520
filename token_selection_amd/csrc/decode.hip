// Decode attention over a compacted KV cache: one new query per sequence
// and query head against the kept keys and values (FastKV section 2B and
// StructKV section 3: the stored cache is what decoding reads), optionally
// with each key's cluster degree as a log term in the softmax (CentroidKV,
// section "Methodologie", part 4: a centroid stands for `degree` tokens).
//
//   out[b, h] = sum_j p_j v[b, g, j],  p = softmax_j(scale * <q[b, h], k[b, g, j]>
//                                                     + ln degree[b, g, j]),
//   g = h / (Hq / Hkv).
//
// The step reads every kept key and value once: it is HBM-bound, and the
// group's G <= 8 query heads are too few rows for matrix cores to matter, so
// the kernel is vector code (the query-key products two bf16 pairs at a time
// with v_dot2_f32_bf16, the rest in fp32). Each work-group takes one (b, g) and one
// split of the keys; its 4 waves walk blocks of 16 keys (8 for G > 4). In a
// block, lane (r, s) owns elements s*D/16 .. (s+1)*D/16 - 1 of rows r, r + 4, ..., for
// the keys and for the values alike: 16 lanes read one row (coalesced), a
// dot product is the lane's partial over its slice summed over its 16 lanes,
// and each lane keeps only its slice of the group's queries. The running value sum is kept normalised (the output so far,
// a convex combination of value rows), so no partial sum of finite values can
// overflow. Splits keep (max, sum of weights, normalised output) in the
// workspace and decode_combine_kernel merges them with weights that sum to 1.
// All arithmetic is fp32 in the log2 domain.

#include <math.h>
#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kDecWaves = 4;
constexpr int kMaxG = 8;
// Rows per lane in a block, so that each wave keeps enough key and value
// slices in flight: 4; 8 for head dim 128 with 3 or 4 heads per group (at two
// waves per SIMD: 7-10% faster than 4 rows at three waves); 2 for groups of
// more than 4 heads, whose per-head state fills the registers.
template <int D, int G>
constexpr int rows_per_lane() {
    return G <= 2 ? 4 : G <= 4 ? (D == 128 ? 8 : 4) : 2;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct DecGeom {
    int32_t B, Hq, Hkv, G;
    int64_t n;
    int32_t splits;
    int64_t split_len;  // keys per split, a multiple of 64
    float c;            // scale * log2(e)
};

// x moved across lanes by the DPP control CTRL (every lane valid).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row, in every lane of it: pairs, quads
// (quad_perm), halves (row_half_mirror), the row (row_mirror). VALU only.
__device__ __forceinline__ float row_sum16(float a) {
    a += dpp<0xB1>(a);   // quad_perm [1, 0, 3, 2]
    a += dpp<0x4E>(a);   // quad_perm [2, 3, 0, 1]
    a += dpp<0x141>(a);  // row_half_mirror
    a += dpp<0x140>(a);  // row_mirror
    return a;
}

// Max / sum over the wave of a value that is uniform within each 16-lane
// row: the four row values read into scalars (no LDS round trip).
__device__ __forceinline__ float rows_max4(float x) {
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float rows_sum4(float x) {
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (a + b) + (c + d);
}

// EL consecutive bf16 elements kept as raw 32-bit words until use.
template <int EL>
struct Slice {
    uint32_t w[EL / 2];
};

template <int EL>
__device__ __forceinline__ Slice<EL> load_slice(const uint16_t* p) {
    Slice<EL> s;
    if constexpr (EL == 8) {
        const uint4 x = *reinterpret_cast<const uint4*>(p);
        s.w[0] = x.x;
        s.w[1] = x.y;
        s.w[2] = x.z;
        s.w[3] = x.w;
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        s.w[0] = x.x;
        s.w[1] = x.y;
    }
    return s;
}

// element e of a slice as fp32
template <int EL>
__device__ __forceinline__ float elem(const Slice<EL>& s, int e) {
    const uint32_t w = s.w[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Waves per SIMD the register state allows without spills (128, 168 or 256
// registers a wave); also the resident work-groups per CU the host plans for
// (a work-group has one wave per SIMD).
__host__ __device__ constexpr int dec_waves(int d, int G) {
    return d == 128 ? (G <= 2 ? 4 : G <= 4 ? 2 : G <= 5 ? 3 : 2) : (G <= 4 ? 4 : 3);
}

template <int D, int G>
constexpr int dec_waves_per_eu() {
    return dec_waves(D, G);
}

template <int D, int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu<D, G>()))) decode_kernel(DecGeom g, const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                     const int32_t* __restrict__ degree, float* part_m,
                                                     float* part_l, float* part_acc) {
    constexpr int EL = D / 16;  // elements of a row per lane
    constexpr int kT = rows_per_lane<D, G>();
    constexpr int kBlock = 4 * kT;  // rows per wave and block
    __shared__ float red_m[kDecWaves][G], red_l[kDecWaves][G];
    __shared__ float red_acc[kDecWaves][G][D];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + kv head
    const int b = bg / g.Hkv;
    const int kvh = bg - b * g.Hkv;
    const int r = lane >> 4;   // rows r, r + 4, ... of a block
    const int sl = lane & 15;  // elements sl*EL .. sl*EL + EL-1 of those rows
    // this lane's slice of the group's queries, raw bf16 pairs (element 2i in the low half, as in a Slice)
    uint32_t qw[G][EL / 2];
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
        for (int e2 = 0; e2 < EL / 2; ++e2)
            qw[gg][e2] = *reinterpret_cast<const uint32_t*>(q + ((int64_t)b * g.Hq + kvh * G + gg) * D + sl * EL + 2 * e2);
    const int64_t key0 = (int64_t)split * g.split_len;
    const int64_t key1 = min(key0 + g.split_len, g.n);
    const uint16_t* kb = k + (int64_t)bg * g.n * D;
    const uint16_t* vb = v + (int64_t)bg * g.n * D;
    const int32_t* db = degree ? degree + (int64_t)bg * g.n : nullptr;
    float m[G], l[G], acc[G][EL];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
        m[gg] = -INFINITY;
        l[gg] = 0.f;
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[gg][e] = 0.f;
    }
    for (int64_t blk = key0 + (int64_t)wave * kBlock; blk < key1; blk += kDecWaves * kBlock) {
        // the block's key and value slices all load first (raw words until use)
        Slice<EL> xk[kT], xv[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const int64_t row = min(blk + 4 * t + r, key1 - 1);  // rows past the end carry weight 0
            xk[t] = load_slice<EL>(kb + row * D + sl * EL);
            xv[t] = load_slice<EL>(vb + row * D + sl * EL);
        }
        // --- logits of rows blk + 4t + r: the lane's partial dot products, summed over its 16 lanes
        float s[kT][G];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                // bf16 pairs multiplied and summed in fp32 by v_dot2_f32_bf16 (the products are exact)
                float a = 0.f;
#pragma unroll
                for (int e2 = 0; e2 < EL / 2; ++e2)
                    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw[gg][e2]),
                                                        __builtin_bit_cast(bf16x2, xk[t].w[e2]), a, false);
                s[t][gg] = a;
            }
        }
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int gg = 0; gg < G; ++gg) s[t][gg] = row_sum16(s[t][gg]);
        // --- online softmax: the block's maximum and weight sum over its rows
        float lb[kT];
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const int64_t row = blk + 4 * t + r;
            lb[t] = row < key1 ? (db ? log2f((float)db[row]) : 0.f) : -INFINITY;
        }
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            float bm = -INFINITY;
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                s[t][gg] = s[t][gg] * g.c + lb[t];
                bm = fmaxf(bm, s[t][gg]);
            }
            bm = rows_max4(bm);
            const float mn = fmaxf(m[gg], bm);
            float ps = 0.f;
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                s[t][gg] = exp2f(s[t][gg] - mn);
                ps += s[t][gg];
            }
            ps = rows_sum4(ps);
            const float kept = l[gg] * exp2f(m[gg] - mn);  // the old weights on the new reference
            const float ln = kept + ps;
            const float inv = 1.0f / ln;
            const float keep = kept * inv;
#pragma unroll
            for (int e = 0; e < EL; ++e) acc[gg][e] *= keep;
#pragma unroll
            for (int t = 0; t < kT; ++t) s[t][gg] *= inv;  // each row's share of the new output
            l[gg] = ln;
            m[gg] = mn;
        }
        // --- values: the same rows and elements
#pragma unroll
        for (int t = 0; t < kT; ++t)
#pragma unroll
            for (int e = 0; e < EL; ++e) {
                const float x = elem<EL>(xv[t], e);
#pragma unroll
                for (int gg = 0; gg < G; ++gg) acc[gg][e] += s[t][gg] * x;
            }
    }
    // --- the four row sets of a wave, then the four waves
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
#pragma unroll
        for (int e = 0; e < EL; ++e) {
            acc[gg][e] += __shfl_xor(acc[gg][e], 16);
            acc[gg][e] += __shfl_xor(acc[gg][e], 32);
        }
    if (lane < 16) {
#pragma unroll
        for (int gg = 0; gg < G; ++gg)
#pragma unroll
            for (int e = 0; e < EL; ++e) red_acc[wave][gg][sl * EL + e] = acc[gg][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int gg = 0; gg < G; ++gg) {
            red_m[wave][gg] = m[gg];
            red_l[wave][gg] = l[gg];
        }
    }
    __syncthreads();
    const int64_t rows_q = (int64_t)g.B * g.Hq;
    for (int i = tid; i < G * D; i += 256) {
        const int gg = i / D, e = i - gg * D;
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < kDecWaves; ++w2) M = fmaxf(M, red_m[w2][gg]);
        float wt[kDecWaves];
        float L = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kDecWaves; ++w2) {
            wt[w2] = red_m[w2][gg] == -INFINITY ? 0.f : red_l[w2][gg] * exp2f(red_m[w2][gg] - M);
            L += wt[w2];
        }
        float A = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < kDecWaves; ++w2) A += (wt[w2] / L) * red_acc[w2][gg][e];
        const int64_t qrow = (int64_t)b * g.Hq + kvh * G + gg;
        part_acc[((int64_t)split * rows_q + qrow) * D + e] = A;
        if (e == 0) {
            part_m[(int64_t)split * rows_q + qrow] = M;
            part_l[(int64_t)split * rows_q + qrow] = L;
        }
    }
}

template <int D>
__global__ void decode_combine_kernel(DecGeom g, const float* part_m, const float* part_l, const float* part_acc,
                                      float* out) {
    const int64_t rows_q = (int64_t)g.B * g.Hq;
    const int64_t qrow = blockIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < g.splits; ++s) M = fmaxf(M, part_m[(int64_t)s * rows_q + qrow]);
    float L = 0.f;
    for (int s = 0; s < g.splits; ++s) {
        const float ms = part_m[(int64_t)s * rows_q + qrow];
        L += ms == -INFINITY ? 0.f : part_l[(int64_t)s * rows_q + qrow] * exp2f(ms - M);
    }
    for (int e = threadIdx.x; e < D; e += blockDim.x) {
        float A = 0.f;
        for (int s = 0; s < g.splits; ++s) {
            const float ms = part_m[(int64_t)s * rows_q + qrow];
            const float w = ms == -INFINITY ? 0.f : part_l[(int64_t)s * rows_q + qrow] * exp2f(ms - M) / L;
            A += w * part_acc[((int64_t)s * rows_q + qrow) * D + e];
        }
        out[qrow * D + e] = A;
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }


DecGeom plan(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n, float scale, int n_cu) {
    DecGeom g;
    g.B = B;
    g.Hq = Hq;
    g.Hkv = Hkv;
    g.G = Hq / Hkv;
    g.n = n;
    // one full wave of resident work-groups (a second, partial wave would run
    // at a fraction of the occupancy), each split at least 256 keys
    const int64_t units = (int64_t)B * Hkv;
    const int64_t target = (int64_t)n_cu * dec_waves(d, g.G);
    int64_t s = (target + units - 1) / units;
    const int64_t max_s = (n + 255) / 256;
    if (s > max_s) s = max_s;
    if (s < 1) s = 1;
    if (s > 65535) s = 65535;
    int64_t len = (n + s - 1) / s;
    len = (len + 63) & ~(int64_t)63;
    g.split_len = len;
    g.splits = (int32_t)((n + len - 1) / len);
    g.c = scale * 1.4426950408889634f;
    return g;
}

template <int D>
bool launch_g(const DecGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* degree,
              float* pm, float* pl, float* pa, hipStream_t st) {
    const dim3 grid((unsigned)g.splits, (unsigned)(g.B * g.Hkv));
    switch (g.G) {
#define KVSEL_DEC_CASE(GG)                                                                                           \
    case GG:                                                                                                         \
        hipLaunchKernelGGL((decode_kernel<D, GG>), grid, dim3(256), 0, st, g, q, k, v, degree, pm, pl, pa);         \
        return true;
        KVSEL_DEC_CASE(1)
        KVSEL_DEC_CASE(2)
        KVSEL_DEC_CASE(3)
        KVSEL_DEC_CASE(4)
        KVSEL_DEC_CASE(5)
        KVSEL_DEC_CASE(6)
        KVSEL_DEC_CASE(7)
        KVSEL_DEC_CASE(8)
#undef KVSEL_DEC_CASE
        default: return false;
    }
}

}  // namespace

int decode_max_group() { return kMaxG; }

size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n, int n_cu) {
    const DecGeom g = plan(B, Hq, Hkv, d, n, 1.f, n_cu);
    const size_t rows = (size_t)g.splits * B * Hq;
    return align256(rows * sizeof(float)) * 2 + align256(rows * d * sizeof(float));
}

hipError_t launch_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n, float scale, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const int32_t* degree, float* out, void* workspace,
                         int n_cu, hipStream_t st) {
    const DecGeom g = plan(B, Hq, Hkv, d, n, scale, n_cu);
    const size_t rows = (size_t)g.splits * B * Hq;
    char* ws = static_cast<char*>(workspace);
    float* pm = reinterpret_cast<float*>(ws);
    float* pl = reinterpret_cast<float*>(ws + align256(rows * sizeof(float)));
    float* pa = reinterpret_cast<float*>(ws + 2 * align256(rows * sizeof(float)));
    const bool ok = d == 128 ? launch_g<128>(g, q, k, v, degree, pm, pl, pa, st)
                             : launch_g<64>(g, q, k, v, degree, pm, pl, pa, st);
    if (!ok) return hipErrorInvalidValue;
    if (d == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)(B * Hq)), dim3(128), 0, st, g, pm, pl, pa, out);
    else
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)(B * Hq)), dim3(64), 0, st, g, pm, pl, pa, out);
    return hipGetLastError();
}

}  // namespace kvsel
