// Register-resident two-pass saliency kernel (bf16, head_dim 64 or 128).
//
// The score of a key needs its window rows' final log-sum-exp, which depends
// on every key of the (layer, sequence, KV head) slab, so the softmax takes
// two passes over K. Re-reading K from HBM for the second pass doubles the
// traffic, and a second read served from the memory-side cache runs no faster
// than HBM on this part. This kernel reads K from HBM once: every slab is
// split across a team of work-groups, each of which keeps its share of K in
// VGPRs as matrix-core operand fragments across both passes.
//
// One slab, seen from one work-group of its team:
//   1. stage the slab's G*w query rows in LDS; load its key range into VGPRs;
//   2. pass 1: logits on v_mfma_f32_16x16x32_bf16, (max, sum of exp2) per
//      row over its keys, merged to one partial per row and published;
//   3. the owner of row r (work-group r mod team size) merges the team's
//      partials of that row into the row's LSE and publishes it;
//   4. every work-group reads all row LSEs, then pass 2 recomputes the
//      logits from the same registers and sums exp2(x - LSE2) over every row
//      per key, times 1/G -> raw scores.
// Two work-groups share each CU and take alternate slabs, so one computes
// while the other waits for its loads or for its slab's LSEs.
//
// Cross-work-group exchange uses no fences and no contended atomics: every
// published value is its own ready flag. Partials (64-bit) and LSEs (32-bit)
// are written with single-copy-atomic agent-scope stores into slots filled
// with an all-ones sentinel before the launch (no real partial or LSE has
// that bit pattern), and readers poll the slots with agent-scope loads, which
// bypass the per-XCD L2. Every poll is bounded by a wall-clock limit; a
// timeout sets a shared abort word, after which every wait returns at once
// and the affected scores are written as NaN, so the grid always drains. The
// grid is sized to the occupancy the device reports, so every work-group of a
// team is resident together.
//
// Operand layout (16x16x32 bf16): lane l supplies row/column (l % 16) and the
// 8 consecutive k-slots of lane group (l / 16). At k-step ks the slot
// (group, v) carries head-dim element ks*32 + group*8 + v, for K and Q alike,
// so each key's four lanes read 64 contiguous bytes per load.

#include <math.h>
#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr uint64_t kEmpty64 = ~0ull;
constexpr uint32_t kEmpty32 = ~0u;

__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll a slot until it leaves the sentinel. Returns false (and sets the abort
// word on a timeout) if the wait is abandoned.
template <typename T>
__device__ bool poll(const T* p, T empty, T& v, uint32_t* abort_word, uint64_t t0, int64_t limit) {
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (uint32_t it = 0; v == empty; ++it) {
        __builtin_amdgcn_s_sleep(1);
        if ((it & 15u) == 15u) {
            if (ld32(abort_word) != 0u) return false;
            if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)limit) {
                st32(abort_word, 1u);
                return false;
            }
        }
        v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return true;
}

__device__ __forceinline__ void merge(float& m, float& z, float mo, float zo) {
    const float mn = fmaxf(m, mo);
    z = z * fexp2(m - mn) + zo * fexp2(mo - mn);
    m = mn;
}

// Pass 1 on one 16-row block: logits of this lane's row against the wave's
// KB*16 keys, reduced to a (reference, sum of exp2(x - reference)) pair.
// Any logit of the row is a valid reference as far as the final LSE goes (the
// merge rescales partials by their references); the maximum only has to keep
// exp2 from overflowing. Away from the window the first logit is the
// reference, so the exponentials can start while later products are still in
// the matrix pipe; if some logit exceeds it by more than 2^64 the block is
// redone with the maximum. Blocks that reach the causal window mask their
// invisible keys and use the maximum directly.
template <int D, int KB, bool EDGE>
__device__ __forceinline__ void pass1_block(const bf16x8 (&kf)[KB][D / 32], const bf16x8 (&qf)[D / 32], float c,
                                            int kfirst, int lim, float& m_out, float& z_out) {
    constexpr int KS = D / 32;
    f32x4 acc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[kb] = mma(kf[kb][ks], qf[ks], acc[kb]);
    }
    if (EDGE) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (kfirst + kb * 16 + v > lim) acc[kb][v] = -INFINITY;
    }
    float mxa = acc[0][0], mxb = acc[0][1];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        mxa = fmaxf(mxa, fmaxf(acc[kb][0], acc[kb][2]));
        mxb = fmaxf(mxb, fmaxf(acc[kb][1], acc[kb][3]));
    }
    const float mx = fmaxf(mxa, mxb) * c;
    float ref = EDGE ? fmaxf(kNegBig, mx) : acc[0][0] * c;
    float zs[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) zs[v] = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) zs[v] += fexp2(acc[kb][v] * c - ref);
    if (!EDGE && __any(mx - ref > 64.f)) {
        ref = fmaxf(ref, mx);
#pragma unroll
        for (int v = 0; v < 4; ++v) zs[v] = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int v = 0; v < 4; ++v) zs[v] += fexp2(acc[kb][v] * c - ref);
    }
    m_out = ref;
    z_out = (zs[0] + zs[1]) + (zs[2] + zs[3]);
}

template <int D, int KB, int RBN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
kres_kernel(KresArgs a) {
    constexpr int KS = D / 32;     // k-steps per fragment
    constexpr int RP = RBN * 16;   // row capacity
    constexpr int QST = D + 8;     // LDS row stride in elements (16 bytes of padding)
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[RP * QST];
    __shared__ float2 red[4][RP];
    __shared__ __attribute__((aligned(16))) float lse_lds[RP];
    __shared__ float2 wred[4];  // per-wave (max, sum) of an owned row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 15;
    const int lg = lane >> 4;
    const int p = blockIdx.x / a.wg_per_stream;
    const int r = blockIdx.x - p * a.wg_per_stream;
    const int team = r / a.team_wgs;
    const int wi = r - team * a.team_wgs;
    if (wi >= a.n_act) return;  // no keys for this work-group
    const int gt = p * a.n_teams + team;
    const int sstride = 2 * a.n_teams;
    const int kbase = wi * (4 * KB * 16) + wave * (KB * 16);  // first key of this wave
    const bool edge = kbase + KB * 16 > a.Np;  // reaches the window (causal mask) or the end
    uint32_t* abort_word = a.abort_word;

    for (int s = gt; s < a.S; s += sstride) {
        const int g = s % a.Hkv;
        const int b = (s / a.Hkv) % a.B;
        const int l = s / (a.Hkv * a.B);
        const uint16_t* kslab = a.k + l * a.ks[0] + b * a.ks[1] + g * a.ks[2];
        const uint16_t* qbase = a.q + l * a.qs[0] + b * a.qs[1];

        __syncthreads();  // the previous slab is done with LDS
        // --- this wave's keys, as operand fragments (clamped loads past the end);
        //     issued first so they are in flight while the queries are staged
        bf16x8 kf[KB][KS];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int j = min(kbase + kb * 16 + col, a.N - 1);
            const uint16_t* row = kslab + (int64_t)j * a.ks[3] + lg * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[kb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + ks * 32));
        }
        // --- stage the query rows of KV head g (row r -> head g*G + r/w, window
        //     index r%w) in LDS: every load is issued before the first store
        {
            constexpr int CH = D / 8;                // 16-byte chunks per row
            constexpr int PER = (RP * CH + 255) / 256;
            constexpr int BATCH = PER < 8 ? PER : 8;  // loads in flight per thread
#pragma unroll
            for (int u0 = 0; u0 < PER; u0 += BATCH) {
                uint4 qv[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int idx = tid + (u0 + u) * 256;
                    const int row = idx / CH;
                    const int ch = idx - row * CH;
                    qv[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (row < a.R) {
                        const int h = g * a.G + row / a.w;
                        const int i = row % a.w;
                        qv[u] = *reinterpret_cast<const uint4*>(qbase + h * a.qs[2] + i * a.qs[3] + ch * 8);
                    }
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const int idx = tid + (u0 + u) * 256;
                    const int row = idx / CH;
                    const int ch = idx - row * CH;
                    if (row < RP) *reinterpret_cast<uint4*>(q_lds + row * QST + ch * 8) = qv[u];
                }
            }
        }
        __syncthreads();

        // --- pass 1: (reference, sum of exp2) per row over this wave's keys, log2 domain
#pragma unroll 1
        for (int rb = 0; rb < a.rbn; ++rb) {
            bf16x8 qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rb * 16 + col) * QST + ks * 32 + lg * 8);
            // lane holds row rb*16 + col and keys kbase + kb*16 + 4*lg + v
            float m, z;
            if (edge) {
                const int row = rb * 16 + col;
                const int lim = row < a.R ? a.Np + row % a.w : -1;
                pass1_block<D, KB, true>(kf, qf, a.c, kbase + 4 * lg, lim, m, z);
            } else {
                pass1_block<D, KB, false>(kf, qf, a.c, kbase + 4 * lg, 0, m, z);
            }
            // merge the four lane groups (same row, other keys)
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) merge(m, z, __shfl_xor(m, off), __shfl_xor(z, off));
            if (lg == 0) red[wave][rb * 16 + col] = make_float2(m, z);
        }
        __syncthreads();
        uint64_t* part_s = a.part + (int64_t)s * a.team_wgs * RP;
        for (int row = tid; row < a.R; row += 256) {
            float2 acc = red[0][row];
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) merge(acc.x, acc.y, red[w2][row].x, red[w2][row].y);
            st64(part_s + (int64_t)wi * RP + row,
                 (uint64_t)__float_as_uint(acc.x) | ((uint64_t)__float_as_uint(acc.y) << 32));
        }
        // --- rows this work-group owns: merge the team's partials into the LSE
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        bool ok = true;
        for (int row = wi; row < a.R; row += a.n_act) {
            float M = kNegBig, Z = 0.f;
            for (int w2 = tid; w2 < a.n_act; w2 += 256) {
                uint64_t v;
                if (poll(part_s + (int64_t)w2 * RP + row, kEmpty64, v, abort_word, t0, a.spin_limit))
                    merge(M, Z, __uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
                else
                    ok = false;
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) merge(M, Z, __shfl_xor(M, off), __shfl_xor(Z, off));
            if (lane == 0) wred[wave] = make_float2(M, Z);
            __syncthreads();
            if (tid == 0) {
#pragma unroll
                for (int w2 = 1; w2 < 4; ++w2) merge(M, Z, wred[w2].x, wred[w2].y);
                const float l2 = M + log2f(Z);
                st32(reinterpret_cast<uint32_t*>(a.lse2) + (int64_t)s * RP + row, __float_as_uint(l2));
                if (a.lse_out) {
                    const int h = g * a.G + row / a.w;
                    const int i = row % a.w;
                    a.lse_out[(((int64_t)l * a.B + b) * a.Hq + h) * a.w + i] = l2 * 0.69314718055994530942f;
                }
            }
            __syncthreads();
        }
        // --- every row's LSE (padded rows: +inf, probability 0 in pass 2)
        for (int row = tid; row < RP; row += 256) {
            float v = INFINITY;
            if (row < a.R) {
                uint32_t u;
                if (poll(reinterpret_cast<const uint32_t*>(a.lse2) + (int64_t)s * RP + row, kEmpty32, u, abort_word,
                         t0, a.spin_limit))
                    v = __uint_as_float(u);
                else
                    ok = false;
            }
            lse_lds[row] = v;
        }
        ok = __syncthreads_and(ok) != 0;

        // --- pass 2: per key, sum over all rows of exp2(x - LSE2)
        float cs[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) cs[kb] = 0.f;
#pragma unroll 1
        for (int rb = 0; rb < a.rbn; ++rb) {
            {
                bf16x8 qf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rb * 16 + col) * QST + ks * 32 + lg * 8);
                const float4 lr = *reinterpret_cast<const float4*>(lse_lds + rb * 16 + 4 * lg);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) acc = mma(qf[ks], kf[kb][ks], acc);
                    // lane holds key kbase + kb*16 + col and rows rb*16 + 4*lg + v
                    cs[kb] += fexp2(acc[0] * a.c - lr.x) + fexp2(acc[1] * a.c - lr.y) +
                              fexp2(acc[2] * a.c - lr.z) + fexp2(acc[3] * a.c - lr.w);
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float v = cs[kb];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            const int j = kbase + kb * 16 + col;
            if (lg == 0 && j < a.Np) a.raw[(int64_t)s * a.Np + j] = ok ? v * a.invG : NAN;
        }
    }
}

// Fill the exchange slots with the all-ones sentinel and clear the abort word.
__global__ void kres_clear_kernel(uint64_t* slots, int64_t n64, uint32_t* abort_word) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n64; i += (int64_t)gridDim.x * blockDim.x)
        st64(slots + i, kEmpty64);
    if (blockIdx.x == 0 && threadIdx.x == 0) st32(abort_word, 0u);
}

typedef void (*kres_fn)(KresArgs);

template <int D, int KB>
kres_fn pick_rbn(int RBN) {
    switch (RBN) {
        case 1: return kres_kernel<D, KB, 1>;
        case 2: return kres_kernel<D, KB, 2>;
        case 4: return kres_kernel<D, KB, 4>;
        case 8: return kres_kernel<D, KB, 8>;
        case 16: return kres_kernel<D, KB, 16>;
        default: return nullptr;
    }
}

template <int D>
kres_fn pick_kb(int KB, int RBN) {
    switch (KB) {
        case 1: return pick_rbn<D, 1>(RBN);
        case 2: return pick_rbn<D, 2>(RBN);
        case 4: return pick_rbn<D, 4>(RBN);
        case 8: return pick_rbn<D, 8>(RBN);
        default: return nullptr;
    }
}

kres_fn pick(int D, int KB, int RBN) { return D == 128 ? pick_kb<128>(KB, RBN) : pick_kb<64>(KB, RBN); }

int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool kres_plan(int dtype, int head_dim, int R, int64_t N, int64_t S, int n_cu, KresPlan& plan) {
    plan.ok = false;
    plan.head_dim = head_dim;
    if (dtype != KVSEL_DTYPE_BF16 || (head_dim != 64 && head_dim != 128)) return false;
    if (R > 256 || n_cu < 1 || N < 1) return false;
    constexpr int kKeysPerWgMax = 4 * 8 * 16;  // 4 waves x 8 key blocks x 16 keys
    const int64_t team = (N + kKeysPerWgMax - 1) / kKeysPerWgMax;
    if (team > n_cu) return false;  // keys do not fit in one team's registers
    plan.team_wgs = (int)team;
    const int64_t per_wave = (N + team * 4 - 1) / (team * 4);
    plan.kb = pow2_at_least((int)((per_wave + 15) / 16));
    plan.n_act = (int)((N + plan.kb * 64 - 1) / (plan.kb * 64));
    int64_t teams = n_cu / plan.team_wgs;
    const int64_t need = (S + 1) / 2;  // teams per stream that have any slab
    if (teams > need) teams = need;
    if (teams < 1) teams = 1;
    plan.n_teams = (int)teams;
    plan.wg_per_stream = plan.n_teams * plan.team_wgs;
    plan.rbn_cap = pow2_at_least((R + 15) / 16);
    plan.rbn = (R + 15) / 16;
    plan.rp = plan.rbn_cap * 16;
    plan.part_off = 0;
    plan.lse2_off = (size_t)S * plan.team_wgs * plan.rp * sizeof(uint64_t);
    plan.slots_end = plan.lse2_off + (((size_t)S * plan.rp * sizeof(float) + 7) & ~(size_t)7);
    plan.abort_off = align256(plan.slots_end);
    plan.raw_off = align256(plan.abort_off + sizeof(uint32_t));
    plan.total = plan.raw_off;  // + raw, added by the caller (shared with the general path)
    plan.ok = true;
    return true;
}

hipError_t launch_kres(const KresPlan& plan, KresArgs a, hipStream_t st) {
    kres_fn fn = pick(plan.head_dim, plan.kb, plan.rbn_cap);
    if (!fn) return hipErrorInvalidValue;
    int64_t blocks = (a.n_slots + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(kres_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.slots, a.n_slots, a.abort_word);
    hipLaunchKernelGGL(fn, dim3(2 * plan.wg_per_stream), dim3(256), 0, st, a);
    return hipGetLastError();
}

bool kres_fits(const KresPlan& plan) {
    kres_fn fn = pick(plan.head_dim, plan.kb, plan.rbn_cap);
    if (!fn) return false;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), 256, 0) !=
        hipSuccess)
        return false;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    return (int64_t)per_cu * n_cu >= 2 * (int64_t)plan.wg_per_stream;
}

}  // namespace kvsel
