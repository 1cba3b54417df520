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
//   2. pass 1: logits on v_mfma_f32_32x32x16_bf16, (reference, sum of exp2)
//      per row over its keys, merged to one partial per row and published;
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
// Operands use the 32x32x16 layout of tile32.h. Keys are read from HBM with
// whole rows per load instruction and reshaped into that layout through a
// per-wave LDS staging area: loading the fragments directly would touch a
// cache line per lane and instruction.
//
// Within a wave the exponentials of one 32-key block are issued while the
// matrix core computes the next block's logits, so the two units overlap.
#include <math.h>
#include <stdint.h>

#include "kvsel.h"
#include "kvsel_internal.h"
#include "tile32.h"

namespace kvsel {
namespace {

using namespace tile;

constexpr uint64_t kEmpty64 = ~0ull;
constexpr uint32_t kEmpty32 = ~0u;

__device__ __forceinline__ uint32_t ld32(const uint32_t* p) {
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

// Dense index of the compute unit this wave runs on: XCC_ID and the SE / SH /
// CU fields of HW_ID (hardware registers 20 and 4), kTurnKeys entries.
constexpr int kTurnKeys = 2048;
__device__ __forceinline__ uint32_t cu_key() {
    const uint32_t hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));
    return ((xcc & 7u) << 8) | (((hw >> 13) & 7u) << 5) | (((hw >> 12) & 1u) << 4) | ((hw >> 8) & 15u);
}

// Load turns of the two work-groups sharing a CU (entry: presence of stream 0
// and 1, loads completed by stream 0 and 1). Stream 0 issues its k-th slab's
// key loads once stream 1 has completed k loads, stream 1 its k-th once stream
// 0 has completed k+1, so the two streams' HBM phases alternate instead of
// colliding. This only orders work: a wait that finds no partner, or lasts
// longer than kTurnTicks, gives up and proceeds.
constexpr uint64_t kTurnTicks = 5000;  // 50 us of the 100 MHz wall clock
__device__ void turn_wait(uint32_t* tent, int p, int k, bool& solo) {
    if (solo) return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    if (p == 0) {
        if (k == 0 || ld32(tent + 1) == 0u) return;
        while (ld32(tent + 3) < (uint32_t)k) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > kTurnTicks) return;
            __builtin_amdgcn_s_sleep(2);
        }
    } else {
        for (;;) {
            if (ld32(tent) != 0u && ld32(tent + 2) >= (uint32_t)(k + 1)) return;
            const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t0;
            if (dt > kTurnTicks || (dt > kTurnTicks / 10 && ld32(tent) == 0u)) {
                solo = ld32(tent) == 0u;  // no partner on this CU: stop waiting
                return;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
}


template <int D, int KB, int RBN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
kres_kernel(KresArgs a) {
    constexpr int KS = D / 16;     // k-steps per fragment
    constexpr int RP = RBN * 32;   // row capacity
    constexpr int QST = D + 8;     // LDS row stride in elements (16 bytes of padding)
    constexpr int CPK = D / 8;     // 16-byte chunks per key row
    constexpr int KPI = 64 / CPK;  // keys per coalesced wave load
    constexpr int NBUF = (RP > 128 ? RP : 128) * QST;
    // q_lds holds the query rows during the passes and, before that, four
    // per-wave staging areas of 32 key rows each (same row stride)
    __shared__ __attribute__((aligned(16))) uint16_t q_lds[NBUF];
    __shared__ float2 red[4][RP];
    __shared__ __attribute__((aligned(16))) float lse_lds[RP];
    __shared__ float2 wred[4];  // per-wave (reference, sum) of an owned row

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int hf = lane >> 5;
    const int p = blockIdx.x / a.wg_per_stream;
    const int r = blockIdx.x - p * a.wg_per_stream;
    const int team = r / a.team_wgs;
    const int wi = r - team * a.team_wgs;
    if (wi >= a.n_act) return;  // no keys for this work-group
    const int gt = p * a.n_teams + team;
    const int sstride = 2 * a.n_teams;
    const int kbase = wi * (4 * KB * 32) + wave * (KB * 32);  // first key of this wave
    const bool edge = kbase + KB * 32 > a.Np;  // reaches the window (causal mask) or the end
    uint32_t* abort_word = a.abort_word;
    uint16_t* stage = q_lds + wave * 32 * QST;
    uint32_t* tent = a.turn + cu_key() * 4u;
    if (tid == 0) __hip_atomic_fetch_add(tent + p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool solo = false;
    int nload = 0;  // slabs whose keys this work-group has loaded

    for (int s = gt; s < a.S; s += sstride) {
        const int g = s % a.Hkv;
        const int b = (s / a.Hkv) % a.B;
        const int l = s / (a.Hkv * a.B);
        const uint16_t* kslab = a.k + l * a.ks[0] + b * a.ks[1] + g * a.ks[2];
        const uint16_t* qbase = a.q + l * a.qs[0] + b * a.qs[1];

        if (tid == 0) turn_wait(tent, p, nload, solo);
        __syncthreads();  // the previous slab is done with LDS; this work-group's turn to load
        // --- this wave's keys: coalesced loads (KPI whole rows per instruction,
        //     clamped past the end), then reshaped through LDS into operand
        //     fragments: fragment (kb, ks) of lane l holds elements
        //     ks*16 + hf*8 .. +7 of key kbase + kb*32 + col
        bf16x8 kst[KB][KS];
        {
            // key kbase + i*KPI + lane/CPK at step i (i = kb*KS + t): one pointer,
            // advanced by a uniform stride and clamped to the last key
            const uint16_t* kp = kslab + (int64_t)(kbase + lane / CPK) * a.ks[3] + (lane % CPK) * 8;
            const uint16_t* klast = kslab + (int64_t)(a.N - 1) * a.ks[3] + (lane % CPK) * 8;
            const int64_t kstep = (int64_t)KPI * a.ks[3];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    kst[kb][t] = *reinterpret_cast<const bf16x8*>(kp < klast ? kp : klast);
                    kp += kstep;
                }
        }
        // --- the query rows of KV head g (row r -> head g*G + r/w, window index
        //     r%w), loaded now and stored to LDS once the keys are reshaped
        constexpr int QPER = (RP * CPK + 255) / 256;
        uint4 qv[QPER];
#pragma unroll
        for (int u = 0; u < QPER; ++u) {
            const int idx = tid + u * 256;
            const int row = idx / CPK;
            const int ch = idx - row * CPK;
            qv[u] = make_uint4(0u, 0u, 0u, 0u);
            if (row < a.R) {
                const int h = g * a.G + row / a.w;
                const int i = row % a.w;
                qv[u] = *reinterpret_cast<const uint4*>(qbase + h * a.qs[2] + i * a.qs[3] + ch * 8);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // every key and query load has landed: the partner may load
        if (tid == 0) st32(tent + 2 + p, (uint32_t)(++nload));
        bf16x8 kf[KB][KS];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int t = 0; t < KS; ++t)
                *reinterpret_cast<bf16x8*>(stage + (t * KPI + lane / CPK) * QST + (lane % CPK) * 8) = kst[kb][t];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[kb][ks] = *reinterpret_cast<const bf16x8*>(stage + col * QST + ks * 16 + hf * 8);
            __builtin_amdgcn_wave_barrier();
        }
        __syncthreads();  // every wave has its fragments; the staging areas become q_lds
#pragma unroll
        for (int u = 0; u < QPER; ++u) {
            const int idx = tid + u * 256;
            const int row = idx / CPK;
            const int ch = idx - row * CPK;
            if (row < RP) *reinterpret_cast<uint4*>(q_lds + row * QST + ch * 8) = qv[u];
        }
        __syncthreads();

        // --- pass 1: (reference, sum of exp2) per row over this wave's keys, log2 domain
#pragma unroll 1
        for (int rb = 0; rb < a.rbn; ++rb) {
            bf16x8 qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rb * 32 + col) * QST + ks * 16 + hf * 8);
            // lane holds row rb*32 + col and keys kbase + kb*32 + tile_row(v, hf)
            float m, z;
            if (edge) {
                const int row = rb * 32 + col;
                const int lim = row < a.R ? a.Np + row % a.w : -1;
                z = pass1_max<D, KB, true>(kf, qf, a.c, kbase, hf, lim, m);
            } else {
                z = pass1_fast<D, KB>(kf, qf, a.c, m);
                if (__any(!(z < kOverflow))) z = pass1_max<D, KB, false>(kf, qf, a.c, kbase, hf, 0, m);
            }
            // merge the two lane halves (same row, other keys)
            merge(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
            if (hf == 0) red[wave][rb * 32 + col] = make_float2(m, z);
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

        // --- pass 2: per key, sum over all rows of exp2(x - LSE2); lane holds
        //     key kbase + kb*32 + col and rows rb*32 + tile_row(v, hf)
        float cs[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) cs[kb] = 0.f;
#pragma unroll 1
        for (int rb = 0; rb < a.rbn; ++rb) {
            bf16x8 qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(q_lds + (rb * 32 + col) * QST + ks * 16 + hf * 8);
            float lr[16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 t = *reinterpret_cast<const float4*>(lse_lds + rb * 32 + 8 * u + 4 * hf);
                lr[4 * u] = t.x;
                lr[4 * u + 1] = t.y;
                lr[4 * u + 2] = t.z;
                lr[4 * u + 3] = t.w;
            }
            f32x16 cur = logits<KS>(qf, kf[0]);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x16 nxt;
                if (kb + 1 < KB) nxt = logits<KS>(qf, kf[kb + 1]);
                float t0s = 0.f, t1s = 0.f;
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    t0s += fexp2(cur[v] * a.c - lr[v]);
                    t1s += fexp2(cur[v + 1] * a.c - lr[v + 1]);
                }
                cs[kb] += t0s + t1s;
                if (kb + 1 < KB) cur = nxt;
            }
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const float v = cs[kb] + __shfl_xor(cs[kb], 32);
            const int j = kbase + kb * 32 + col;
            if (hf == 0 && j < a.Np) a.raw[(int64_t)s * a.Np + j] = ok ? v * a.invG : NAN;
        }
    }
    if (tid == 0) st32(tent + 2 + p, 0x7fffffffu);  // no more loads from this work-group
}

// Fill the exchange slots with the all-ones sentinel and clear the abort word.
__global__ void kres_clear_kernel(uint64_t* slots, int64_t n64, uint32_t* abort_word, uint32_t* turn) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n64; i += (int64_t)gridDim.x * blockDim.x)
        st64(slots + i, kEmpty64);
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kTurnKeys * 4; i += gridDim.x * blockDim.x)
        st32(turn + i, 0u);
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
        default: return nullptr;
    }
}

template <int D>
kres_fn pick_kb(int KB, int RBN) {
    switch (KB) {
        case 1: return pick_rbn<D, 1>(RBN);
        case 2: return pick_rbn<D, 2>(RBN);
        case 4: return pick_rbn<D, 4>(RBN);
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
    constexpr int kKeysPerWgMax = 4 * 4 * 32;  // 4 waves x 4 key blocks x 32 keys
    const int64_t team = (N + kKeysPerWgMax - 1) / kKeysPerWgMax;
    if (team > n_cu) return false;  // keys do not fit in one team's registers
    plan.team_wgs = (int)team;
    const int64_t per_wave = (N + team * 4 - 1) / (team * 4);
    plan.kb = pow2_at_least((int)((per_wave + 31) / 32));
    plan.n_act = (int)((N + plan.kb * 128 - 1) / (plan.kb * 128));
    int64_t teams = n_cu / plan.team_wgs;
    const int64_t need = (S + 1) / 2;  // teams per stream that have any slab
    if (teams > need) teams = need;
    if (teams < 1) teams = 1;
    plan.n_teams = (int)teams;
    plan.wg_per_stream = plan.n_teams * plan.team_wgs;
    plan.rbn_cap = pow2_at_least((R + 31) / 32);
    plan.rbn = (R + 31) / 32;
    plan.rp = plan.rbn_cap * 32;
    plan.part_off = 0;
    plan.lse2_off = (size_t)S * plan.team_wgs * plan.rp * sizeof(uint64_t);
    plan.slots_end = plan.lse2_off + (((size_t)S * plan.rp * sizeof(float) + 7) & ~(size_t)7);
    plan.abort_off = align256(plan.slots_end);
    plan.turn_off = align256(plan.abort_off + sizeof(uint32_t));
    plan.raw_off = align256(plan.turn_off + (size_t)kTurnKeys * 4 * sizeof(uint32_t));
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
    hipLaunchKernelGGL(kres_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.slots, a.n_slots, a.abort_word,
                       a.turn);
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
