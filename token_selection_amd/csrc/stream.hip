// Streaming two-pass saliency kernels (bf16, head_dim 64 or 128).
//
// The score of a prefix key needs the final log-sum-exp of every window row,
// which depends on every key of the (layer, sequence, KV head) slab. These
// kernels take the two passes literally and stream K from HBM in each:
//
//   stream_kernel<PASS=1>  per-row (reference, sum of exp2) partials of every
//                          segment of a slab, causal mask applied;
//   stream_merge_kernel    the partials of a slab's segments -> row LSE2 (and
//                          the natural-log LSE the caller may ask for), or
//                          the same merge done by pass 2 as it stages a slab;
//   stream_kernel<PASS=2>  per prefix key, sum over the rows of
//                          exp2(c*x - LSE2), times 1/G -> raw scores.
//
// With ST (the pivot statistics of StructKV section 2) pass 1 also carries
// each row's sum of e*x and e^2 (tile32.h), the merge turns them into the
// row's entropy and sum of p^2, and pass 2 runs over all N keys and also counts
// the keys each row sees with p below a threshold: the exponent it already
// has decides (c*x - LSE2 < log2 threshold), into packed per-lane counters
// that are summed over the lanes once per segment.
//
// A slab holds at most 256 window rows: when a KV head's G*w rows exceed
// that, its query heads split into head groups, each a slab of its own over
// the same keys (StreamArgs::T, Gs, S0).
//
// With LS (calls of several layers, average pool, one head group) pass 2 adds
// up groups of layers itself: a work-group walks the layers of a group over
// one key range, keeps each key's running sum in LDS and writes it once, so
// raw holds one row per layer group instead of one per layer (pooling the sum
// equals summing the pooled layers).
//
// No work-group waits for another: every slab is cut into segments of whole
// 256-key chunks, work-group g takes segments g, g + grid, ..., and while it
// computes one chunk the loads of its next chunk are in flight into a second
// register buffer, so HBM sees a continuous stream of requests. Each wave
// holds 64 keys of a chunk as 32x32x16 operand fragments (tile32.h) and
// reads its query fragments from the slab's rows staged in LDS.

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kvsel.h"
#include "kvsel_internal.h"
#include "tile32.h"

namespace kvsel {
namespace {

using namespace tile;

constexpr int kWaves = 4;
constexpr int kKB = 2;                     // 32-key blocks per wave and chunk
constexpr int kWaveKeys = kKB * 32;        // 64
constexpr int kChunk = kWaves * kWaveKeys; // 256 keys per work-group chunk

template <int D>
struct Frag {
    bf16x8 v[kKB][D / 16];
};

// Pass 1 without statistics: each lane's running (reference, sum) of its row
// in every row block, over the keys of its lane half, held in registers for
// the whole segment (the halves and the waves merge when the segment ends).
// Interior chunks index the slots statically; the rolled loop of a chunk at
// the causal window works on slot 0 and rotates, RBN times per chunk, so that
// every block is back in its own slot afterwards.
template <int RBN>
struct RowState {
    float m[RBN], z[RBN];
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int rb = 0; rb < RBN; ++rb) {
            m[rb] = kNegBig;
            z[rb] = 0.f;
        }
    }
    // Slot 0 is the current row block's; after RBN rotations every row
    // block is back in its own slot (static register indices only).
    __device__ __forceinline__ void rotate() {
        const float m0 = m[0], z0 = z[0];
#pragma unroll
        for (int rb = 0; rb + 1 < RBN; ++rb) {
            m[rb] = m[rb + 1];
            z[rb] = z[rb + 1];
        }
        m[RBN - 1] = m0;
        z[RBN - 1] = z0;
    }
};

// Pass 2 with statistics: per lane, for every row block and result register
// v (row rb*32 + tile_row(v, half)), how many of the lane's keys had p below
// the threshold: 8-bit fields, four to a register, in rotating slots like
// RowState. A field grows by at most kKB per chunk and segments hold at most
// kMaxSegChunks chunks, so it cannot overflow before the segment's flush.
constexpr int kMaxSegChunks = 127;

template <int RBN>
struct CountState {
    uint32_t c[RBN][4];
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int rb = 0; rb < RBN; ++rb)
#pragma unroll
            for (int w = 0; w < 4; ++w) c[rb][w] = 0u;
    }
    __device__ __forceinline__ void rotate() {
        uint32_t c0[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) c0[w] = c[0][w];
#pragma unroll
        for (int rb = 0; rb + 1 < RBN; ++rb)
#pragma unroll
            for (int w = 0; w < 4; ++w) c[rb][w] = c[rb + 1][w];
#pragma unroll
        for (int w = 0; w < 4; ++w) c[RBN - 1][w] = c0[w];
    }
};

// Layer-sum pass 2 (LS): a unit is one key range of kLsKeys keys of one
// (b, KV head) in a group of a.lg consecutive layers; its work-group walks the
// group's layers over that range (the unit's slices) and keeps each key's sum
// over them in LDS, one slot per lane and key (no other lane touches it), so
// that raw holds one row per layer group instead of one per layer.
constexpr int kLsChunks = 32;
constexpr int kLsKeys = kLsChunks * kChunk;  // 8192 keys, 32 KB of LDS sums

// Position in a work-group's sequence of chunks.
struct Cursor {
    int seg;    // segment index: slab * spp + part, or with LS unit * lg + slice
    int first;  // first key of the chunk
    int end;    // end of the segment's key range
    int slab;   // the segment's slab
    int base;   // LS: the segment's first key
    int out;    // LS: raw row of the unit (layer group * B*Hkv + b*Hkv + g)
    int lsm;    // LS: bit 0 the group's first layer, bit 1 its last
};

template <bool LS>
__device__ __forceinline__ bool seg_range(const StreamArgs& a, int seg, Cursor& c) {
    int part;
    c.seg = seg;
    if constexpr (LS) {
        // seg = unit * lg + slice, unit = (grp * B*Hkv + bg) * spp + part, layer = grp * lg + slice
        const int unit = seg / a.lg, sl = seg - unit * a.lg;
        const int gb = unit / a.spp;
        part = unit - gb * a.spp;
        const int BH = a.B * a.Hkv;
        const int grp = gb / BH, bg = gb - grp * BH;
        const int l = grp * a.lg + sl;
        if (l >= a.n_lyr) return false;  // the last group holds fewer layers
        c.slab = l * BH + bg;
        c.out = gb;
        c.lsm = (sl == 0 ? 1 : 0) | (sl == a.lg - 1 || l == a.n_lyr - 1 ? 2 : 0);
    } else {
        c.slab = seg / a.spp;
        part = seg - c.slab * a.spp;
        c.out = 0;
        c.lsm = 0;
    }
    c.first = part * a.seg_len;
    c.base = c.first;
    c.end = min(c.first + a.seg_len, a.n_range);
    return c.first < c.end;
}

// The chunk after c in this work-group's sequence; seg = -1 when there is none.
template <bool LS>
__device__ __forceinline__ Cursor advance(const StreamArgs& a, Cursor c) {
    if (c.first + kChunk < c.end) {
        c.first += kChunk;
        return c;
    }
    Cursor n;
    if constexpr (LS) {
        // the unit's next slice, else this work-group's next unit
        int seg = c.seg + 1;
        for (;;) {
            if (seg % a.lg == 0) seg += ((int)gridDim.x - 1) * a.lg;
            if (seg >= a.n_seg) break;
            if (seg_range<true>(a, seg, n)) return n;
            seg = (seg / a.lg + 1) * a.lg;  // past the last layer: the unit is done
        }
    } else {
        for (int seg = c.seg + (int)gridDim.x; seg < a.n_seg; seg += gridDim.x)
            if (seg_range<false>(a, seg, n)) return n;
    }
    n.seg = -1;
    return n;
}

// Slabs are [T][S0]: head group t = slab / S0 of the (layer, b, KV head)
// slab s0 = slab % S0 (s0 = (l*B + b)*Hkv + g) holds query heads
// g*G + t*Gs + (0 .. slab_rows/w - 1).
__device__ __forceinline__ const uint16_t* slab_keys(const StreamArgs& a, int slab) {
    const int s0 = slab % a.S0;
    const int g = s0 % a.Hkv;
    const int b = (s0 / a.Hkv) % a.B;
    const int l = s0 / (a.Hkv * a.B);
    return a.k + l * a.ks[0] + b * a.ks[1] + g * a.ks[2];
}

__device__ __forceinline__ int slab_rows(const StreamArgs& a, int slab) {
    return min(a.Gs, a.G - slab / a.S0 * a.Gs) * a.w;
}

// This wave's 64 keys of a chunk as operand fragments: lane (col, hf) reads
// elements ks*16 + hf*8 .. +7 of key kbase + kb*32 + col (clamped to the last key).
template <int D>
__device__ __forceinline__ void load_chunk(Frag<D>& f, const StreamArgs& a, const Cursor& c, int wave, int col,
                                           int hf) {
    const uint16_t* kslab = slab_keys(a, c.slab);
    const int kbase = c.first + wave * kWaveKeys;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
        const int j = min(kbase + kb * 32 + col, a.N - 1);
        const uint16_t* row = kslab + (int64_t)j * a.ks[3] + hf * 8;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            f.v[kb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(row + ks * 16));
    }
}

template <int D, int RBN, bool ST>
struct Smem {
    static constexpr int RP = RBN * 32;
    static constexpr int QST = D + 8;  // LDS row stride in elements (16 bytes of padding)
    static constexpr int SP = ST ? RP : 1;
    using State = typename std::conditional<ST, float4, float2>::type;
    uint16_t q[RP * QST];
    State st[kWaves][RP];     // pass 1: running (reference, sum[, s, q]) per wave and row
    float lse[RP];            // pass 2: row LSE2 (+inf on padded rows)
    uint32_t cnt[kWaves][SP]; // pass 2 with ST: per wave and row, keys counted so far
};

// Stage the query rows of a segment's slab (row r -> head g*G + r/w, window
// index r%w; rows past R are zero) and reset or load the per-row state. The
// rows pass through registers kStageLoads 16-byte loads per thread at a time,
// which keeps this code (run once per segment) clear of the registers that
// hold the next chunk's keys.
constexpr int kStageLoads = 4;
// Pass 2 merges the partials as it stages a slab while that costs each
// thread at most this many of them (and without layer sums); otherwise a
// merge launch runs first.
constexpr int kStageMerge = 16;

// Pass 2 of the two-pass call with a.spp1 > 0 also merges the slab's pass-1
// partials into its row LSEs here (no merge launch): 256/RP threads per row,
// each over every (256/RP)-th segment, their states merged across adjacent
// lanes; the work-group staging key range 0 of the slab (`first`) also writes
// the rows' natural-log LSE where the caller asked for it.
template <int D, int RBN, int PASS, bool ST>
__device__ void stage(Smem<D, RBN, ST>& sm, const StreamArgs& a, int slab, int tid, bool first) {
    constexpr int RP = RBN * 32;
    constexpr int QST = D + 8;
    constexpr int CPK = D / 8;  // 16-byte chunks per row
    constexpr int QPER = (RP * CPK + 255) / 256;
    const int s0 = slab % a.S0;
    const int g = s0 % a.Hkv;
    const int b = (s0 / a.Hkv) % a.B;
    const int l = s0 / (a.Hkv * a.B);
    const int h0 = g * a.G + slab / a.S0 * a.Gs;  // the head group's first query head
    const int rows = slab_rows(a, slab);
    const uint16_t* qbase = a.q + l * a.qs[0] + b * a.qs[1];
    __syncthreads();  // every wave is done with the previous segment's rows
    if (PASS == 1) {
        if constexpr (ST) {
            for (int i = tid; i < kWaves * RP; i += 256) (&sm.st[0][0])[i] = make_float4(kNegBig, 0.f, 0.f, 0.f);
        } else {
            for (int i = tid; i < kWaves * RP; i += 256) (&sm.st[0][0])[i] = make_float2(kNegBig, 0.f);
        }
    } else if (!ST && a.spp1 > 0) {
        constexpr int NSUB = 256 / RP;
        const int row = tid / NSUB, sub = tid % NSUB;
        float M = kNegBig, Z = 0.f;
        if (row < rows) {
            const float2* pp = a.part + (int64_t)slab * a.spp1 * RP + row;
#pragma unroll 4
            for (int p = sub; p < a.spp1; p += NSUB) {
                const float2 v = pp[(int64_t)p * RP];
                merge(M, Z, v.x, v.y);
            }
        }
#pragma unroll
        for (int off = 1; off < NSUB; off <<= 1) {
            const float om = __shfl_xor(M, off), oz = __shfl_xor(Z, off);
            merge(M, Z, om, oz);
        }
        if (sub == 0) {
            const float l2 = row < rows ? M + log2f(Z) : INFINITY;
            sm.lse[row] = l2;
            if (first && a.lse_out && row < rows)
                a.lse_out[(((int64_t)l * a.B + b) * a.Hq + h0 + row / a.w) * a.w + row % a.w] =
                    l2 * 0.69314718055994530942f;
        }
    } else {
        for (int row = tid; row < RP; row += 256) {
            const float l2 = row < rows ? a.lse2[(int64_t)slab * RP + row] : INFINITY;
            sm.lse[row] = l2;
        }
        if constexpr (ST)
            for (int i = tid; i < kWaves * RP; i += 256) (&sm.cnt[0][0])[i] = 0u;
    }
#pragma unroll 1
    for (int u0 = 0; u0 < QPER; u0 += kStageLoads) {
        uint4 qv[kStageLoads];
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int idx = tid + (u0 + u) * 256;
            const int row = idx / CPK;
            const int ch = idx - row * CPK;
            qv[u] = make_uint4(0u, 0u, 0u, 0u);
            if (u0 + u < QPER && row < rows) {
                const int h = h0 + row / a.w;
                const int i = row % a.w;
                qv[u] = *reinterpret_cast<const uint4*>(qbase + h * a.qs[2] + i * a.qs[3] + ch * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < kStageLoads; ++u) {
            const int idx = tid + (u0 + u) * 256;
            const int row = idx / CPK;
            const int ch = idx - row * CPK;
            if (u0 + u < QPER && row < RP) *reinterpret_cast<uint4*>(sm.q + row * QST + ch * 8) = qv[u];
        }
    }
    __syncthreads();
}

// Pass 1 on one chunk: merge this wave's (reference, sum) of every row into
// its running state (registers without statistics, LDS with them).
template <int D, int RBN, bool ST>
__device__ __forceinline__ void pass1_chunk(Smem<D, RBN, ST>& sm, const StreamArgs& a, const Frag<D>& f,
                                            const Cursor& c, int wave, int col, int hf, RowState<RBN>& rs) {
    constexpr int KS = D / 16;
    constexpr int QST = D + 8;
    const int kbase = c.first + wave * kWaveKeys;
    if (kbase >= a.N) return;  // the chunk ends before this wave's keys
    const bool edge = kbase + kWaveKeys > a.Np;  // reaches the window (causal mask) or the end
    const int rows = slab_rows(a, c.slab);
    const int rbn = (rows + 31) >> 5;  // row blocks holding this slab's rows
    if constexpr (!ST) {
        if (!edge) {
            // interior chunk: the row-block loop unrolled, each block's state in its own slot
            // (512K workload: 3-6% faster per score call than the rotating slots below)
#pragma unroll
            for (int rb = 0; rb < RBN; ++rb) {
                if (rb >= rbn) break;
                bf16x8 qf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qf[ks] = *reinterpret_cast<const bf16x8*>(sm.q + (rb * 32 + col) * QST + ks * 16 + hf * 8);
                // lane holds row rb*32 + col and keys kbase + kb*32 + tile_row(v, hf);
                // summed on the running reference, the block just adds to the running sum
                float m;
                float z = pass1_fast<D, kKB>(f.v, qf, a.c, rs.m[rb], m);
                if (__any(!(z < kOverflow))) {
                    z = pass1_max<D, kKB, false>(f.v, qf, a.c, kbase, hf, 0, m);
                    merge(rs.m[rb], rs.z[rb], m, z);
                } else {
                    rs.z[rb] = rs.m[rb] > kNegBig ? rs.z[rb] + z : z;
                    rs.m[rb] = m;
                }
            }
            return;
        }
        // the chunk reaching the causal window (one per segment at most): a rolled loop over
        // rotating slots keeps the masked variant's code out of the unrolled one
#pragma unroll 1
        for (int rb = 0; rb < rbn; ++rb) {
            bf16x8 qf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ks] = *reinterpret_cast<const bf16x8*>(sm.q + (rb * 32 + col) * QST + ks * 16 + hf * 8);
            const int row = rb * 32 + col;
            const int lim = row < rows ? a.Np + row % a.w : -1;
            float m;
            const float z = pass1_max<D, kKB, true>(f.v, qf, a.c, kbase, hf, lim, m);
            merge(rs.m[0], rs.z[0], m, z);
            rs.rotate();
        }
        for (int rb = rbn; rb < RBN; ++rb) rs.rotate();
        return;
    }
#pragma unroll 1
    for (int rb = 0; rb < rbn; ++rb) {
        bf16x8 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(sm.q + (rb * 32 + col) * QST + ks * 16 + hf * 8);
        // lane holds row rb*32 + col and keys kbase + kb*32 + tile_row(v, hf)
        float m, z;
        if constexpr (ST) {
            Moments mo;
            if (edge) {
                const int row = rb * 32 + col;
                const int lim = row < rows ? a.Np + row % a.w : -1;
                z = pass1_max_st<D, kKB, true>(f.v, qf, a.c, kbase, hf, lim, m, mo);
            } else {
                z = pass1_fast_st<D, kKB>(f.v, qf, a.c, m, mo);
                if (__any(!(z < kOverflowSt))) z = pass1_max_st<D, kKB, false>(f.v, qf, a.c, kbase, hf, 0, m, mo);
            }
            merge_st(m, z, mo, __shfl_xor(m, 32), __shfl_xor(z, 32),
                     Moments{__shfl_xor(mo.s, 32), __shfl_xor(mo.q, 32)});
            if (hf == 0) {
                float4 st = sm.st[wave][rb * 32 + col];
                Moments sa{st.z, st.w};
                merge_st(st.x, st.y, sa, m, z, mo);
                sm.st[wave][rb * 32 + col] = make_float4(st.x, st.y, sa.s, sa.q);
            }
        }
    }
}

// Pass 2 on one chunk: raw score of each of this wave's prefix keys (with LS
// added to the key's sum over the layer group, stored at the group's last).
template <int D, int RBN, bool ST, bool LS>
__device__ __forceinline__ void pass2_chunk(Smem<D, RBN, ST>& sm, float* lsum, const StreamArgs& a,
                                            const Frag<D>& f, const Cursor& c, int wave, int col, int hf,
                                            CountState<RBN>& cn) {
    constexpr int KS = D / 16;
    constexpr int QST = D + 8;
    const int kbase = c.first + wave * kWaveKeys;
    if (kbase >= a.n_range) return;  // no keys of this pass in this wave's range
    const int slab = c.slab;
    const int rows = slab_rows(a, slab);
    const int rbn = (rows + 31) >> 5;  // row blocks holding this slab's rows
    float cs[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) cs[kb] = 0.f;
#pragma unroll 1
    for (int rb = 0; rb < rbn; ++rb) {
        bf16x8 qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = *reinterpret_cast<const bf16x8*>(sm.q + (rb * 32 + col) * QST + ks * 16 + hf * 8);
        float lr[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 t = *reinterpret_cast<const float4*>(sm.lse + rb * 32 + 8 * u + 4 * hf);
            lr[4 * u] = t.x;
            lr[4 * u + 1] = t.y;
            lr[4 * u + 2] = t.z;
            lr[4 * u + 3] = t.w;
        }
        // lane holds key kbase + kb*32 + col and rows rb*32 + tile_row(v, hf)
        f32x16 x[kKB];
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) x[kb] = logits<KS>(qf, f.v[kb]);
        if constexpr (!ST) {
#pragma unroll
            for (int kb = 0; kb < kKB; ++kb) {
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    s0 += fexp2(x[kb][v] * a.c - lr[v]);
                    s1 += fexp2(x[kb][v + 1] * a.c - lr[v + 1]);
                }
                cs[kb] += s0 + s1;
            }
        } else {
            // the same exponent decides the count: p < small_p  <=>  c*x - LSE2 < log2(small_p);
            // a key past the causal limit of the row (or past N) is not counted
            const bool edge = kbase + kWaveKeys > a.Np;  // reaches the window (causal mask) or the end
            if (!edge) {  // every key of the chunk is visible to every row
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb) {
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; v += 2) {
                        const float t0 = x[kb][v] * a.c - lr[v];
                        const float t1 = x[kb][v + 1] * a.c - lr[v + 1];
                        s0 += fexp2(t0);
                        s1 += fexp2(t1);
                        cn.c[0][v >> 2] += ((uint32_t)(t0 < a.l2tau) << (8 * (v & 3))) +
                                           ((uint32_t)(t1 < a.l2tau) << (8 * ((v + 1) & 3)));
                    }
                    cs[kb] += s0 + s1;
                }
            } else {
#pragma unroll
                for (int kb = 0; kb < kKB; ++kb) {
                    const int j = kbase + kb * 32 + col;
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; v += 2) {
                        const float t0 = x[kb][v] * a.c - lr[v];
                        const float t1 = x[kb][v + 1] * a.c - lr[v + 1];
                        s0 += fexp2(t0);
                        s1 += fexp2(t1);
                        const int r0 = rb * 32 + tile_row(v, hf), r1 = rb * 32 + tile_row(v + 1, hf);
                        const bool in0 = r0 < rows && j <= a.Np + r0 % a.w;
                        const bool in1 = r1 < rows && j <= a.Np + r1 % a.w;
                        cn.c[0][v >> 2] += ((uint32_t)(in0 && t0 < a.l2tau) << (8 * (v & 3))) +
                                           ((uint32_t)(in1 && t1 < a.l2tau) << (8 * ((v + 1) & 3)));
                    }
                    cs[kb] += s0 + s1;
                }
            }
            cn.rotate();
        }
    }
    if constexpr (ST)
        for (int rb = rbn; rb < RBN; ++rb) cn.rotate();
    // one store per wave and chunk: lane half hf writes key block hf, 64
    // consecutive raw scores (two half-wave stores measured about 1% slower on
    // the 128K workload; without any store the pass would be about 4% faster)
    static_assert(kKB == 2, "one key block per lane half");
    const float v0 = cs[0] + __shfl_xor(cs[0], 32);
    const float v1 = cs[1] + __shfl_xor(cs[1], 32);
    const int j = kbase + hf * 32 + col;
    const float val = (hf ? v1 : v0) * a.invG;
    if constexpr (LS) {
        float* p = lsum + (j - c.base);  // this lane's slot for key j
        if (c.lsm & 2) {
            if (j < a.Np) a.raw[(int64_t)c.out * a.Np + j] = ((c.lsm & 1) ? 0.f : *p) + val;
        } else {
            *p = (c.lsm & 1) ? val : *p + val;
        }
    } else if (j < a.Np) {
        a.raw[(int64_t)slab * a.Np + j] = val;
    }
}

// Pass 1, end of a segment: merge the waves' states and publish the partials.
template <int D, int RBN, bool ST>
__device__ __forceinline__ void pass1_finish(Smem<D, RBN, ST>& sm, const StreamArgs& a, int seg, int tid,
                                             RowState<RBN>& rs) {
    constexpr int RP = RBN * 32;
    if constexpr (!ST) {
        // the two lane halves (same row, other keys), then this wave's row states to LDS
        const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
        for (int rb = 0; rb < RBN; ++rb) {
            float m = rs.m[rb], z = rs.z[rb];
            merge(m, z, __shfl_xor(m, 32), __shfl_xor(z, 32));
            if (lane < 32) sm.st[wave][rb * 32 + lane] = make_float2(m, z);
        }
        rs.reset();
    }
    __syncthreads();
    for (int row = tid; row < RP; row += 256) {
        if constexpr (ST) {
            float4 acc = sm.st[0][row];
            Moments ma{acc.z, acc.w};
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2) {
                const float4 o = sm.st[w2][row];
                merge_st(acc.x, acc.y, ma, o.x, o.y, Moments{o.z, o.w});
            }
            a.part4[(int64_t)seg * RP + row] = make_float4(acc.x, acc.y, ma.s, ma.q);
        } else {
            float2 acc = sm.st[0][row];
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2) merge(acc.x, acc.y, sm.st[w2][row].x, sm.st[w2][row].y);
            a.part[(int64_t)seg * RP + row] = acc;
        }
    }
}

// Pass 2 with ST, end of a segment: each field summed over the 32 lanes of its
// lane half (keys) into the wave's per-row count in LDS, then cleared.
template <int D, int RBN>
__device__ __forceinline__ void count_flush(Smem<D, RBN, true>& sm, int wave, int col, int hf, CountState<RBN>& cn) {
#pragma unroll
    for (int rb = 0; rb < RBN; ++rb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t lo = cn.c[rb][w] & 0x00FF00FFu;         // fields of v = 4w and 4w + 2
            uint32_t hi = (cn.c[rb][w] >> 8) & 0x00FF00FFu;  // fields of v = 4w + 1 and 4w + 3
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) {
                lo += __shfl_xor(lo, off);
                hi += __shfl_xor(hi, off);
            }
            if (col == 0) {
                sm.cnt[wave][rb * 32 + tile_row(4 * w, hf)] += lo & 0xFFFFu;
                sm.cnt[wave][rb * 32 + tile_row(4 * w + 1, hf)] += hi & 0xFFFFu;
                sm.cnt[wave][rb * 32 + tile_row(4 * w + 2, hf)] += lo >> 16;
                sm.cnt[wave][rb * 32 + tile_row(4 * w + 3, hf)] += hi >> 16;
            }
        }
    cn.reset();
}

// Pass 2 with ST, end of a segment: the waves' counts of every row.
template <int D, int RBN>
__device__ __forceinline__ void pass2_finish(Smem<D, RBN, true>& sm, const StreamArgs& a, int seg, int tid) {
    constexpr int RP = RBN * 32;
    __syncthreads();
    for (int row = tid; row < RP; row += 256) {
        uint32_t n = 0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) n += sm.cnt[w2][row];
        a.cnt_part[(int64_t)seg * RP + row] = n;
    }
}

// One chunk with its keys in `f` while the next chunk's keys load into `g`.
// Returns false once the work-group's sequence ends.
template <int D, int RBN, int PASS, bool ST, bool LS>
__device__ __forceinline__ bool step(Smem<D, RBN, ST>& sm, float* lsum, const StreamArgs& a, Cursor& cur,
                                     Frag<D>& f, Frag<D>& g, int tid, int wave, int col, int hf, RowState<RBN>& rs,
                                     CountState<RBN>& cn) {
    const Cursor nx = advance<LS>(a, cur);
    // Issued on every step (the last one re-reads the current chunk): with a
    // fixed number of loads in flight the wait for `f` leaves `g`'s in flight.
    load_chunk<D>(g, a, nx.seg >= 0 ? nx : cur, wave, col, hf);
    if (PASS == 1)
        pass1_chunk<D, RBN, ST>(sm, a, f, cur, wave, col, hf, rs);
    else
        pass2_chunk<D, RBN, ST, LS>(sm, lsum, a, f, cur, wave, col, hf, cn);
    if (nx.seg != cur.seg) {
        if (PASS == 1) pass1_finish<D, RBN, ST>(sm, a, cur.seg, tid, rs);
        if constexpr (ST && PASS == 2) {
            count_flush<D, RBN>(sm, wave, col, hf, cn);
            pass2_finish<D, RBN>(sm, a, cur.seg, tid);
        }
        if (nx.seg < 0) return false;
        stage<D, RBN, PASS, ST>(sm, a, nx.slab, tid, nx.base == 0);
    }
    cur = nx;
    return true;
}

// The kernel's LDS: the passes' own, and with LS the layer group's key sums.
template <int D, int RBN, bool ST, bool LS>
struct SmemK : Smem<D, RBN, ST> {
    float lsum[LS ? kLsKeys : 1];
};

template <int D, int RBN, int PASS, bool ST, bool LS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
stream_kernel(StreamArgs a) {
    __shared__ __attribute__((aligned(16))) SmemK<D, RBN, ST, LS> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps chunk bounds scalar
    const int col = lane & 31;
    const int hf = lane >> 5;

    // the first segment of this work-group's first unit (LS: a unit's first
    // slice always holds a layer) or its first segment with keys
    const int lg = LS ? a.lg : 1;
    Cursor cur;
    bool found = false;
    for (int seg = blockIdx.x * lg; seg < a.n_seg && !found; seg += gridDim.x * lg)
        found = seg_range<LS>(a, seg, cur);
    if (!found) return;
    Frag<D> fa, fb;
    RowState<RBN> rs;
    rs.reset();
    CountState<RBN> cn;
    cn.reset();
    load_chunk<D>(fa, a, cur, wave, col, hf);
    stage<D, RBN, PASS, ST>(sm, a, cur.slab, tid, cur.base == 0);

    for (;;) {
        if (!step<D, RBN, PASS, ST, LS>(sm, sm.lsum, a, cur, fa, fb, tid, wave, col, hf, rs, cn)) break;
        if (!step<D, RBN, PASS, ST, LS>(sm, sm.lsum, a, cur, fb, fa, tid, wave, col, hf, rs, cn)) break;
    }
}

// Rows of a slab and where its row statistics go: slab = t*S0 + s0 with
// s0 = (l*B + b)*Hkv + g, row r -> query head g*G + t*Gs + r/w, window
// index r%w, output index ((l*B + b)*Hq + head)*w + r%w.
struct RowMap {
    int w, B, Hq, Hkv, G, S0, Gs;
    __device__ int rows(int slab) const { return min(Gs, G - slab / S0 * Gs) * w; }
    __device__ int64_t out(int slab, int row) const {
        const int s0 = slab % S0;
        const int g = s0 % Hkv;
        const int b = (s0 / Hkv) % B;
        const int l = s0 / (Hkv * B);
        const int h = g * G + slab / S0 * Gs + row / w;
        return (((int64_t)l * B + b) * Hq + h) * w + row % w;
    }
};

RowMap row_map(const StreamArgs& a) { return RowMap{a.w, a.B, a.Hq, a.Hkv, a.G, a.S0, a.Gs}; }

// The merge kernels below take blocks of 256 threads over RQ rows of a slab
// each (grid: slabs x row tiles): RQ is the power of two at or above the
// slab's row count, at most 32, and thread t takes row t % RQ of the tile and
// every (256/RQ)-th segment from t / RQ on. A wave reads consecutive rows of
// a segment, a long segment list is spread over at least 8 threads per row,
// and the per-thread states then merge through LDS.
constexpr int kMergeRows = 32;

__device__ __forceinline__ int row_span(int R) {
    int q = 1;
    while (q < R && q < kMergeRows) q <<= 1;
    return q;
}

dim3 merge_grid(const StreamArgs& a) { return dim3((unsigned)a.S, (unsigned)((a.R + kMergeRows - 1) / kMergeRows)); }

// Row LSE2 of every slab from its segments' partials; padded rows are left
// alone (pass 2 stages +inf for them).
__global__ __launch_bounds__(256) void stream_merge_kernel(const float2* part, int spp, int rp, RowMap m, float* lse2,
                                                           float* lse_out) {
    __shared__ float2 red[256];
    const int slab = blockIdx.x;
    const int R = m.rows(slab);
    const int rq = row_span(R), nsub = 256 / rq;
    if ((int)blockIdx.y * rq >= R) return;  // the whole tile is past this slab's rows
    const int row = blockIdx.y * rq + threadIdx.x % rq, sub = threadIdx.x / rq;
    float M = kNegBig, Z = 0.f;
    if (row < R)
#pragma unroll 4
        for (int p = sub; p < spp; p += nsub) {
            const float2 v = part[((int64_t)slab * spp + p) * rp + row];
            merge(M, Z, v.x, v.y);
        }
    red[threadIdx.x] = make_float2(M, Z);
    __syncthreads();
    if (sub == 0 && row < R) {
        for (int s2 = 1; s2 < nsub; ++s2) {
            const float2 o = red[s2 * rq + threadIdx.x % rq];
            merge(M, Z, o.x, o.y);
        }
        const float l2 = M + log2f(Z);
        lse2[(int64_t)slab * rp + row] = l2;
        if (lse_out) lse_out[m.out(slab, row)] = l2 * 0.69314718055994530942f;
    }
}

// ST merge: row LSE2 as above, plus the row's entropy
// -sum p ln p = ln2 * (LSE2 - c * sum p*x) and sum p^2 = q / z^2.
__global__ __launch_bounds__(256) void stream_merge_st_kernel(const float4* part, int spp, int rp, RowMap m, float c,
                                                              float* lse2, float* lse_out, float* entropy,
                                                              float* sum_p2) {
    __shared__ float4 red[256];
    const int slab = blockIdx.x;
    const int R = m.rows(slab);
    const int rq = row_span(R), nsub = 256 / rq;
    if ((int)blockIdx.y * rq >= R) return;  // the whole tile is past this slab's rows
    const int row = blockIdx.y * rq + threadIdx.x % rq, sub = threadIdx.x / rq;
    float M = kNegBig, Z = 0.f;
    Moments mo{0.f, 0.f};
    if (row < R)
#pragma unroll 4
        for (int p = sub; p < spp; p += nsub) {
            const float4 v = part[((int64_t)slab * spp + p) * rp + row];
            merge_st(M, Z, mo, v.x, v.y, Moments{v.z, v.w});
        }
    red[threadIdx.x] = make_float4(M, Z, mo.s, mo.q);
    __syncthreads();
    if (sub == 0 && row < R) {
        for (int s2 = 1; s2 < nsub; ++s2) {
            const float4 o = red[s2 * rq + threadIdx.x % rq];
            merge_st(M, Z, mo, o.x, o.y, Moments{o.z, o.w});
        }
        const float l2 = M + log2f(Z);
        lse2[(int64_t)slab * rp + row] = l2;
        const int64_t o = m.out(slab, row);
        constexpr float kLn2 = 0.69314718055994530942f;
        if (lse_out) lse_out[o] = l2 * kLn2;
        entropy[o] = kLn2 * (l2 - c * (mo.s / Z));
        sum_p2[o] = mo.q / (Z * Z);
    }
}

// ST: every row's count of keys below the threshold, summed over segments.
__global__ __launch_bounds__(256) void stream_count_kernel(const uint32_t* cnt_part, int spp, int rp, RowMap m,
                                                           int32_t* n_below) {
    __shared__ uint32_t red[256];
    const int slab = blockIdx.x;
    const int R = m.rows(slab);
    const int rq = row_span(R), nsub = 256 / rq;
    if ((int)blockIdx.y * rq >= R) return;  // the whole tile is past this slab's rows
    const int row = blockIdx.y * rq + threadIdx.x % rq, sub = threadIdx.x / rq;
    uint32_t n = 0;
    if (row < R)
        for (int p = sub; p < spp; p += nsub) n += cnt_part[((int64_t)slab * spp + p) * rp + row];
    red[threadIdx.x] = n;
    __syncthreads();
    if (sub == 0 && row < R) {
        for (int s2 = 1; s2 < nsub; ++s2) n += red[s2 * rq + threadIdx.x % rq];
        n_below[m.out(slab, row)] = (int32_t)n;
    }
}

typedef void (*stream_fn)(StreamArgs);

template <int D, int PASS, bool ST>
stream_fn pick_rbn(int RBN) {
    switch (RBN) {
        case 1: return stream_kernel<D, 1, PASS, ST, false>;
        case 2: return stream_kernel<D, 2, PASS, ST, false>;
        case 4: return stream_kernel<D, 4, PASS, ST, false>;
        case 8: return stream_kernel<D, 8, PASS, ST, false>;
        default: return nullptr;
    }
}

// Layer-sum pass 2: the instances whose LDS (query rows plus the 32 KB of key
// sums) leaves room for two work-groups per compute unit.
stream_fn pick_ls(int D, int RBN) {
    if (D == 128) {
        switch (RBN) {
            case 1: return stream_kernel<128, 1, 2, false, true>;
            case 2: return stream_kernel<128, 2, 2, false, true>;
            case 4: return stream_kernel<128, 4, 2, false, true>;
            default: return nullptr;
        }
    }
    switch (RBN) {
        case 1: return stream_kernel<64, 1, 2, false, true>;
        case 2: return stream_kernel<64, 2, 2, false, true>;
        case 4: return stream_kernel<64, 4, 2, false, true>;
        case 8: return stream_kernel<64, 8, 2, false, true>;
        default: return nullptr;
    }
}
static_assert(sizeof(SmemK<128, 4, false, true>) <= 80 * 1024 && sizeof(SmemK<64, 8, false, true>) <= 80 * 1024,
              "two layer-sum work-groups per compute unit");

stream_fn pick(int D, int RBN, int PASS, bool ST = false) {
    if (ST) {
        if (D == 128) return PASS == 1 ? pick_rbn<128, 1, true>(RBN) : pick_rbn<128, 2, true>(RBN);
        return PASS == 1 ? pick_rbn<64, 1, true>(RBN) : pick_rbn<64, 2, true>(RBN);
    }
    if (D == 128) return PASS == 1 ? pick_rbn<128, 1, false>(RBN) : pick_rbn<128, 2, false>(RBN);
    return PASS == 1 ? pick_rbn<64, 1, false>(RBN) : pick_rbn<64, 2, false>(RBN);
}

int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segments per slab for `keys` keys, each a whole number of chunks: as few
// as keep every segment within kMaxSegChunks, at most m per work-group slot
// of the grid in total for the smallest such m (m = 1 unless the slabs are
// long), so that no work-group stages a slab's rows more often than it must
// and none takes an extra full segment.
void segments(int64_t keys, int64_t S, int n_wg, int& spp, int& seg_len) {
    const int64_t chunks = (keys + kChunk - 1) / kChunk;
    int64_t per = chunks;  // chunks per segment
    for (int64_t m = 1;; ++m) {
        int64_t want = m * n_wg / S;
        if (want > chunks) want = chunks;
        if (want < 1) want = 1;
        per = (chunks + want - 1) / want;
        if (per <= kMaxSegChunks || want == chunks) break;
    }
    if (per > kMaxSegChunks) per = kMaxSegChunks;
    seg_len = (int)(per * kChunk);
    spp = (int)((keys + seg_len - 1) / seg_len);
    if (spp < 1) spp = 1;
}

}  // namespace

bool stream_plan(int dtype, int head_dim, int R, int64_t N, int64_t Np, int64_t S, int n_cu, StreamPlan& plan) {
    plan.ok = false;
    if (dtype != KVSEL_DTYPE_BF16 || (head_dim != 64 && head_dim != 128)) return false;
    if (R < 1 || R > 256 || N < 1 || S < 1 || n_cu < 1) return false;
    plan.head_dim = head_dim;
    plan.rbn = (R + 31) / 32;
    plan.rbn_cap = pow2_at_least(plan.rbn);
    plan.rp = plan.rbn_cap * 32;
    plan.n_wg = 2 * n_cu;
    segments(N, S, plan.n_wg, plan.spp1, plan.seg_len1);
    segments(Np > 0 ? Np : 1, S, plan.n_wg, plan.spp2, plan.seg_len2);
    plan.part_off = 0;  // float2 partials, or float4 with the pivot statistics
    plan.cnt_off = align256((size_t)S * plan.spp1 * plan.rp * sizeof(float4));
    plan.lse2_off = align256(plan.cnt_off + (size_t)S * plan.spp1 * plan.rp * sizeof(uint32_t));
    plan.raw_off = align256(plan.lse2_off + (size_t)S * plan.rp * sizeof(float));
    plan.ok = pick(head_dim, plan.rbn_cap, 1) != nullptr;
    return plan.ok;
}

hipError_t launch_stream(const StreamPlan& plan, StreamArgs a, float* lse_out, hipStream_t st) {
    stream_fn f1 = pick(plan.head_dim, plan.rbn_cap, 1);
    stream_fn f2 = pick(plan.head_dim, plan.rbn_cap, 2);
    if (!f1 || !f2) return hipErrorInvalidValue;
    // pass 1 over every key (window included)
    a.spp = plan.spp1;
    a.seg_len = plan.seg_len1;
    a.n_range = a.N;
    a.n_seg = a.S * plan.spp1;
    hipLaunchKernelGGL(f1, dim3((unsigned)(a.n_seg < plan.n_wg ? a.n_seg : plan.n_wg)), dim3(256), 0, st, a);
    if ((int64_t)plan.spp1 * plan.rp <= 256 * kStageMerge && a.Np > 0 && a.lg == 0) {
        // pass 2 merges each slab's partials itself as it stages the slab (not
        // with layer sums: a work-group restages there every 32 chunks, and the
        // merges then cost what the launch saves)
        a.spp1 = plan.spp1;
        a.lse_out = lse_out;
    } else {
        hipLaunchKernelGGL(stream_merge_kernel, merge_grid(a), dim3(256), 0, st, a.part, plan.spp1, plan.rp,
                           row_map(a), a.lse2, lse_out);
    }
    return launch_stream_pass2(plan, a, st);
}

hipError_t launch_stream_stats(const StreamPlan& plan, StreamArgs a, float* lse_out, float* entropy, float* sum_p2,
                               int32_t* n_below, hipStream_t st) {
    stream_fn f1 = pick(plan.head_dim, plan.rbn_cap, 1, true);
    stream_fn f2 = pick(plan.head_dim, plan.rbn_cap, 2, true);
    if (!f1 || !f2) return hipErrorInvalidValue;
    // both passes over every key: pass 2 also counts the window keys each row sees
    a.spp = plan.spp1;
    a.seg_len = plan.seg_len1;
    a.n_range = a.N;
    a.n_seg = a.S * plan.spp1;
    const unsigned grid = (unsigned)(a.n_seg < plan.n_wg ? a.n_seg : plan.n_wg);
    hipLaunchKernelGGL(f1, dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL(stream_merge_st_kernel, merge_grid(a), dim3(256), 0, st, a.part4, plan.spp1, plan.rp,
                       row_map(a), a.c, a.lse2, lse_out, entropy, sum_p2);
    hipLaunchKernelGGL(f2, dim3(grid), dim3(256), 0, st, a);
    hipLaunchKernelGGL(stream_count_kernel, merge_grid(a), dim3(256), 0, st, a.cnt_part, plan.spp1, plan.rp,
                       row_map(a), n_below);
    return hipGetLastError();
}

int stream_layer_groups(const StreamPlan& plan, StreamArgs& a, int L) {
    a.lg = 0;
    a.n_lyr = L;
    if (L < 2 || a.T != 1 || a.Np <= 0 || !pick_ls(plan.head_dim, plan.rbn_cap)) return L * a.T;
    // as many layers per group as leave every work-group slot of the grid a unit
    const int64_t per_group = (int64_t)a.B * a.Hkv * ((a.Np + kLsKeys - 1) / kLsKeys);
    const int64_t n_groups = (plan.n_wg + per_group - 1) / per_group;
    if (n_groups >= L) return L;  // one layer per unit: the per-layer pass does the same work
    a.lg = (int)((L + n_groups - 1) / n_groups);
    return (L + a.lg - 1) / a.lg;
}

hipError_t launch_stream_pass2(const StreamPlan& plan, StreamArgs a, hipStream_t st) {
    if (a.lg > 0 && a.Np > 0) {
        // layer sums: units of kLsKeys keys of one (b, KV head) over a group of a.lg layers
        stream_fn f2 = pick_ls(plan.head_dim, plan.rbn_cap);
        if (!f2) return hipErrorInvalidValue;
        a.seg_len = kLsKeys;
        a.spp = (a.Np + kLsKeys - 1) / kLsKeys;
        a.n_range = a.Np;
        const int n_groups = (a.n_lyr + a.lg - 1) / a.lg;
        const int units = n_groups * a.B * a.Hkv * a.spp;
        a.n_seg = units * a.lg;
        hipLaunchKernelGGL(f2, dim3((unsigned)(units < plan.n_wg ? units : plan.n_wg)), dim3(256), 0, st, a);
        return hipGetLastError();
    }
    stream_fn f2 = pick(plan.head_dim, plan.rbn_cap, 2);
    if (!f2) return hipErrorInvalidValue;
    // pass 2 over the prefix keys
    if (a.Np > 0) {
        a.spp = plan.spp2;
        a.seg_len = plan.seg_len2;
        a.n_range = a.Np;
        a.n_seg = a.S * plan.spp2;
        hipLaunchKernelGGL(f2, dim3((unsigned)(a.n_seg < plan.n_wg ? a.n_seg : plan.n_wg)), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace kvsel
