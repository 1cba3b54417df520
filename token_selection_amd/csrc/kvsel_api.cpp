// C ABI of libkvsel: argument validation, geometry, kernel dispatch.
//
// Every entry point validates its arguments on the host before enqueuing any
// work, so an error return means nothing was launched and nothing written.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "kvsel.h"
#include "kvsel_internal.h"

using kvsel::ScoreGeom;
using kvsel::ScoreWs;

namespace {

constexpr int64_t kMaxKeys = (int64_t)1 << 31;  // positions are int32 on the device

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kvsel_status_t validate_desc(const kvsel_score_desc_t* d) {
    if (!d) return KVSEL_ERR_INVALID_ARG;
    if (d->n_layers < 1 || d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1) return KVSEL_ERR_INVALID_ARG;
    if (d->n_q_heads % d->n_kv_heads != 0) return KVSEL_ERR_INVALID_ARG;
    if (d->window < 1 || d->n_keys < d->window || d->n_keys >= kMaxKeys) return KVSEL_ERR_INVALID_ARG;
    if (d->pool_kernel < 1 || d->pool_kernel % 2 == 0 || d->pool_kernel > 255) return KVSEL_ERR_INVALID_ARG;
    if ((int64_t)d->n_layers * d->batch * d->n_kv_heads > 65535) return KVSEL_ERR_INVALID_ARG;
    if ((int64_t)(d->n_q_heads / d->n_kv_heads) * d->window > (1 << 20)) return KVSEL_ERR_INVALID_ARG;
    if (!isfinite(d->softmax_scale)) return KVSEL_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
        if (d->q_strides[i] < 0 || d->k_strides[i] < 0) return KVSEL_ERR_INVALID_ARG;
    if (d->dtype != KVSEL_DTYPE_F32 && d->dtype != KVSEL_DTYPE_BF16) return KVSEL_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
    if (d->pool_type != KVSEL_POOL_AVG && d->pool_type != KVSEL_POOL_MAX) return KVSEL_ERR_UNSUPPORTED;
    if (d->path != KVSEL_PATH_AUTO && d->path != KVSEL_PATH_STREAM && d->path != KVSEL_PATH_GENERAL)
        return KVSEL_ERR_INVALID_ARG;
    if (d->reserved != 0) return KVSEL_ERR_INVALID_ARG;
    const int64_t e = d->dtype == KVSEL_DTYPE_F32 ? 4 : 2;
    for (int i = 0; i < 4; ++i)
        if ((d->q_strides[i] * e) % 16 != 0 || (d->k_strides[i] * e) % 16 != 0) return KVSEL_ERR_INVALID_ARG;
    return KVSEL_OK;
}

void make_geom(const kvsel_score_desc_t* d, ScoreGeom& g, int& RB) {
    g.L = d->n_layers;
    g.B = d->batch;
    g.Hq = d->n_q_heads;
    g.Hkv = d->n_kv_heads;
    g.G = d->n_q_heads / d->n_kv_heads;
    g.w = d->window;
    g.R = g.G * g.w;
    RB = kvsel::score_row_blocks(d->dtype, d->head_dim, g.R);
    const int nb = (g.R + 15) / 16;
    g.n_groups = (nb + RB - 1) / RB;
    g.Rpad = g.n_groups * RB * 16;
    g.S = g.L * g.B * g.Hkv;
    g.N = d->n_keys;
    g.Np = d->n_keys - d->window;
    // general path: halve the chunk until the grid has ~2 work-groups per
    // compute unit (or the chunk reaches its minimum)
    g.chunk = kvsel::kScoreChunk;
    while (g.chunk > kvsel::kScoreChunkMin && (int64_t)g.S * ((g.N + g.chunk - 1) / g.chunk) < 512) g.chunk >>= 1;
    g.n_chunks1 = (int32_t)((g.N + g.chunk - 1) / g.chunk);
    g.n_chunks2 = (int32_t)((g.Np + g.chunk - 1) / g.chunk);
    const double scale = d->softmax_scale > 0.f ? (double)d->softmax_scale : 1.0 / sqrt((double)d->head_dim);
    g.c = (float)(scale * 1.4426950408889634074);  // log2(e)
    g.invG = (float)(1.0 / (double)g.G);
    for (int i = 0; i < 4; ++i) {
        g.qs[i] = d->q_strides[i];
        g.ks[i] = d->k_strides[i];
    }
    g.q = nullptr;
    g.k = nullptr;
    g.part = nullptr;
    g.lse2 = nullptr;
    g.raw = nullptr;
    g.lse_out = nullptr;
    g.lse_in = nullptr;
}

ScoreWs ws_layout(const ScoreGeom& g) { return kvsel::score_workspace_layout(g.S, g.n_chunks1, g.Rpad, g.Np); }

// Compute units of the current device; 256 (MI355X) when no device answers,
// so that workspace queries also work on a host without a GPU.
int device_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return 256;
    }
    return n;
}

struct Plan {
    ScoreGeom g;
    int RB;
    ScoreWs gen;               // general two-pass layout (any dtype)
    kvsel::StreamPlan stream;  // streaming bf16 layout (stream.ok when eligible)
    int T, Gs;                 // streaming head groups: T groups of at most Gs query heads per KV head
    size_t stream_total, total;
};

size_t raw_bytes(int64_t S, int64_t Np) { return ((size_t)S * Np * sizeof(float) + 255) & ~(size_t)255; }
size_t raw_bytes(const ScoreGeom& g) { return raw_bytes(g.S, g.Np); }

// The streaming kernels hold at most 256 window rows per slab. Past that, a
// KV head's query heads split into T head groups of at most Gs heads each
// (Gs*w <= 256, sizes balanced), each streamed as a slab of its own over the
// same keys; their raw scores add up like extra layers.
void head_groups(const ScoreGeom& g, int& T, int& Gs) {
    T = 1;
    Gs = g.G;
    if (g.R <= 256 || g.w > 256) return;
    Gs = 256 / g.w;
    T = (g.G + Gs - 1) / Gs;
    Gs = (g.G + T - 1) / T;
}

void make_plan(const kvsel_score_desc_t* d, Plan& p) {
    make_geom(d, p.g, p.RB);
    p.gen = ws_layout(p.g);
    p.total = p.gen.total;
    const int n_cu = device_cu_count();
    p.stream_total = 0;
    head_groups(p.g, p.T, p.Gs);
    const int64_t S_groups = (int64_t)p.g.S * p.T;
    p.stream.ok = false;
    if (S_groups <= 65535 &&
        kvsel::stream_plan(d->dtype, d->head_dim, p.Gs * p.g.w, p.g.N, p.g.Np, S_groups, n_cu, p.stream)) {
        p.stream_total = p.stream.raw_off + raw_bytes(S_groups, p.g.Np);
        if (p.stream_total > p.total) p.total = p.stream_total;
    }
}

// Scoring path of a call: the descriptor's explicit choice, or for
// KVSEL_PATH_AUTO the streaming kernels wherever they apply (bf16, head_dim 64
// or 128, w <= 256), else the general kernels. -1: an explicit streaming
// choice on a shape the streaming kernels do not take.
int resolve_path(const kvsel_score_desc_t* d, const Plan& p) {
    if (d->path == KVSEL_PATH_GENERAL) return KVSEL_PATH_GENERAL;
    if (d->path == KVSEL_PATH_STREAM) return p.stream.ok ? KVSEL_PATH_STREAM : -1;
    return p.stream.ok ? KVSEL_PATH_STREAM : KVSEL_PATH_GENERAL;
}

kvsel_status_t from_hip(hipError_t e) { return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP; }

// Pivot-statistics outputs of kvsel_score_stats.
struct StatsOut {
    float small_p;
    float* entropy;
    float* sum_p2;
    int32_t* n_below;
};

// The scoring call. lse_in == null: both softmax passes (a1-a3). lse_in !=
// null: the row LSEs are handed in and only the second pass runs.
kvsel_status_t score_impl(const kvsel_score_desc_t* desc, const void* q_win, const void* k, float* scores,
                          int32_t accumulate, float* lse_out, const float* lse_in, void* workspace,
                          size_t workspace_bytes, void* stream, const StatsOut* stats = nullptr) {
    const kvsel_status_t st = validate_desc(desc);
    if (st != KVSEL_OK) return st;
    if (!q_win || !k || !aligned16(q_win) || !aligned16(k)) return KVSEL_ERR_INVALID_ARG;
    if (desc->n_keys > desc->window && !scores) return KVSEL_ERR_INVALID_ARG;
    Plan p;
    make_plan(desc, p);
    if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace & 255u)) return KVSEL_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    ScoreGeom& g = p.g;
    g.q = q_win;
    g.k = k;
    g.lse_out = lse_out;
    g.lse_in = lse_in;
    float* raw = nullptr;
    int raw_layers = g.L;  // slices of raw that the pool sums (layers, times head groups)
    bool done = false;
    const int path = resolve_path(desc, p);
    if (path < 0) return KVSEL_ERR_UNSUPPORTED;
    // the statistics ride on the streaming passes
    if (stats && path != KVSEL_PATH_STREAM) return KVSEL_ERR_UNSUPPORTED;
    if (path == KVSEL_PATH_STREAM) {
        kvsel::StreamArgs a;
        a.q = static_cast<const uint16_t*>(q_win);
        a.k = static_cast<const uint16_t*>(k);
        for (int i = 0; i < 4; ++i) {
            a.qs[i] = g.qs[i];
            a.ks[i] = g.ks[i];
        }
        a.B = g.B;
        a.Hq = g.Hq;
        a.Hkv = g.Hkv;
        a.G = g.G;
        a.w = g.w;
        a.T = p.T;
        a.Gs = p.Gs;
        a.S0 = g.S;
        a.R = p.Gs * g.w;
        a.N = (int32_t)g.N;
        a.Np = (int32_t)g.Np;
        a.S = g.S * p.T;
        a.c = g.c;
        a.invG = g.invG;
        a.part = reinterpret_cast<float2*>(ws + p.stream.part_off);
        a.part4 = reinterpret_cast<float4*>(ws + p.stream.part_off);
        a.cnt_part = reinterpret_cast<uint32_t*>(ws + p.stream.cnt_off);
        a.lse2 = reinterpret_cast<float*>(ws + p.stream.lse2_off);
        a.raw = reinterpret_cast<float*>(ws + p.stream.raw_off);
        a.l2tau = stats ? log2f(stats->small_p) : 0.f;
        a.lg = 0;
        a.n_lyr = g.L;
        a.spp1 = 0;
        a.lse_out = nullptr;
        // pass 2 may sum the layers itself where pooling the sum equals summing the pooled layers
        raw_layers = g.L * p.T;
        if (!stats && desc->pool_type == KVSEL_POOL_AVG) raw_layers = kvsel::stream_layer_groups(p.stream, a, g.L);
        if (stats) {
            if (kvsel::launch_stream_stats(p.stream, a, lse_out, stats->entropy, stats->sum_p2, stats->n_below, hs) !=
                hipSuccess)
                return KVSEL_ERR_HIP;
        } else if (lse_in) {
            if (kvsel::launch_lse_from_input(lse_in, a.lse2, a.S, p.stream.rp, a.R, g.w, g.B, g.Hq, g.Hkv, g.G, g.S,
                                             p.Gs, hs) != hipSuccess ||
                kvsel::launch_stream_pass2(p.stream, a, hs) != hipSuccess)
                return KVSEL_ERR_HIP;
        } else if (kvsel::launch_stream(p.stream, a, lse_out, hs) != hipSuccess) {
            return KVSEL_ERR_HIP;
        }
        raw = a.raw;
        if (p.T > 1 && desc->pool_type == KVSEL_POOL_MAX && g.Np > 0) {
            // the max pool is not linear: add the head groups into the first
            // group's slices first, then pool layer by layer
            for (int t = 1; t < p.T; ++t)
                if (kvsel::launch_accumulate(1, g.S, g.Np, raw + (int64_t)t * g.S * g.Np, raw, KVSEL_ACC_ADD, hs) !=
                    hipSuccess)
                    return KVSEL_ERR_HIP;
            raw_layers = g.L;
        }
        done = true;
    }
    if (!done) {
        g.part = reinterpret_cast<float2*>(ws + p.gen.part_off);
        g.lse2 = reinterpret_cast<float*>(ws + p.gen.lse2_off);
        g.raw = reinterpret_cast<float*>(ws + p.gen.raw_off);
        const hipError_t e = kvsel::launch_score_passes(g, desc->dtype, desc->head_dim, p.RB, hs);
        if (e != hipSuccess) return KVSEL_ERR_HIP;
        raw = g.raw;
    }
    return from_hip(kvsel::launch_pool(raw, scores, raw_layers, (int64_t)g.B * g.Hkv, g.Np, desc->pool_kernel,
                                       desc->pool_type, accumulate ? 1 : 0, hs));
}

}  // namespace

extern "C" {

const char* kvsel_status_string(kvsel_status_t status) {
    switch (status) {
        case KVSEL_OK: return "KVSEL_OK";
        case KVSEL_ERR_INVALID_ARG: return "KVSEL_ERR_INVALID_ARG: invalid argument";
        case KVSEL_ERR_UNSUPPORTED: return "KVSEL_ERR_UNSUPPORTED: unsupported head_dim, dtype or pool type";
        case KVSEL_ERR_WORKSPACE: return "KVSEL_ERR_WORKSPACE: workspace missing or too small";
        case KVSEL_ERR_HIP: return "KVSEL_ERR_HIP: HIP runtime error";
        case KVSEL_ERR_TOO_LARGE:
            return "KVSEL_ERR_TOO_LARGE: the problem needs more scratch than the no-allocation entry point holds";
        default: return "KVSEL: unknown status";
    }
}

const char* kvsel_version(void) { return "kvsel 0.1.0 (gfx950)"; }

size_t kvsel_score_workspace_bytes(const kvsel_score_desc_t* desc) {
    if (validate_desc(desc) != KVSEL_OK) return 0;
    Plan p;
    make_plan(desc, p);
    return p.total;
}

int32_t kvsel_score_path(const kvsel_score_desc_t* desc) {
    if (validate_desc(desc) != KVSEL_OK) return -1;
    Plan p;
    make_plan(desc, p);
    return resolve_path(desc, p);
}

kvsel_status_t kvsel_score(const kvsel_score_desc_t* desc, const void* q_win, const void* k, float* scores,
                           int32_t accumulate, float* lse_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return score_impl(desc, q_win, k, scores, accumulate, lse_out, nullptr, workspace, workspace_bytes, stream);
}

kvsel_status_t kvsel_score_lse(const kvsel_score_desc_t* desc, const void* q_win, const void* k, const float* lse_in,
                               float* scores, int32_t accumulate, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!lse_in) return KVSEL_ERR_INVALID_ARG;
    return score_impl(desc, q_win, k, scores, accumulate, nullptr, lse_in, workspace, workspace_bytes, stream);
}

kvsel_status_t kvsel_score_stats(const kvsel_score_desc_t* desc, const void* q_win, const void* k, float* scores,
                                 int32_t accumulate, float* lse_out, float small_p, float* entropy, float* sum_p2,
                                 int32_t* n_below, void* workspace, size_t workspace_bytes, void* stream) {
    if (!entropy || !sum_p2 || !n_below) return KVSEL_ERR_INVALID_ARG;
    if (!(small_p > 0.f && small_p <= 1.f)) return KVSEL_ERR_INVALID_ARG;  // also rejects NaN
    const StatsOut so{small_p, entropy, sum_p2, n_below};
    return score_impl(desc, q_win, k, scores, accumulate, lse_out, nullptr, workspace, workspace_bytes, stream, &so);
}

kvsel_status_t kvsel_layer_summary(int32_t n_layers, int32_t rows_per_layer, int32_t window, int64_t n_keys,
                                   const float* entropy, const float* sum_p2, const int32_t* n_below, float* summary,
                                   void* stream) {
    if (n_layers < 1 || n_layers > 65535 || rows_per_layer < 1 || window < 1 || n_keys < window ||
        n_keys >= kMaxKeys || rows_per_layer % window != 0)
        return KVSEL_ERR_INVALID_ARG;
    if (!entropy || !sum_p2 || !n_below || !summary) return KVSEL_ERR_INVALID_ARG;
    return from_hip(kvsel::launch_layer_summary(n_layers, rows_per_layer, window, n_keys, entropy, sum_p2, n_below,
                                                summary, static_cast<hipStream_t>(stream)));
}

kvsel_status_t kvsel_pivot_layer(int32_t n_layers, const float* mean_entropy, const float* mean_sparsity,
                                 float min_drop, float min_rise, int32_t* pivot) {
    if (n_layers < 1 || !mean_entropy || !mean_sparsity || !pivot) return KVSEL_ERR_INVALID_ARG;
    if (!isfinite(min_drop) || !isfinite(min_rise)) return KVSEL_ERR_INVALID_ARG;
    for (int32_t l = 1; l < n_layers; ++l) {
        const double e0 = mean_entropy[l - 1], e1 = mean_entropy[l];
        const double s0 = mean_sparsity[l - 1], s1 = mean_sparsity[l];
        if (e0 - e1 >= (double)min_drop * e0 && s1 - s0 >= (double)min_rise) {
            *pivot = l;
            return KVSEL_OK;
        }
    }
    *pivot = n_layers - 1;
    return KVSEL_OK;
}

kvsel_status_t kvsel_accumulate(int32_t batch, int32_t n_heads, int64_t n, const float* src, float* dst,
                                int32_t mode, void* stream) {
    if (batch < 1 || n_heads < 1 || n < 0 || !src || !dst) return KVSEL_ERR_INVALID_ARG;
    if (mode != KVSEL_ACC_ADD && mode != KVSEL_ACC_HEAD_MEAN) return KVSEL_ERR_INVALID_ARG;
    return from_hip(kvsel::launch_accumulate(batch, n_heads, n, src, dst, mode, static_cast<hipStream_t>(stream)));
}

size_t kvsel_topk_workspace_bytes(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget) {
    if (batch < 1 || rows < 1 || (int64_t)batch * rows > 65535) return 0;
    if (window < 1 || budget < window || n_keys < budget || n_keys >= kMaxKeys) return 0;
    return kvsel::topk_workspace_bytes(batch * rows, n_keys - window);
}

kvsel_status_t kvsel_topk_sinks(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                                int32_t n_sink, const float* scores, int32_t* idx, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (batch < 1 || rows < 1 || (int64_t)batch * rows > 65535) return KVSEL_ERR_INVALID_ARG;
    if (window < 1 || budget < window || n_keys < budget || n_keys >= kMaxKeys) return KVSEL_ERR_INVALID_ARG;
    if (n_sink < 0 || n_sink > budget - window) return KVSEL_ERR_INVALID_ARG;
    if (!idx || (n_keys > window && !scores)) return KVSEL_ERR_INVALID_ARG;
    const size_t need = kvsel::topk_workspace_bytes(batch * rows, n_keys - window);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return KVSEL_ERR_WORKSPACE;
    return from_hip(kvsel::launch_topk(batch * rows, n_keys, window, budget, n_sink, scores, idx, workspace,
                                       static_cast<hipStream_t>(stream)));
}

static_assert(KVSEL_TOPK_NOALLOC_MAX_BYTES == kvsel::kTopkScratchBytes, "the header states the scratch size");

kvsel_status_t kvsel_topk_noalloc(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                                  int32_t n_sink, const float* scores, int32_t* idx, void* stream) {
    if (batch < 1 || rows < 1 || (int64_t)batch * rows > 65535) return KVSEL_ERR_INVALID_ARG;
    if (window < 1 || budget < window || n_keys < budget || n_keys >= kMaxKeys) return KVSEL_ERR_INVALID_ARG;
    if (n_sink < 0 || n_sink > budget - window) return KVSEL_ERR_INVALID_ARG;
    if (!idx || (n_keys > window && !scores)) return KVSEL_ERR_INVALID_ARG;
    if (kvsel::topk_workspace_bytes(batch * rows, n_keys - window) > kvsel::kTopkScratchBytes)
        return KVSEL_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (kvsel::topk_scratch(&ws) != hipSuccess) return KVSEL_ERR_HIP;
    return from_hip(kvsel::launch_topk(batch * rows, n_keys, window, budget, n_sink, scores, idx, ws,
                                       static_cast<hipStream_t>(stream)));
}

kvsel_status_t kvsel_topk(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                          const float* scores, int32_t* idx, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return kvsel_topk_sinks(batch, rows, n_keys, window, budget, 0, scores, idx, workspace, workspace_bytes, stream);
}

int64_t kvsel_csm_candidates(int64_t n_tokens, int32_t chunk, int32_t n_sink, int32_t n_recent) {
    if (n_tokens < 1 || n_tokens >= kMaxKeys || chunk < 2 || chunk > 64 || chunk % 2 || n_sink < 0 || n_recent < 0 ||
        (int64_t)n_sink + n_recent > n_tokens)
        return -1;
    return kvsel::csm_candidates(n_tokens, chunk, n_sink, n_recent);
}

size_t kvsel_csm_workspace_bytes(int32_t n_slabs, int64_t n_tokens, int32_t chunk, int32_t n_sink, int32_t n_recent,
                                 int32_t n_merge) {
    const int64_t cand = kvsel_csm_candidates(n_tokens, chunk, n_sink, n_recent);
    if (n_slabs < 1 || n_slabs > 65535 || cand < 0 || n_merge < 0 || n_merge > cand) return 0;
    return kvsel::csm_workspace_bytes(n_slabs, n_tokens, chunk, n_sink, n_recent, n_merge);
}

kvsel_status_t kvsel_csm(int32_t n_slabs, int64_t n_tokens, int32_t head_dim, int32_t chunk, int32_t n_sink,
                         int32_t n_recent, int32_t n_merge, const void* k, const void* v, const int32_t* degree,
                         void* k_out, void* v_out, int32_t* degree_out, float* score_out, int32_t* match_out,
                         int32_t* chosen_out, void* workspace, size_t workspace_bytes, void* stream) {
    const int64_t cand = kvsel_csm_candidates(n_tokens, chunk, n_sink, n_recent);
    if (n_slabs < 1 || n_slabs > 65535 || cand < 0 || n_merge < 0 || n_merge > cand) return KVSEL_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return KVSEL_ERR_UNSUPPORTED;
    if (!k || !v || !k_out || !v_out || !degree_out) return KVSEL_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out)) return KVSEL_ERR_INVALID_ARG;
    const size_t need = kvsel::csm_workspace_bytes(n_slabs, n_tokens, chunk, n_sink, n_recent, n_merge);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return KVSEL_ERR_WORKSPACE;
    return from_hip(kvsel::launch_csm(n_slabs, n_tokens, head_dim, chunk, n_sink, n_recent, n_merge,
                                      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), degree,
                                      static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), degree_out,
                                      score_out, match_out, chosen_out, workspace, static_cast<hipStream_t>(stream)));
}

size_t kvsel_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t n_keys) {
    if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_keys < 1 || n_keys >= kMaxKeys ||
        (head_dim != 64 && head_dim != 128) || (int64_t)batch * n_kv_heads > 65535 ||
        n_q_heads / n_kv_heads > kvsel::decode_max_group())
        return 0;
    return kvsel::decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_keys, device_cu_count());
}

kvsel_status_t kvsel_decode_attention(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int64_t n_keys, float softmax_scale, const void* q, const void* k, const void* v,
                                      const int32_t* degree, float* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (batch < 1 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || n_keys < 1 || n_keys >= kMaxKeys ||
        (int64_t)batch * n_kv_heads > 65535 || (int64_t)batch * n_q_heads > 0x7fffffff || !isfinite(softmax_scale))
        return KVSEL_ERR_INVALID_ARG;
    if ((head_dim != 64 && head_dim != 128) || n_q_heads / n_kv_heads > kvsel::decode_max_group())
        return KVSEL_ERR_UNSUPPORTED;
    if (!q || !k || !v || !out || !aligned16(k) || !aligned16(v)) return KVSEL_ERR_INVALID_ARG;
    const int n_cu = device_cu_count();
    const size_t need = kvsel::decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, n_keys, n_cu);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return KVSEL_ERR_WORKSPACE;
    const float scale = softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
    return from_hip(kvsel::launch_decode(batch, n_q_heads, n_kv_heads, head_dim, n_keys, scale,
                                         static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(v), degree, out, workspace, n_cu,
                                         static_cast<hipStream_t>(stream)));
}

kvsel_status_t kvsel_gather(int32_t n_layers, int32_t batch, int32_t n_heads, int32_t idx_heads, int32_t budget,
                            int64_t n_src_rows, int64_t row_bytes, const void* src,
                            const int64_t src_strides_bytes[4], const int32_t* idx, void* dst, void* stream) {
    if (n_layers < 1 || batch < 1 || n_heads < 1 || budget < 1 || n_src_rows < 1 || row_bytes < 1)
        return KVSEL_ERR_INVALID_ARG;
    if (idx_heads != 1 && idx_heads != n_heads) return KVSEL_ERR_INVALID_ARG;
    if (!src || !dst || !idx || !src_strides_bytes) return KVSEL_ERR_INVALID_ARG;
    for (int i = 0; i < 4; ++i)
        if (src_strides_bytes[i] < 0) return KVSEL_ERR_INVALID_ARG;
    return from_hip(kvsel::launch_gather(n_layers, batch, n_heads, idx_heads, budget, n_src_rows, row_bytes, src,
                                         src_strides_bytes, idx, dst, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
