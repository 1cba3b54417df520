// Internal declarations shared by the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

// Geometry of one scoring call, resolved on the host and passed by value.
struct ScoreGeom {
    const void* q;
    const void* k;
    int64_t qs[4];  // element strides over (layer, b, head, t)
    int64_t ks[4];
    int32_t L, B, Hq, Hkv, G, w;
    int32_t R;         // query rows per KV head: G * w
    int32_t Rpad;      // R rounded up to whole row groups
    int32_t n_groups;  // row groups of RB * 16 rows
    int32_t S;         // slabs: L * B * Hkv
    int64_t N, Np;
    int32_t chunk;      // keys per work-group chunk
    int32_t n_chunks1;  // chunks over [0, N)   (LSE pass)
    int32_t n_chunks2;  // chunks over [0, Np)  (score pass)
    float c;            // softmax scale * log2(e)
    float invG;
    float2* part;     // [S][n_chunks1][Rpad] (max, sum) in the log2 domain
    float* lse2;      // [S][Rpad] row LSE in the log2 domain (+inf on padded rows)
    float* raw;       // [S][Np] window-summed, group-averaged probabilities
    float* lse_out;   // [L][B][Hq][w] natural-log LSE, or null
    const float* lse_in;  // [L][B][Hq][w] natural-log LSE handed in (pass 1 skipped), or null
};

// Workspace layout of the scoring call.
struct ScoreWs {
    size_t part_off, lse2_off, raw_off, total;
};

// Keys per work-group chunk of the general path: kScoreChunk, or a smaller
// power of two (down to kScoreChunkMin) when the call has too few chunks to
// give every compute unit a couple of work-groups.
constexpr int kScoreChunk = 1024;
constexpr int kScoreChunkMin = 64;

int score_row_blocks(int dtype, int head_dim, int R);  // RB (row blocks of 16 per group)
ScoreWs score_workspace_layout(int64_t S, int64_t n_chunks1, int64_t Rpad, int64_t Np);

// General path: two launches over K (LSE partials + combine, then scores).
hipError_t launch_score_passes(const ScoreGeom& g, int dtype, int head_dim, int RB, hipStream_t stream);

// Row LSE2 [S][stride] (log2 domain, +inf past R) from a handed-in natural-log
// LSE [L][B][Hq][w].
// Slabs are [T][S0] head groups of Gs heads each (T = 1, Gs = G without
// groups); R is the row count of a full group.
hipError_t launch_lse_from_input(const float* lse_in, float* lse2, int S, int stride, int R, int w, int B, int Hq,
                                 int Hkv, int G, int S0, int Gs, hipStream_t stream);

// Pool (KVSEL_POOL_AVG or _MAX) of raw [L][B*Hkv][Np], summed over layers,
// written or added to scores.
hipError_t launch_pool(const float* raw, float* scores, int L, int64_t BH, int64_t Np, int pool_kernel, int pool_type,
                       int accumulate, hipStream_t stream);

// Streaming path (bf16): pass 1 partials, merge, pass 2, each streaming K.
struct StreamArgs {
    const uint16_t* q;
    const uint16_t* k;
    int64_t qs[4];
    int64_t ks[4];
    int32_t B, Hq, Hkv, G, w, R;
    int32_t N, Np, S;
    // Head groups: when the G*w rows of a KV head exceed the kernels' 256,
    // its query heads split into T groups of Gs heads (the last may hold
    // fewer), each a slab of its own. Slabs are [T][S0] with S0 = L*B*Hkv;
    // R = Gs*w is the row count of a full group.
    int32_t T, Gs, S0;
    int32_t spp;      // segments per slab (set per pass)
    int32_t seg_len;  // keys per segment, a multiple of the 256-key chunk
    int32_t n_range;  // keys the pass covers: N (pass 1, and pass 2 with statistics) or Np (pass 2)
    int32_t n_seg;    // S * spp (layer-sum pass 2: units * lg)
    // Layer-sum pass 2 (set by stream_layer_groups): the prefix keys' raw
    // scores summed over groups of lg consecutive layers of the n_lyr, raw
    // then [ceil(n_lyr / lg)][B*Hkv][Np]; lg = 0: one raw row per slab.
    int32_t lg, n_lyr;
    float c, invG;
    float l2tau;   // statistics: log2 of the probability threshold of the count
    float2* part;  // [S][spp1][rp] per-segment (reference, sum) of every row, log2 domain
    float4* part4; // statistics: [S][spp1][rp] (reference, sum, sum e*x, sum e^2), same place as part
    uint32_t* cnt_part;  // statistics: [S][spp1][rp] per-segment counts of keys below the threshold
    float* lse2;   // [S][rp] row LSE2
    float* raw;    // [S][Np]
    // Pass 2 of the two-pass call: > 0 when it merges pass 1's spp1 partials
    // of a slab into the row LSEs itself (then writing lse_out [L][B][Hq][w]
    // natural-log LSE, or nothing if null); 0: the row LSEs are read from lse2.
    int32_t spp1;
    float* lse_out;
};

struct StreamPlan {
    bool ok;
    int head_dim, rbn, rbn_cap, rp, n_wg;
    int spp1, seg_len1, spp2, seg_len2;
    size_t part_off, cnt_off, lse2_off, raw_off;  // raw: [S][Np] floats at raw_off
};

bool stream_plan(int dtype, int head_dim, int R, int64_t N, int64_t Np, int64_t S, int n_cu, StreamPlan& plan);
hipError_t launch_stream(const StreamPlan& plan, StreamArgs a, float* lse_out, hipStream_t stream);
// Both passes with the pivot statistics of every row: entropy, sum of p^2
// ([L][B][Hq][w] floats) and the count of keys with p below the threshold
// ([L][B][Hq][w] int32), besides the raw scores and the optional LSE.
hipError_t launch_stream_stats(const StreamPlan& plan, StreamArgs a, float* lse_out, float* entropy, float* sum_p2,
                               int32_t* n_below, hipStream_t stream);
// Pass 2 alone, on row LSEs already in a.lse2.
hipError_t launch_stream_pass2(const StreamPlan& plan, StreamArgs a, hipStream_t stream);
// Whether pass 2 sums the layers of an L-layer call itself (average pool
// only: pooling is linear; one head group): sets a.lg (0: no) and a.n_lyr and
// returns the number of raw rows per (b, KV head) the pool then sums.
int stream_layer_groups(const StreamPlan& plan, StreamArgs& a, int L);

hipError_t launch_accumulate(int32_t B, int32_t H, int64_t n, const float* src, float* dst, int mode,
                             hipStream_t stream);

// Per-layer means [L][3] (entropy, sparsity, variance) of the row statistics.
hipError_t launch_layer_summary(int32_t L, int32_t rows, int32_t w, int64_t N, const float* entropy,
                                const float* sum_p2, const int32_t* n_below, float* summary, hipStream_t stream);

size_t topk_workspace_bytes(int32_t rows, int64_t n_prefix);
// The no-allocation top-k's static scratch: its size, and its device address
// on the current device (looked up once per device).
constexpr size_t kTopkScratchBytes = (size_t)16 << 20;
hipError_t topk_scratch(void** out);
hipError_t launch_topk(int32_t rows, int64_t n_keys, int32_t window, int32_t budget, int32_t n_sink,
                       const float* scores, int32_t* idx, void* workspace, hipStream_t stream);

// CentroidKV chunked soft matching (centroid.hip).
int64_t csm_candidates(int64_t n, int32_t chunk, int32_t n_sink, int32_t n_recent);
size_t csm_workspace_bytes(int32_t S, int64_t n, int32_t chunk, int32_t n_sink, int32_t n_recent, int32_t n_merge);
hipError_t launch_csm(int32_t S, int64_t n, int32_t d, int32_t chunk, int32_t n_sink, int32_t n_recent,
                      int32_t n_merge, const uint16_t* k, const uint16_t* v, const int32_t* degree, uint16_t* k_out,
                      uint16_t* v_out, int32_t* degree_out, float* score_out, int32_t* match_out,
                      int32_t* chosen_out, void* workspace, hipStream_t stream);

// Decode attention over a compacted cache (decode.hip).
int decode_max_group();
size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n, int n_cu);
hipError_t launch_decode(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int64_t n, float scale, const uint16_t* q,
                         const uint16_t* k, const uint16_t* v, const int32_t* degree, float* out, void* workspace,
                         int n_cu, hipStream_t stream);

hipError_t launch_gather(int32_t L, int32_t B, int32_t H, int32_t idx_heads, int32_t budget, int64_t n_src_rows,
                         int64_t row_bytes, const void* src, const int64_t s[4], const int32_t* idx, void* dst,
                         hipStream_t stream);

}  // namespace kvsel
