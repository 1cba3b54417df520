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
};

// Workspace layout of the scoring call.
struct ScoreWs {
    size_t part_off, lse2_off, raw_off, total;
};

constexpr int kScoreChunk = 1024;  // keys per work-group in both passes

int score_row_blocks(int dtype, int head_dim, int R);  // RB (row blocks of 16 per group)
ScoreWs score_workspace_layout(int64_t S, int64_t n_chunks1, int64_t Rpad, int64_t Np);

hipError_t launch_score(const ScoreGeom& g, int dtype, int head_dim, int RB, float* scores, int accumulate,
                        int pool_kernel, hipStream_t stream);

hipError_t launch_accumulate(int32_t B, int32_t H, int64_t n, const float* src, float* dst, int mode,
                             hipStream_t stream);

hipError_t launch_topk(int32_t rows, int64_t n_keys, int32_t window, int32_t budget, const float* scores,
                       int32_t* idx, hipStream_t stream);

hipError_t launch_gather(int32_t L, int32_t B, int32_t H, int32_t idx_heads, int32_t budget, int64_t n_src_rows,
                         int64_t row_bytes, const void* src, const int64_t s[4], const int32_t* idx, void* dst,
                         hipStream_t stream);

}  // namespace kvsel
