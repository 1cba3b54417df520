/*
 * kvsel.h - attention-saliency KV token selection on MI355X (gfx950).
 *
 * C ABI of libkvsel.so. Every pointer argument named as device memory must be
 * memory the caller allocated on the current HIP device (hipMalloc, or a torch
 * tensor); the library never allocates, frees or keeps a pointer after a call
 * returns. Its only mutable global state is kvsel_topk_noalloc's per-GPU
 * scratch array and the cached address of that array (described there).
 * Work is enqueued on the caller's HIP stream (`stream` is a hipStream_t;
 * NULL means the default stream) and runs asynchronously; calls on one
 * stream run in order.
 *
 * Errors are return codes. Arguments are validated on the host before any
 * launch; when a call returns anything but KVSEL_OK nothing was enqueued and
 * no output was written. A launch failure reported by the HIP runtime returns
 * KVSEL_ERR_HIP. Inputs must be finite (NaN / Inf scores or keys give
 * unspecified, but memory-safe, results).
 *
 * What is computed (the pages: "FastKV: Decoupling of Context Reduction and KV
 * Cache Compression for Prefill-Decoding Acceleration", section 2A
 * Token-Selective Propagation and section 2B decoupled KV reduction;
 * "StructKV: Preserving the Structural Skeleton for Scalable Long-Context
 * Inference", sections 1 global in-degree centrality and 3 decoupled compute
 * and storage budgets). With G = Hq / Hkv, query head h reading KV head
 * floor(h / G), Np = N - w, and window query i sitting at position Np + i:
 *
 *   logit[h,i,j] = scale * <q[h,i,:], k[floor(h/G), j, :]>        for j <= Np + i
 *   p[h,i,j]     = exp(logit[h,i,j] - LSE[h,i])                  (row softmax)
 *   raw[g,j]     = (1/G) * sum_{h in group g} sum_{i<w} p[h,i,j]  for j < Np
 *   score[g,j]   = (1/kp) * sum_{t=-r..r} raw[g,j+t]  (raw = 0 outside [0,Np))
 *                  (KVSEL_POOL_MAX: max_{t=-r..r} raw[g,j+t] inside [0,Np))
 *   C[g,j]       = sum over layers of score[g,j]                  (StructKV)
 *   kept         = the (budget - w) prefix positions of largest score, ties to
 *                  the lower position, plus the window Np .. N-1, ascending.
 */
#ifndef KVSEL_H_
#define KVSEL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvsel_status_t;

#define KVSEL_OK 0              /* success */
#define KVSEL_ERR_INVALID_ARG 1 /* a null pointer, bad size, bad stride or alignment */
#define KVSEL_ERR_UNSUPPORTED 2 /* valid but not implemented: head_dim, dtype, pool type */
#define KVSEL_ERR_WORKSPACE 3   /* workspace missing or smaller than the queried size */
#define KVSEL_ERR_HIP 4         /* the HIP runtime reported a launch error */
#define KVSEL_ERR_TOO_LARGE 5   /* more scratch than kvsel_topk_noalloc holds (KVSEL_TOPK_NOALLOC_MAX_BYTES) */

#define KVSEL_DTYPE_F32 0  /* IEEE binary32 */
#define KVSEL_DTYPE_BF16 1 /* bfloat16 (upper half of a binary32) */

#define KVSEL_POOL_AVG 0 /* stride-1 average pool, zero padded, divisor = kernel */
#define KVSEL_POOL_MAX 1 /* stride-1 max pool over the positions inside [0, N-w), per layer */

#define KVSEL_PATH_AUTO 0    /* streaming kernels where they apply, else the general ones */
#define KVSEL_PATH_STREAM 1  /* streaming two-pass kernels: bf16, head_dim 64/128, w <= 256 */
#define KVSEL_PATH_GENERAL 2 /* general kernels: any supported dtype and head_dim */

#define KVSEL_ACC_ADD 0       /* dst[b,h,:] += src[b,h,:] */
#define KVSEL_ACC_HEAD_MEAN 1 /* dst[b,0,:]  = mean over h of src[b,h,:] */

/*
 * Shape of one scoring call. Q holds the w window queries of every layer,
 * sequence and query head, post-RoPE: element (l, b, h, i, e) lives at
 * q_win + l*q_strides[0] + b*q_strides[1] + h*q_strides[2] + i*q_strides[3] + e
 * (strides in elements; the head-dim stride is 1), so q_win may be a strided
 * view of the caller's full query tensor. K is addressed the same way with
 * k_strides over (layer, b, kv_head, position).
 */
typedef struct kvsel_score_desc {
    int32_t n_layers;    /* L >= 1: layers scored and summed in this call */
    int32_t batch;       /* B >= 1 */
    int32_t n_q_heads;   /* Hq >= 1, a multiple of n_kv_heads */
    int32_t n_kv_heads;  /* Hkv >= 1; L * B * Hkv <= 65535 */
    int32_t head_dim;    /* d: 64 or 128 (others: KVSEL_ERR_UNSUPPORTED) */
    int32_t window;      /* w: 1 <= w <= n_keys */
    int64_t n_keys;      /* N: cached keys per sequence, N < 2^31 */
    int32_t pool_kernel; /* odd, >= 1 (1 = no pool), <= 255 */
    int32_t pool_type;   /* KVSEL_POOL_AVG or KVSEL_POOL_MAX */
    int32_t dtype;       /* KVSEL_DTYPE_F32 or KVSEL_DTYPE_BF16, for Q and K */
    float softmax_scale; /* > 0, or <= 0 for 1/sqrt(head_dim) */
    int64_t q_strides[4];
    int64_t k_strides[4];
    int32_t path;        /* KVSEL_PATH_AUTO (0), _STREAM or _GENERAL: which kernels score */
    int32_t reserved;    /* must be 0 */
} kvsel_score_desc_t;

/* Device workspace, in bytes, that kvsel_score needs for `desc` (0 on an
 * invalid descriptor). */
size_t kvsel_score_workspace_bytes(const kvsel_score_desc_t* desc);

/* The scoring kernels a call with `desc` runs: KVSEL_PATH_STREAM or
 * KVSEL_PATH_GENERAL (what KVSEL_PATH_AUTO resolves to), or -1 when the
 * descriptor is invalid or asks for the streaming kernels on a shape they do
 * not take (kvsel_score then returns KVSEL_ERR_UNSUPPORTED). Host only. */
int32_t kvsel_score_path(const kvsel_score_desc_t* desc);

/*
 * Saliency scores of every prefix key (FastKV section 2A; StructKV section 1).
 *
 * q_win   device, see kvsel_score_desc_t; 16-byte aligned rows.
 * k       device, see kvsel_score_desc_t; 16-byte aligned rows.
 * scores  device float[B][Hkv][N - w], contiguous. accumulate == 0: written
 *         with the sum over the L layers of the pooled score; accumulate != 0:
 *         that sum is added to what scores holds (StructKV accumulation across
 *         calls, layer by layer or in groups of layers).
 * lse_out device float[L][B][Hq][w] or NULL: the natural-log LSE of every
 *         window row.
 * workspace  device, >= kvsel_score_workspace_bytes(desc) bytes, 256-byte
 *         aligned; its content is scratch between calls.
 * Paths (desc->path): KVSEL_PATH_AUTO streams K in two passes for bf16 with
 * head_dim 64/128 and w <= 256 (when G*w > 256 the group's query heads are
 * streamed in head groups of at most 256 rows, each reading the keys) and
 * takes the general two-pass kernels for other shapes; KVSEL_PATH_STREAM or
 * _GENERAL asks for one of them explicitly (the streaming choice on a shape
 * it does not take returns UNSUPPORTED). Both compute the same result to the
 * stated tolerance.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
kvsel_status_t kvsel_score(const kvsel_score_desc_t* desc, const void* q_win, const void* k, float* scores,
                           int32_t accumulate, float* lse_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Saliency scores with the window rows' LSEs handed in: prefill attention
 * (FastKV section 2A; StructKV section 1) has already normalised every window
 * row, so only the second softmax pass runs and K is read once.
 *
 * Same arguments as kvsel_score, except:
 * lse_in  device float[L][B][Hq][w], required: the natural-log LSE of every
 *         window row under the same scale and causal mask (the layout
 *         kvsel_score writes to lse_out). Values must be finite.
 * workspace  >= kvsel_score_workspace_bytes(desc) bytes, 256-byte aligned.
 * Scores equal kvsel_score's to the stated tolerance when lse_in is the LSE
 * kvsel_score would compute. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
kvsel_status_t kvsel_score_lse(const kvsel_score_desc_t* desc, const void* q_win, const void* k, const float* lse_in,
                               float* scores, int32_t accumulate, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Saliency scores plus the attention statistics of every window row that
 * StructKV's dynamic pivot detection watches (StructKV section 2: attention
 * entropy, sparsity and variance during the first pass, layer by layer).
 *
 * Same arguments and scores as kvsel_score, and:
 * small_p  probability threshold of the count, 0 < small_p <= 1.
 * entropy  device float[L][B][Hq][w]: -sum_j p_j ln p_j over the keys row i
 *          sees (j <= N - w + i), p_j = exp(l_j - LSE), in nats.
 * sum_p2   device float[L][B][Hq][w]: sum_j p_j^2 (the row's variance of
 *          weights is sum_p2 / n - 1 / n^2 with n = N - w + i + 1).
 * n_below  device int32[L][B][Hq][w]: the number of keys the row sees with
 *          p_j < small_p (decided in fp32 on the exponent: c*x - LSE2 <
 *          log2(small_p), c = scale*log2(e); keys within rounding of the
 *          threshold may fall either way).
 * Only the streaming path computes them: bf16, head_dim 64/128, w <= 256;
 * other shapes return UNSUPPORTED. Both passes read every key.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
kvsel_status_t kvsel_score_stats(const kvsel_score_desc_t* desc, const void* q_win, const void* k, float* scores,
                                 int32_t accumulate, float* lse_out, float small_p, float* entropy, float* sum_p2,
                                 int32_t* n_below, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-layer means of the row statistics (StructKV section 2).
 *
 * entropy, sum_p2, n_below  device [n_layers][rows_per_layer] as written by
 *          kvsel_score_stats, rows_per_layer = B*Hq*w (window index r % w).
 * summary  device float[n_layers][3]: the means over the layer's rows of the
 *          entropy, of the sparsity n_below / n and of the variance
 *          sum_p2 / n - 1 / n^2, n = n_keys - window + 1 + (r % window).
 * Errors: INVALID_ARG (rows_per_layer not a multiple of window, null
 * pointers, sizes out of range), HIP.
 */
kvsel_status_t kvsel_layer_summary(int32_t n_layers, int32_t rows_per_layer, int32_t window, int64_t n_keys,
                                   const float* entropy, const float* sum_p2, const int32_t* n_below, float* summary,
                                   void* stream);

/*
 * StructKV's pivot layer (section 2, the phase transition where entropy falls
 * and sparsity rises), on HOST arrays: the first layer l >= 1 with
 *   mean_entropy[l-1] - mean_entropy[l] >= min_drop * mean_entropy[l-1]   and
 *   mean_sparsity[l] - mean_sparsity[l-1] >= min_rise,
 * compared in double; n_layers - 1 when there is none. Layers 0 .. *pivot are
 * the ones whose scores are accumulated. Runs on the host only.
 * Errors: INVALID_ARG (n_layers < 1, null pointers, non-finite thresholds).
 */
kvsel_status_t kvsel_pivot_layer(int32_t n_layers, const float* mean_entropy, const float* mean_sparsity,
                                 float min_drop, float min_rise, int32_t* pivot);

/*
 * Accumulate score vectors (StructKV section 1: a token's scores added up over
 * layers; FastKV section 2A: one token set per sequence for propagation).
 *
 * src  device float[batch][n_heads][n]; dst device float.
 * KVSEL_ACC_ADD:       dst[batch][n_heads][n] += src.
 * KVSEL_ACC_HEAD_MEAN: dst[batch][1][n] = (1/n_heads) * sum over heads of src
 *                      (the token-set score ranked for propagation).
 * src and dst must not overlap. Errors: INVALID_ARG, HIP.
 */
kvsel_status_t kvsel_accumulate(int32_t batch, int32_t n_heads, int64_t n, const float* src, float* dst,
                                int32_t mode, void* stream);

/* Device workspace, in bytes, that kvsel_topk needs (0 on invalid sizes): the
 * per-chunk digit histograms, selection state and chunk counts of the
 * multi-work-group radix select. */
size_t kvsel_topk_workspace_bytes(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget);

/*
 * Keep `budget` positions per selection row (FastKV section 2A: the most
 * salient tokens plus a window of the newest; section 2B and StructKV section
 * 3: the TSP / compute budget and the KV / storage budget are separate calls).
 *
 * scores  device float[batch][rows][n_keys - window], contiguous, >= 0.
 * idx     device int32[batch][rows][budget], contiguous: per row the
 *         (budget - window) prefix positions with the largest score (ties go
 *         to the lower position), then window positions n_keys - window ..
 *         n_keys - 1; strictly ascending, window last.
 * The TSP token set calls this with rows = 1 on the head-mean score; the KV
 * set with rows = n_kv_heads.
 * workspace  device, >= kvsel_topk_workspace_bytes(...) bytes, 256-byte aligned.
 * Preconditions: 1 <= window <= budget <= n_keys < 2^31; batch * rows <= 65535.
 * Errors: INVALID_ARG, WORKSPACE, HIP.
 */
kvsel_status_t kvsel_topk(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                          const float* scores, int32_t* idx, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * kvsel_topk with attention sinks protected (CentroidKV, section 2
 * inference pipeline: attention sinks and the newest tokens are preserved):
 * positions 0 .. n_sink-1 are always kept, and they count against the
 * (budget - window) slots chosen by score. 0 <= n_sink <= budget - window
 * (and n_sink <= n_keys - window); n_sink = 0 is kvsel_topk. Same workspace
 * as kvsel_topk. Errors: INVALID_ARG, WORKSPACE, HIP.
 */
kvsel_status_t kvsel_topk_sinks(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                                int32_t n_sink, const float* scores, int32_t* idx, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kvsel_topk_sinks without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments (minus the workspace),
 * result and errors as kvsel_topk_sinks (n_sink = 0 is kvsel_topk).
 *
 * Its scratch (digit histograms, per-pass states, per-chunk counts) is a
 * static device array of KVSEL_TOPK_NOALLOC_MAX_BYTES bytes (16 MiB), one
 * copy per GPU, held until the process ends; the call allocates nothing. A
 * problem whose scratch, kvsel_topk_workspace_bytes(batch, rows, n_keys,
 * window, budget), exceeds that returns KVSEL_ERR_TOO_LARGE before any launch
 * (about 680 selection rows at 131072 keys). Every call on a GPU shares that
 * GPU's array: calls that can overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller; calls on one stream are
 * ordered. The kernels clear what must start at zero, so a call never sees
 * the previous call's contents. The first call on each device looks up the
 * array's device address (hipGetSymbolAddress, no allocation).
 */
#define KVSEL_TOPK_NOALLOC_MAX_BYTES ((size_t)16 << 20)
kvsel_status_t kvsel_topk_noalloc(int32_t batch, int32_t rows, int64_t n_keys, int32_t window, int32_t budget,
                                  int32_t n_sink, const float* scores, int32_t* idx, void* stream);

/*
 * CentroidKV chunked soft matching, one clustering round (page "Technische
 * Samenvatting: CentroidKV", section "Methodologie": part 2 keeps sinks and
 * recent tokens out of the partition, part 3 matches inside chunks and merges
 * only the best-ranked matches, part 4 builds degree-weighted centroids).
 *
 * Per slab (layer, sequence, KV head) of n_tokens tokens, the middle
 * [n_sink, n_tokens - n_recent) is cut into chunks of `chunk` tokens (even,
 * 2..64; the last chunk may be shorter). In a chunk, offsets 0, 2, ... form
 * set A and 1, 3, ... set B. Each A token's candidate is the B token of its
 * chunk with the highest cosine similarity of keys (0 when a key is zero;
 * ties to the lower position). The n_merge candidates of highest similarity
 * (ties to the lower A position) merge into their B tokens; a cluster's key
 * and value become the degree-weighted means of its members (fp32, rounded
 * to bf16 to nearest even) and its degree their sum. Every other token is
 * copied bit for bit. Survivors keep position order: n_out = n_tokens -
 * n_merge rows per slab.
 *
 * k, v         device bf16 [n_slabs][n_tokens][head_dim], 16-byte aligned.
 * degree       device int32 [n_slabs][n_tokens] (>= 1), or NULL for all 1.
 * k_out, v_out device bf16 [n_slabs][n_out][head_dim]; degree_out device int32
 *              [n_slabs][n_out]. Outputs must not overlap the inputs.
 * score_out    device float [n_slabs][n_A] or NULL: each A token's best
 *              similarity (-inf without a candidate); A tokens are numbered in
 *              position order.
 * match_out    device int32 [n_slabs][n_A] or NULL: that candidate's position
 *              (-1 without one).
 * chosen_out   device int32 [n_slabs][n_merge] or NULL: the merged A numbers,
 *              ascending.
 * n_merge must not exceed kvsel_csm_candidates(...). head_dim 64 or 128.
 * Keys must be finite: a key with NaN or Inf has NaN similarities, so its A
 * token may rank among the chosen with no partner (score -inf, match -1); such
 * a token is dropped without merging (its row and degree leave the output).
 * The output stays n_out rows and no access leaves the buffers.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 *
 * kvsel_csm_candidates: host-only; the number of A tokens that have a B
 * partner (n_merge's upper bound), or -1 for invalid sizes (n_tokens outside
 * [1, 2^31), chunk odd or outside 2..64, n_sink or n_recent negative or
 * together above n_tokens). kvsel_csm_workspace_bytes: 0 on invalid
 * arguments.
 */
int64_t kvsel_csm_candidates(int64_t n_tokens, int32_t chunk, int32_t n_sink, int32_t n_recent);
size_t kvsel_csm_workspace_bytes(int32_t n_slabs, int64_t n_tokens, int32_t chunk, int32_t n_sink, int32_t n_recent,
                                 int32_t n_merge);
kvsel_status_t kvsel_csm(int32_t n_slabs, int64_t n_tokens, int32_t head_dim, int32_t chunk, int32_t n_sink,
                         int32_t n_recent, int32_t n_merge, const void* k, const void* v, const int32_t* degree,
                         void* k_out, void* v_out, int32_t* degree_out, float* score_out, int32_t* match_out,
                         int32_t* chosen_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over a compacted cache (FastKV section 2B and StructKV
 * section 3: decoding reads the kept cache; CentroidKV part 4: a centroid's
 * degree enters the softmax as a log term).
 *
 * out[b][h][:] = sum_j p_j v[b][g][j][:], p = softmax over j of
 *   scale * <q[b][h], k[b][g][j]> + ln degree[b][g][j],  g = h / (Hq / Hkv).
 * q       device bf16 [batch][n_q_heads][head_dim] (one new query each).
 * k, v    device bf16 [batch][n_kv_heads][n_keys][head_dim], 16-byte aligned.
 * degree  device int32 [batch][n_kv_heads][n_keys] (>= 1), or NULL (no term).
 * out     device float [batch][n_q_heads][head_dim].
 * softmax_scale > 0, or <= 0 for 1/sqrt(head_dim). Fold layers into batch to
 * run a step over every layer at once. head_dim 64 or 128; at most 8 query
 * heads per KV head. Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
size_t kvsel_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                    int64_t n_keys);
kvsel_status_t kvsel_decode_attention(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int64_t n_keys, float softmax_scale, const void* q, const void* k, const void* v,
                                      const int32_t* degree, float* out, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Compact the cache (FastKV section 2A: only the kept tokens are passed on;
 * section 2B / StructKV section 3: the kept KV entries are stored).
 *
 * Copies rows bit for bit: dst[l][b][h][t][:] = src row (l, b, h,
 * idx[b][idx_heads == 1 ? 0 : h][t]) for every layer l < n_layers; a row is
 * `row_bytes` bytes. The source row (l, b, h, j) starts at
 * src + l*s[0] + b*s[1] + h*s[2] + j*s[3] bytes, s = src_strides_bytes.
 * dst is device memory, contiguous [n_layers][batch][n_heads][budget][row_bytes].
 * idx is device int32[batch][idx_heads][budget] with idx_heads 1 (one token set
 * shared by every head, e.g. hidden states) or n_heads (per KV head). An index
 * outside [0, n_src_rows) yields an all-zero row.
 * Rows whose size, base and strides are multiples of 16 bytes are copied with
 * 16-byte accesses, otherwise byte by byte. src and dst must not overlap.
 * Errors: INVALID_ARG, HIP.
 */
kvsel_status_t kvsel_gather(int32_t n_layers, int32_t batch, int32_t n_heads, int32_t idx_heads, int32_t budget,
                            int64_t n_src_rows, int64_t row_bytes, const void* src,
                            const int64_t src_strides_bytes[4], const int32_t* idx, void* dst, void* stream);

/* Static, human-readable name of a status code. */
const char* kvsel_status_string(kvsel_status_t status);

/* Library version string. */
const char* kvsel_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H_ */
