/*
 * nsa.h -- C ABI of the MI355X (gfx950) library for block-sparse attention
 * driven by top-k KV-tile selection.
 *
 * Two calls make up the path:
 *   nsa_select             query/key tiles -> int8 keep flags + per-row CSR list
 *   nsa_block_sparse_attn  attention over the kept tiles -> output + logsumexp
 * plus host-only sizing, two stage entry points (pooling, scores) and status
 * strings.
 *
 * What the selection computes is defined by the page
 * "automatic/modules/attention/sparse/selector.py" (functions SparseSpec,
 * BlockSelection, pool_blocks, diagonal_blocks, score_blocks, selection_plan,
 * select_blocks). The attention consumer is not printed on any page; its
 * definition here is the usual scaled softmax attention restricted to the kept
 * tiles (see nsa_block_sparse_attn).
 *
 * Conventions common to every call
 *   - Tensors are dense, contiguous, row-major (B, H, S, D) in device memory.
 *   - The caller allocates and owns every buffer; the library keeps no pointer
 *     after a call returns. All device work is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and runs asynchronously; nothing
 *     synchronises the device.
 *   - Every argument is validated before any work is enqueued; on an error the
 *     call returns a negative nsa_status and leaves all outputs untouched.
 *   - No C++ exception crosses this interface.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. 0 = success; NSA_DENSE is informational (> 0); errors < 0. */
enum nsa_status {
    NSA_OK = 0,
    NSA_DENSE = 1,                /* the budget covers every candidate: attend densely */
    NSA_ERR_NULL_ARG = -1,        /* a required pointer is NULL */
    NSA_ERR_BAD_SHAPE = -2,       /* inconsistent sizes, Hq % Hkv != 0, mask not broadcastable */
    NSA_ERR_BAD_DTYPE = -3,       /* dtype not F32/BF16, or q/k/v/out dtypes differ */
    NSA_ERR_UNSUPPORTED = -4,     /* valid request this library does not run (see each call) */
    NSA_ERR_WORKSPACE = -5,       /* workspace missing or smaller than nsa_sizes.workspace_bytes */
    NSA_ERR_BAD_SPEC = -6,        /* block size <= 0, budget < 0 or NaN, chunk bytes < 0 */
    NSA_ERR_HIP = -7,             /* a HIP runtime call failed: see nsa_last_hip_error() */
    NSA_ERR_CAPACITY = -8         /* col_idx capacity below the selection's nnz */
};

enum nsa_dtype { NSA_F32 = 0, NSA_BF16 = 1 };

/* A device tensor of shape (B, H, S, D), contiguous. */
typedef struct nsa_tensor {
    void* data;      /* device pointer */
    int32_t dtype;   /* enum nsa_dtype */
    int32_t B, H, S, D;
} nsa_tensor;

/* Selection spec; the fields and defaults of SparseSpec on the selection page:
 * budget 0.30, block_q 128, block_kv 64, head_shared 0, force 0,
 * score_chunk_bytes 256 MiB. budget is the fraction of each row's candidate
 * tiles (neither must-keep nor dropped) chosen by score; pinned and diagonal
 * tiles come on top. head_shared scores once for all heads with the head-mean
 * of the pooled queries and of the pooled keys. force skips the dense short
 * circuit. score_chunk_bytes bounds the fp32 score buffer per head chunk. */
typedef struct nsa_spec {
    float budget;
    int32_t block_q;
    int32_t block_kv;
    int32_t head_shared;
    int32_t force;
    int64_t score_chunk_bytes;
} nsa_spec;

/* Optional tile mask in HOST memory (pins or drops), int8, nonzero = set,
 * contiguous (b_dim, h_dim, nq, nk) and broadcast over the selection shape
 * (B, H', NQ, NK): b_dim in {1, B}, h_dim in {1, H'}, nq == NQ, nk == NK.
 * H' = 1 when head_shared, else Hq. */
typedef struct nsa_mask {
    const int8_t* data;
    int32_t b_dim, h_dim, nq, nk;
} nsa_mask;

/* A block selection (the BlockSelection of the selection page plus its CSR
 * form). Device buffers are caller-owned:
 *   keep    int8  (B, H', NQ, NK)     1 = tile kept
 *   row_ptr int32 (B*H'*NQ + 1)       row r = (b*H' + h')*NQ + i
 *   col_idx int32 (capacity >= nnz)   kept kv tiles per row, strictly ascending
 * nsa_select fills the buffers and every geometry field. */
typedef struct nsa_selection {
    int8_t* keep;
    int32_t* row_ptr;
    int32_t* col_idx;
    int64_t col_capacity;   /* entries available in col_idx (set by the caller) */
    int64_t nnz;            /* number of kept tiles (set by nsa_select) */
    int32_t B, H, NQ, NK;   /* H = H' (selection heads: 1 or Hq) */
    int32_t block_q, block_kv;
    int32_t seq_q, seq_kv;
    float budget;
} nsa_selection;

/* Sizes of a selection, from geometry and masks only (no tensor data). */
typedef struct nsa_sizes {
    int32_t NQ, NK;          /* ceil(S / block_q), ceil(S / block_kv) */
    int32_t sel_heads;       /* H' */
    int32_t dense;           /* 1 when the dense short circuit applies (and force is 0) */
    int64_t rows;            /* B * H' * NQ */
    int64_t nnz;             /* exact number of kept tiles */
    int64_t workspace_bytes; /* device workspace nsa_select needs */
} nsa_sizes;

/* Host only. Computes the plan of selection_plan on the selection page: NQ,
 * NK, must = diagonal OR pins, forbidden = drops, candidates c_r, per-row
 * budget k_r = ceil(fl32(c_r) * fl32(budget)), the exact nnz
 * = sum_r |must_r \ forbidden_r| + min(k_r, c_r), and the dense decision (every
 * k_r >= c_r and force == 0). q and k are read for their shapes only; pins and
 * drops may be NULL. If row_ptr_host is non-NULL it receives rows+1 int32
 * offsets. Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_SPEC, UNSUPPORTED
 * (nnz >= 2^31). */
int nsa_select_sizes(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec,
                     const nsa_mask* pins, const nsa_mask* drops, nsa_sizes* out,
                     int32_t* row_ptr_host);

/* select_blocks of the selection page. Pools q over block_q tokens and k over
 * block_kv tokens (fp32 means; a tail tile is averaged over its real length),
 * scores every (query tile, kv tile) pair by the pooled dot product (no scale,
 * no softmax; head_shared: head-means of both operands; GQA: query head h uses
 * kv head h / (Hq/Hkv)), then per row keeps must, plus the k_r best candidates
 * (score descending, ties to the lower kv index, -0.0 == +0.0), minus drops.
 *   q: (B, Hq, Sq, D), k: (B, Hkv, Skv, D), same dtype (F32 or BF16), finite.
 *   out: keep / row_ptr / col_idx buffers and col_capacity set by the caller.
 *   workspace: device scratch of at least nsa_sizes.workspace_bytes, 256-byte
 *   aligned; its contents are undefined after the call.
 * Returns NSA_DENSE (outputs untouched, nothing enqueued) when the dense short
 * circuit applies. Errors as nsa_select_sizes, plus WORKSPACE, CAPACITY, HIP.
 * UNSUPPORTED: D not in {64, 128, 256}, NK > 4096. Result on non-finite
 * inputs is unspecified. */
int nsa_select(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec,
               const nsa_mask* pins, const nsa_mask* drops, nsa_selection* out,
               void* workspace, size_t workspace_bytes, void* stream);

/* Attention over the kept tiles. For query head h, kv head g = h / (Hq/Hkv)
 * and selection head h' = h (or 0 when sel->H == 1); a selection with
 * sel->B == 1 applies to every batch entry (as radial_blocks returns it). Key u is visible to query
 * t iff tile (t / block_q, u / block_kv) is kept in row (b, h', t / block_q)
 * and, when causal != 0, u <= t. With l_tu = D^-1/2 q_t . k_u:
 *   lse[t] = ln sum_{visible u} exp(l_tu)            (fp32, natural log)
 *   out[t] = sum_{visible u} exp(l_tu - lse[t]) v_u   (dtype of q)
 * A query with no visible key gets out = 0 and lse = -inf. sel == NULL means
 * dense (every tile kept: the consumer side of NSA_DENSE).
 *   q, out: (B, Hq, S, D); k, v: (B, Hkv, S, D); lse: device fp32 (B, Hq, S).
 * UNSUPPORTED: Sq != Skv (the selection page pools both from equal-length
 * sequences in every workload here), D not in {64, 128}. */
int nsa_block_sparse_attn(const nsa_tensor* q, const nsa_tensor* k, const nsa_tensor* v,
                          const nsa_selection* sel, int causal, nsa_tensor* out,
                          float* lse, void* stream);

/* ---- Plan reuse --------------------------------------------------------------
 * selection_plan on the selection page depends only on geometry, the spec and
 * the pin / drop masks, and the page caches it under a caller-supplied key
 * that leaves the mask contents out. Here the plan is an explicit handle built
 * from all of them, so a reused plan can never be stale. */
typedef struct nsa_plan nsa_plan;

/* Host only. Builds the plan nsa_select would build for tensors shaped like q
 * and k (read for shape and dtype only) and copies what it needs from pins and
 * drops (the caller may free them afterwards). Errors as nsa_select_sizes.
 * The plan never changes and the handle may be used by several threads at once. */
int nsa_plan_create(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec,
                    const nsa_mask* pins, const nsa_mask* drops, nsa_plan** out);

/* Host only. The sizes of the planned selection (as nsa_select_sizes). */
int nsa_plan_sizes(const nsa_plan* plan, nsa_sizes* out, int32_t* row_ptr_host);

/* Host only. Bytes of the plan's device image (its row offsets and bit-packed
 * pin / drop words): the size of the buffer nsa_plan_upload fills. */
int nsa_plan_device_bytes(const nsa_plan* plan, int64_t* bytes);

/* Copies the plan's device image into plan_dev, a caller-owned device buffer
 * of at least nsa_plan_device_bytes bytes, 256-byte aligned, enqueued on
 * `stream` through a pinned host staging slot of the library (no device
 * allocation, no synchronisation). The image stays valid while the caller
 * keeps the buffer; it does not depend on tensor data. Errors: NULL_ARG,
 * WORKSPACE (plan_dev NULL, misaligned or too small), HIP. */
int nsa_plan_upload(const nsa_plan* plan, void* plan_dev, size_t bytes, void* stream);

/* nsa_select with a prebuilt plan: q and k must have the plan's shapes and
 * dtype (BAD_SHAPE / BAD_DTYPE otherwise). Result, outputs, workspace and
 * errors as nsa_select with the plan's spec, pins and drops. plan_dev: the
 * plan's device image written by nsa_plan_upload (on this or an earlier
 * point of the same stream), read by the selection kernels, which copy its
 * row offsets into out->row_ptr; nothing is then copied from the host. NULL:
 * the image is uploaded into the workspace by this call, as nsa_select does.
 * WORKSPACE also when plan_dev is not 256-byte aligned. */
int nsa_select_planned(const nsa_plan* plan, const void* plan_dev, const nsa_tensor* q, const nsa_tensor* k,
                       nsa_selection* out, void* workspace, size_t workspace_bytes, void* stream);

/* Frees a plan (NULL is allowed). Host memory only: device buffers holding
 * its image are the caller's. */
void nsa_plan_destroy(nsa_plan* plan);

/* ---- Plan cache of nsa_select and nsa_select_sizes ---------------------------
 * Both calls look their plan up in a process-wide cache before building it
 * (the plan cache of selection_plan on the selection page). The key is the
 * whole request: q and k shapes and dtypes, every nsa_spec field, and the
 * shape and bytes of pins and drops, so a request whose masks differ in one
 * byte builds its own plan (the page's key leaves the masks out). Entries are
 * host memory only (the plan is uploaded per call on the caller's stream, as
 * without the cache); the least recently used entry is replaced when the
 * cache is full. Each entry keeps a copy of its masks, so requests whose pins
 * and drops hold more than 64 MiB together are built per call and not cached.
 * Thread-safe. */

/* Host only. Keeps at most `capacity` plans (default 8; 0 disables caching).
 * Lowering it drops the least recently used entries. BAD_SPEC if capacity < 0. */
int nsa_plan_cache_config(int32_t capacity);

/* Host only. Drops every cached plan and zeroes the counters. */
void nsa_plan_cache_clear(void);

/* Host only. Lookups that found a plan, lookups that built one, and the entries
 * held now. NULL_ARG if any pointer is NULL. */
int nsa_plan_cache_stats(int64_t* hits, int64_t* misses, int32_t* entries);

/* ---- Controls (selection page: schedule, radial_blocks, BlockSelection.density) */

/* Host only. Per-step budgets: out[i] = budget, raised to min(1, budget + bump)
 * on the first and last edge steps, edge = min(bump_steps, ceil(steps / 2)),
 * when bump > 0, bump_steps > 0 and steps > 0. Writes max(steps, 0) values
 * (fp64, as the page's Python floats). NULL_ARG if steps > 0 and out is NULL. */
int nsa_schedule(int32_t steps, double budget, double bump, int32_t bump_steps, double* out);

/* Host only. Sizes of radial_blocks(seq_q, seq_kv, density): NQ, NK,
 * sel_heads = 1, rows = NQ, nnz; row_ptr_host (NQ + 1 int32) if non-NULL.
 * BAD_SPEC for block sizes <= 0 or negative lengths. */
int nsa_radial_sizes(int32_t seq_q, int32_t seq_kv, double density, const nsa_spec* spec,
                     nsa_sizes* out, int32_t* row_ptr_host);

/* radial_blocks of the selection page: the static control at a given density.
 * A tile is kept when the centres of its query and kv token ranges are at
 * most a bandwidth apart; the bandwidth is bisected 40 times over
 * [0, max(seq_q, seq_kv)] until the kept fraction reaches density (distances
 * in fp32, the kept fraction an fp32 mean compared in fp64). Computed on the
 * host (geometry only) and copied on `stream` into out->keep (1, 1, NQ, NK)
 * int8, out->row_ptr (NQ + 1) and out->col_idx (capacity out->col_capacity);
 * the other fields of out are set (B = H = 1, budget = density). Errors:
 * NULL_ARG, BAD_SPEC, CAPACITY, HIP. */
int nsa_radial_blocks(int32_t seq_q, int32_t seq_kv, double density, const nsa_spec* spec,
                      nsa_selection* out, void* stream);

/* Host only. BlockSelection.density: kept tiles / (B * H * NQ * NK), from the
 * selection's nnz (no device readback). 0 for an empty selection. */
int nsa_selection_density(const nsa_selection* sel, double* out);

/* ---- Token reordering ("Optimal ordering with block mask") -------------------
 * For tokens on a grid (an image, a video), laying the sequence out along a
 * space-filling curve before a series of attention calls keeps neighbouring
 * tokens in the same tiles, so local patterns touch fewer blocks. */
enum { NSA_CURVE_MORTON = 0, NSA_CURVE_HILBERT = 1 };

/* Host only. perm[m] = raster index (last axis fastest) of the grid point at
 * position m of the curve, for a grid of ndim (1..4) axes of sizes dims[].
 * Morton: the key interleaves coordinate bits (bit b of axis a, a = 0 the
 * last axis, to bit b * ndim + a). Hilbert: J. Skilling's transpose method
 * on the enclosing 2^p cube ("Programming the Hilbert curve", 2004); a grid
 * that is not a full cube keeps the cube's order restricted to its points.
 * perm holds prod(dims) int32. Errors: NULL_ARG, BAD_SPEC (kind),
 * BAD_SHAPE (negative size), UNSUPPORTED (ndim, or more than 2^31 points). */
int nsa_curve_order(int32_t kind, int32_t ndim, const int32_t* dims, int32_t* perm);

/* y[b, h, m, :] = x[b, h, perm[m], :] (inverse == 0), or
 * y[b, h, perm[m], :] = x[b, h, m, :] (inverse != 0), on `stream`.
 * x, y: device (B, H, S, D), same shape and dtype, not the same buffer,
 * 16-byte aligned, D * sizeof(dtype) a power of two from 64 to 1024 bytes.
 * perm: device int32 (S), a permutation of [0, S); rows whose entry is
 * outside [0, S) are left untouched. Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE,
 * UNSUPPORTED, HIP. */
int nsa_permute_tokens(const nsa_tensor* x, const int32_t* perm, int32_t inverse, nsa_tensor* y,
                       void* stream);

/* ---- Decoding over a KV cache ------------------------------------------------
 * The inference pathways of "todo" (native-sparse-attention-pytorch issue #1):
 * a running pooled key sequence, the importance score of the new query tokens
 * and attention over only the selected blocks of the cache. Reading (the
 * selection page aligns queries at position 0): n new query tokens sit at
 * absolute positions q_pos0 .. q_pos0 + n - 1 of the cache, q_pos0 + n <=
 * length; query tiles are counted from q_pos0, the diagonal is measured at the
 * queries' absolute positions, and attention is causal in absolute positions. */

/* Keeps pooled (B, Hkv, tiles_capacity, D) fp32 equal to pool_blocks of the
 * first len_new tokens of k_cache (B, Hkv, capacity, D), given that it held
 * those of the first len_old: only the kv tiles holding a new token are
 * recomputed (each averaged over its real length). 0 <= len_old <= len_new
 * <= capacity; ceil(len_new / block_kv) <= tiles_capacity. Errors: BAD_SHAPE,
 * BAD_SPEC, BAD_DTYPE, NULL_ARG, UNSUPPORTED (D), HIP. */
int nsa_decode_pool_update(const nsa_tensor* k_cache, int32_t len_old, int32_t len_new, int32_t block_kv,
                           float* pooled, int32_t tiles_capacity, void* stream);

/* Host only. Sizes of nsa_decode_select (as nsa_select_sizes); pins / drops
 * are (1|B, 1|H', ceil(n / block_q), ceil(length / block_kv)). */
int nsa_decode_select_sizes(const nsa_tensor* q, const nsa_tensor* pooled_k, int32_t length, int32_t q_pos0,
                            const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops,
                            nsa_sizes* out, int32_t* row_ptr_host);

/* select_blocks for the new query tokens q (B, Hq, n, D) against the first
 * `length` cached keys, whose pooled means are pooled_k (F32 nsa_tensor
 * (B, Hkv, tiles_capacity, D), kept by nsa_decode_pool_update). Outputs,
 * workspace, NSA_DENSE and errors as nsa_select; the selection records
 * seq_q = n and seq_kv = length. */
int nsa_decode_select(const nsa_tensor* q, const nsa_tensor* pooled_k, int32_t length, int32_t q_pos0,
                      const nsa_spec* spec, const nsa_mask* pins, const nsa_mask* drops, nsa_selection* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Host only. Device workspace nsa_decode_attn needs for these shapes and this
 * selection (sel may be NULL). */
int nsa_decode_attn_workspace_size(const nsa_tensor* q, const nsa_tensor* k_cache, int32_t length, int32_t q_pos0,
                                   const nsa_selection* sel, int64_t* bytes);

/* Attention of the new query tokens q (B, Hq, n, D) over the kept tiles of the
 * first `length` keys of k_cache / v_cache (B, Hkv, capacity, D): key u is
 * visible to query t iff its tile is kept and u <= q_pos0 + t. sel from
 * nsa_decode_select, or NULL for every tile. out (B, Hq, n, D), lse (B, Hq, n)
 * as nsa_block_sparse_attn. With few query rows, each row's tiles are split
 * over several workgroups whose partial results (unnormalised output, exponent
 * reference and sum) go to `workspace` and are then merged, so the whole GPU
 * streams the cache. workspace: device scratch of
 * nsa_decode_attn_workspace_size bytes. Errors as nsa_block_sparse_attn, plus
 * WORKSPACE. */
int nsa_decode_attn(const nsa_tensor* q, const nsa_tensor* k_cache, const nsa_tensor* v_cache, int32_t length,
                    int32_t q_pos0, const nsa_selection* sel, nsa_tensor* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

/* nsa_decode_attn without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. The split partials go
 * to a static device buffer of the library, NSA_DECODE_SCRATCH_BYTES (16 MiB)
 * per GPU, held until the process ends; its address on the current device is
 * looked up on the first call there. Every call on one GPU shares that buffer
 * (each call writes every partial it reads, so nothing carries over), so calls
 * that overlap on one GPU -- from several threads or streams -- race and must be
 * serialised by the caller. Arguments, result and errors as nsa_decode_attn
 * with no workspace; NSA_ERR_WORKSPACE when nsa_decode_attn_workspace_size
 * for the request exceeds NSA_DECODE_SCRATCH_BYTES. The tensors must live on
 * the current device. */
#define NSA_DECODE_SCRATCH_BYTES (16u << 20)
int nsa_decode_attn_static(const nsa_tensor* q, const nsa_tensor* k_cache, const nsa_tensor* v_cache,
                           int32_t length, int32_t q_pos0, const nsa_selection* sel, nsa_tensor* out, float* lse,
                           void* stream);

/* Device workspace, in bytes, that nsa_block_sparse_attn_bwd needs for these
 * shapes and this selection (sel may be NULL for dense). Host only. */
int nsa_attn_bwd_workspace_size(const nsa_tensor* q, const nsa_tensor* k, const nsa_selection* sel,
                                int64_t* bytes);

/* Gradients of nsa_block_sparse_attn (same visibility, same selection). With
 * P_tu = exp(l_tu - lse[t]) on visible pairs and dO the upstream gradient:
 *   Delta_t = dO_t . out_t,  dS_tu = P_tu (dO_t . v_u - Delta_t)
 *   dq[t] = D^-1/2 sum_u dS_tu k_u
 *   dk[u] = D^-1/2 sum_t dS_tu q_t,  dv[u] = sum_t P_tu dO_t
 * where the sums for dk and dv also run over the query heads of the kv head's
 * GQA group. Queries with no visible key (lse = -inf) contribute nothing.
 * This differentiates the consumer of the selection page's BlockSelection;
 * the selection itself (a top-k) has no gradient.
 *   q, out, dout, dq: (B, Hq, S, D); k, v, dk, dv: (B, Hkv, S, D); all the
 *   dtype of q. lse: device fp32 (B, Hq, S) as returned by the forward.
 *   sel: the forward's selection, or NULL for dense. Its keep flags are read
 *   to build a kv-tile-major index and row_ptr / col_idx for the query-major
 *   walk, so both must describe the same selection (nsa_select writes both).
 *   workspace: device scratch of nsa_attn_bwd_workspace_size bytes, 256-byte
 *   aligned; contents undefined afterwards.
 * Every element of dq, dk and dv is written. Errors as the forward, plus
 * WORKSPACE. */
int nsa_block_sparse_attn_bwd(const nsa_tensor* q, const nsa_tensor* k, const nsa_tensor* v,
                              const nsa_tensor* out, const float* lse, const nsa_tensor* dout,
                              const nsa_selection* sel, int causal, nsa_tensor* dq, nsa_tensor* dk,
                              nsa_tensor* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Stage entry point: pool_blocks of the selection page on its own.
 * x: (B, H, S, D) F32/BF16 device; out: device fp32 (B, H, ceil(S/block), D). */
int nsa_pool_blocks(const nsa_tensor* x, int32_t block, float* out, void* stream);

/* Stage entry point: the full fp32 score tensor of score_blocks on the
 * selection page, (B, H', NQ, NK), written to scores (device). Needs a
 * workspace of nsa_sizes.workspace_bytes (as nsa_select). Each score is the
 * pooled dot product to within fp32 rounding of the products and their sum
 * (|error| <= 2 D 2^-24 sum |q_d k_d|); with more than 64 query tiles per
 * head it is computed from exact three-term bf16 splits of the pooled
 * operands on the bf16 matrix cores. */
int nsa_score_blocks(const nsa_tensor* q, const nsa_tensor* k, const nsa_spec* spec,
                     float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* ---- Stage timing (measurement) ----------------------------------------------
 * Between nsa_stage_timing_begin and nsa_stage_timing_end, the selection calls
 * (nsa_select, nsa_select_planned, nsa_decode_select) made on the calling
 * thread record a HIP event on their stream at their start and after each
 * stage: "pool_q", "pool_k", "head_mean" (head_shared), then "scores" and
 * "topk" once per head chunk. nsa_block_sparse_attn_bwd records "delta",
 * "kv_index" (with a selection), then "dq" and "dkdv" on its MFMA path.
 * Host only; the events are created by the library and destroyed by _end. */
typedef struct nsa_stage_time {
    const char* name;   /* static string: the stage that ended at this mark */
    float ms;           /* device time since the previous mark of the same call */
} nsa_stage_time;

/* Starts recording on this thread (drops any marks of an unfinished run). */
int nsa_stage_timing_begin(void);

/* Stops recording, waits for the last recorded event, and writes up to
 * `capacity` stages in the order they were enqueued; *count receives the
 * number recorded (which may exceed capacity). NULL_ARG if count is NULL, or
 * out is NULL with capacity > 0; HIP if an event query fails. */
int nsa_stage_timing_end(nsa_stage_time* out, int32_t capacity, int32_t* count);

/* Static description of a status code. Never NULL. */
const char* nsa_status_string(int status);

/* The hipError_t of the last NSA_ERR_HIP returned on this thread (0 if none). */
int nsa_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* nsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
