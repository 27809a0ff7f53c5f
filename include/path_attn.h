/*
 * path_attn.h -- C ABI of libpath_attn: PaTH attention prefill and decode on
 * AMD Instinct MI355X (gfx950).
 *
 * Citations name a page and a section of it:
 *   [Notes s2.x]   reading-notes page "PaTH Attention:通过累积 Householder
 *                  变换编码位置" (cc.laoqi.cc, notes on arXiv 2505.16381v2);
 *   [Explainer s3] explainer page "PaTH Attention: Position Encoding via
 *                  Accumulating Householder Transformations" (gist.science),
 *                  section 3 on efficient training and inference.
 *
 * The operation [Notes s2.1, s2.5]: for each (batch n, head h) and query
 * position i, with transitions H_t = I - beta_t w_t w_t^T,
 *   logit(i, j) = scale * k_j^T H_{j+1} ... H_i q_i + sum_{s=j+1..i} log f_s,
 *   j <= i (causal), o_i = softmax_j(logit) . v,  lse_i = log sum_j exp(logit).
 * The forget-gate term is present only when a log f array is given (PaTH-FoX);
 * it is added after scaling and is not scaled.  Positions are 0-based.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers owned by the caller.  The library
 *   allocates nothing, frees nothing, keeps no per-call global state, and
 *   never synchronises the host with the device.  Work is enqueued on the
 *   caller's stream; results are visible after the caller synchronises it.
 *   (path_decode_step_noalloc alone uses a fixed scratch array that the
 *   library holds in device memory, one per GPU, instead of a workspace.)
 * - Layouts are dense and row-major:
 *     q, k, v, w, o          [N, H, L, d]  in desc->dtype
 *     beta, logf, lse        [N, H, L]     float32
 *     per-token decode args  [N, H, d] (q_t, k_t, v_t, w_t, o_t) in
 *                            desc->dtype; [N, H] float32 (beta_t, logf_t, lse_t)
 * - Supported: dtype PATH_F32 with d in {16, 32, 64}; dtype PATH_BF16 with
 *   d in {16, 32, 64} (d = 32 and 64 use the matrix-core kernels).
 * - beta and log f are used as given: no clipping, no renormalisation of w.
 *   NaN and Inf propagate.  beta in [0, 2] is the meaningful range.
 * - Argument errors are reported synchronously, before anything is enqueued:
 *   null pointers, sizes < 1 (or L > 8388608), unsupported d or dtype, pointers that are not
 *   16-byte aligned (4-byte for float32 arrays), a workspace smaller than the
 *   matching *_workspace() result, or a cache index beyond its capacity.
 *   A failed kernel launch returns PATH_E_LAUNCH.  Faults inside a kernel
 *   surface at the caller's next synchronisation.  path_last_error() gives a
 *   message for the last failure on the calling thread.
 * - Outputs must not alias inputs.  Calls on different streams are
 *   independent as long as their buffers (including workspaces and caches)
 *   are distinct.
 */
#ifndef PATH_ATTN_H
#define PATH_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PATH_ATTN_ABI_VERSION 5

typedef enum {
    PATH_OK = 0,
    PATH_E_NULL = 1,         /* a required pointer is NULL */
    PATH_E_SHAPE = 2,        /* N, H, L or a length argument out of range */
    PATH_E_DTYPE = 3,        /* unknown dtype enum value */
    PATH_E_UNSUPPORTED = 4,  /* valid but unsupported (d, block size) */
    PATH_E_ALIGN = 5,        /* pointer not aligned as required */
    PATH_E_WORKSPACE = 6,    /* workspace NULL or smaller than required */
    PATH_E_CAPACITY = 7,     /* cache capacity exceeded */
    PATH_E_LAUNCH = 8        /* a kernel launch failed */
} path_status;

typedef enum { PATH_F32 = 0, PATH_BF16 = 1 } path_dtype;

/* Problem description.  L is the sequence length for the forward pass and is
 * ignored by the decode entry points.  block = 0 selects the default block
 * size (64); the float32 path also accepts 16 and 32, which must give the same
 * result up to rounding (the block decomposition is exact [Notes s2.7]). */
typedef struct {
    int N, H, L, d;
    path_dtype dtype;
    float scale;
    int block;
} path_fwd_desc;

/* Decode cache [Notes s2.8; Explainer s3].  Keys are stored already rewritten
 * by every transition after them: after position t has been processed, slot j
 * holds H_t ... H_{j+1} k_j, so a plain softmax decode over it gives PaTH
 * scores.  No w or beta history is kept.
 *   kcache [N, H, cap, d] in k_dtype (PATH_F32 or PATH_BF16)
 *   vcache [N, H, cap, d] in desc->dtype
 *   gcache [N, H, cap] float32: inclusive prefix sums of log f (slot j holds
 *          sum_{s<=j} log f_s), or NULL for plain PaTH (no forget gate). */
typedef struct {
    int cap;
    path_dtype k_dtype;
    void *kcache;
    void *vcache;
    float *gcache;
} path_cache;

int path_abi_version(void);
const char *path_status_str(path_status s);
/* Message for the last failure on the calling thread ("" if none). */
const char *path_last_error(void);

/* Bytes of device workspace path_attn_fwd needs for this description
 * (0 if the description is invalid).  with_cache != 0 sizes it for a call
 * that also fills a decode cache (cache_out != NULL). */
size_t path_attn_fwd_workspace(const path_fwd_desc *desc, int with_cache);

/*
 * Prefill forward pass [Notes s2.1, s2.5 (definition); s2.6-s2.7 (blockwise
 * UT form and right-to-left scan, the algorithm used)].
 *   q, k, v, w : [N, H, L, d] desc->dtype      beta : [N, H, L] float32
 *   logf       : [N, H, L] float32 log forget gates, or NULL (plain PaTH)
 *   o          : [N, H, L, d] desc->dtype (written; bf16 rounds to nearest even)
 *   lse        : [N, H, L] float32 natural-log log-sum-exp of each row's
 *                final logits (after scale and bias), or NULL
 *   cache_out  : NULL, or a cache with cap >= L to fill with the prompt's keys
 *                aligned to position L-1 (H_{L-1}...H_{j+1} k_j), its values,
 *                and (if gcache != NULL and logf != NULL) the log f prefix.
 *                This is the prefill-to-decode alignment of [Notes s2.8].
 *   ws, ws_bytes : workspace of at least path_attn_fwd_workspace(desc,
 *                cache_out != NULL) bytes,
 *                256-byte aligned; its contents need not be initialised.
 */
path_status path_attn_fwd(const path_fwd_desc *desc, const void *q,
                          const void *k, const void *v, const void *w,
                          const float *beta, const float *logf, void *o,
                          float *lse, const path_cache *cache_out, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* path_attn_fwd with phase timing, for measurement.  Identical work, plus
 * four events recorded on `stream` (created by the caller): ev[0] before the
 * block preconditioning, ev[1] before the right-to-left scan, ev[2] after it,
 * ev[3] after the cache alignment (right after ev[2] when cache_out is NULL). */
path_status path_attn_fwd_timed(const path_fwd_desc *desc, const void *q,
                                const void *k, const void *v, const void *w,
                                const float *beta, const float *logf, void *o,
                                float *lse, const path_cache *cache_out,
                                void *ws, size_t ws_bytes, hipStream_t stream,
                                hipEvent_t ev[4]);

/* Bytes of device workspace path_attn_bwd needs (0 if the description is
 * invalid or its block is not 64).  It holds the recomputed preconditioning,
 * per-block gradients, and per block pair of a bounded group of slices (the
 * call walks the slices in groups so this part stays within 4 GiB) the
 * queries carried to each key block and the gradient chain. */
size_t path_attn_bwd_workspace(const path_fwd_desc *desc);

/*
 * Backward pass (training): gradients of a scalar loss with respect to q, k,
 * v, w, beta and log f, given dL/do.  The pages give no backward formulas;
 * this differentiates the forward's block algorithm [Notes s2.6-s2.7], the
 * same function as the definition [Notes s2.1, s2.5], so the gradients are
 * those of the definition.  The loss is taken not to depend on lse.
 *   desc       : as for path_attn_fwd; block must be 0 or 64.
 *   q, k, v, w, beta, logf : the forward's inputs (logf NULL: plain PaTH)
 *   o, lse     : the forward's outputs for these inputs (lse required)
 *   dout       : [N, H, L, d] desc->dtype, dL/do
 *   dq, dk, dv, dw : [N, H, L, d] desc->dtype (written)
 *   dbeta      : [N, H, L] float32 (written)
 *   dlogf      : [N, H, L] float32 (written; dlogf[.., 0] = 0, since log f at
 *                the first position never reaches an output), given exactly
 *                when logf is given
 *   ws, ws_bytes : at least path_attn_bwd_workspace(desc) bytes, 256-byte
 *                aligned; contents need not be initialised.
 * Same conventions as path_attn_fwd (device pointers, no allocation, no
 * synchronisation, argument errors before launch).  Products run on the
 * matrix cores from fp32 operands split into bf16 parts (two for bf16 data,
 * three for fp32 data).
 */
path_status path_attn_bwd(const path_fwd_desc *desc, const void *q,
                          const void *k, const void *v, const void *w,
                          const float *beta, const float *logf, const void *o,
                          const float *lse, const void *dout, void *dq, void *dk,
                          void *dv, void *dw, float *dbeta, float *dlogf,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* Cache rewrite for a new position [Notes s2.8, eq. (1) of the paper]:
 *   k_j <- k_j - beta_t (w_t^T k_j) w_t   for every slot j in [0, n).
 * w_t [N, H, d] desc->dtype; beta_t [N, H] float32.  In place on kcache. */
path_status path_kv_update(const path_fwd_desc *desc, const path_cache *cache,
                           int n, const void *w_t, const float *beta_t,
                           hipStream_t stream);

/* Appends one token at slot n (n < cap): kcache[n] = k_t (not rewritten: its
 * own transition is not on its path [Notes s2.1]), vcache[n] = v_t, and, if
 * gcache != NULL, gcache[n] = gcache[n-1] + logf_t (logf_t alone when n = 0;
 * logf_t may be NULL only if gcache is NULL). */
path_status path_kv_append(const path_fwd_desc *desc, const path_cache *cache,
                           int n, const void *k_t, const void *v_t,
                           const float *logf_t, hipStream_t stream);

/* Bytes of workspace the decode entry points need for up to n_keys keys. */
size_t path_decode_workspace(const path_fwd_desc *desc, int n_keys);

/* Single-query attention over slots [0, n_keys) of a rewritten cache
 * [Notes s2.8]: with t = n_keys - 1,
 *   s_j = scale * q_t^T kcache[j] + (gcache[t] - gcache[j])   (bias 0 if
 *   gcache is NULL), o_t = softmax(s) . vcache, lse_t = log sum exp s.
 * q_t, o_t [N, H, d] desc->dtype; lse_t [N, H] float32 or NULL.
 * Split over key chunks of 128; ws holds the per-chunk partial softmax
 * states.  At most 131072 keys per call (PATH_E_UNSUPPORTED beyond). */
path_status path_decode(const path_fwd_desc *desc, const path_cache *cache,
                        int n_keys, const void *q_t, void *o_t, float *lse_t,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* One fused decode step at position t = n (n keys already cached, n < cap)
 * [Notes s2.8, eq. (1) of the paper: every cached key is rewritten by the new
 * transition, the new key enters unrewritten, and a plain softmax over the
 * cache then gives the PaTH(-FoX) logits of query t; Explainer s3]:
 * path_kv_update(n, w_t, beta_t), path_kv_append(n, k_t, v_t, logf_t) and
 * path_decode(n + 1, q_t) in one pass over the cache.  Afterwards the cache
 * holds n + 1 keys.  logf_t may be NULL only if gcache is NULL.
 * ws: at least path_decode_workspace(desc, n + 1) bytes. */
path_status path_decode_step(const path_fwd_desc *desc,
                             const path_cache *cache, int n, const void *q_t,
                             const void *k_t, const void *v_t,
                             const void *w_t, const float *beta_t,
                             const float *logf_t, void *o_t, float *lse_t,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/* path_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, semantics and results as path_decode_step
 * (bit for bit: the same kernels), without the workspace arguments: the
 * split-K partial states go to a scratch array that the library holds in
 * device memory, one per GPU, for the life of the process
 * (path_decode_step_noalloc_limit() bytes, 16 MiB).  Neither call allocates
 * or frees anything.
 *   - A step whose partial states need more than that (path_decode_workspace
 *     (desc, n + 1) > the limit; at d = 64 about 63 500 chunks of 128 keys
 *     over all N * H slices) returns PATH_E_WORKSPACE before any launch.
 *   - The first call on a GPU looks the array's device address up (with that
 *     GPU current; the GPU is the one `stream` belongs to) and keeps it.
 *   - Every call on one GPU shares the array: calls that overlap on one GPU
 *     (on different streams or from different threads) race and must be
 *     ordered by the caller.  The array keeps the last call's contents;
 *     nothing in it needs clearing. */
size_t path_decode_step_noalloc_limit(void);
path_status path_decode_step_noalloc(const path_fwd_desc *desc,
                                     const path_cache *cache, int n,
                                     const void *q_t, const void *k_t,
                                     const void *v_t, const void *w_t,
                                     const float *beta_t, const float *logf_t,
                                     void *o_t, float *lse_t, hipStream_t stream);

/* Paged decode cache for a batch of sequences of different lengths
 * [Notes s2.8; Explainer s3: the in-place key rewrite keeps decoding
 * compatible with paged caches and FlashDecoding-style split-K kernels].
 * Keys, values and log-f prefixes of a sequence live in fixed-size pages
 * taken from one pool; a per-sequence page table maps the slot range
 * [i*page_size, (i+1)*page_size) to a page.  Within a page the H heads are
 * separate contiguous [page_size, d] slabs:
 *   kpages [num_pages, H, page_size, d] in k_dtype (PATH_F32 or PATH_BF16)
 *   vpages [num_pages, H, page_size, d] in desc->dtype
 *   gpages [num_pages, H, page_size] float32 inclusive log-f prefixes of the
 *          sequence (as gcache of path_cache), or NULL (no forget gate).
 * Slots hold rewritten keys exactly as path_cache does. */
typedef struct {
    int num_pages;
    int page_size;      /* 16, 32, 64 or 128 */
    path_dtype k_dtype;
    void *kpages;
    void *vpages;
    float *gpages;
} path_paged_cache;

/* Bytes of workspace path_paged_decode_step needs for desc->N sequences of up
 * to max_keys keys each (0 if the arguments are invalid). */
size_t path_paged_decode_workspace(const path_fwd_desc *desc, int max_keys);

/*
 * One fused decode step for a batch of S = desc->N sequences at their own
 * positions [Notes s2.8]: for each sequence s with n = seq_lens[s] keys
 * cached, path_decode_step's work at position t = n (every cached key
 * rewritten in place by H_t, the token appended at slot n, single-query
 * attention over slots [0, n]), with the page indirection.
 *   page_table   : [S, table_stride] int32, device; entry i of row s is the
 *                  page holding slots [i*page_size, (i+1)*page_size) of s.
 *   seq_lens     : [S] int32, device; keys cached per sequence on entry,
 *                  advanced by one on exit (so the same call, or a captured
 *                  graph of it, serves the next position).
 *   max_keys     : bound on seq_lens[s] + 1 over the batch (sets the grid);
 *                  table_stride >= ceil(max_keys / page_size); at most 131072.
 *   q_t, k_t, v_t, w_t : [S, H, d] desc->dtype; beta_t, logf_t : [S, H]
 *                  float32 (logf_t may be NULL only if gpages is NULL).
 *   o_t [S, H, d] desc->dtype, lse_t [S, H] float32 or NULL (written).
 *   ws           : at least path_paged_decode_workspace(desc, max_keys)
 *                  bytes, 256-byte aligned; contents need not be initialised.
 * Split over chunks of 128 keys per (sequence, head), then a combine.
 * Device-side values are checked where they are read: a sequence whose
 * seq_lens entry is outside [0, max_keys) is left untouched (seq_lens too)
 * and gets NaN outputs; a chunk of 128 keys that reaches a page-table entry
 * outside [0, num_pages) (one of its own pages or, with the gate, the page of
 * slot n - 1) touches no cache memory, and its (sequence, head) gets NaN
 * outputs while seq_lens still advances.  Same conventions as
 * path_decode_step otherwise.
 */
path_status path_paged_decode_step(const path_fwd_desc *desc,
                                   const path_paged_cache *cache,
                                   const int *page_table, int table_stride,
                                   int *seq_lens, int max_keys, const void *q_t,
                                   const void *k_t, const void *v_t,
                                   const void *w_t, const float *beta_t,
                                   const float *logf_t, void *o_t, float *lse_t,
                                   void *ws, size_t ws_bytes, hipStream_t stream);

/* Copies slots [0, seq_lens[s]) of each sequence s of a contiguous cache (for
 * example the one path_attn_fwd aligns a prefill into, desc->N = S
 * sequences) into its pages, so that paged decoding can continue from a
 * prefill.  Key dtypes must match, and gcache / gpages be given together.
 * seq_lens and page_table as for path_paged_decode_step (seq_lens is only
 * read); sequences with seq_lens[s] outside [0, min(max_keys, src->cap)] and
 * table entries outside [0, num_pages) are skipped. */
path_status path_paged_import(const path_fwd_desc *desc, const path_cache *src,
                              const path_paged_cache *dst, const int *page_table,
                              int table_stride, const int *seq_lens, int max_keys,
                              hipStream_t stream);

/* Plain causal softmax attention (every beta = 0, no gate): the in-library
 * baseline the PaTH kernels are timed against.  Same layouts as
 * path_attn_fwd; no workspace.  bf16 with d in {32, 64} only (other
 * descriptions return PATH_E_UNSUPPORTED). */
path_status path_causal_attn_fwd(const path_fwd_desc *desc, const void *q,
                                 const void *k, const void *v, void *o,
                                 float *lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Parameter front-end [Notes s2.1, s2.5]: the branch that turns a layer input
 * x_t into the transition parameters consumed by path_attn_fwd and the decode
 * calls.  Per sequence n and token t (0-based), with C = H * d channels:
 *   p_t      = Wd x_t                                   (rank R)
 *   r_t      = Wu p_t                                   (C channels)
 *   c_t      = kc[:,0] r_t + kc[:,1] r_{t-1} + kc[:,2] r_{t-2}
 *              (depthwise causal convolution of width 3; r_s = 0 for s < 0,
 *              no activation)
 *   w_t      = c_t / |c_t| per head (the head's d channels; 0 if c_t = 0)
 *   beta_t   = 2 / (1 + exp(-(ub . x_t + bb)))          per head, in (0, 2)
 *   logf_t   = log sigma(uf . x_t + bf)                 per head (optional)
 * The pages give the structure (low-rank linear layer, width-3 short
 * convolution, L2 normalisation, 2 sigma, log sigma) but not the rank or the
 * convolution's exact form; the above is the plainest reading.
 *
 * Layouts (row-major, weights in the out-by-in layout of a linear layer):
 *   x [N, L, Dm], Wd [R, Dm], Wu [C, R], ub and uf [H, Dm]  in desc->dtype;
 *   kc [C, 3], bb and bf [H]                                  float32;
 *   outputs w [N, H, L, d] in desc->dtype (bf16: round to nearest even),
 *   beta and logf [N, H, L] float32.
 * uf, bf and logf are all NULL (no forget gate) or all given.
 * Supported: d in {16, 32, 64}, Dm a multiple of 16 and at most 65536, R a
 * multiple of 16 with 16 <= R <= 256; otherwise PATH_E_UNSUPPORTED.
 * N, L, H >= 1; PATH_E_SHAPE when one sequence's rows of the intermediate
 * would pass 1 GiB (L * Rp * 4 bytes).
 * ws: at least path_param_workspace(desc) bytes, 256-byte aligned; it holds
 * the projected float32 intermediate [N*L, Rp]: R low-rank columns, then H
 * beta and (with a gate) H gate columns, each block padded to a multiple of
 * 8, Rp the total rounded up to 32.
 * Same conventions as every other entry point (device pointers, no
 * allocation, no synchronisation, errors before launch). */
typedef struct {
    int N, L;          /* sequences, tokens per sequence */
    int Dm;            /* layer input width */
    int R;             /* rank of the low-rank layer */
    int H, d;          /* heads, head dim */
    path_dtype dtype;  /* of x, the weight matrices and w */
} path_param_desc;

size_t path_param_workspace(const path_param_desc *desc, int with_gate);

path_status path_param_fwd(const path_param_desc *desc, const void *x,
                           const void *Wd, const void *Wu, const float *kc,
                           const void *ub, const float *bb, const void *uf,
                           const float *bf, void *w, float *beta, float *logf,
                           void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PATH_ATTN_H */
