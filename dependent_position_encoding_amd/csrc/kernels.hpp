// kernels.hpp -- internal interface between the C-ABI host layer and the
// kernel translation units of libpath_attn.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pa {

// Per-block products of the preconditioning step, carved from the caller's
// workspace by the host layer.  "blk" = slice * nb + c with slice = n*H + h.
struct FwdWs {
    void* kr;     // f32 path: keys moved to their block's right edge [blk][B][d]
                  //   (the bf16 backward keeps scale * Kright here as bf16, see kb16)
    void* em;     // f32 path: block transition I - E, E as [blk][d][d]
                  //   (the bf16 backward keeps -E here as bf16, see eb16)
    void* img;    // bf16 path: per-block tile images (Kright, V^T, -E, gate
                  //   cumsum) in the scan's LDS layout [blk][image bytes]
    float* ql;    // queries moved to their block's left edge [blk][B][d]
    float* dg;    // in-block logits lower(QK^T) - P M [blk][B][B]
    float* gl;    // in-block inclusive cumsum of log f [blk][B]
    float* tot;   // block sum of log f [blk]
    // cache alignment only (NULL otherwise)
    float* k32;   // Kright in float32 [blk][B][d]
    float* e32;   // E in float32 [blk][d][d]
    float* suf;   // suffix transitions S_c [blk][d][d]
    float* gpre;  // log f sum of all blocks before c [blk]
    float* grp;   // per group of blocks: whole transition and suffix [slice][g][2][d][d]
    // backward (bf16 pair kernels) only (NULL otherwise): bf16 copies of
    // scale * Kright [blk][B][d] and of -E [blk][d][d], row-major
    void* kb16;
    void* eb16;
};

struct FwdArgs {
    int N, H, L, d, block;
    bool bf16;
    float scale;
    const void *q, *k, *v, *w;
    const float *beta, *logf;
    void* o;
    float* lse;
    FwdWs ws;
    hipEvent_t* ev;   // optional phase events; ev[1] is recorded before the scan
};

struct CacheArgs {
    int N, H, d, cap;
    bool k_bf16, v_bf16;
    void* kcache;
    void* vcache;
    float* gcache;
};

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st);
bool fwd_bf16_supported(int d, int block);
size_t fwd_bf16_image_bytes(int d);

// prefill -> decode alignment (uses ws.k32 / ws.e32 written by the forward)
hipError_t launch_kv_align(const FwdArgs& a, const CacheArgs& c, hipStream_t st);
int suffix_groups(int nb);   // number of block groups the alignment chain uses

hipError_t launch_kv_update(const CacheArgs& c, int n, const void* w_t,
                            const float* beta_t, hipStream_t st);
hipError_t launch_kv_append(const CacheArgs& c, int n, const void* k_t,
                            const void* v_t, const float* logf_t, hipStream_t st);
// decode: fused = 1 also rewrites slots [0, n_keys-1) with (w_t, beta_t) and
// appends (k_t, v_t, logf_t) at slot n_keys-1 before attending.
hipError_t launch_decode(const CacheArgs& c, int n_keys, float scale,
                         const void* q_t, void* o_t, float* lse_t, float* part,
                         int chunk, bool fused, const void* k_t, const void* v_t,
                         const void* w_t, const float* beta_t,
                         const float* logf_t, hipStream_t st);
int decode_chunk(int n_keys);
int decode_max_keys();   // longest cache one decode call can attend over
// Bytes of the device-resident scratch array (one per GPU) that
// path_decode_step_noalloc uses in place of a workspace, and its device
// address on the GPU of `stream` (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
hipError_t static_scratch(hipStream_t stream, float** out);

// paged cache [page][H][P][d] (P = 1 << lp) for a batch of S sequences
struct PagedArgs {
    int S, H, d, num_pages, lp, table_stride, max_keys;
    bool k_bf16, v_bf16;
    float scale;
    void *kpages, *vpages;
    float* gpages;
    const int* tables;    // [S][table_stride] page of each P-slot range
    int* seq_lens;        // [S] keys cached (advanced by one by the step)
    const void *q_t, *k_t, *v_t, *w_t;
    const float *beta_t, *logf_t;
    void* o_t;
    float* lse_t;
    float* ws;            // partials [S*H][chunks][d+2], then n_keys [S*H] (int)
};
hipError_t launch_paged_step(const PagedArgs& a, hipStream_t st);
hipError_t launch_paged_import(const PagedArgs& a, const CacheArgs& src, hipStream_t st);
size_t paged_workspace_bytes(int S, int H, int d, int max_keys);

bool causal_supported(int d, bool bf16);
hipError_t launch_causal(const FwdArgs& a, hipStream_t st);

// the preconditioning step alone (block 64, fp32 products in ws.ql/kr/em/dg/gl/tot)
hipError_t launch_precond_f32(const FwdArgs& a, hipStream_t st);
// same on the matrix cores for bf16 d in {32, 64}: Kright and E in fp32 go to
// ws.k32 / ws.e32 (ws.img receives the scan's tile images)
hipError_t launch_precond_bf16(const FwdArgs& a, hipStream_t st);

// backward pass (block 64)
struct BwdArgs {
    int N, H, L, d;
    bool bf16;
    float scale;
    const void *q, *k, *v, *w, *o, *dout;
    const float *beta, *logf, *lse;
    void *dq, *dk, *dv, *dw;
    float *dbeta, *dlogf;
    FwdWs fw;            // recomputed preconditioning (ql, kr, em, dg, gl, tot; fp32,
                         // kr and em as bf16 rows on the bf16 matrix-core path)
    float *X, *Z;        // per block pair of a chunk of slices [slice][pair][B][d] (bf16
                         // elements for bf16 inputs at d >= 32)
    float *dQl, *dKr, *dEm, *dDg;   // per block: gradients of the preconditioned products
    float *rowsum, *colsum, *delta; // per position [blk][B]
    float* scr;          // per block of a chunk: scratch of the preconditioning's backward
    void* img;           // bf16 d in {32, 64}: tile images of the matrix-core preconditioning
    int chunk;           // slices per pass over the pair buffers
};
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);
size_t bwd_pair_floats(int L, int d, int chunk);     // X (and Z) for a chunk
size_t bwd_scratch_floats(int L, int chunk);         // scr for a chunk
int bwd_block();

// parameter front-end (w, beta, log f from a layer input)
struct ParamArgs {
    int N, L, Dm, R, H, d, Rp;
    bool bf16;
    const void *x, *Wd, *Wu, *ub, *uf;   // uf NULL: no forget gate
    const float *kc, *bb, *bf;
    void* w;
    float *beta, *logf;
    float* P;                            // workspace [N*L, Rp]
};
int param_columns(int R, int H, bool gate);   // Rp
hipError_t launch_param(const ParamArgs& a, hipStream_t st);

}  // namespace pa
