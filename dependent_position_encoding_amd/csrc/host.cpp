// host.cpp -- the C ABI of libpath_attn (declared in include/path_attn.h):
// argument validation, workspace sizing and carving, kernel dispatch.
// Every argument error is detected here, before anything is enqueued.
#include "path_attn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <string>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

path_status fail(path_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

path_status ok() {
    g_last_error.clear();
    return PATH_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// A C caller may store any int in an enum field; in C++ loading a value outside
// the enumerators' range as the enum type is undefined, so the field's bytes
// are read as an int before anything compares them.
int raw_enum(const void* field) {
    int v;
    memcpy(&v, field, sizeof v);
    return v;
}

bool valid_dtype(const path_dtype* t) {
    const int v = raw_enum(t);
    return v == PATH_F32 || v == PATH_BF16;
}

size_t esize(path_dtype t) { return t == PATH_F32 ? 4 : 2; }

int block_of(const path_fwd_desc* d) { return d->block == 0 ? 64 : d->block; }

// Which forward kernels serve this description.
bool use_mfma(const path_fwd_desc* d) {
    return d->dtype == PATH_BF16 && pa::fwd_bf16_supported(d->d, block_of(d));
}

path_status check_desc(const path_fwd_desc* d, bool need_L) {
    if (!d) return fail(PATH_E_NULL, "desc is NULL");
    if (d->N < 1 || d->H < 1 || (need_L && d->L < 1))
        return fail(PATH_E_SHAPE, "N, H and L must be >= 1");
    if (!valid_dtype(&d->dtype)) return fail(PATH_E_DTYPE, "unknown dtype");
    if (d->d != 16 && d->d != 32 && d->d != 64)
        return fail(PATH_E_UNSUPPORTED, "head dim must be 16, 32 or 64");
    const int B = block_of(d);
    if (B != 16 && B != 32 && B != 64)
        return fail(PATH_E_UNSUPPORTED, "block must be 0, 16, 32 or 64");
    if (d->dtype == PATH_BF16 && B != 64)
        return fail(PATH_E_UNSUPPORTED, "bf16 inputs use block 64");
    if ((size_t)d->N * d->H * (need_L ? d->L : 1) * d->d > ((size_t)1 << 40))
        return fail(PATH_E_SHAPE, "problem too large");
    // one slice's tile images must stay below 4 GiB (32-bit buffer offsets)
    if (need_L && d->L > (1 << 23))
        return fail(PATH_E_SHAPE, "L must be at most 8388608");
    return PATH_OK;
}

struct Layout {
    size_t kr, em, img, ql, dg, gl, tot, k32, e32, suf, gpre, grp, total;
};

Layout fwd_layout(const path_fwd_desc* d, bool with_cache) {
    const int B = block_of(d), D = d->d;
    const size_t nb = (size_t)(d->L + B - 1) / B;
    const size_t nblk = (size_t)d->N * d->H * nb;
    const bool mf = use_mfma(d);
    const size_t op = mf ? 2 : 4;       // operand element size
    Layout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
    if (mf) {
        l.img = take(nblk * pa::fwd_bf16_image_bytes(D));
    } else {
        l.kr = take(nblk * B * D * op);
        l.em = take(nblk * D * D * op);
    }
    l.ql = take(nblk * B * D * 4);
    l.dg = take(nblk * B * B * 4);
    l.gl = take(nblk * B * 4);
    l.tot = take(nblk * 4);
    if (with_cache) {
        l.k32 = take(nblk * B * D * 4);
        l.e32 = take(nblk * D * D * 4);
        l.suf = take(nblk * D * D * 4);
        l.gpre = take(nblk * 4);
        l.grp = take((size_t)d->N * d->H * pa::suffix_groups((int)nb) * 2 * D * D * 4);
    }
    l.total = off;
    return l;
}

path_status check_cache(const path_fwd_desc* d, const path_cache* c) {
    if (!c) return fail(PATH_E_NULL, "cache is NULL");
    if (!c->kcache || !c->vcache) return fail(PATH_E_NULL, "kcache/vcache is NULL");
    if (c->cap < 1) return fail(PATH_E_SHAPE, "cache capacity must be >= 1");
    if (!valid_dtype(&c->k_dtype)) return fail(PATH_E_DTYPE, "unknown kcache dtype");
    if (!aligned(c->kcache, 16) || !aligned(c->vcache, 16) || !aligned(c->gcache, 4))
        return fail(PATH_E_ALIGN, "cache pointers must be 16-byte aligned (gcache 4)");
    (void)d;
    return PATH_OK;
}

pa::CacheArgs cache_args(const path_fwd_desc* d, const path_cache* c) {
    pa::CacheArgs a;
    a.N = d->N; a.H = d->H; a.d = d->d; a.cap = c->cap;
    a.k_bf16 = c->k_dtype == PATH_BF16;
    a.v_bf16 = d->dtype == PATH_BF16;
    a.kcache = c->kcache; a.vcache = c->vcache; a.gcache = c->gcache;
    return a;
}

path_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess)
        return fail(PATH_E_LAUNCH, std::string(what) + ": " + hipGetErrorString(e));
    return ok();
}

// Backward workspace: the recomputed preconditioning, per-block gradients,
// per-position sums, then the pair buffers and scratch for `chunk` slices at a
// time (chunk chosen so those stay within kBwdChunkBytes).
constexpr size_t kBwdChunkBytes = (size_t)4 << 30;

struct BwdLayout {
    size_t ql, kr, em, dg, gl, tot, dQl, dKr, dEm, dDg, rowsum, colsum, delta, X, Z, scr, img, total;
    bool mfma_precond;
    int chunk;
};

BwdLayout bwd_layout(const path_fwd_desc* d) {
    const int B = pa::bwd_block(), D = d->d;
    const size_t nb = (size_t)(d->L + B - 1) / B, ns = (size_t)d->N * d->H, nblk = ns * nb;
    // bf16 at d >= 32: the pair buffers hold bf16 and the preconditioning's
    // backward keeps its intermediates in LDS (no scratch area)
    const bool b16 = d->dtype == PATH_BF16 && D >= 32;
    const size_t pair_el = b16 ? 2 : 4;
    const size_t scr_el = b16 ? 0 : 4;
    const size_t per_slice = 2 * pair_el * pa::bwd_pair_floats(d->L, D, 1) +
                             scr_el * pa::bwd_scratch_floats(d->L, 1);
    size_t chunk = per_slice ? kBwdChunkBytes / per_slice : ns;
    chunk = chunk < 1 ? 1 : (chunk > ns ? ns : chunk);
    BwdLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += up256(bytes); return o; };
    l.ql = take(nblk * B * D * 4);
    l.kr = take(nblk * B * D * 4);
    l.em = take(nblk * D * D * 4);
    l.dg = take(nblk * B * B * 4);
    l.gl = take(nblk * B * 4);
    l.tot = take(nblk * 4);
    l.dQl = take(nblk * B * D * 4);
    l.dKr = take(nblk * B * D * 4);
    l.dEm = take(nblk * D * D * 4);
    l.dDg = take(nblk * B * B * 4);
    l.rowsum = take(nblk * B * 4);
    l.colsum = take(nblk * B * 4);
    l.delta = take(nblk * B * 4);
    l.X = take(pair_el * pa::bwd_pair_floats(d->L, D, (int)chunk));
    l.Z = take(pair_el * pa::bwd_pair_floats(d->L, D, (int)chunk));
    l.scr = take(scr_el * pa::bwd_scratch_floats(d->L, (int)chunk));
    l.mfma_precond = d->dtype == PATH_BF16 && pa::fwd_bf16_supported(D, B);
    if (l.mfma_precond) l.img = take(nblk * pa::fwd_bf16_image_bytes(D));
    l.total = off;
    l.chunk = (int)chunk;
    return l;
}

path_status check_param(const path_param_desc* d) {
    if (!d) return fail(PATH_E_NULL, "desc is NULL");
    if (d->N < 1 || d->L < 1 || d->H < 1 || d->Dm < 1 || d->R < 1)
        return fail(PATH_E_SHAPE, "N, L, H, Dm and R must be >= 1");
    if (!valid_dtype(&d->dtype)) return fail(PATH_E_DTYPE, "unknown dtype");
    if (d->d != 16 && d->d != 32 && d->d != 64)
        return fail(PATH_E_UNSUPPORTED, "head dim must be 16, 32 or 64");
    if (d->Dm % 16 != 0) return fail(PATH_E_UNSUPPORTED, "Dm must be a multiple of 16");
    if (d->R % 16 != 0 || d->R > 256)
        return fail(PATH_E_UNSUPPORTED, "R must be a multiple of 16, at most 256");
    if (d->Dm > 65536) return fail(PATH_E_UNSUPPORTED, "Dm must be at most 65536");
    // the kernels address x rows, weight matrices and a sequence's rows of the
    // intermediate through 32-bit buffer ranges
    if ((size_t)d->N * d->L > ((size_t)1 << 31) || (size_t)d->H * d->d > 65536 ||
        (size_t)d->N * d->L * d->Dm > ((size_t)1 << 40) ||
        (size_t)d->L * pa::param_columns(d->R, d->H, true) * 4 > ((size_t)1 << 30))
        return fail(PATH_E_SHAPE, "problem too large");
    return PATH_OK;
}

size_t param_ws(const path_param_desc* d, bool gate) {
    return up256((size_t)d->N * d->L * pa::param_columns(d->R, d->H, gate) * 4);
}

}  // namespace

extern "C" {

int path_abi_version(void) { return PATH_ATTN_ABI_VERSION; }

const char* path_status_str(path_status s) {
    switch (raw_enum(&s)) {
        case PATH_OK: return "ok";
        case PATH_E_NULL: return "null pointer";
        case PATH_E_SHAPE: return "bad shape";
        case PATH_E_DTYPE: return "bad dtype";
        case PATH_E_UNSUPPORTED: return "unsupported";
        case PATH_E_ALIGN: return "misaligned pointer";
        case PATH_E_WORKSPACE: return "workspace too small";
        case PATH_E_CAPACITY: return "cache capacity exceeded";
        case PATH_E_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

const char* path_last_error(void) { return g_last_error.c_str(); }

size_t path_attn_fwd_workspace(const path_fwd_desc* desc, int with_cache) {
    if (check_desc(desc, true) != PATH_OK) return 0;
    return fwd_layout(desc, with_cache != 0).total;
}

static path_status fwd_impl(const path_fwd_desc* desc, const void* q, const void* k,
                            const void* v, const void* w, const float* beta,
                            const float* logf, void* o, float* lse,
                            const path_cache* cache_out, void* ws, size_t ws_bytes,
                            hipStream_t stream, hipEvent_t* ev) {
    path_status s = check_desc(desc, true);
    if (s != PATH_OK) return s;
    if (!q || !k || !v || !w || !beta || !o) return fail(PATH_E_NULL, "q, k, v, w, beta and o are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(w, 16) || !aligned(o, 16))
        return fail(PATH_E_ALIGN, "q, k, v, w and o must be 16-byte aligned");
    if (!aligned(beta, 4) || !aligned(logf, 4) || !aligned(lse, 4))
        return fail(PATH_E_ALIGN, "beta, logf and lse must be 4-byte aligned");
    if (cache_out) {
        s = check_cache(desc, cache_out);
        if (s != PATH_OK) return s;
        if (cache_out->cap < desc->L) return fail(PATH_E_CAPACITY, "cache capacity below L");
    }
    const Layout lay = fwd_layout(desc, cache_out != nullptr);
    if (!ws) return fail(PATH_E_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(PATH_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < lay.total) return fail(PATH_E_WORKSPACE, "workspace smaller than path_attn_fwd_workspace()");

    char* base = static_cast<char*>(ws);
    pa::FwdArgs a{};
    a.N = desc->N; a.H = desc->H; a.L = desc->L; a.d = desc->d; a.block = block_of(desc);
    a.bf16 = desc->dtype == PATH_BF16; a.scale = desc->scale;
    a.q = q; a.k = k; a.v = v; a.w = w; a.beta = beta; a.logf = logf; a.o = o; a.lse = lse;
    const bool mf = use_mfma(desc);
    a.ws.kr = mf ? nullptr : base + lay.kr;
    a.ws.em = mf ? nullptr : base + lay.em;
    a.ws.img = mf ? base + lay.img : nullptr;
    a.ws.ql = reinterpret_cast<float*>(base + lay.ql);
    a.ws.dg = reinterpret_cast<float*>(base + lay.dg);
    a.ws.gl = reinterpret_cast<float*>(base + lay.gl);
    a.ws.tot = reinterpret_cast<float*>(base + lay.tot);
    if (cache_out) {
        a.ws.k32 = reinterpret_cast<float*>(base + lay.k32);
        a.ws.e32 = reinterpret_cast<float*>(base + lay.e32);
        a.ws.suf = reinterpret_cast<float*>(base + lay.suf);
        a.ws.gpre = reinterpret_cast<float*>(base + lay.gpre);
        a.ws.grp = reinterpret_cast<float*>(base + lay.grp);
    }
    a.ev = ev;
    hipError_t e = hipSuccess;
    if (ev && (e = hipEventRecord(ev[0], stream)) != hipSuccess)
        return launched(e, "path_attn_fwd_timed (event 0)");
    e = use_mfma(desc) ? pa::launch_fwd_bf16(a, stream) : pa::launch_fwd_f32(a, stream);
    if (e != hipSuccess) return launched(e, "path_attn_fwd");
    if (ev && (e = hipEventRecord(ev[2], stream)) != hipSuccess)
        return launched(e, "path_attn_fwd_timed (event 2)");
    if (cache_out) {
        e = pa::launch_kv_align(a, cache_args(desc, cache_out), stream);
        if (e != hipSuccess) return launched(e, "path_attn_fwd (cache alignment)");
    }
    if (ev && (e = hipEventRecord(ev[3], stream)) != hipSuccess)
        return launched(e, "path_attn_fwd_timed (event 3)");
    return ok();
}

path_status path_attn_fwd(const path_fwd_desc* desc, const void* q, const void* k,
                          const void* v, const void* w, const float* beta,
                          const float* logf, void* o, float* lse,
                          const path_cache* cache_out, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    return fwd_impl(desc, q, k, v, w, beta, logf, o, lse, cache_out, ws, ws_bytes, stream,
                    nullptr);
}

path_status path_attn_fwd_timed(const path_fwd_desc* desc, const void* q, const void* k,
                                const void* v, const void* w, const float* beta,
                                const float* logf, void* o, float* lse,
                                const path_cache* cache_out, void* ws, size_t ws_bytes,
                                hipStream_t stream, hipEvent_t ev[4]) {
    if (!ev || !ev[0] || !ev[1] || !ev[2] || !ev[3]) return fail(PATH_E_NULL, "four events are required");
    return fwd_impl(desc, q, k, v, w, beta, logf, o, lse, cache_out, ws, ws_bytes, stream, ev);
}

path_status path_kv_update(const path_fwd_desc* desc, const path_cache* cache, int n,
                           const void* w_t, const float* beta_t, hipStream_t stream) {
    path_status s = check_desc(desc, false);
    if (s != PATH_OK) return s;
    if ((s = check_cache(desc, cache)) != PATH_OK) return s;
    if (!w_t || !beta_t) return fail(PATH_E_NULL, "w_t and beta_t are required");
    if (!aligned(w_t, 16) || !aligned(beta_t, 4)) return fail(PATH_E_ALIGN, "w_t must be 16-byte aligned");
    if (n < 0) return fail(PATH_E_SHAPE, "n must be >= 0");
    if (n > cache->cap) return fail(PATH_E_CAPACITY, "n exceeds cache capacity");
    return launched(pa::launch_kv_update(cache_args(desc, cache), n, w_t, beta_t, stream),
                    "path_kv_update");
}

path_status path_kv_append(const path_fwd_desc* desc, const path_cache* cache, int n,
                           const void* k_t, const void* v_t, const float* logf_t,
                           hipStream_t stream) {
    path_status s = check_desc(desc, false);
    if (s != PATH_OK) return s;
    if ((s = check_cache(desc, cache)) != PATH_OK) return s;
    if (!k_t || !v_t) return fail(PATH_E_NULL, "k_t and v_t are required");
    if (cache->gcache && !logf_t) return fail(PATH_E_NULL, "logf_t is required when gcache is set");
    if (!aligned(k_t, 16) || !aligned(v_t, 16) || !aligned(logf_t, 4))
        return fail(PATH_E_ALIGN, "k_t and v_t must be 16-byte aligned");
    if (n < 0) return fail(PATH_E_SHAPE, "n must be >= 0");
    if (n >= cache->cap) return fail(PATH_E_CAPACITY, "slot n is beyond the cache capacity");
    return launched(pa::launch_kv_append(cache_args(desc, cache), n, k_t, v_t, logf_t, stream),
                    "path_kv_append");
}

size_t path_decode_workspace(const path_fwd_desc* desc, int n_keys) {
    if (check_desc(desc, false) != PATH_OK || n_keys < 1) return 0;
    const int chunk = pa::decode_chunk(n_keys);
    const size_t nch = (size_t)(n_keys + chunk - 1) / chunk;
    return up256((size_t)desc->N * desc->H * nch * (desc->d + 2) * 4);
}

static path_status decode_common(const path_fwd_desc* desc, const path_cache* cache,
                                 int n_keys, const void* q_t, void* o_t, float* lse_t,
                                 void* ws, size_t ws_bytes, bool fused, const void* k_t,
                                 const void* v_t, const void* w_t, const float* beta_t,
                                 const float* logf_t, hipStream_t stream, const char* name,
                                 bool validate_only = false) {
    path_status s = check_desc(desc, false);
    if (s != PATH_OK) return s;
    if ((s = check_cache(desc, cache)) != PATH_OK) return s;
    if (!q_t || !o_t) return fail(PATH_E_NULL, "q_t and o_t are required");
    if (!aligned(q_t, 16) || !aligned(o_t, 16) || !aligned(lse_t, 4))
        return fail(PATH_E_ALIGN, "q_t and o_t must be 16-byte aligned");
    if (n_keys < 1) return fail(PATH_E_SHAPE, "at least one key is required");
    if (n_keys > cache->cap) return fail(PATH_E_CAPACITY, "keys exceed cache capacity");
    if (n_keys > pa::decode_max_keys())
        return fail(PATH_E_UNSUPPORTED, "decode attends over at most 131072 keys per call");
    if (validate_only) return PATH_OK;
    if (!ws) return fail(PATH_E_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(PATH_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < path_decode_workspace(desc, n_keys))
        return fail(PATH_E_WORKSPACE, "workspace smaller than path_decode_workspace()");
    return launched(pa::launch_decode(cache_args(desc, cache), n_keys, desc->scale, q_t, o_t,
                                      lse_t, static_cast<float*>(ws),
                                      pa::decode_chunk(n_keys), fused, k_t, v_t, w_t, beta_t,
                                      logf_t, stream),
                    name);
}

path_status path_decode(const path_fwd_desc* desc, const path_cache* cache, int n_keys,
                        const void* q_t, void* o_t, float* lse_t, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
    return decode_common(desc, cache, n_keys, q_t, o_t, lse_t, ws, ws_bytes, false, nullptr,
                         nullptr, nullptr, nullptr, nullptr, stream, "path_decode");
}

// The token arguments of a fused step (shared by path_decode_step and
// path_decode_step_noalloc).
static path_status check_step_token(const path_cache* cache, int n, const void* k_t,
                                    const void* v_t, const void* w_t, const float* beta_t,
                                    const float* logf_t) {
    if (!k_t || !v_t || !w_t || !beta_t) return fail(PATH_E_NULL, "k_t, v_t, w_t and beta_t are required");
    if (!aligned(k_t, 16) || !aligned(v_t, 16) || !aligned(w_t, 16) || !aligned(beta_t, 4) ||
        !aligned(logf_t, 4))
        return fail(PATH_E_ALIGN, "k_t, v_t and w_t must be 16-byte aligned");
    if (cache && cache->gcache && !logf_t) return fail(PATH_E_NULL, "logf_t is required when gcache is set");
    if (n < 0) return fail(PATH_E_SHAPE, "n must be >= 0");
    if (cache && n >= cache->cap) return fail(PATH_E_CAPACITY, "slot n is beyond the cache capacity");
    return PATH_OK;
}

path_status path_decode_step(const path_fwd_desc* desc, const path_cache* cache, int n,
                             const void* q_t, const void* k_t, const void* v_t,
                             const void* w_t, const float* beta_t, const float* logf_t,
                             void* o_t, float* lse_t, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    path_status s = check_step_token(cache, n, k_t, v_t, w_t, beta_t, logf_t);
    if (s != PATH_OK) return s;
    return decode_common(desc, cache, n + 1, q_t, o_t, lse_t, ws, ws_bytes, true, k_t, v_t,
                         w_t, beta_t, logf_t, stream, "path_decode_step");
}

size_t path_decode_step_noalloc_limit(void) { return pa::kStaticScratchBytes; }

path_status path_decode_step_noalloc(const path_fwd_desc* desc, const path_cache* cache, int n,
                                     const void* q_t, const void* k_t, const void* v_t,
                                     const void* w_t, const float* beta_t, const float* logf_t,
                                     void* o_t, float* lse_t, hipStream_t stream) {
    path_status s = check_step_token(cache, n, k_t, v_t, w_t, beta_t, logf_t);
    if (s != PATH_OK) return s;
    if ((s = check_desc(desc, false)) != PATH_OK) return s;
    const size_t need = path_decode_workspace(desc, n + 1);
    if (need > pa::kStaticScratchBytes)
        return fail(PATH_E_WORKSPACE,
                    "this step needs " + std::to_string(need) + " bytes of scratch; the "
                    "library's static scratch holds " + std::to_string(pa::kStaticScratchBytes) +
                    " (use path_decode_step with a workspace)");
    // Everything else is checked (and reported) exactly as path_decode_step
    // checks it before the scratch address is looked up.
    if ((s = decode_common(desc, cache, n + 1, q_t, o_t, lse_t, nullptr, 0, true, k_t, v_t,
                           w_t, beta_t, logf_t, stream, "path_decode_step_noalloc",
                           /*validate_only=*/true)) != PATH_OK)
        return s;
    float* scratch = nullptr;
    hipError_t e = pa::static_scratch(stream, &scratch);
    if (e != hipSuccess) return launched(e, "path_decode_step_noalloc (scratch address)");
    return decode_common(desc, cache, n + 1, q_t, o_t, lse_t, scratch, pa::kStaticScratchBytes,
                         true, k_t, v_t, w_t, beta_t, logf_t, stream, "path_decode_step_noalloc");
}

// ---- paged cache

static path_status check_paged(const path_fwd_desc* d, const path_paged_cache* c,
                               const int* table, int table_stride, const int* seq_lens,
                               int max_keys, int* lp) {
    if (!c) return fail(PATH_E_NULL, "paged cache is NULL");
    if (!c->kpages || !c->vpages) return fail(PATH_E_NULL, "kpages/vpages is NULL");
    if (!table || !seq_lens) return fail(PATH_E_NULL, "page_table and seq_lens are required");
    if (!valid_dtype(&c->k_dtype)) return fail(PATH_E_DTYPE, "unknown kpages dtype");
    int l = 0;
    while (l < 8 && (1 << l) != c->page_size) ++l;
    if (l < 4 || l > 7) return fail(PATH_E_UNSUPPORTED, "page_size must be 16, 32, 64 or 128");
    if (c->num_pages < 1) return fail(PATH_E_SHAPE, "num_pages must be >= 1");
    if ((size_t)c->num_pages * d->H * c->page_size * d->d > ((size_t)1 << 40))
        return fail(PATH_E_SHAPE, "paged cache too large");
    if (max_keys < 1) return fail(PATH_E_SHAPE, "max_keys must be >= 1");
    if (max_keys > pa::decode_max_keys())
        return fail(PATH_E_UNSUPPORTED, "decode attends over at most 131072 keys per sequence");
    if (table_stride < (max_keys + c->page_size - 1) / c->page_size)
        return fail(PATH_E_SHAPE, "table_stride below ceil(max_keys / page_size)");
    if (!aligned(c->kpages, 16) || !aligned(c->vpages, 16) || !aligned(c->gpages, 4) ||
        !aligned(table, 4) || !aligned(seq_lens, 4))
        return fail(PATH_E_ALIGN, "page pointers must be 16-byte aligned (gpages, tables 4)");
    *lp = l;
    return PATH_OK;
}

static pa::PagedArgs paged_args(const path_fwd_desc* d, const path_paged_cache* c,
                                const int* table, int table_stride, int* seq_lens,
                                int max_keys, int lp) {
    pa::PagedArgs a{};
    a.S = d->N; a.H = d->H; a.d = d->d; a.num_pages = c->num_pages; a.lp = lp;
    a.table_stride = table_stride; a.max_keys = max_keys;
    a.k_bf16 = c->k_dtype == PATH_BF16; a.v_bf16 = d->dtype == PATH_BF16;
    a.scale = d->scale;
    a.kpages = c->kpages; a.vpages = c->vpages; a.gpages = c->gpages;
    a.tables = table; a.seq_lens = seq_lens;
    return a;
}

size_t path_paged_decode_workspace(const path_fwd_desc* desc, int max_keys) {
    if (check_desc(desc, false) != PATH_OK || max_keys < 1 || max_keys > pa::decode_max_keys())
        return 0;
    return up256(pa::paged_workspace_bytes(desc->N, desc->H, desc->d, max_keys));
}

path_status path_paged_decode_step(const path_fwd_desc* desc, const path_paged_cache* cache,
                                   const int* page_table, int table_stride, int* seq_lens,
                                   int max_keys, const void* q_t, const void* k_t,
                                   const void* v_t, const void* w_t, const float* beta_t,
                                   const float* logf_t, void* o_t, float* lse_t, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
    path_status s = check_desc(desc, false);
    if (s != PATH_OK) return s;
    int lp = 0;
    if ((s = check_paged(desc, cache, page_table, table_stride, seq_lens, max_keys, &lp)) != PATH_OK)
        return s;
    if (!q_t || !k_t || !v_t || !w_t || !beta_t || !o_t)
        return fail(PATH_E_NULL, "q_t, k_t, v_t, w_t, beta_t and o_t are required");
    if (cache->gpages && !logf_t) return fail(PATH_E_NULL, "logf_t is required when gpages is set");
    if (!aligned(q_t, 16) || !aligned(k_t, 16) || !aligned(v_t, 16) || !aligned(w_t, 16) ||
        !aligned(o_t, 16) || !aligned(beta_t, 4) || !aligned(logf_t, 4) || !aligned(lse_t, 4))
        return fail(PATH_E_ALIGN, "q_t, k_t, v_t, w_t and o_t must be 16-byte aligned");
    if (!ws) return fail(PATH_E_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(PATH_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < path_paged_decode_workspace(desc, max_keys))
        return fail(PATH_E_WORKSPACE, "workspace smaller than path_paged_decode_workspace()");
    pa::PagedArgs a = paged_args(desc, cache, page_table, table_stride, seq_lens, max_keys, lp);
    a.q_t = q_t; a.k_t = k_t; a.v_t = v_t; a.w_t = w_t; a.beta_t = beta_t;
    a.logf_t = cache->gpages ? logf_t : nullptr;
    a.o_t = o_t; a.lse_t = lse_t;
    a.ws = static_cast<float*>(ws);
    return launched(pa::launch_paged_step(a, stream), "path_paged_decode_step");
}

path_status path_paged_import(const path_fwd_desc* desc, const path_cache* src,
                              const path_paged_cache* dst, const int* page_table,
                              int table_stride, const int* seq_lens, int max_keys,
                              hipStream_t stream) {
    path_status s = check_desc(desc, false);
    if (s != PATH_OK) return s;
    if ((s = check_cache(desc, src)) != PATH_OK) return s;
    int lp = 0;
    if ((s = check_paged(desc, dst, page_table, table_stride, seq_lens, max_keys, &lp)) != PATH_OK)
        return s;
    if (src->k_dtype != dst->k_dtype) return fail(PATH_E_DTYPE, "kcache and kpages dtypes differ");
    if ((src->gcache == nullptr) != (dst->gpages == nullptr))
        return fail(PATH_E_NULL, "gcache and gpages must be given together");
    pa::PagedArgs a = paged_args(desc, dst, page_table, table_stride,
                                 const_cast<int*>(seq_lens), max_keys, lp);
    return launched(pa::launch_paged_import(a, cache_args(desc, src), stream), "path_paged_import");
}

path_status path_causal_attn_fwd(const path_fwd_desc* desc, const void* q, const void* k,
                                 const void* v, void* o, float* lse, hipStream_t stream) {
    path_status s = check_desc(desc, true);
    if (s != PATH_OK) return s;
    if (!q || !k || !v || !o) return fail(PATH_E_NULL, "q, k, v and o are required");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return fail(PATH_E_ALIGN, "q, k, v and o must be 16-byte aligned");
    if (!pa::causal_supported(desc->d, desc->dtype == PATH_BF16))
        return fail(PATH_E_UNSUPPORTED, "the causal baseline takes bf16 with head dim 32 or 64");
    pa::FwdArgs a{};
    a.N = desc->N; a.H = desc->H; a.L = desc->L; a.d = desc->d; a.block = 64;
    a.bf16 = desc->dtype == PATH_BF16; a.scale = desc->scale;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    return launched(pa::launch_causal(a, stream), "path_causal_attn_fwd");
}

size_t path_attn_bwd_workspace(const path_fwd_desc* desc) {
    if (check_desc(desc, true) != PATH_OK || block_of(desc) != pa::bwd_block()) return 0;
    return bwd_layout(desc).total;
}

path_status path_attn_bwd(const path_fwd_desc* desc, const void* q, const void* k,
                          const void* v, const void* w, const float* beta, const float* logf,
                          const void* o, const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* dw, float* dbeta, float* dlogf, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    path_status s = check_desc(desc, true);
    if (s != PATH_OK) return s;
    if (block_of(desc) != pa::bwd_block())
        return fail(PATH_E_UNSUPPORTED, "the backward pass uses block 64");
    if (!q || !k || !v || !w || !beta || !o || !lse || !dout || !dq || !dk || !dv || !dw ||
        !dbeta)
        return fail(PATH_E_NULL, "q, k, v, w, beta, o, lse, dout, dq, dk, dv, dw and dbeta are required");
    if ((logf != nullptr) != (dlogf != nullptr))
        return fail(PATH_E_NULL, "logf and dlogf must be given together");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(w, 16) ||
        !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dv, 16) || !aligned(dw, 16))
        return fail(PATH_E_ALIGN, "tensors of [N,H,L,d] must be 16-byte aligned");
    if (!aligned(beta, 4) || !aligned(logf, 4) || !aligned(lse, 4) || !aligned(dbeta, 4) ||
        !aligned(dlogf, 4))
        return fail(PATH_E_ALIGN, "beta, logf, lse, dbeta and dlogf must be 4-byte aligned");
    const BwdLayout lay = bwd_layout(desc);
    if (!ws) return fail(PATH_E_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(PATH_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < lay.total) return fail(PATH_E_WORKSPACE, "workspace smaller than path_attn_bwd_workspace()");
    char* base = static_cast<char*>(ws);
    auto at = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
    pa::BwdArgs a{};
    a.N = desc->N; a.H = desc->H; a.L = desc->L; a.d = desc->d;
    a.bf16 = desc->dtype == PATH_BF16; a.scale = desc->scale;
    a.q = q; a.k = k; a.v = v; a.w = w; a.o = o; a.dout = dout;
    a.beta = beta; a.logf = logf; a.lse = lse;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dw = dw; a.dbeta = dbeta; a.dlogf = dlogf;
    a.fw.ql = at(lay.ql); a.fw.kr = at(lay.kr); a.fw.em = at(lay.em); a.fw.dg = at(lay.dg);
    a.fw.gl = at(lay.gl); a.fw.tot = at(lay.tot);
    a.X = at(lay.X); a.Z = at(lay.Z);
    a.dQl = at(lay.dQl); a.dKr = at(lay.dKr); a.dEm = at(lay.dEm); a.dDg = at(lay.dDg);
    a.rowsum = at(lay.rowsum); a.colsum = at(lay.colsum); a.delta = at(lay.delta);
    a.scr = at(lay.scr);
    a.img = lay.mfma_precond ? base + lay.img : nullptr;
    a.chunk = lay.chunk;
    return launched(pa::launch_bwd(a, stream), "path_attn_bwd");
}

size_t path_param_workspace(const path_param_desc* desc, int with_gate) {
    if (check_param(desc) != PATH_OK) return 0;
    return param_ws(desc, with_gate != 0);
}

path_status path_param_fwd(const path_param_desc* desc, const void* x, const void* Wd,
                           const void* Wu, const float* kc, const void* ub, const float* bb,
                           const void* uf, const float* bf, void* w, float* beta, float* logf,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    path_status s = check_param(desc);
    if (s != PATH_OK) return s;
    if (!x || !Wd || !Wu || !kc || !ub || !bb || !w || !beta || !ws)
        return fail(PATH_E_NULL, "x, Wd, Wu, kc, ub, bb, w, beta and ws are required");
    const bool gate = uf != nullptr;
    if (gate != (bf != nullptr) || gate != (logf != nullptr))
        return fail(PATH_E_NULL, "uf, bf and logf must be given together");
    if (!aligned(x, 16) || !aligned(Wd, 16) || !aligned(Wu, 16) || !aligned(ub, 16) ||
        !aligned(uf, 16) || !aligned(w, 16))
        return fail(PATH_E_ALIGN, "x, Wd, Wu, ub, uf and w must be 16-byte aligned");
    if (!aligned(kc, 4) || !aligned(bb, 4) || !aligned(bf, 4) || !aligned(beta, 4) ||
        !aligned(logf, 4))
        return fail(PATH_E_ALIGN, "kc, bb, bf, beta and logf must be 4-byte aligned");
    if (!aligned(ws, 256)) return fail(PATH_E_ALIGN, "workspace must be 256-byte aligned");
    if (ws_bytes < param_ws(desc, gate)) return fail(PATH_E_WORKSPACE, "workspace too small");
    pa::ParamArgs a{};
    a.N = desc->N; a.L = desc->L; a.Dm = desc->Dm; a.R = desc->R; a.H = desc->H; a.d = desc->d;
    a.Rp = pa::param_columns(desc->R, desc->H, gate);
    a.bf16 = desc->dtype == PATH_BF16;
    a.x = x; a.Wd = Wd; a.Wu = Wu; a.ub = ub; a.uf = uf;
    a.kc = kc; a.bb = bb; a.bf = bf;
    a.w = w; a.beta = beta; a.logf = logf;
    a.P = static_cast<float*>(ws);
    return launched(pa::launch_param(a, stream), "path_param_fwd");
}

}  // extern "C"
