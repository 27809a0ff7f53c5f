// decode.hip -- decoding over a rewritten key cache, and the prefill-to-cache
// alignment.  All kernels here are bound by HBM bandwidth: each cached key
// row is read (and, for the rewrite, written) once per call with 16-byte
// vector accesses.
//
// Citations: [Notes s2.x] = reading-notes page "PaTH Attention:通过累积
// Householder 变换编码位置" (cc.laoqi.cc), section 2.x; [Explainer s3] =
// explainer page "PaTH Attention: Position Encoding via Accumulating
// Householder Transformations" (gist.science), section 3.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace pa {

// 16 bytes of a row: 8 bf16 or 4 float32 values.
template <typename T> struct Vec;
template <> struct Vec<bf16> {
    static constexpr int n = 8;
    uint4 raw;
    __device__ void load(const bf16* p) { raw = *reinterpret_cast<const uint4*>(p); }
    __device__ void store(bf16* p) const { *reinterpret_cast<uint4*>(p) = raw; }
    __device__ float get(int i) const {
        uint32_t wd = (&raw.x)[i >> 1];
        union { uint32_t u; float f; } c;
        c.u = (i & 1) ? (wd & 0xffff0000u) : (wd << 16);
        return c.f;
    }
    __device__ void set(int i, float f) {
        uint32_t b = f32_to_bf16(f).bits;
        uint32_t& wd = (&raw.x)[i >> 1];
        wd = (i & 1) ? ((wd & 0x0000ffffu) | (b << 16)) : ((wd & 0xffff0000u) | b);
    }
};
template <> struct Vec<float> {
    static constexpr int n = 4;
    float4 raw;
    __device__ void load(const float* p) { raw = *reinterpret_cast<const float4*>(p); }
    __device__ void store(float* p) const { *reinterpret_cast<float4*>(p) = raw; }
    __device__ float get(int i) const { return (&raw.x)[i]; }
    __device__ void set(int i, float f) { (&raw.x)[i] = f; }
};

// N values of type T kept as raw bits (loaded with one wide access).
template <typename T, int N>
struct Raw {
    static constexpr int W = N * (int)sizeof(T) / 4;
    uint32_t w[W];
    __device__ void load(const T* p) {
        if constexpr (W == 4) {
            const uint4 x = *reinterpret_cast<const uint4*>(p);
            w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        } else if constexpr (W == 2) {
            const uint2 x = *reinterpret_cast<const uint2*>(p);
            w[0] = x.x; w[1] = x.y;
        } else {
#pragma unroll
            for (int i = 0; i < W; i += 4) {
                const uint4 x = reinterpret_cast<const uint4*>(p)[i / 4];
                w[i] = x.x; w[i + 1] = x.y; w[i + 2] = x.z; w[i + 3] = x.w;
            }
        }
    }
    __device__ float get(int i) const {
        union { uint32_t u; float f; } c;
        if constexpr (sizeof(T) == 2) c.u = (i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16);
        else c.u = w[i];
        return c.f;
    }
};

// Sum over the TPR consecutive lanes that share one row.
template <int TPR>
__device__ inline float group_sum(float x) {
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------------------
// Cache rewrite for a new position [Notes s2.8, eq. (1)]:
//   k_j <- k_j - beta_t (w_t . k_j) w_t  for j in [0, n).
// Grid: (row tiles, slices).  Each group of TPR lanes owns one row.
template <typename K, typename T, int D>
__global__ void __launch_bounds__(256)
kv_update_kernel(K* __restrict__ kc, int cap, int n, const T* __restrict__ w_t,
                 const float* __restrict__ beta_t, int rows_per_block) {
    constexpr int VN = Vec<K>::n, TPR = D / VN, GROUPS = 256 / TPR;
    const int slice = blockIdx.y;
    const int lane_in = threadIdx.x % TPR, grp = threadIdx.x / TPR;
    float wv[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) wv[e] = to_f32(w_t[(size_t)slice * D + lane_in * VN + e]);
    const float bt = beta_t[slice];
    K* base = kc + (size_t)slice * cap * D;
    const int j0 = blockIdx.x * rows_per_block;
    const int j1 = min(n, j0 + rows_per_block);
    for (int j = j0 + grp; j < j1; j += GROUPS) {
        Vec<K> x;
        x.load(base + (size_t)j * D + lane_in * VN);
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < VN; ++e) p += wv[e] * x.get(e);
        const float cf = bt * group_sum<TPR>(p);
#pragma unroll
        for (int e = 0; e < VN; ++e) x.set(e, x.get(e) - cf * wv[e]);
        x.store(base + (size_t)j * D + lane_in * VN);
    }
}

// Append one token at slot n: its key unrewritten, its value, and the
// inclusive log-f prefix.  One block per slice.
template <typename K, typename T, int D>
__global__ void kv_append_kernel(K* __restrict__ kc, T* __restrict__ vc,
                                 float* __restrict__ gc, int cap, int n,
                                 const T* __restrict__ k_t, const T* __restrict__ v_t,
                                 const float* __restrict__ logf_t) {
    const int slice = blockIdx.x;
    const size_t slot = ((size_t)slice * cap + n) * D;
    for (int x = threadIdx.x; x < D; x += blockDim.x) {
        kc[slot + x] = from_f32<K>(to_f32(k_t[(size_t)slice * D + x]));
        vc[slot + x] = v_t[(size_t)slice * D + x];
    }
    if (gc && threadIdx.x == 0) {
        const float prev = n > 0 ? gc[(size_t)slice * cap + n - 1] : 0.f;
        gc[(size_t)slice * cap + n] = prev + logf_t[slice];
    }
}

// ---------------------------------------------------------------------------
// Single-query attention over one chunk of cached keys, optionally fused with
// the rewrite and the append of the current token [Notes s2.8].
//   score_j = scale * q_t . k_j + (C_t - C_j),  C = inclusive log-f prefix.
// A chunk is kDecChunk keys; each group of TPR lanes owns one 16-byte slice
// of a row and handles KPG keys spaced GROUPS apart.  All of a group's key,
// value and prefix loads are issued before any arithmetic (KPG rows in flight
// per group), then one max / sum / weighted value sum over its keys.  Groups
// are merged through LDS and the chunk's partial softmax state
// (m, l, acc[D]) goes to `out`.
//
// Where slot j of a slice lives is a policy: its key row starts at element
// Rows::off(j) of Rows::k0 and its value row at the same offset of Rows::v0;
// Rows::g(j) points at its log-f prefix entry (Rows::gate() false: no gate).
constexpr int kDecChunk = 128;
// keys per workgroup of the paged step (256, with its doubled registers, is
// slower at every page size)
constexpr int kPagedChunk = 128;

// one slice of a contiguous cache [slice][cap][D]
template <typename K, typename T, int D>
struct ContigRows {
    static constexpr bool kSlotPointers = false;
    K* k0;            // the slice's slot 0
    T* v0;
    float* g0;        // its log-f prefix (NULL: no gate)
    __device__ size_t off(int j) const { return (size_t)j * D; }
    __device__ float* g(int j) const { return g0 + j; }
    // the same for key j in key slot i of the chunk body (the slot is not needed here)
    __device__ size_t off_i(int, int j) const { return off(j); }
    __device__ float* g_i(int, int j) const { return g(j); }
    __device__ float prev_prefix(int t) const { return g0[t - 1]; }
    __device__ bool gate() const { return g0 != nullptr; }
};

// one (sequence, head) of a paged cache [page][H][P][D], seen from one chunk:
// slot j is in page pages[(j >> lp) - p0] (the chunk's page-table entries,
// staged in LDS) at position j & (P - 1)
template <typename K, typename T, int D>
struct PagedRows {
    static constexpr bool kSlotPointers = false;
    K* k0;             // the page pool
    T* v0;
    float* gp;         // log-f pages [page][H][P] (NULL: no gate)
    const int* pages;  // page-table entries p0, p0 + 1, ... of the sequence
    const float* gprev;  // log-f prefix of slot t - 1, wherever its page is
    int p0, lp, H, h;
    __device__ size_t slab(int j) const {
        return ((size_t)pages[(j >> lp) - p0] * H + h) << lp | (size_t)(j & ((1 << lp) - 1));
    }
    __device__ size_t off(int j) const { return slab(j) * D; }
    __device__ float* g(int j) const { return gp + slab(j); }
    __device__ size_t off_i(int, int j) const { return off(j); }
    __device__ float* g_i(int, int j) const { return g(j); }
    __device__ float prev_prefix(int) const { return *gprev; }
    __device__ bool gate() const { return gp != nullptr; }
};

// A paged cache whose pages hold at least as many slots as the chunk body's
// lane groups step over (GROUPS): then key slot i of the chunk (keys
// j0 + i GROUPS .. j0 + (i + 1) GROUPS - 1, an aligned run no longer than a
// page) lies in one page, and that page's slab start is the same for every
// lane, so it is kept per slot in scalar registers and a key's offset is the
// slab start plus its position in the page, as in a contiguous slice.
template <typename K, typename T, int D, int NS>
struct PagedSlotRows {
    static constexpr bool kSlotPointers = true;
    K* kb[NS];          // slot i's page slab: keys, values, log-f prefixes
    T* vb[NS];
    float* gb[NS];
    const float* gprev;
    float* gp;          // the log-f pool (NULL: no gate)
    int mask;           // P - 1
    // a row in its page: a 32-bit byte offset from the slot's base, so that
    // the access takes the base from scalar registers and one offset VGPR
    template <typename E>
    __device__ static E* at(E* base, uint32_t bytes) {
        return reinterpret_cast<E*>(reinterpret_cast<char*>(base) + bytes);
    }
    __device__ uint32_t row_bytes(int j, int e, uint32_t esize) const {
        return ((uint32_t)(j & mask) * D + (uint32_t)e) * esize;
    }
    __device__ K* kp_i(int i, int j, int e) const { return at(kb[i], row_bytes(j, e, sizeof(K))); }
    __device__ T* vp_i(int i, int j, int e) const { return at(vb[i], row_bytes(j, e, sizeof(T))); }
    __device__ float* g_i(int i, int j) const { return at(gb[i], (uint32_t)(j & mask) * 4u); }
    __device__ float prev_prefix(int) const { return *gprev; }
    __device__ bool gate() const { return gp != nullptr; }
};

template <typename K, typename T, int D, bool FUSED, int CH, typename Rows>
__device__ inline void chunk_attend(const Rows& rows, int slice, int ch, int n_keys, float scale,
                                    const T* __restrict__ q_t, const T* __restrict__ k_t,
                                    const T* __restrict__ v_t, const T* __restrict__ w_t,
                                    const float* __restrict__ beta_t,
                                    const float* __restrict__ logf_t, float* __restrict__ out) {
    constexpr int VN = Vec<K>::n, TPR = D / VN, GROUPS = 256 / TPR;
    constexpr int KPG = CH / GROUPS;             // keys per group
    const int lane_in = threadIdx.x % TPR, grp = threadIdx.x / TPR;
    const int t = n_keys - 1;                     // query position
    const size_t sd = (size_t)slice * D + lane_in * VN;

    float qv[VN], wv[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) {
        qv[e] = to_f32(q_t[sd + e]);
        wv[e] = FUSED ? to_f32(w_t[sd + e]) : 0.f;
    }
    const float bt = FUSED ? beta_t[slice] : 0.f;
    const bool gate = rows.gate();
    float ct = 0.f;                               // C_t
    if (gate) {
        if constexpr (FUSED) ct = (t > 0 ? rows.prev_prefix(t) : 0.f) + logf_t[slice];
        else ct = *rows.g(t);
    }
    const int j0 = ch * CH;

    // ---- loads (every key of this group in flight at once)
    Vec<K> kx[KPG];
    Raw<T, VN> vr[KPG];
    float gj[KPG];
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
        const int j = j0 + grp + GROUPS * i;
        const bool live = j < n_keys && !(FUSED && j == t);
        if (live) {
            if constexpr (Rows::kSlotPointers) {
                kx[i].load(rows.kp_i(i, j, lane_in * VN));
                vr[i].load(rows.vp_i(i, j, lane_in * VN));
            } else {
                const size_t off = rows.off_i(i, j) + lane_in * VN;
                kx[i].load(rows.k0 + off);
                vr[i].load(rows.v0 + off);
            }
            gj[i] = gate ? *rows.g_i(i, j) : 0.f;
        } else {
            // keys past the end get weight 0; their values must be finite
#pragma unroll
            for (int e = 0; e < Raw<T, VN>::W; ++e) vr[i].w[e] = 0u;
            gj[i] = 0.f;
        }
    }
    // ---- scores (rewriting the keys first when fused)
    float sc[KPG];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < KPG; ++i) {
        const int j = j0 + grp + GROUPS * i;
        float kf[VN], bias = 0.f;
        if (j >= n_keys) {
            sc[i] = -INFINITY;
            continue;
        }
        // the key's and value's row (formed where used, as the loads formed them)
        auto krow = [&]() -> K* {
            if constexpr (Rows::kSlotPointers) return rows.kp_i(i, j, lane_in * VN);
            else return rows.k0 + (rows.off_i(i, j) + lane_in * VN);
        };
        auto vrow = [&]() -> T* {
            if constexpr (Rows::kSlotPointers) return rows.vp_i(i, j, lane_in * VN);
            else return rows.v0 + (rows.off_i(i, j) + lane_in * VN);
        };
        if (FUSED && j == t) {
            // the new token: stored as given, its own transition excluded
#pragma unroll
            for (int e = 0; e < VN; ++e) {
                kf[e] = to_f32(from_f32<K>(to_f32(k_t[sd + e])));
                krow()[e] = from_f32<K>(kf[e]);
                vrow()[e] = v_t[sd + e];
            }
            vr[i].load(v_t + sd);
            if (gate && lane_in == 0) *rows.g_i(i, t) = ct;
        } else {
            if (FUSED) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < VN; ++e) p += wv[e] * kx[i].get(e);
                const float cf = bt * group_sum<TPR>(p);
#pragma unroll
                for (int e = 0; e < VN; ++e) kx[i].set(e, kx[i].get(e) - cf * wv[e]);
                kx[i].store(krow());
            }
#pragma unroll
            for (int e = 0; e < VN; ++e) kf[e] = kx[i].get(e);
            bias = gate ? ct - gj[i] : 0.f;
        }
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < VN; ++e) p += qv[e] * kf[e];
        sc[i] = scale * group_sum<TPR>(p) + bias;
        m = fmaxf(m, sc[i]);
    }
    float l = 0.f, acc[VN];
#pragma unroll
    for (int e = 0; e < VN; ++e) acc[e] = 0.f;
    if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < KPG; ++i) {
            const float pe = __expf(sc[i] - m);       // 0 for keys past the end
            l += pe;
#pragma unroll
            for (int e = 0; e < VN; ++e) acc[e] += pe * vr[i].get(e);
        }
    }

    // merge the groups of this block
    __shared__ float sm[GROUPS], sl[GROUPS];
    __shared__ float sacc[GROUPS][D + 1];
    if (lane_in == 0) { sm[grp] = m; sl[grp] = l; }
#pragma unroll
    for (int e = 0; e < VN; ++e) sacc[grp][lane_in * VN + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        const int x = threadIdx.x;
        float M = -INFINITY;
        for (int g = 0; g < GROUPS; ++g) M = fmaxf(M, sm[g]);
        float a = 0.f, ls = 0.f;
        for (int g = 0; g < GROUPS; ++g) {
            const float f = (sm[g] == -INFINITY) ? 0.f : __expf(sm[g] - M);
            a += sacc[g][x] * f;
            ls += sl[g] * f;
        }
        out[2 + x] = a;
        if (x == 0) { out[0] = M; out[1] = ls; }
    }
}

// Contiguous cache: grid (chunks, slices); partials part[slice][chunk].
template <typename K, typename T, int D, bool FUSED>
__global__ void __launch_bounds__(256)
decode_chunk_kernel(K* __restrict__ kc, T* __restrict__ vc, float* __restrict__ gc,
                    int cap, int n_keys, float scale,
                    const T* __restrict__ q_t, const T* __restrict__ k_t,
                    const T* __restrict__ v_t, const T* __restrict__ w_t,
                    const float* __restrict__ beta_t, const float* __restrict__ logf_t,
                    float* __restrict__ part) {
    const int slice = blockIdx.y, ch = blockIdx.x, nch = gridDim.x;
    const ContigRows<K, T, D> rows{kc + (size_t)slice * cap * D, vc + (size_t)slice * cap * D,
                                   gc ? gc + (size_t)slice * cap : nullptr};
    chunk_attend<K, T, D, FUSED, kDecChunk>(rows, slice, ch, n_keys, scale, q_t, k_t, v_t, w_t,
                                            beta_t, logf_t,
                                            part + ((size_t)slice * nch + ch) * (D + 2));
}

// Paged cache, one fused step for a batch of sequences of their own lengths
// [Notes s2.8]: grid (chunks of the longest sequence, S * H); slice = s*H + h.
// Sequence s has n_keys = seq_lens[s] + 1 keys (the new token at slot
// seq_lens[s]); chunks past its end exit at once.  The chunk-0 workgroup
// records n_keys (or -1 when seq_lens[s] is out of [0, max_keys)) in nk[slice]
// for the combine.  A chunk that reaches a page-table entry outside
// [0, num_pages) (its own pages, or with the gate the page of slot t - 1)
// touches no cache memory and leaves m = +inf, which makes the combine's
// result NaN for that (sequence, head).
template <typename K, typename T, int D, bool SLOTS>
__device__ inline void paged_chunk(K* __restrict__ kp, T* __restrict__ vp, float* __restrict__ gp,
                                   int num_pages, int lp, int H, const int* __restrict__ tables,
                                   int table_stride, const int* __restrict__ seq_lens,
                                   int max_keys, float scale, const T* __restrict__ q_t,
                                   const T* __restrict__ k_t, const T* __restrict__ v_t,
                                   const T* __restrict__ w_t, const float* __restrict__ beta_t,
                                   const float* __restrict__ logf_t, float* __restrict__ part,
                                   int* __restrict__ nk) {
    // chunk-major grid: every slice's chunk 0, then every slice's chunk 1, ...,
    // so the chunks past the shorter sequences' ends, which exit at once,
    // come at the end of the dispatch instead of between working ones
    const int slice = blockIdx.x, ch = blockIdx.y, nch = gridDim.y;
    const int s = slice / H, h = slice % H;
    const int len = seq_lens[s];
    const bool ok = len >= 0 && len < max_keys;
    const int n_keys = len + 1;
    if (ch == 0 && threadIdx.x == 0) nk[slice] = ok ? n_keys : -1;
    if (!ok || ch * kPagedChunk >= n_keys) return;
    const int* table = tables + (size_t)s * table_stride;
    float* out = part + ((size_t)slice * nch + ch) * (D + 2);
    // The chunk's page-table entries into LDS (one lane per page) and, on the
    // last lane, with the gate, the entry of slot t - 1's page (the new
    // token's log-f prefix continues that slot's, which need not be on one of
    // this chunk's pages), loaded together and each checked against the pool;
    // the key rows then read their page from LDS.
    __shared__ int sPage[kPagedChunk / 16];
    __shared__ int sPrev;
    const int p0 = (ch * kPagedChunk) >> lp, p1 = (min(n_keys, (ch + 1) * kPagedChunk) - 1) >> lp;
    const int tp = n_keys - 2;                    // slot t - 1
    bool bad = false;
    if (threadIdx.x <= p1 - p0) {                 // at most kPagedChunk / 16 lanes
        const int pg = table[p0 + threadIdx.x];
        sPage[threadIdx.x] = pg;
        bad = (unsigned)pg >= (unsigned)num_pages;
    }
    if (threadIdx.x == blockDim.x - 1) {
        int prev = 0;
        if (gp && tp >= 0) prev = table[tp >> lp];
        sPrev = prev;
        bad = bad || (unsigned)prev >= (unsigned)num_pages;
    }
    if (__syncthreads_or(bad)) {
        if (threadIdx.x < D + 2) out[threadIdx.x] = threadIdx.x == 0 ? INFINITY : 0.f;
        return;
    }
    const float* gprev = gp && tp >= 0
        ? gp + ((((size_t)sPrev * H + h) << lp) | (size_t)(tp & ((1 << lp) - 1))) : nullptr;
    if constexpr (SLOTS) {
        // pages of at least GROUPS slots (checked by the launch): one page per key slot
        constexpr int GROUPS = 256 / (D / Vec<K>::n), NS = kPagedChunk / GROUPS;
        static_assert(NS <= kPagedChunk / 16, "slot pages among the staged entries");
        PagedSlotRows<K, T, D, NS> rows{{}, {}, {}, gprev, gp, (1 << lp) - 1};
        const int j0 = ch * kPagedChunk;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            // slots past the sequence end may name an unstaged entry: their keys are never read
            const int pg = __builtin_amdgcn_readfirstlane(sPage[((j0 + GROUPS * i) >> lp) - p0]);
            const size_t slab = ((size_t)pg * H + h) << lp;
            rows.kb[i] = kp + slab * D;
            rows.vb[i] = vp + slab * D;
            rows.gb[i] = gp ? gp + slab : nullptr;
        }
        chunk_attend<K, T, D, true, kPagedChunk>(rows, slice, ch, n_keys, scale, q_t, k_t, v_t,
                                                 w_t, beta_t, logf_t, out);
    } else {
        const PagedRows<K, T, D> rows{kp, vp, gp, sPage, gprev, p0, lp, H, h};
        chunk_attend<K, T, D, true, kPagedChunk>(rows, slice, ch, n_keys, scale, q_t, k_t, v_t,
                                                 w_t, beta_t, logf_t, out);
    }
}
#define PA_PAGED_PARAMS                                                                         \
    K *__restrict__ kp, T *__restrict__ vp, float *__restrict__ gp, int num_pages, int lp,      \
        int H, const int *__restrict__ tables, int table_stride,                                \
        const int *__restrict__ seq_lens, int max_keys, float scale, const T *__restrict__ q_t, \
        const T *__restrict__ k_t, const T *__restrict__ v_t, const T *__restrict__ w_t,        \
        const float *__restrict__ beta_t, const float *__restrict__ logf_t,                     \
        float *__restrict__ part, int *__restrict__ nk
#define PA_PAGED_ARGS                                                                         \
    kp, vp, gp, num_pages, lp, H, tables, table_stride, seq_lens, max_keys, scale, q_t, k_t, \
        v_t, w_t, beta_t, logf_t, part, nk
template <typename K, typename T, int D, bool SLOTS>
__global__ void __launch_bounds__(256) paged_chunk_kernel(PA_PAGED_PARAMS) {
    paged_chunk<K, T, D, SLOTS>(PA_PAGED_ARGS);
}
// The same at six waves per SIMD (registers capped at 80), for the cache
// types whose step fits that without spilling: bf16 keys and values at d = 64
// (measured 4-5 % faster than at the five waves its 84 registers would give).
template <typename K, typename T, int D, bool SLOTS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6)))
paged_chunk6_kernel(PA_PAGED_PARAMS) {
    paged_chunk<K, T, D, SLOTS>(PA_PAGED_ARGS);
}
#undef PA_PAGED_PARAMS
#undef PA_PAGED_ARGS

// Merge the chunk partials of one slice: o = sum acc_c e^{m_c - M} / l,
// lse = M + log l.  One 1024-thread block per slice, one chunk per thread for
// the maxima and sums (wave shuffles, then one LDS exchange of the 16 wave
// results), and 1024/D groups of D lanes each summing a strided share of the
// chunks' accumulators (every load of a group in flight at once).
// Contiguous cache: every slice has nch chunks (nk NULL).  Paged cache: slice
// s*H + h has ceil(nk[slice] / kDecChunk) of the pstride chunk rows (nk < 0:
// the output is NaN), and the head-0 block of a sequence then advances
// seq_lens[s] to nk (the chunk kernel, which reads it, has finished).
constexpr int kCombineMaxChunks = 1024;
constexpr int kCombineThreads = 1024;
constexpr int kCombinePre = 24;  // chunks per thread whose accumulators are loaded up front

template <typename T, int D>
__global__ void __launch_bounds__(kCombineThreads)
decode_combine_kernel(const float* __restrict__ part, int nch, int pstride, int chunk,
                      const int* __restrict__ nk, int H, int* __restrict__ seq_lens,
                      T* __restrict__ o_t, float* __restrict__ lse_t) {
    constexpr int NTH = kCombineThreads, NW = NTH / 64, G = NTH / D;
    __shared__ float wmax[NW], wsum[NW];
    __shared__ float sf[kCombineMaxChunks];
    __shared__ float sacc[G][D];
    const int slice = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    if (nk) {
        const int n = nk[slice];
        if (n < 1) {
            if (tid < D) o_t[(size_t)slice * D + tid] = from_f32<T>(NAN);
            if (tid == 0 && lse_t) lse_t[slice] = NAN;
            return;
        }
        nch = (n + chunk - 1) / chunk;
        if (tid == 0 && seq_lens && slice % H == 0) seq_lens[slice / H] = n;
    }
    const float* p = part + (size_t)slice * pstride * (D + 2);
    const int g = tid / D, x = tid % D;
    // this thread's share of the accumulators, loaded beside the maxima and
    // sums (they do not depend on them), for up to kCombinePre chunks
    float pre[kCombinePre];
#pragma unroll
    for (int i = 0; i < kCombinePre; ++i) {
        const int c = g + G * i;
        pre[i] = c < nch ? p[(size_t)c * (D + 2) + 2 + x] : 0.f;
    }
    const float mc = tid < nch ? p[(size_t)tid * (D + 2)] : -INFINITY;
    const float lc = tid < nch ? p[(size_t)tid * (D + 2) + 1] : 0.f;
    float mx = mc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    if (ln == 0) wmax[wv] = mx;
    __syncthreads();
    float M = wmax[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, wmax[i]);
    const float f = (mc == -INFINITY) ? 0.f : __expf(mc - M);
    if (tid < nch) sf[tid] = f;
    float sl = f * lc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sl += __shfl_xor(sl, off, 64);
    if (ln == 0) wsum[wv] = sl;
    __syncthreads();
    float lt = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) lt += wsum[i];
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < kCombinePre; ++i) {
        const int c = g + G * i;
        if (c < nch) a += sf[c] * pre[i];
    }
#pragma unroll 8
    for (int c = g + G * kCombinePre; c < nch; c += G) a += sf[c] * p[(size_t)c * (D + 2) + 2 + x];
    sacc[g][x] = a;
    __syncthreads();
    if (tid < D) {
        float sum = 0.f;
#pragma unroll
        for (int gg = 0; gg < G; ++gg) sum += sacc[gg][tid];
        o_t[(size_t)slice * D + tid] = from_f32<T>(sum / lt);
        if (tid == 0 && lse_t) lse_t[slice] = M + logf(lt);
    }
}

// ---------------------------------------------------------------------------
// Prefill -> decode alignment [Notes s2.8]: the cache must hold every prompt
// key moved to the prompt end, H_{L-1} ... H_{j+1} k_j.  Keys already sit at
// their block's right edge (Kright); the rest of the way is the product of
// the later blocks' transitions.  In row form, kcache_c = Kright_c S_c with
//   S_{nb-1} = I,  S_c = F_{c+1} S_{c+1},  F_c = I - E_c.
// The chain is split into groups of kSufGroup blocks so that it runs in
// parallel: inside group g (blocks first..last)
//   T_last = I,  T_c = F_{c+1} T_{c+1}          (suffix_local_kernel)
// and the group's whole transition G_g = F_first T_first; across groups
//   Z_{ng-1} = I,  Z_g = G_{g+1} Z_{g+1}         (suffix_groups_kernel)
// so that S_c = T_c Z_{g(c)} (align_apply_kernel).  All in fp32.
constexpr int kSufGroup = 32;

// The d x d products run on the matrix cores on matrices padded to
// DP = max(d, 32), with fp32 operands split into bf16 parts: three parts and
// six partial products (tile_mm_f32, fp32 accuracy) for an fp32 key cache;
// two parts and three partial products (tile_mm, ~16 significant bits) for a
// bf16 cache, whose own rounding (2^-9) is far coarser than what a chain of
// at most kSufGroup + ceil(nb / kSufGroup) such products accumulates.  The
// chain is kept transposed (S^T <- S^T - S^T E^T) so that every product reads
// both operands row-major from LDS.  Stored: suf[c] = T_c^T, grp[g][0] = G_g,
// grp[g][1] = Z_g^T.
constexpr int kMS = 68;   // LDS row stride (floats) of the padded matrices

template <int D>
struct Pad {
    static constexpr int DP = D < 32 ? 32 : D, DT = DP / 32;
};

template <int D>
__device__ inline void mat_identity(float* dst, int tid) {
    constexpr int DP = Pad<D>::DP;
    for (int e = tid; e < DP * DP; e += 256) dst[(e / DP) * kMS + e % DP] = (e / DP == e % DP) ? 1.f : 0.f;
}

// A thread's share of a D x D row-major matrix (element e = tid + 256 i of
// the padded DP x DP matrix), held in registers so that the next matrix of a
// chain is in flight while the current product runs.
template <int D>
struct MatRegs {
    static constexpr int DP = Pad<D>::DP, N = DP * DP / 256;
    float v[N];
    __device__ void load(const float* src, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int e = tid + 256 * i, x = e / DP, y = e % DP;
            v[i] = (x < D && y < D) ? src[x * D + y] : 0.f;
        }
    }
    __device__ void store(float* dst, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int e = tid + 256 * i;
            dst[(e / DP) * kMS + e % DP] = v[i];
        }
    }
};

// acc += A B^T over a DP x DP tile pair at the chain's precision
template <int DP, bool F32>
__device__ inline void chain_mm(f32x16& acc, const float* A, const float* Bn, int m0, int n0,
                                int lane) {
    if constexpr (F32) tile_mm_f32<DP>(acc, A, kMS, Bn, kMS, m0, n0, lane);
    else tile_mm<DP, float, float>(acc, A, kMS, Bn, kMS, m0, n0, lane);
}

template <int D, bool F32>
__global__ void __launch_bounds__(256)
suffix_local_kernel(int nb, int ngroups, FwdWs ws) {
    using P = Pad<D>;
    __shared__ __attribute__((aligned(16))) float sSt[64 * kMS], sE[64 * kMS];
    const int slice = blockIdx.x / ngroups, gi = blockIdx.x % ngroups, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int first = gi * kSufGroup, last = min(nb - 1, first + kSufGroup - 1);
    const size_t b0 = (size_t)slice * nb;
    mat_identity<D>(sSt, tid);
    for (int e = tid; e < D * D; e += 256) ws.suf[(b0 + last) * D * D + e] = (e / D == e % D) ? 1.f : 0.f;
    // c = first - 1 yields the group total: G^T = T_first^T F_first^T
    MatRegs<D> nextE;
    if (last - 1 >= first - 1) nextE.load(ws.e32 + (b0 + last) * D * D, tid);
    for (int c = last - 1; c >= first - 1; --c) {
        __syncthreads();
        nextE.store(sE, tid);
        if (c - 1 >= first - 1) nextE.load(ws.e32 + (b0 + c) * D * D, tid);
        __syncthreads();
        f32x16 acc = zero16();
        const int mt = wave / P::DT, nt = wave % P::DT;
        const bool mine = wave < P::DT * P::DT;
        if (mine) chain_mm<P::DP, F32>(acc, sSt, sE, 32 * mt, 32 * nt, lane);
        const int h = lane >> 5, y = 32 * nt + (lane & 31);
        float nv[16];
        if (mine) {
#pragma unroll
            for (int r = 0; r < 16; ++r) nv[r] = sSt[(32 * mt + crow(r, h)) * kMS + y] - acc[r];
        }
        __syncthreads();
        if (mine) {
            float* dst = c >= first ? ws.suf + (b0 + c) * D * D
                                    : ws.grp + ((size_t)slice * ngroups + gi) * 2 * D * D;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int x = 32 * mt + crow(r, h);
                sSt[x * kMS + y] = nv[r];
                if (x < D && y < D) {
                    if (c >= first) dst[x * D + y] = nv[r];   // T_c^T
                    else dst[y * D + x] = nv[r];              // G (transposed back)
                }
            }
        }
    }
}

template <int D, bool F32>
__global__ void __launch_bounds__(256)
suffix_groups_kernel(int nb, int ngroups, FwdWs ws) {
    using P = Pad<D>;
    __shared__ __attribute__((aligned(16))) float sZt[64 * kMS], sG[64 * kMS];
    __shared__ double sScan[256];
    const int slice = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t b0 = (size_t)slice * nb, g0 = (size_t)slice * ngroups;
    // block prefix of log f, gpre[c] = sum_{c' < c} tot[c'], accumulated in double
    double carry = 0.0;
    for (int c0 = 0; c0 < nb; c0 += 256) {
        const int c = c0 + tid;
        const double tv = c < nb ? (double)ws.tot[b0 + c] : 0.0;
        sScan[tid] = tv;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const double add = tid >= off ? sScan[tid - off] : 0.0;
            __syncthreads();
            sScan[tid] += add;
            __syncthreads();
        }
        if (c < nb) ws.gpre[b0 + c] = (float)(carry + sScan[tid] - tv);
        carry += sScan[255];
        __syncthreads();
    }
    mat_identity<D>(sZt, tid);
    for (int e = tid; e < D * D; e += 256)
        ws.grp[((g0 + ngroups - 1) * 2 + 1) * D * D + e] = (e / D == e % D) ? 1.f : 0.f;
    // Z_g^T = Z_{g+1}^T G_{g+1}^T
    MatRegs<D> nextG;
    if (ngroups >= 2) nextG.load(ws.grp + ((g0 + ngroups - 1) * 2) * D * D, tid);
    for (int g = ngroups - 2; g >= 0; --g) {
        __syncthreads();
        nextG.store(sG, tid);
        if (g >= 1) nextG.load(ws.grp + ((g0 + g) * 2) * D * D, tid);
        __syncthreads();
        f32x16 acc = zero16();
        const int mt = wave / P::DT, nt = wave % P::DT;
        const bool mine = wave < P::DT * P::DT;
        if (mine) chain_mm<P::DP, F32>(acc, sZt, sG, 32 * mt, 32 * nt, lane);
        __syncthreads();
        if (mine) {
            const int h = lane >> 5, y = 32 * nt + (lane & 31);
            float* dst = ws.grp + ((g0 + g) * 2 + 1) * D * D;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int x = 32 * mt + crow(r, h);
                sZt[x * kMS + y] = acc[r];
                if (x < D && y < D) dst[x * D + y] = acc[r];
            }
        }
    }
}

// Eight fp32 values of row `row` of a row-major matrix (stride ld) as a bf16
// hi + lo operand pair: columns c0 + 8h .. +7, or with PERM the columns
// c0 + swap23(8h + e) that match a C tile reused as the other operand.  Rows
// at or beyond nr and column groups at or beyond nc read as zero.
// The load (ld8_raw) and the split (split8) are separate so that a product's
// operand loads can all be in flight before its first matrix instruction.
struct F8 {
    f32x4 a, b;
};
template <bool PERM>
__device__ inline F8 ld8_raw(const float* base, int ld, int row, int nr, int c0, int nc, int h) {
    F8 v;
    v.a = f32x4{0.f, 0.f, 0.f, 0.f};
    v.b = v.a;
    if (row < nr && c0 < nc) {
        const float* p = base + (size_t)row * ld + c0;
        const int o0 = PERM ? 4 * h : 8 * h, o1 = PERM ? 8 + 4 * h : 8 * h + 4;
        v.a = *reinterpret_cast<const f32x4*>(p + o0);
        v.b = *reinterpret_cast<const f32x4*>(p + o1);
    }
    return v;
}
__device__ inline void split8(const F8& v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? v.a[e] : v.b[e - 4];
        hi[e] = (__bf16)x;
        lo[e] = (__bf16)(x - (float)hi[e]);
    }
}

// kcache rows of block c = (Kright_c T_c) Z_g; values copied; gcache = block
// prefix + in-block cumsum.  Register-only: a wave owns 32 keys of one block
// and forms X^T = T_c^T Kright_c^T (operands read from HBM as they are
// stored), then kcache^T = Z_g^T X^T with X^T's C tiles reused directly as
// the B operand.  Each product's operand loads are all issued before its
// first matrix instruction (two memory round trips per wave, not one per
// k-step).  Products use fp32 operands split into bf16 hi + lo (about
// 16 significant bits), well below the bf16 or fp32 rounding of the cache.
// Workgroups go to the 8 XCDs round-robin; the workgroups of one XCD take
// consecutive block pairs, so that the blocks of a suffix group, which all
// read that group's Z_g, run in one XCD and find it in its L2.
__device__ inline int xcd_major(int b, int n) {
    const int full = n & ~7;
    if (b >= full) return b;
    return (b & 7) * (full >> 3) + (b >> 3);
}

template <typename K, typename T, int B, int D>
__global__ void __launch_bounds__(256)
align_apply_kernel(int L, int nb, int ngroups, int nblk, FwdWs ws, const T* __restrict__ v,
                   int has_gate, K* __restrict__ kc, T* __restrict__ vc,
                   float* __restrict__ gc, int cap) {
    constexpr int DP = Pad<D>::DP, XT = DP / 32, KS = DP / 16;
    constexpr int BP = B < 32 ? 32 : B, RT = BP / 32, BPW = 4 / RT;   // blocks per workgroup
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int col = lane & 31;
    const int wg = xcd_major(blockIdx.x, gridDim.x);
    const int blk = wg * BPW + wave / RT, rt = wave % RT;
    // value unit i of this thread: (its slice, its position, its 16-byte unit x)
    constexpr int UPR = D * (int)sizeof(T) / 16, NU = BPW * B * UPR, NVU = (NU + 255) / 256;
    auto vunit = [&](int i, int& slice, int& pos, int& x) {
        const int u = tid + 256 * i, b2 = wg * BPW + u / (B * UPR), rr = (u / UPR) % B;
        x = u % UPR;
        slice = b2 / nb;
        pos = (b2 % nb) * B + rr;
        return u < NU && b2 < nblk && pos < L;
    };
    const int slice = blk / nb, c = blk % nb, g = c / kSufGroup;
    const int r = 32 * rt + col;                 // this lane's key (B-operand column)
    // X^T's C tiles as the B operand of the second product: k-step ks holds
    // rows 16 ks + swap23(slot)
    bf16x8 bh[KS], bl[KS];
    if (blk < nblk) {
        const float* Tt = ws.suf + (size_t)blk * D * D;
        const float* kr = ws.k32 + (size_t)blk * B * D;
        F8 kv[KS], tv[XT][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kv[ks] = ld8_raw<false>(kr, D, r, B, 16 * ks, D, h);
#pragma unroll
        for (int t = 0; t < XT; ++t)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                tv[t][ks] = ld8_raw<false>(Tt, D, 32 * t + col, D, 16 * ks, D, h);
        __builtin_amdgcn_sched_barrier(0);   // every load above issued before the products
        bf16x8 kh[KS], kl[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) split8(kv[ks], kh[ks], kl[ks]);
        f32x16 xt[XT];
#pragma unroll
        for (int t = 0; t < XT; ++t) {
            xt[t] = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah, al;
                split8(tv[t][ks], ah, al);
                xt[t] = mfma_split(ah, al, kh[ks], kl[ks], xt[t]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = xt[ks >> 1][8 * (ks & 1) + e];
                bh[ks][e] = (__bf16)x;
                bl[ks][e] = (__bf16)(x - (float)bh[ks][e]);
            }
    }
    // values (16-byte units) and the gate prefix of this workgroup's blocks,
    // loaded beside the second product's operands and stored at the end
    u32x4 vv[NVU];
#pragma unroll
    for (int i = 0; i < NVU; ++i) {
        int vs, vp, x;
        vv[i] = vunit(i, vs, vp, x) ? reinterpret_cast<const u32x4*>(v + ((size_t)vs * L + vp) * D)[x]
                                    : u32x4{0u, 0u, 0u, 0u};
    }
    float gpre = 0.f, gin = 0.f;     // added at the store, so nothing waits on them here
    size_t gdst = ~(size_t)0;
    if (gc && tid < BPW * B) {
        const int b2 = wg * BPW + tid / B, rr = tid % B;
        const int gs = b2 / nb, gp = (b2 % nb) * B + rr;
        if (b2 < nblk && gp < L) {
            gdst = (size_t)gs * cap + gp;
            if (has_gate) {
                gpre = ws.gpre[b2];
                gin = ws.gl[(size_t)b2 * B + rr];
            }
        }
    }
    if (blk < nblk) {
        const float* Zt = ws.grp + (((size_t)slice * ngroups + g) * 2 + 1) * D * D;
        const int pos = c * B + r;
        K* krow = kc + ((size_t)slice * cap + pos) * D;
        F8 zv[XT][KS];
#pragma unroll
        for (int yt = 0; yt < XT; ++yt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                zv[yt][ks] = ld8_raw<true>(Zt, D, 32 * yt + col, D, 16 * ks, D, h);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int yt = 0; yt < XT; ++yt) {
            f32x16 acc = zero16();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                bf16x8 ah, al;
                split8(zv[yt][ks], ah, al);
                acc = mfma_split(ah, al, bh[ks], bl[ks], acc);
            }
            if (r < B && pos < L) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int y0 = 32 * yt + 8 * i + 4 * h;
                    if (y0 < D) {
                        if constexpr (sizeof(K) == 2) {
                            typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                            bf16x4 pk;
#pragma unroll
                            for (int j = 0; j < 4; ++j) pk[j] = (__bf16)acc[4 * i + j];
                            *reinterpret_cast<bf16x4*>(krow + y0) = pk;
                        } else {
                            f32x4 pk;
#pragma unroll
                            for (int j = 0; j < 4; ++j) pk[j] = acc[4 * i + j];
                            *reinterpret_cast<f32x4*>(krow + y0) = pk;
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NVU; ++i) {
        int vs, vp, x;
        if (vunit(i, vs, vp, x)) reinterpret_cast<u32x4*>(vc + ((size_t)vs * cap + vp) * D)[x] = vv[i];
    }
    if (gdst != ~(size_t)0) gc[gdst] = gpre + gin;
}

// ---------------------------------------------------------------------------
template <typename K, typename T, int D>
static hipError_t kv_update_t(const CacheArgs& c, int n, const void* w_t,
                              const float* beta_t, hipStream_t st) {
    const int rows = 256;
    dim3 grid((n + rows - 1) / rows, c.N * c.H);
    hipLaunchKernelGGL((kv_update_kernel<K, T, D>), grid, dim3(256), 0, st,
                       (K*)c.kcache, c.cap, n, (const T*)w_t, beta_t, rows);
    return hipGetLastError();
}

template <typename K, typename T>
static hipError_t kv_update_d(const CacheArgs& c, int n, const void* w_t,
                              const float* beta_t, hipStream_t st) {
    switch (c.d) {
        case 16: return kv_update_t<K, T, 16>(c, n, w_t, beta_t, st);
        case 32: return kv_update_t<K, T, 32>(c, n, w_t, beta_t, st);
        case 64: return kv_update_t<K, T, 64>(c, n, w_t, beta_t, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_kv_update(const CacheArgs& c, int n, const void* w_t,
                            const float* beta_t, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    if (c.k_bf16)
        return c.v_bf16 ? kv_update_d<bf16, bf16>(c, n, w_t, beta_t, st)
                        : kv_update_d<bf16, float>(c, n, w_t, beta_t, st);
    return c.v_bf16 ? kv_update_d<float, bf16>(c, n, w_t, beta_t, st)
                    : kv_update_d<float, float>(c, n, w_t, beta_t, st);
}

template <typename K, typename T, int D>
static hipError_t kv_append_t(const CacheArgs& c, int n, const void* k_t,
                              const void* v_t, const float* logf_t, hipStream_t st) {
    hipLaunchKernelGGL((kv_append_kernel<K, T, D>), dim3(c.N * c.H), dim3(64), 0, st,
                       (K*)c.kcache, (T*)c.vcache, c.gcache, c.cap, n,
                       (const T*)k_t, (const T*)v_t, logf_t);
    return hipGetLastError();
}

template <typename K, typename T>
static hipError_t kv_append_d(const CacheArgs& c, int n, const void* k_t,
                              const void* v_t, const float* logf_t, hipStream_t st) {
    switch (c.d) {
        case 16: return kv_append_t<K, T, 16>(c, n, k_t, v_t, logf_t, st);
        case 32: return kv_append_t<K, T, 32>(c, n, k_t, v_t, logf_t, st);
        case 64: return kv_append_t<K, T, 64>(c, n, k_t, v_t, logf_t, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_kv_append(const CacheArgs& c, int n, const void* k_t,
                            const void* v_t, const float* logf_t, hipStream_t st) {
    if (c.k_bf16)
        return c.v_bf16 ? kv_append_d<bf16, bf16>(c, n, k_t, v_t, logf_t, st)
                        : kv_append_d<bf16, float>(c, n, k_t, v_t, logf_t, st);
    return c.v_bf16 ? kv_append_d<float, bf16>(c, n, k_t, v_t, logf_t, st)
                    : kv_append_d<float, float>(c, n, k_t, v_t, logf_t, st);
}

int decode_chunk(int n_keys) {
    (void)n_keys;
    return kDecChunk;
}

int decode_max_keys() { return kDecChunk * kCombineMaxChunks; }

template <typename K, typename T, int D>
static hipError_t decode_t(const CacheArgs& c, int n_keys, float scale, const void* q_t,
                           void* o_t, float* lse_t, float* part, int chunk, bool fused,
                           const void* k_t, const void* v_t, const void* w_t,
                           const float* beta_t, const float* logf_t, hipStream_t st) {
    const int nch = (n_keys + chunk - 1) / chunk;
    dim3 grid(nch, c.N * c.H);
    if (fused)
        hipLaunchKernelGGL((decode_chunk_kernel<K, T, D, true>), grid, dim3(256), 0, st,
                           (K*)c.kcache, (T*)c.vcache, c.gcache, c.cap, n_keys, scale,
                           (const T*)q_t, (const T*)k_t, (const T*)v_t, (const T*)w_t,
                           beta_t, logf_t, part);
    else
        hipLaunchKernelGGL((decode_chunk_kernel<K, T, D, false>), grid, dim3(256), 0, st,
                           (K*)c.kcache, (T*)c.vcache, c.gcache, c.cap, n_keys, scale,
                           (const T*)q_t, nullptr, nullptr, nullptr, nullptr, nullptr, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(c.N * c.H), dim3(kCombineThreads), 0, st,
                       (const float*)part, nch, nch, kDecChunk, nullptr, c.H, nullptr, (T*)o_t,
                       lse_t);
    return hipGetLastError();
}

template <typename K, typename T>
static hipError_t decode_d(const CacheArgs& c, int n_keys, float scale, const void* q_t,
                           void* o_t, float* lse_t, float* part, int chunk, bool fused,
                           const void* k_t, const void* v_t, const void* w_t,
                           const float* beta_t, const float* logf_t, hipStream_t st) {
    switch (c.d) {
        case 16: return decode_t<K, T, 16>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st);
        case 32: return decode_t<K, T, 32>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st);
        case 64: return decode_t<K, T, 64>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const CacheArgs& c, int n_keys, float scale, const void* q_t,
                         void* o_t, float* lse_t, float* part, int chunk, bool fused,
                         const void* k_t, const void* v_t, const void* w_t,
                         const float* beta_t, const float* logf_t, hipStream_t st) {
    if (c.k_bf16)
        return c.v_bf16 ? decode_d<bf16, bf16>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st)
                        : decode_d<bf16, float>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st);
    return c.v_bf16 ? decode_d<float, bf16>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st)
                    : decode_d<float, float>(c, n_keys, scale, q_t, o_t, lse_t, part, chunk, fused, k_t, v_t, w_t, beta_t, logf_t, st);
}

// ---------------------------------------------------------------------------
// Paged cache: one fused step for a batch of sequences, and the import of a
// contiguous (prefill-aligned) cache into pages.

// Slots [0, n) of sequence s (n = seq_lens[s], at most min(max_keys, cap)) of a
// contiguous cache [S][H][cap][D] copied into the sequence's pages.  Grid
// (pages of the longest sequence, S * H).  Pages whose table entry is outside
// [0, num_pages), and sequences whose length is out of range, are skipped.
template <typename K, typename T, int D>
__global__ void __launch_bounds__(256)
paged_import_kernel(const K* __restrict__ kc, const T* __restrict__ vc,
                    const float* __restrict__ gc, int cap, K* __restrict__ kp,
                    T* __restrict__ vp, float* __restrict__ gp, int num_pages, int lp, int H,
                    const int* __restrict__ tables, int table_stride,
                    const int* __restrict__ seq_lens, int max_keys) {
    constexpr int KU = 16 / (int)sizeof(K), VU = 16 / (int)sizeof(T);   // elements per 16 B
    const int slice = blockIdx.y, pg = blockIdx.x, s = slice / H, h = slice % H;
    const int P = 1 << lp;
    const int n = seq_lens[s];
    if (n < 0 || n > max_keys || n > cap || pg * P >= n) return;
    const int page = tables[(size_t)s * table_stride + pg];
    if ((unsigned)page >= (unsigned)num_pages) return;
    const int rows = min(P, n - pg * P);
    const size_t src = ((size_t)slice * cap + (size_t)pg * P) * D;
    const size_t dst = ((size_t)page * H + h) * P * D;
    for (int e = threadIdx.x; e < rows * (D / KU); e += blockDim.x)
        *reinterpret_cast<uint4*>(kp + dst + (size_t)e * KU) =
            *reinterpret_cast<const uint4*>(kc + src + (size_t)e * KU);
    for (int e = threadIdx.x; e < rows * (D / VU); e += blockDim.x)
        *reinterpret_cast<uint4*>(vp + dst + (size_t)e * VU) =
            *reinterpret_cast<const uint4*>(vc + src + (size_t)e * VU);
    if (gc && gp)
        for (int r = threadIdx.x; r < rows; r += blockDim.x)
            gp[((size_t)page * H + h) * P + r] = gc[(size_t)slice * cap + pg * P + r];
}

template <typename K, typename T, int D>
static hipError_t paged_step_t(const PagedArgs& a, hipStream_t st) {
    const int mch = (a.max_keys + kPagedChunk - 1) / kPagedChunk;
    const int S = a.S * a.H;
    float* part = a.ws;
    int* nk = reinterpret_cast<int*>(a.ws + (size_t)S * mch * (D + 2));
    // pages of at least as many slots as the chunk body's lane groups step over
    // take the scalar per-slot page bases
    constexpr int GROUPS = 256 / (D / Vec<K>::n);
    constexpr bool SIX = std::is_same_v<K, bf16> && std::is_same_v<T, bf16> && D == 64;
    const bool slots = (1 << a.lp) >= GROUPS;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(S, mch), dim3(256), 0, st, (K*)a.kpages, (T*)a.vpages,
                           a.gpages, a.num_pages, a.lp, a.H, a.tables, a.table_stride,
                           (const int*)a.seq_lens, a.max_keys, a.scale, (const T*)a.q_t,
                           (const T*)a.k_t, (const T*)a.v_t, (const T*)a.w_t, a.beta_t, a.logf_t,
                           part, nk);
    };
    if constexpr (SIX) {
        if (slots) launch(paged_chunk6_kernel<K, T, D, true>);
        else launch(paged_chunk6_kernel<K, T, D, false>);
    } else {
        if (slots) launch(paged_chunk_kernel<K, T, D, true>);
        else launch(paged_chunk_kernel<K, T, D, false>);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(S), dim3(kCombineThreads), 0, st,
                       (const float*)part, mch, mch, kPagedChunk, (const int*)nk, a.H, a.seq_lens,
                       (T*)a.o_t, a.lse_t);
    return hipGetLastError();
}

template <typename K, typename T, int D>
static hipError_t paged_import_t(const PagedArgs& a, const CacheArgs& c, hipStream_t st) {
    const int mp = (a.max_keys + (1 << a.lp) - 1) >> a.lp;
    hipLaunchKernelGGL((paged_import_kernel<K, T, D>), dim3(mp, a.S * a.H), dim3(256), 0, st,
                       (const K*)c.kcache, (const T*)c.vcache, (const float*)c.gcache, c.cap,
                       (K*)a.kpages, (T*)a.vpages, a.gpages, a.num_pages, a.lp, a.H, a.tables,
                       a.table_stride, (const int*)a.seq_lens, a.max_keys);
    return hipGetLastError();
}

// dispatch over (key type, value type, d)
template <template <typename, typename, int> class F, typename... Args>
static hipError_t paged_dispatch(const PagedArgs& a, Args&&... args) {
    auto by_d = [&](auto kt, auto vt) -> hipError_t {
        using K = decltype(kt);
        using T = decltype(vt);
        switch (a.d) {
            case 16: return F<K, T, 16>::run(a, args...);
            case 32: return F<K, T, 32>::run(a, args...);
            case 64: return F<K, T, 64>::run(a, args...);
        }
        return hipErrorInvalidValue;
    };
    if (a.k_bf16) return a.v_bf16 ? by_d(bf16{}, bf16{}) : by_d(bf16{}, float{});
    return a.v_bf16 ? by_d(float{}, bf16{}) : by_d(float{}, float{});
}
template <typename K, typename T, int D>
struct PagedStep {
    static hipError_t run(const PagedArgs& a, hipStream_t st) { return paged_step_t<K, T, D>(a, st); }
};
template <typename K, typename T, int D>
struct PagedImport {
    static hipError_t run(const PagedArgs& a, const CacheArgs& c, hipStream_t st) {
        return paged_import_t<K, T, D>(a, c, st);
    }
};

hipError_t launch_paged_step(const PagedArgs& a, hipStream_t st) {
    return paged_dispatch<PagedStep>(a, st);
}
hipError_t launch_paged_import(const PagedArgs& a, const CacheArgs& c, hipStream_t st) {
    return paged_dispatch<PagedImport>(a, c, st);
}
size_t paged_workspace_bytes(int S, int H, int d, int max_keys) {
    const size_t mch = (size_t)(max_keys + kPagedChunk - 1) / kPagedChunk;
    return (size_t)S * H * (mch * (d + 2) * 4 + 4);
}

int suffix_groups(int nb) { return (nb + kSufGroup - 1) / kSufGroup; }

template <typename K, typename T, int B, int D>
static hipError_t align_t(const FwdArgs& a, const CacheArgs& c, hipStream_t st) {
    const int nb = (a.L + B - 1) / B;
    const int ng = suffix_groups(nb);
    const int NH = a.N * a.H;
    constexpr bool F32 = sizeof(K) == 4;   // the chain at the key cache's precision
    hipLaunchKernelGGL((suffix_local_kernel<D, F32>), dim3(NH * ng), dim3(256), 0, st, nb, ng, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((suffix_groups_kernel<D, F32>), dim3(NH), dim3(256), 0, st, nb, ng, a.ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    constexpr int BPW = 4 / ((B < 32 ? 32 : B) / 32);   // blocks per workgroup
    const int nblk = NH * nb;
    hipLaunchKernelGGL((align_apply_kernel<K, T, B, D>), dim3((nblk + BPW - 1) / BPW), dim3(256), 0,
                       st, a.L, nb, ng, nblk, a.ws, (const T*)a.v, a.logf ? 1 : 0, (K*)c.kcache,
                       (T*)c.vcache, c.gcache, c.cap);
    return hipGetLastError();
}

template <typename K, typename T, int B>
static hipError_t align_d(const FwdArgs& a, const CacheArgs& c, hipStream_t st) {
    switch (a.d) {
        case 16: return align_t<K, T, B, 16>(a, c, st);
        case 32: return align_t<K, T, B, 32>(a, c, st);
        case 64: return align_t<K, T, B, 64>(a, c, st);
    }
    return hipErrorInvalidValue;
}

template <typename K, typename T>
static hipError_t align_b(const FwdArgs& a, const CacheArgs& c, hipStream_t st) {
    switch (a.block) {
        case 16: return align_d<K, T, 16>(a, c, st);
        case 32: return align_d<K, T, 32>(a, c, st);
        case 64: return align_d<K, T, 64>(a, c, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_kv_align(const FwdArgs& a, const CacheArgs& c, hipStream_t st) {
    if (c.k_bf16)
        return a.bf16 ? align_b<bf16, bf16>(a, c, st) : align_b<bf16, float>(a, c, st);
    return a.bf16 ? align_b<float, bf16>(a, c, st) : align_b<float, float>(a, c, st);
}

// ---------------------------------------------------------------------------
// Device-resident scratch for the entry point that allocates nothing
// (path_decode_step_noalloc): the split-K partial softmax states of a fused
// decode step go here instead of into a caller workspace.  The array exists
// once on every GPU the library's code object is loaded on and lives until
// the process ends; all calls on one GPU share it and it keeps the last
// call's contents (nothing in it needs to start at zero: every partial a
// combine reads is written by the same call's chunk kernel).  Calls that
// overlap on one GPU (different streams, or threads) race on it.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];     // device address of `scratch`, per device
}  // namespace

// The device address of `scratch` on the GPU that `stream` belongs to.  The
// host-side name of the array is only a stand-in for the symbol, never a
// device address: the address is looked up once per device (with that device
// current) and kept.
hipError_t static_scratch(hipStream_t stream, float** out) {
    int dev = -1, cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (stream) {
        if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    } else {
        dev = cur;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float*>(g_scratch_ptr[dev]);
    return hipSuccess;
}

}  // namespace pa
