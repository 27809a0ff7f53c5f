// frontend.hip -- the parameter front-end [Notes s2.1, s2.5]: from a layer
// input x_t, the transition parameters of PaTH attention:
//   w_t     = per-head L2 normalisation of a width-3 causal short
//             convolution of a low-rank linear layer's output,
//             c_t = sum_tau kc[:, tau] (Wu Wd x_{t - tau})
//   beta_t  = 2 sigma(ub . x_t + bb)
//   log f_t = log sigma(uf . x_t + bf)           (only with a forget gate)
// Citations: [Notes s2.x] = reading-notes page "PaTH Attention:通过累积
// Householder 变换编码位置" (cc.laoqi.cc), section 2.x.
//
// Two kernels, both on the matrix cores, both streaming their operands
// HBM -> LDS with direct buffer loads (no registers in between):
//   project: P = x [Wd; ub; uf]^T, one GEMM over the input width Dm, fp32
//            [N*L, Rp] in the workspace.  Columns: [0, R) the low-rank p,
//            then the H beta logits and (with a gate) the H gate logits, each
//            block padded to H8 = H rounded up to 8 columns; Rp = the total
//            rounded up to 32.
//   finish:  per (token tile of 32, head): y_tau = Wu P_{t - tau}^T for the
//            three taps, c = sum_tau kc[:, tau] y_tau, the norm over the
//            head's channels (a lane owns one token: a sum over its registers
//            and one exchange with the other lane half), beta and log f from
//            P's gate columns.
// Products are formed transposed (weights as the A operand) so that a lane
// ends up owning one token.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Direct HBM -> LDS loads through buffer resources.  One instruction moves 16
// bytes per lane and the wave's 64 lanes land contiguously from a uniform LDS
// address; each lane's source offset is free, so a permutation or a padding
// of the units inside that 1 KB is a matter of addressing.  A lane offset past
// the resource's range reads zeros: kOob marks units outside the data
// (sequence edges, the tail of a row, padding).  The host keeps every
// resource range below 2^31 bytes, so kOob plus a chunk offset stays past it.
constexpr uint32_t kOob = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                  char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                             voff, soff, 0, 0);
}
// Vector-memory waits.  The counter drains in issue order, so waiting until
// at most N operations are pending completes everything but the last N.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void wait_vm0() { wait_vm<0>(); }
// wait for a chunk when `ahead` later chunks of IPW loads each may stay pending
template <int IPW, int J>
__device__ inline void wait_ahead(int ahead) {
    if constexpr (J == 0) {
        wait_vm<0>();
    } else {
        if (ahead >= J) wait_vm<IPW * J>();
        else wait_ahead<IPW, J - 1>(ahead);
    }
}
// a workgroup barrier without the memory fence of __syncthreads (which would
// also drain every load in flight); the empty asm statements keep the
// compiler from moving memory accesses across it
__device__ inline void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 8 consecutive fp32 values split into bf16 parts: two (hi + lo, ~16
// mantissa bits) or three (hi + mid + lo, fp32 accuracy).
template <int PARTS>
__device__ inline void split8(const f32x4& a, const f32x4& b, bf16x8 (&o)[3]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a[e] : b[e - 4];
        o[0][e] = (__bf16)x;
        const float r = x - (float)o[0][e];
        o[1][e] = (__bf16)r;
        if constexpr (PARTS == 3) o[2][e] = (__bf16)(r - (float)o[1][e]);
    }
}

// acc += A B over bf16 operand parts: bf16 data is exact (one part); fp32
// data is split three ways and the six partial products that matter at fp32
// precision are taken, smallest first.
template <typename T>
__device__ inline f32x16 mfma_parts(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x16 acc) {
    if constexpr (sizeof(T) == 4) {
        acc = mfma32(a[1], b[1], acc);
        acc = mfma32(a[2], b[0], acc);
        acc = mfma32(a[0], b[2], acc);
        acc = mfma32(a[1], b[0], acc);
        acc = mfma32(a[0], b[1], acc);
    }
    return mfma32(a[0], b[0], acc);
}

// ---------------------------------------------------------------------------
// The projection GEMM.  One 256-thread workgroup (4 waves) per 128 tokens and
// NT 32-column tiles of P.  The input width is walked in chunks of 128 bytes
// per row; a chunk of the 128 x rows and the 32 NT weight rows fills one stage
// of an LDS ring as deep as LDS allows, so all but one of its stages are in
// flight while the oldest is multiplied.  The stage's 1 KB groups of 8 rows
// are dealt to the waves, 4 + NT loads each per chunk (always that many, so
// the waits count statically).  Each wave forms 32 tokens x 32 NT columns of
// P^T, one x fragment serving all its column tiles.  Weight rows come in
// groups of 8 from Wd, ub or uf (R is a multiple of 16 and the gate blocks are
// padded to 8), so a group's load has one source; rows past the data read
// zeros.  Workgroups start at different chunks (and wrap around), so that at
// any moment they read different 128-byte columns of rows that lie Dm
// elements apart.
constexpr int kProjTM = 128;
constexpr int kProjMaxTiles = 4;
constexpr int kProjLds = 140 * 1024;          // LDS budget of the ring

template <int NT>
struct ProjGeom {
    static constexpr int IPW = 4 + NT;                      // loads per wave per chunk
    static constexpr int STAGE = (kProjTM + 32 * NT) * 128;
    static constexpr int STAGES = kProjLds / STAGE < 8 ? kProjLds / STAGE : 8;
};

// byte offset of 16-byte unit u of row r of a stage region: 8 units per row,
// XOR-swizzled with bits 1..3 of the row, so that 16 consecutive rows read at
// one unit (a quarter wave) fall into 16 different bank groups
__device__ inline int proj_off(int r, int u) { return r * 128 + 16 * (u ^ ((r >> 1) & 7)); }

// the 8 values k = 16 ks + 8 h .. +7 of row r of a region as operand parts
__device__ inline void proj_parts(const char* reg, int r, int ks, int h, const bf16* /*tag*/,
                                  bf16x8 (&o)[3]) {
    o[0] = *reinterpret_cast<const bf16x8*>(reg + proj_off(r, 2 * ks + h));
}
__device__ inline void proj_parts(const char* reg, int r, int ks, int h, const float* /*tag*/,
                                  bf16x8 (&o)[3]) {
    const int u = 4 * ks + 2 * h;
    split8<3>(*reinterpret_cast<const f32x4*>(reg + proj_off(r, u)),
              *reinterpret_cast<const f32x4*>(reg + proj_off(r, u + 1)), o);
}

template <typename T, int NT>
__global__ void __launch_bounds__(256)
param_project_kernel(const T* __restrict__ x, const T* __restrict__ Wd, const T* __restrict__ ub,
                     const T* __restrict__ uf, int M, int Dm, int R, int H, int H8, int Rp,
                     float* __restrict__ P) {
    using G = ProjGeom<NT>;
    constexpr int IPW = G::IPW, S = G::STAGES;
    __shared__ __attribute__((aligned(1024))) char lds[S][G::STAGE];
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ngroups = (Rp / 32 + NT - 1) / NT;
    const int tb = blockIdx.x / ngroups, jg = blockIdx.x % ngroups;
    const int t0 = kProjTM * tb, jt0 = jg * NT;
    const uint32_t rowb = (uint32_t)Dm * sizeof(T);
    // load i of this wave fills the stage's 1 KB group gi = IPW wave + i: x rows
    // 8 gi .. (gi < 16) or weight rows 8 (gi - 16) ..; lane -> row + lane / 8,
    // stored unit lane % 8 (holding unit u)
    __amdgpu_buffer_rsrc_t rs[IPW];
    uint32_t voff[IPW];
    int lim[IPW];   // the chunk's byte offset must not exceed this (tail of a row)
    const int rl = lane >> 3, pu = lane & 7;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int gi = IPW * wave + i;
        const bool isx = gi < 16;
        const int r = 8 * (isx ? gi : gi - 16) + rl, u = pu ^ ((r >> 1) & 7);
        uint32_t row = 0;
        lim[i] = (int)rowb - 16 * u - 16;
        if (isx) {
            rs[i] = rsrc_of(x + (size_t)t0 * Dm, (uint32_t)min(kProjTM, M - t0) * rowb);
            row = r;
        } else {
            const int col0 = 32 * jt0 + 8 * (gi - 16);   // the group's first column of P
            if (col0 < R) {
                rs[i] = rsrc_of(Wd, (uint32_t)R * rowb);
                row = col0 + rl;
            } else if (col0 < R + H8) {
                rs[i] = rsrc_of(ub, (uint32_t)H * rowb);
                row = col0 - R + rl;
            } else if (uf && col0 < R + 2 * H8) {
                rs[i] = rsrc_of(uf, (uint32_t)H * rowb);
                row = col0 - R - H8 + rl;
            } else {
                rs[i] = rsrc_of(Wd, 0u);             // padding columns: zeros
                lim[i] = -1;
            }
        }
        voff[i] = row * rowb + 16 * u;
    }
    const int nch = (int)((rowb + 127) / 128), rot = tb % nch;
    auto issue = [&](int j, int st) {
        const int kc = j + rot < nch ? j + rot : j + rot - nch;
        char* dst = lds[st] + IPW * wave * 1024;
        const int off = kc * 128;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            lds_load16(rs[i], off <= lim[i] ? voff[i] : kOob, (uint32_t)off, dst + i * 1024);
    };
    f32x16 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[q] = zero16();
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        if (s < nch) issue(s, s);
    int st = 0;
    for (int j = 0; j < nch; ++j) {
        // chunk j has landed once at most the chunks issued after it are pending
        wait_ahead<IPW, S - 2>(min(nch - 1, j + S - 2) - j);
        // every wave's part of chunk j has landed, and every wave is done with
        // the stage of chunk j - 1 (its operands were consumed by its products)
        bare_barrier();
        if (j + S - 1 < nch) issue(j + S - 1, st == 0 ? S - 1 : st - 1);
        const char* xs = lds[st];
        const char* wsr = xs + kProjTM * 128;
        // all of the chunk's operands first, then the products
        constexpr int KS = 128 / (16 * (int)sizeof(T));
        bf16x8 b[KS][3], a[KS][NT][3];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            proj_parts(xs, 32 * wave + c, ks, h, (const T*)nullptr, b[ks]);
#pragma unroll
            for (int q = 0; q < NT; ++q) proj_parts(wsr, 32 * q + c, ks, h, (const T*)nullptr, a[ks][q]);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int q = 0; q < NT; ++q) acc[q] = mfma_parts<T>(a[ks][q], b[ks], acc[q]);
        st = st + 1 == S ? 0 : st + 1;
    }
    const int t = t0 + 32 * wave + c, nt = min(NT, Rp / 32 - jt0);
    if (t < M) {
        // lane: token t; registers 4i..4i+3 of tile q: columns 32(jt0+q) + 8i + 4h.
        // Low-rank columns go out split: each group of 8 holds its 8 bf16 hi
        // parts, then its 8 lo parts (the bytes of 8 floats), the operand
        // layout of the finish; gate columns stay float.
        char* prow = reinterpret_cast<char*>(P + (size_t)t * Rp);
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            if (q < nt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = 32 * (jt0 + q) + 8 * i;
                    const f32x4 v = {acc[q][4 * i], acc[q][4 * i + 1], acc[q][4 * i + 2],
                                     acc[q][4 * i + 3]};
                    if (col < R) {
                        bf16x4 hi, lo;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            hi[e] = (__bf16)v[e];
                            lo[e] = (__bf16)(v[e] - (float)hi[e]);
                        }
                        *reinterpret_cast<bf16x4*>(prow + 4 * col + 8 * h) = hi;
                        *reinterpret_cast<bf16x4*>(prow + 4 * col + 16 + 8 * h) = lo;
                    } else {
                        *reinterpret_cast<f32x4*>(prow + 4 * (col + 4 * h)) = v;
                    }
                }
            }
        }
    }
}

// beta = 2 sigma(z) and log sigma(z) = min(z, 0) - log(1 + e^-|z|), with the
// hardware exp, log and reciprocal (relative errors of a few ulp; the log's
// argument lies in (1, 2], so its absolute error stays near 1e-7)
__device__ inline float sigmoid2(float z) { return 2.f * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
__device__ inline float log_sigmoid(float z) {
    return fminf(z, 0.f) - __logf(1.f + __expf(-fabsf(z)));
}

// ---------------------------------------------------------------------------
// The finish.  A workgroup owns a group of four heads (one per wave) and walks
// a sequence of 32-token tiles; tiles are dealt so that the head groups of one
// tile run on the same XCD (blockIdx % 8), which then reads the tile's rows
// of P once into its L2.  Per tile, the 34 rows of P it needs (its tokens and
// the two before, zeros outside the sequence) are loaded straight into an LDS
// stage while the previous tile is computed.  A stage row holds R/4 units of
// p, then one unit with the group's four beta logits and one with its four
// gate logits, its unit count made odd so that consecutive rows start in
// different bank groups.  Per head: y_tau = Wu P_{t - tau}^T (Wu the A
// operand; bf16 Wu exact, P split into hi + lo at the read), then
// c = sum_tau kc[:, tau] y_tau, the norm, and w written through the wave's
// LDS tile as whole rows -- a head's 32 tokens are one contiguous block of w.
constexpr int kFinishHeads = 4;
constexpr int kOutPad = 8;      // row padding (elements) of a wave's output tile

struct FinishGeom {
    int U, IPW;                  // units per stage row; loads per wave per stage
    __host__ __device__ FinishGeom(int R, bool gate) {
        U = (R / 4 + 1 + (gate ? 1 : 0)) | 1;
        IPW = (34 * U + 255) / 256;
    }
    __host__ __device__ int stage_bytes() const { return IPW * 4096; }
};

template <typename T, int D>
__host__ __device__ constexpr int finish_out_bytes() {
    return kFinishHeads * 32 * (D + kOutPad) * (int)sizeof(T);
}
template <typename T, int D>
__host__ __device__ inline int finish_lds_bytes(int R, bool gate) {
    return 2 * FinishGeom(R, gate).stage_bytes() + finish_out_bytes<T, D>() +
           3 * kFinishHeads * D * 4;
}

// WS > 0: the wave's Wu fragments for R <= 16 WS held in registers (bf16);
// WS == 0: loaded per rank step (any R, any dtype).
template <typename T, int D, int WS>
__global__ void __launch_bounds__(256)
param_finish_kernel(const float* __restrict__ P, const T* __restrict__ Wu,
                    const float* __restrict__ kc, const float* __restrict__ bb,
                    const float* __restrict__ bf, int N, int L, int R, int H, int H8, int Rp,
                    int nseq, T* __restrict__ w, float* __restrict__ beta,
                    float* __restrict__ logf) {
    static_assert(WS == 0 || sizeof(T) == 2, "register-held Wu is the bf16 path");
    constexpr int CT = D < 32 ? 1 : D / 32;     // 32-channel tiles per head
    constexpr int MAXI = WS > 0 ? 3 : 9;        // loads per wave per stage, bound
    extern __shared__ __attribute__((aligned(1024))) char dyn[];
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, c = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool gate = logf != nullptr;
    const FinishGeom geo(R, gate);
    const int U = geo.U, IPW = geo.IPW, SB = geo.stage_bytes();
    T* sOut = reinterpret_cast<T*>(dyn + 2 * SB) + wave * 32 * (D + kOutPad);
    float* sKc = reinterpret_cast<float*>(dyn + 2 * SB + finish_out_bytes<T, D>());
    const int ntt = (L + 31) / 32, ntiles = N * ntt, nhg = (H + kFinishHeads - 1) / kFinishHeads;
    const int x8 = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int hg = j % nhg, seq = x8 + 8 * (j / nhg);
    if (seq >= ntiles) return;
    const int hh = kFinishHeads * hg + wave;     // this wave's head
    const bool hok = hh < H;

    // this lane's stage units: row and float column of P (-1: padding)
    int prow[MAXI], pcol[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int slot = (wave * IPW + i) * 64 + lane, row = slot / U, u = slot - row * U;
        int col = -1;
        if (row < 34) {
            if (u < R / 4) col = 4 * u;
            else if (u == R / 4) col = R + kFinishHeads * hg;
            else if (gate && u == R / 4 + 1) col = R + H8 + kFinishHeads * hg;
        }
        prow[i] = row;
        pcol[i] = col;
    }
    auto issue = [&](int g, char* st) {
        const int n = g / ntt, t0 = 32 * (g - n * ntt);
        const auto rs = rsrc_of(P + (size_t)n * L * Rp, (uint32_t)L * Rp * 4);
        char* dst = st + wave * IPW * 1024;
#pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            if (i < IPW) {
                const int t = t0 - 2 + prow[i];
                const bool ok = pcol[i] >= 0 && t >= 0 && t < L;
                lds_load16(rs, ok ? (uint32_t)(t * Rp + pcol[i]) * 4u : kOob, 0u, dst + i * 1024);
            }
        }
    };
    // the group's taps, [tau][head-local channel], read before the first
    // stage is requested and written after, so the reads overlap it
    constexpr int KI = (3 * kFinishHeads * D + 255) / 256;
    float kv[KI];
#pragma unroll
    for (int q = 0; q < KI; ++q) {
        const int e = tid + 256 * q, tau = e / (kFinishHeads * D), cl = e - tau * kFinishHeads * D;
        const int ch = kFinishHeads * hg * D + cl;
        kv[q] = e < 3 * kFinishHeads * D && ch < H * D ? kc[(size_t)(ch < H * D ? ch : 0) * 3 + tau] : 0.f;
    }
    const float bbh = hok ? bb[hh] : 0.f, bfh = hok && gate ? bf[hh] : 0.f;
    bf16x8 wreg[CT][WS > 0 ? WS : 1];
    if constexpr (WS > 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int chl = 32 * ct + c;
            const bool ok = hok && chl < D;
            const bf16* wp = reinterpret_cast<const bf16*>(Wu) + (size_t)(ok ? hh * D + chl : 0) * R;
#pragma unroll
            for (int s = 0; s < WS; ++s) {
                const int r0 = 16 * s < R ? 16 * s : 0;
                wreg[ct][s] = *reinterpret_cast<const bf16x8*>(wp + r0 + 8 * h);
                if (!ok) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) wreg[ct][s][e] = (__bf16)0.f;
                }
            }
        }
    }

    issue(seq, dyn);
#pragma unroll
    for (int q = 0; q < KI; ++q)
        if (tid + 256 * q < 3 * kFinishHeads * D) sKc[tid + 256 * q] = kv[q];
    // per tile, a head's wave stores exactly NROW + 1 (+ 1 with a gate) times:
    // whole rows of w, then beta (and log f); lanes past the data are dropped
    // by the buffer ranges.  The wait for a tile's stage therefore leaves the
    // previous tile's stores in flight.
    constexpr int UPR = D * (int)sizeof(T) / 16;      // 16-byte units per row of w
    constexpr int NROW = 32 * UPR / 64;
    int k = 0;
    for (int g = seq; g < ntiles; g += nseq, ++k) {
        if (k == 0 || !hok) wait_vm0();
        else if (gate) wait_vm<NROW + 2>();
        else wait_vm<NROW + 1>();
        // this tile's stage has landed; the other stage is free
        if (k == 0) __syncthreads();    // also publishes the taps
        else bare_barrier();
        char* st = dyn + (k & 1) * SB;
        if (g + nseq < ntiles) issue(g + nseq, dyn + ((k + 1) & 1) * SB);
        if (!hok) continue;
        const int n = g / ntt, t0 = 32 * (g - n * ntt);
        // B operand of tap tau, rank step r0: P row t - tau (stage row c + 2 - tau),
        // ranks r0 + 8h .. +7: one group of 8, its hi unit then its lo unit
        auto bpart = [&](int tau, int r0, bf16x8 (&o)[3]) {
            const char* rp = st + ((c + 2 - tau) * U + r0 / 4 + 2 * h) * 16;
            o[0] = *reinterpret_cast<const bf16x8*>(rp);
            o[1] = *reinterpret_cast<const bf16x8*>(rp + 16);
        };
        // c = sum_tau kc[:, tau] y_tau; lane: token t0 + c, registers 4i..4i+3
        // of tile ct: channels 32ct + 8i + 4h + j
        f32x16 acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = zero16();
        auto fold = [&](int tau, const f32x16 (&y)[CT]) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch0 = 32 * ct + 8 * i + 4 * h;
                    f32x4 kt = {0.f, 0.f, 0.f, 0.f};
                    if (ch0 < D) kt = *reinterpret_cast<const f32x4*>(sKc + (tau * kFinishHeads + wave) * D + ch0);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc[ct][4 * i + jj] += kt[jj] * y[ct][4 * i + jj];
                }
            }
        };
        // rank step by rank step, a Wu fragment serving the three taps
        f32x16 y[3][CT];
#pragma unroll
        for (int tau = 0; tau < 3; ++tau)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) y[tau][ct] = zero16();
        auto step = [&](const bf16x8 (&a)[CT][3], int r0) {
#pragma unroll
            for (int tau = 0; tau < 3; ++tau) {
                bf16x8 b[3];
                bpart(tau, r0, b);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    if constexpr (sizeof(T) == 2) {
                        y[tau][ct] = mfma32(a[ct][0], b[1], y[tau][ct]);
                        y[tau][ct] = mfma32(a[ct][0], b[0], y[tau][ct]);
                    } else {
                        y[tau][ct] = mfma_split(a[ct][0], a[ct][1], b[0], b[1], y[tau][ct]);
                    }
                }
            }
        };
        if constexpr (WS > 0) {
#pragma unroll
            for (int s = 0; s < WS; ++s) {
                if (s == 0 || 16 * s < R) {       // R >= 16: the first step always runs
                    bf16x8 a[CT][3];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) a[ct][0] = wreg[ct][s];
                    step(a, 16 * s);
                }
            }
        } else {
            for (int r0 = 0; r0 < R; r0 += 16) {
                bf16x8 a[CT][3];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int chl = 32 * ct + c;
                    const bool ok = chl < D;
                    const T* wp = Wu + (size_t)(hh * D + (ok ? chl : 0)) * R + r0 + 8 * h;
                    if constexpr (sizeof(T) == 2) {
                        a[ct][0] = *reinterpret_cast<const bf16x8*>(wp);
                        if (!ok) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) a[ct][0][e] = (__bf16)0.f;
                        }
                    } else {
                        f32x4 lo = *reinterpret_cast<const f32x4*>(wp);
                        f32x4 hi = *reinterpret_cast<const f32x4*>(wp + 4);
                        if (!ok) lo = hi = f32x4{0.f, 0.f, 0.f, 0.f};
                        split8<2>(lo, hi, a[ct]);
                    }
                }
                step(a, r0);
            }
        }
#pragma unroll
        for (int tau = 0; tau < 3; ++tau) fold(tau, y[tau]);
        float ss = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) ss += acc[ct][r] * acc[ct][r];
        ss = pair_sum(ss);
        const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
        // the wave's 32 x D tile of w through its LDS tile, out as whole rows
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * ct + 8 * i + 4 * h;
                if (ch0 < D) {
                    T* o = sOut + c * (D + kOutPad) + ch0;
                    if constexpr (sizeof(T) == 2) {
                        *reinterpret_cast<bf16x4*>(o) =
                            bf16x4{(__bf16)(acc[ct][4 * i] * inv), (__bf16)(acc[ct][4 * i + 1] * inv),
                                   (__bf16)(acc[ct][4 * i + 2] * inv), (__bf16)(acc[ct][4 * i + 3] * inv)};
                    } else {
                        *reinterpret_cast<f32x4*>(o) =
                            f32x4{acc[ct][4 * i] * inv, acc[ct][4 * i + 1] * inv,
                                  acc[ct][4 * i + 2] * inv, acc[ct][4 * i + 3] * inv};
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        const int nrows = min(32, L - t0);
        const size_t o = ((size_t)n * H + hh) * L + t0;     // the head's first row of the tile
        const auto wr = rsrc_of(w + o * D, (uint32_t)(nrows * D * (int)sizeof(T)));
#pragma unroll
        for (int q = 0; q < NROW; ++q) {
            const int u = lane + 64 * q, rr = u / UPR, xu = u - rr * UPR;
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                reinterpret_cast<const char*>(sOut + rr * (D + kOutPad)) + 16 * xu);
            __builtin_amdgcn_raw_buffer_store_b128(v, wr, 16 * u, 0, 0);
        }
        __builtin_amdgcn_wave_barrier();
        const float* zr = reinterpret_cast<const float*>(st + ((c + 2) * U + R / 4) * 16);
        const int bo = h == 0 ? 4 * c : (int)kOob;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sigmoid2(zr[wave] + bbh)),
                                              rsrc_of(beta + o, (uint32_t)nrows * 4), bo, 0, 0);
        if (gate)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(log_sigmoid(zr[4 + wave] + bfh)),
                                                  rsrc_of(logf + o, (uint32_t)nrows * 4), bo, 0, 0);
    }
    wait_vm0();
}

// finish workgroups: each head group gets 8 m tile sequences (a multiple of
// the XCD count), about three workgroups per CU in all
constexpr int kFinishWgs = 768;

template <typename T, int D, int WS>
hipError_t finish_t(const ParamArgs& a, int H8, hipStream_t st) {
    const bool gate = a.logf != nullptr;
    const long ntiles = (long)a.N * ((a.L + 31) / 32);
    const int nhg = (a.H + kFinishHeads - 1) / kFinishHeads;
    const long m = std::max(1L, std::min((ntiles + 7) / 8, (long)kFinishWgs / (8 * nhg)));
    const int nseq = (int)(8 * m);
    const int lds = finish_lds_bytes<T, D>(a.R, gate);
    if (lds > 65536) {   // beyond the default dynamic LDS limit (large ranks)
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&param_finish_kernel<T, D, WS>),
            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((param_finish_kernel<T, D, WS>), dim3((unsigned)(nhg * nseq)), dim3(256),
                       (size_t)lds, st, a.P, (const T*)a.Wu, a.kc, a.bb, a.bf, a.N, a.L, a.R,
                       a.H, H8, a.Rp, nseq, (T*)a.w, a.beta, a.logf);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t finish_d(const ParamArgs& a, int H8, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        if (a.R <= 32) return finish_t<T, D, 2>(a, H8, st);
        if (a.R <= 64) return finish_t<T, D, 4>(a, H8, st);
    }
    return finish_t<T, D, 0>(a, H8, st);
}

// column tiles per projection workgroup: the fewest groups of at most
// kProjMaxTiles, then as even as they go
template <typename T, int NT>
hipError_t project_nt(const ParamArgs& a, long M, int H8, hipStream_t st) {
    const long ngroups = (a.Rp / 32 + NT - 1) / NT;
    hipLaunchKernelGGL((param_project_kernel<T, NT>),
                       dim3((unsigned)(((M + kProjTM - 1) / kProjTM) * ngroups)), dim3(256), 0,
                       st, (const T*)a.x, (const T*)a.Wd, (const T*)a.ub, (const T*)a.uf,
                       (int)M, a.Dm, a.R, a.H, H8, a.Rp, a.P);
    return hipGetLastError();
}
template <typename T>
hipError_t project_t(const ParamArgs& a, long M, int H8, hipStream_t st) {
    const int ntn = a.Rp / 32, ngroups = (ntn + kProjMaxTiles - 1) / kProjMaxTiles;
    switch ((ntn + ngroups - 1) / ngroups) {
        case 1: return project_nt<T, 1>(a, M, H8, st);
        case 2: return project_nt<T, 2>(a, M, H8, st);
        case 3: return project_nt<T, 3>(a, M, H8, st);
        default: return project_nt<T, 4>(a, M, H8, st);
    }
}

template <typename T>
hipError_t launch_param_t(const ParamArgs& a, hipStream_t st) {
    const long M = (long)a.N * a.L;
    const int H8 = (a.H + 7) / 8 * 8;
    hipError_t e = project_t<T>(a, M, H8, st);
    if (e != hipSuccess) return e;
    switch (a.d) {
        case 16: return finish_d<T, 16>(a, H8, st);
        case 32: return finish_d<T, 32>(a, H8, st);
        case 64: return finish_d<T, 64>(a, H8, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int param_columns(int R, int H, bool gate) {
    const int H8 = (H + 7) / 8 * 8;
    return (R + H8 * (gate ? 2 : 1) + 31) / 32 * 32;
}

hipError_t launch_param(const ParamArgs& a, hipStream_t st) {
    return a.bf16 ? launch_param_t<bf16>(a, st) : launch_param_t<float>(a, st);
}

}  // namespace pa
