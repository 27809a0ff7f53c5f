// bwd.hip -- backward pass of PaTH(-FoX) attention: gradients of a loss with
// respect to q, k, v, w, beta and log f, given dL/do.
//
// Citations: [Notes s2.x] = reading-notes page "PaTH Attention:通过累积
// Householder 变换编码位置" (cc.laoqi.cc), section 2.x.
//
// The pages give no backward formulas.  This is reverse-mode differentiation
// of the forward's block algorithm -- the per-block UT solve and boundary
// preconditioning [Notes s2.6], the right-to-left scan [Notes s2.7] -- with
// blocks of B = 64.  Per slice (batch, head), query block b, key block c < b:
//   forward   S_bc = scale Qw_c Kr_c^T + bias, Qw_{b-1} = Ql_b,
//             Qw_{c-1} = Qw_c (I - E_c)^T; diagonal S_bb = scale Dg_b + bias;
//             P = exp(S - lse); o = P V.
//   backward  Delta_i = do_i . o_i;  dS = P (do V^T - Delta);
//             dV_c = sum_b P_bc^T do_b;  dKr_c = scale sum_b dS_bc^T Qw_c;
//             A_0 = scale dS_b0 Kr_0, A_c = scale dS_bc Kr_c + A_{c-1} (I - E_c),
//             dQl_b = A_{b-1};  dE_c = -sum_b A_{c-1}^T Qw_c  (c >= 1);
//             dDg_b = scale dS_bb;  the gate bias of logit (i, j) is C_i - C_j
//             with C the running sum of log f, so dC_t = rowsum_t(dS) -
//             colsum_t(dS) and dlogf_s = sum_{t >= s} dC_t (log f_0 is never
//             read: dlogf_0 = 0);
//             then each block's (dQl, dKr, dE, dDg) back through the
//             preconditioning and the UT solve to dq, dk, dw, dbeta.
// Kernels: the forward's preconditioning (recomputed), `chain` (query-major:
// the Qw_c of every block pair, kept in the workspace), `query` (query-major,
// left to right: dS, the A chain, dQl, dDg, row sums), `key` (key-major: dV,
// dKr, dE, column sums -- accumulated in LDS, no atomics), `precond_bwd`
// (per block), `gate_bwd` (per slice).  All products run on the matrix cores
// from fp32 tiles split into bf16 parts (two for bf16 data, three for fp32).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "img.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace pa {

namespace {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kB = 64;          // block size
constexpr int kLdB = kB + 4;    // LDS row stride of a B x B tile (floats)

template <int D>
struct Dims {
    static constexpr int DP = D < 32 ? 32 : D;   // head dim padded to the 32-wide tiles
    static constexpr int LD = DP + 4;            // LDS row stride of a B x DP / DP x DP tile
};

// 8 fp32 values as bf16 operand parts: hi (1: exact for bf16 data), hi + lo
// (2) or hi + mid + lo (3)
template <int PARTS>
__device__ inline void parts8(const float (&v)[8], bf16x8 (&o)[3]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[0][e] = (__bf16)v[e];
        if constexpr (PARTS >= 2) {
            const float r = v[e] - (float)o[0][e];
            o[1][e] = (__bf16)r;
            if constexpr (PARTS == 3) o[2][e] = (__bf16)(r - (float)o[1][e]);
        }
    }
}
// acc += A B over the partial products that matter (a part of order i times
// one of order j kept when i + j < the larger part count), smallest first
template <int PA, int PB>
__device__ inline f32x16 mma(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x16 c) {
    constexpr int P = PA > PB ? PA : PB;
    if constexpr (P == 3) {
        if constexpr (PA >= 2 && PB >= 2) c = mfma32(a[1], b[1], c);
        if constexpr (PA == 3) c = mfma32(a[2], b[0], c);
        if constexpr (PB == 3) c = mfma32(a[0], b[2], c);
    }
    if constexpr (PA >= 2) c = mfma32(a[1], b[0], c);
    if constexpr (PB >= 2) c = mfma32(a[0], b[1], c);
    return mfma32(a[0], b[0], c);
}

// Operand views over fp32 tiles, read 8 values along the contraction at once.
// Rows (index i) past imax and contraction indices past kmax read zero; kmax
// is a multiple of 8.
struct Cont {           // value (i, k) = p[i * ld + k]: contiguous along k, vector loads
    const float* p;
    int ld, imax, kmax;
    __device__ void ld8(int i, int k0, float (&v)[8]) const {
        if (i < imax && k0 < kmax) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(p + (size_t)i * ld + k0);
            const f32x4 b = *reinterpret_cast<const f32x4*>(p + (size_t)i * ld + k0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = a[e];
                v[e + 4] = b[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        }
    }
};
struct Strd {           // value (i, k) = p[k * ld + i]: strided along k
    const float* p;
    int ld, imax, kmax;
    __device__ void ld8(int i, int k0, float (&v)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = i < imax && k0 < kmax ? p[(size_t)(k0 + e) * ld + i] : 0.f;
    }
};
// the same over bf16 storage (the caller's exact bf16 data in LDS)
struct ContH {
    const __bf16* p;
    int ld;
    __device__ void ld8(int i, int k0, float (&v)[8]) const {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + i * ld + k0);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
    }
};
struct StrdH {
    const __bf16* p;
    int ld;
    __device__ void ld8(int i, int k0, float (&v)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (float)p[(k0 + e) * ld + i];
    }
};
// views of an LDS tile of element type E (float or bf16) with row stride ld
__device__ inline Cont contv(const float* p, int ld) { return Cont{p, ld, 1 << 30, 1 << 30}; }
__device__ inline Strd strdv(const float* p, int ld) { return Strd{p, ld, 1 << 30, 1 << 30}; }
__device__ inline ContH contv(const __bf16* p, int ld) { return ContH{p, ld}; }
__device__ inline StrdH strdv(const __bf16* p, int ld) { return StrdH{p, ld}; }
__device__ inline Cont cont(const float* p, int ld, int imax = 1 << 30, int kmax = 1 << 30) {
    return Cont{p, ld, imax, kmax};
}
__device__ inline Strd strd(const float* p, int ld, int imax = 1 << 30, int kmax = 1 << 30) {
    return Strd{p, ld, imax, kmax};
}

// C (M x N) = sum_k A(m, k) B(k, n) on the matrix cores, A and B given as
// views indexed (row of the product's operand, contraction index): A by m, B
// by n.  The 32 x 32 output tiles are dealt to the workgroup's waves and
// out(m, n, value) receives each element (one lane per element; gemms of the
// same M x N deal their tiles identically, so a lane may accumulate into an
// element across such gemms without a barrier).  M, N multiples of 32, K of 16.
template <int PA, int PB, int K, typename VA, typename VB, typename FO>
__device__ inline void gemm(int M, int N, const VA& A, const VB& Bv, FO out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32, nt = (M / 32) * tn;
    for (int t = wave; t < nt; t += nw) {
        const int m0 = (t / tn) * 32, n0 = (t % tn) * 32;
        f32x16 c = zero16();
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 16) {
            float av[8], bv[8];
            A.ld8(m0 + r, k0 + 8 * h, av);
            Bv.ld8(n0 + r, k0 + 8 * h, bv);
            bf16x8 ap[3], bp[3];
            parts8<PA>(av, ap);
            parts8<PB>(bv, bp);
            c = mma<PA, PB>(ap, bp, c);
        }
        // C layout: lane -> column n0 + r, register 4i + j -> row m0 + 8i + 4h + j
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) out(m0 + 8 * i + 4 * h + j, n0 + r, c[4 * i + j]);
    }
}

// The wave's own 32 x 32 tile (tile index = wave) of C = sum_k A(m, k) B(k, n),
// accumulated into acc; waves past the tile count do nothing.  Its elements
// are visited with for_acc.  Callers use it where M x N has at most one tile
// per wave.
template <int PA, int PB, int K, typename VA, typename VB>
__device__ inline void gemm_acc(int M, int N, const VA& A, const VB& Bv, f32x16& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32;
    if (wave >= (M / 32) * tn) return;
    const int m0 = (wave / tn) * 32, n0 = (wave % tn) * 32;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        float av[8], bv[8];
        A.ld8(m0 + r, k0 + 8 * h, av);
        Bv.ld8(n0 + r, k0 + 8 * h, bv);
        bf16x8 ap[3], bp[3];
        parts8<PA>(av, ap);
        parts8<PB>(bv, bp);
        acc = mma<PA, PB>(ap, bp, acc);
    }
}
template <typename FO>
__device__ inline void for_acc(int M, int N, const f32x16& acc, FO f) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32;
    if (wave >= (M / 32) * tn) return;
    const int m0 = (wave / tn) * 32, n0 = (wave % tn) * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) f(m0 + 8 * i + 4 * h + j, n0 + r, acc[4 * i + j]);
}

__device__ inline size_t pair_index(int b, int c) { return (size_t)b * (b - 1) / 2 + c; }

// F: operand parts of fp32 intermediates (2 for bf16 data, 3 for fp32 data);
// X: parts of the caller's own data (v, do): 1 for bf16 (exact), else F.
template <typename T, int PARTS>
struct Parts {
    static constexpr int F = PARTS;
    static constexpr int X = sizeof(T) == 2 ? 1 : PARTS;
};

// Register prefetch of an [R][D] row-major tile (element type S) from global
// memory, in 16-byte units, later written into an fp32 LDS tile of row stride
// ld (columns past D are left alone: the caller zeroes them once).
template <typename S, int R, int D>
struct TilePf {
    static constexpr int EPU = 16 / (int)sizeof(S);     // elements per unit
    static constexpr int UPR = D / EPU;                 // units per row
    static constexpr int NU = (R * UPR + 255) / 256;
    u32x4 u[NU];
    __device__ void load(const S* src, int rows_valid) {
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = threadIdx.x + 256 * i, r = e / UPR, x = e % UPR;
            u[i] = u32x4{0u, 0u, 0u, 0u};
            if (e < R * UPR && r < rows_valid)
                u[i] = *reinterpret_cast<const u32x4*>(src + (size_t)r * D + x * EPU);
        }
    }
    __device__ void store(float* dst, int ld) const {
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = threadIdx.x + 256 * i, r = e / UPR, x = e % UPR;
            if (e >= R * UPR) continue;
            if constexpr (sizeof(S) == 4) {
                *reinterpret_cast<u32x4*>(dst + r * ld + 4 * x) = u[i];
            } else {   // 8 bf16 -> 8 floats (exact)
                f32x4 a, b;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    a[2 * q] = __uint_as_float(u[i][q] << 16);
                    a[2 * q + 1] = __uint_as_float(u[i][q] & 0xffff0000u);
                    b[2 * q] = __uint_as_float(u[i][q + 2] << 16);
                    b[2 * q + 1] = __uint_as_float(u[i][q + 2] & 0xffff0000u);
                }
                *reinterpret_cast<f32x4*>(dst + r * ld + 8 * x) = a;
                *reinterpret_cast<f32x4*>(dst + r * ld + 8 * x + 4) = b;
            }
        }
    }
};

// ---------------------------------------------------------------------------
// chain: for query block b >= 1 of a slice, the queries Qw_c used against every
// key block c < b, carried right to left as in the forward scan; stored per
// block pair in X [slice][pair][B][d].  Longest chains first.  (fp32 inputs
// and d = 16; bf16 at d 32/64 takes bwd_chain_b16_kernel.)
template <int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_chain_kernel(int nb, int nsc, int slice0, const float* __restrict__ ql,
                 const float* __restrict__ em, float* __restrict__ X) {
    using Dm = Dims<D>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ __attribute__((aligned(16))) float sQ[kB * LD], sT[kB * LD], sE[DP * LD];
    const int tid = threadIdx.x;
    const int b = nb - 1 - (int)(blockIdx.x / nsc), sl = (int)(blockIdx.x % nsc);
    const size_t slice = (size_t)slice0 + sl, npairs = (size_t)nb * (nb - 1) / 2;
    float* Xs = X + (size_t)sl * npairs * kB * D;
    const float* qlb = ql + (slice * nb + b) * kB * D;
    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP;
        sQ[r * LD + x] = x < D ? qlb[r * D + x] : 0.f;
    }
    for (int e = tid; e < DP * LD; e += 256) sE[e] = 0.f;   // the padding stays zero
    TilePf<float, D, D> pfE;                                 // the next step's E, in flight
    if (b - 1 >= 1) pfE.load(em + (slice * nb + b - 1) * D * D, D);
    for (int c = b - 1; c >= 0; --c) {
        __syncthreads();
        for (int e = tid; e < kB * (D / 4); e += 256) {
            const int r = e / (D / 4), x = 4 * (e % (D / 4));
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(sQ + r * LD + x);
            float* xo = Xs + pair_index(b, c) * kB * D;
            *reinterpret_cast<f32x4*>(xo + (size_t)r * D + x) = q4;
        }
        if (c == 0) break;
        pfE.store(sE, LD);
        __syncthreads();
        if (c - 1 >= 1) pfE.load(em + (slice * nb + c - 1) * D * D, D);
        // Qw_{c-1} = Qw_c - Qw_c E_c^T:  B(k, n) = E[n][k]
        gemm<PARTS, PARTS, DP>(kB, DP, cont(sQ, LD), cont(sE, LD),
                         [&](int m, int n, float v) { sT[m * LD + n] = v; });
        __syncthreads();
        for (int e = tid; e < kB * DP; e += 256) {
            const int r = e / DP, x = e % DP;
            sQ[r * LD + x] -= sT[r * LD + x];
        }
    }
}

// ---------------------------------------------------------------------------
// query: for query block b of a slice, left to right over the key blocks:
// the diagonal tile's dS (-> dDg_b), then for c = 0 .. b-1 the pair's dS and
// the chain A_c (A_{c-1} kept in Z for the transitions' gradients); dQl_b,
// the rows' dS sums and Delta.  Longest rows of pairs first.
template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_query_kernel(int L, int nb, int nsc, int slice0, float scale, int fox,
                 const T* __restrict__ v, const T* __restrict__ o, const T* __restrict__ dout,
                 const float* __restrict__ lse, FwdWs fw, const float* __restrict__ X,
                 float* __restrict__ Z, float* __restrict__ dQl, float* __restrict__ dDg,
                 float* __restrict__ rowsum, float* __restrict__ delta) {
    using Dm = Dims<D>;
    using Pt = Parts<T, PARTS>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ __attribute__((aligned(16))) float sdO[kB * LD], sV[kB * LD], sA[kB * LD],
        sK[kB * LD], sX[kB * LD], sE[DP * LD], sS[kB * kLdB], sP[kB * kLdB];
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB], sRow[kB];
    __shared__ float sTb;
    const int tid = threadIdx.x;
    const int b = nb - 1 - (int)(blockIdx.x / nsc), sl = (int)(blockIdx.x % nsc);
    const size_t slice = (size_t)slice0 + sl, blk_b = slice * nb + b, base = slice * L;
    const size_t npairs = (size_t)nb * (nb - 1) / 2;
    const float* Xs = X + (size_t)sl * npairs * kB * D;
    float* Zs = Z + (size_t)sl * npairs * kB * D;
    const float* kr = static_cast<const float*>(fw.kr);
    const float* em = static_cast<const float*>(fw.em);

    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP, pos = b * kB + r;
        sdO[r * LD + x] = x < D && pos < L ? to_f32(dout[(base + pos) * D + x]) : 0.f;
    }
    if (tid < kB) {
        const int pos = b * kB + tid;
        float dl = 0.f;
        if (pos < L)
            for (int x = 0; x < D; ++x)
                dl += to_f32(dout[(base + pos) * D + x]) * to_f32(o[(base + pos) * D + x]);
        sDel[tid] = dl;
        sLse[tid] = pos < L ? lse[base + pos] : 0.f;
        sGb[tid] = fox ? fw.gl[blk_b * kB + tid] : 0.f;
        sRow[tid] = 0.f;
        delta[blk_b * kB + tid] = dl;
    }
    if (tid == 0) {
        float s = 0.f;
        if (fox)
            for (int c = 0; c < b; ++c) s += fw.tot[slice * nb + c];
        sTb = s;
    }
    auto load_v = [&](int c) {
        for (int e = tid; e < kB * DP; e += 256) {
            const int r = e / DP, x = e % DP, pos = c * kB + r;
            sV[r * LD + x] = x < D && pos < L ? to_f32(v[(base + pos) * D + x]) : 0.f;
        }
    };
    auto row_sums = [&]() {   // four lanes per row, 16 columns each
        const int i = tid >> 2, q = tid & 3;
        float s = 0.f;
        for (int j = 16 * q; j < 16 * q + 16; ++j) s += sS[i * kLdB + j];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        if (q == 0) sRow[i] += s;
    };
    // the next key block's V, Kr, X_bc and E, in flight in registers while the
    // current one is processed
    TilePf<T, kB, D> pfV;
    TilePf<float, kB, D> pfK, pfX;
    TilePf<float, D, D> pfE;
    float pGc = 0.f;
    for (int e = tid; e < kB * LD; e += 256) sK[e] = sX[e] = 0.f;   // pad columns
    for (int e = tid; e < DP * LD; e += 256) sE[e] = 0.f;
    auto prefetch = [&](int c) {
        const size_t blk_c = slice * nb + c;
        pfV.load(v + (base + (size_t)c * kB) * D, min(kB, L - c * kB));
        pfK.load(kr + blk_c * kB * D, kB);
        pfX.load(Xs + pair_index(b, c) * kB * D, kB);
        if (c >= 1) pfE.load(em + blk_c * D * D, D);
        if (tid < kB) pGc = fox ? fw.gl[blk_c * kB + tid] : 0.f;
    };
    if (b > 0) prefetch(0);

    // diagonal tile: P from the in-block logits, then dS = P (dP - Delta)
    load_v(b);
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) {
        const int i = e / kB, j = e % kB;
        sS[i * kLdB + j] = j <= i && b * kB + i < L
            ? __expf(scale * fw.dg[blk_b * kB * kB + e] + (sGb[i] - sGb[j]) - sLse[i]) : 0.f;
    }
    __syncthreads();
    gemm<Pt::X, Pt::X, DP>(kB, kB, cont(sdO, LD), cont(sV, LD), [&](int m, int n, float val) {
        sP[m * kLdB + n] = val;
    });
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) {
        const int i = e / kB, j = e % kB;
        const float ds = sS[i * kLdB + j] * (sP[i * kLdB + j] - sDel[i]);
        sS[i * kLdB + j] = ds;
        dDg[blk_b * kB * kB + e] = scale * ds;
    }
    for (int e = tid; e < kB * DP; e += 256) sA[(e / DP) * LD + e % DP] = 0.f;
    __syncthreads();
    row_sums();

    float Tc = 0.f;                 // sum of the gate totals of blocks before c
    for (int c = 0; c < b; ++c) {
        const size_t blk_c = slice * nb + c;
        __syncthreads();
        pfV.store(sV, LD);
        pfK.store(sK, LD);
        pfX.store(sX, LD);
        if (c >= 1) pfE.store(sE, LD);
        if (tid < kB) sGc[tid] = pGc;
        __syncthreads();
        if (c + 1 < b) prefetch(c + 1);
        const float shift = fox ? sTb - Tc : 0.f;   // sum of the totals of blocks c .. b-1
        // P = exp(scale X Kr^T + bias - lse), then dS = P (dO V^T - Delta) in place
        // (the two products deal their tiles alike: each lane finishes its own P)
        gemm<Pt::F, Pt::F, DP>(kB, kB, cont(sX, LD), cont(sK, LD), [&](int m, int n, float val) {
            sS[m * kLdB + n] = b * kB + m < L
                ? __expf(scale * val + (sGb[m] + shift - sGc[n]) - sLse[m]) : 0.f;
        });
        gemm<Pt::X, Pt::X, DP>(kB, kB, cont(sdO, LD), cont(sV, LD), [&](int m, int n, float val) {
            sS[m * kLdB + n] *= val - sDel[m];
        });
        __syncthreads();
        row_sums();
        // G = scale dS Kr_c and (c >= 1) A_{c-1} E_c, in registers
        f32x16 gt = zero16(), ae = zero16();
        gemm_acc<Pt::F, Pt::F, kB>(kB, DP, cont(sS, kLdB), strd(sK, LD), gt);
        if (c >= 1) {
            float* zo = Zs + pair_index(b, c) * kB * D;
            for (int e = tid; e < kB * (D / 4); e += 256) {
                const int r = e / (D / 4), x = 4 * (e % (D / 4));
                *reinterpret_cast<f32x4*>(zo + (size_t)r * D + x) =
                    *reinterpret_cast<const f32x4*>(sA + r * LD + x);
            }
            gemm_acc<Pt::F, Pt::F, DP>(kB, DP, cont(sA, LD), strd(sE, LD, D, D), ae);
        }
        __syncthreads();   // every read of A_{c-1} is done
        // A_c = scale dS Kr_c + A_{c-1} - A_{c-1} E_c
        const bool first = c == 0;
        {
            const int lane = tid & 63, wave = tid >> 6, r = lane & 31, h = lane >> 5;
            const int tn = DP / 32;
            if (wave < 2 * tn) {
                const int m0 = (wave / tn) * 32, n0 = (wave % tn) * 32;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float* a = sA + (m0 + 8 * i + 4 * h + j) * LD + n0 + r;
                        *a = scale * gt[4 * i + j] + (first ? 0.f : *a - ae[4 * i + j]);
                    }
            }
        }
        if (fox) Tc += fw.tot[blk_c];
    }
    __syncthreads();
    for (int e = tid; e < kB * D; e += 256) dQl[blk_b * kB * D + e] = sA[(e / D) * LD + e % D];
    if (tid < kB) rowsum[blk_b * kB + tid] = sRow[tid];
}

// ---------------------------------------------------------------------------
// key: for key block c of a slice, over the query blocks b >= c: dV_c, dKr_c,
// dE_c (matrix-core accumulators held in registers across the loop, a wave per
// output tile) and the keys' dS column sums.  Longest first.
template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_key_kernel(int L, int nb, int nsc, int slice0, float scale, int fox,
               const T* __restrict__ v, const T* __restrict__ dout,
               const float* __restrict__ lse, const float* __restrict__ delta, FwdWs fw,
               const float* __restrict__ X, const float* __restrict__ Z,
               float* __restrict__ dKr, float* __restrict__ dEm, T* __restrict__ dv,
               float* __restrict__ colsum) {
    using Dm = Dims<D>;
    using Pt = Parts<T, PARTS>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ __attribute__((aligned(16))) float sV[kB * LD], sK[kB * LD], sdO[kB * LD],
        sX[kB * LD], sZ[kB * LD], sS[kB * kLdB], sP[kB * kLdB];
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB], sCol[kB], sCp[4][kB];
    const int tid = threadIdx.x;
    const int c = (int)(blockIdx.x / nsc), sl = (int)(blockIdx.x % nsc);
    const size_t slice = (size_t)slice0 + sl, blk_c = slice * nb + c, base = slice * L;
    const size_t npairs = (size_t)nb * (nb - 1) / 2;
    const float* Xs = X + (size_t)sl * npairs * kB * D;
    const float* Zs = Z + (size_t)sl * npairs * kB * D;
    auto stage = [&](float* dst, const float* src) {
        for (int e = tid; e < kB * (DP / 4); e += 256) {
            const int r = e / (DP / 4), x = 4 * (e % (DP / 4));
            *reinterpret_cast<f32x4*>(dst + r * LD + x) =
                x < D ? *reinterpret_cast<const f32x4*>(src + (size_t)r * D + x)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP, pos = c * kB + r;
        sV[r * LD + x] = x < D && pos < L ? to_f32(v[(base + pos) * D + x]) : 0.f;
    }
    stage(sK, static_cast<const float*>(fw.kr) + blk_c * kB * D);
    if (tid < kB) {
        sGc[tid] = fox ? fw.gl[blk_c * kB + tid] : 0.f;
        sCol[tid] = 0.f;
    }
    f32x16 accV = zero16(), accK = zero16(), accE = zero16();
    // the next query block's dO, X_bc, Z_bc and row terms, in flight in
    // registers while the current block is processed
    TilePf<T, kB, D> pfO;
    TilePf<float, kB, D> pfX, pfZ;
    float pLse = 0.f, pDel = 0.f, pGb = 0.f;
    for (int e = tid; e < kB * LD; e += 256) sX[e] = sZ[e] = 0.f;   // pad columns
    auto prefetch = [&](int b) {
        const size_t blk_b = slice * nb + b;
        pfO.load(dout + (base + (size_t)b * kB) * D, min(kB, L - b * kB));
        pfX.load(Xs + pair_index(b, c) * kB * D, kB);
        if (c >= 1) pfZ.load(Zs + pair_index(b, c) * kB * D, kB);
        if (tid < kB) {
            const int pos = b * kB + tid;
            pLse = pos < L ? lse[base + pos] : 0.f;
            pDel = delta[blk_b * kB + tid];
            pGb = fox ? fw.gl[blk_b * kB + tid] : 0.f;
        }
    };
    // per query block b: its dO, lse, Delta and gate cumsum
    auto load_rows = [&](int b) {
        const size_t blk_b = slice * nb + b;
        for (int e = tid; e < kB * DP; e += 256) {
            const int r = e / DP, x = e % DP, pos = b * kB + r;
            sdO[r * LD + x] = x < D && pos < L ? to_f32(dout[(base + pos) * D + x]) : 0.f;
        }
        if (tid < kB) {
            const int pos = b * kB + tid;
            sLse[tid] = pos < L ? lse[base + pos] : 0.f;
            sDel[tid] = delta[blk_b * kB + tid];
            sGb[tid] = fox ? fw.gl[blk_b * kB + tid] : 0.f;
        }
    };
    // sS holds P: dV += P^T dO; dP -> sP; dS -> sS; columns summed
    auto backprop = [&]() {
        __syncthreads();   // P is complete
        gemm_acc<Pt::F, Pt::X, kB>(kB, DP, strd(sS, kLdB), strd(sdO, LD), accV);
        gemm<Pt::X, Pt::X, DP>(kB, kB, cont(sdO, LD), cont(sV, LD),
                           [&](int m, int n, float val) { sP[m * kLdB + n] = val; });
        __syncthreads();
        // a thread keeps one column (tid % 64) and every fourth row
        float cs = 0.f;
        for (int e = tid; e < kB * kB; e += 256) {
            const int i = e / kB, j = e % kB;
            const float ds = sS[i * kLdB + j] * (sP[i * kLdB + j] - sDel[i]);
            sS[i * kLdB + j] = ds;
            cs += ds;
        }
        sCp[tid >> 6][tid & 63] = cs;
        __syncthreads();
        if (tid < kB) sCol[tid] += sCp[0][tid] + sCp[1][tid] + sCp[2][tid] + sCp[3][tid];
    };

    // diagonal tile (b = c)
    load_rows(c);
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) {
        const int i = e / kB, j = e % kB;
        sS[i * kLdB + j] = j <= i && c * kB + i < L
            ? __expf(scale * fw.dg[blk_c * kB * kB + e] + (sGc[i] - sGc[j]) - sLse[i]) : 0.f;
    }
    if (c + 1 < nb) prefetch(c + 1);
    backprop();

    float shift = 0.f;              // sum of the gate totals of blocks c .. b-1
    for (int b = c + 1; b < nb; ++b) {
        if (fox) shift += fw.tot[slice * nb + b - 1];
        __syncthreads();
        pfO.store(sdO, LD);
        pfX.store(sX, LD);
        if (c >= 1) pfZ.store(sZ, LD);
        if (tid < kB) {
            sLse[tid] = pLse;
            sDel[tid] = pDel;
            sGb[tid] = pGb;
        }
        __syncthreads();
        if (b + 1 < nb) prefetch(b + 1);
        // P = exp(scale X Kr^T + bias - lse)
        gemm<Pt::F, Pt::F, DP>(kB, kB, cont(sX, LD), cont(sK, LD), [&](int m, int n, float val) {
            sS[m * kLdB + n] = b * kB + m < L
                ? __expf(scale * val + (sGb[m] + shift - sGc[n]) - sLse[m]) : 0.f;
        });
        backprop();
        // dKr += dS^T X (scaled at the end);  dE -= A_{c-1}^T X
        gemm_acc<Pt::F, Pt::F, kB>(kB, DP, strd(sS, kLdB), strd(sX, LD), accK);
        if (c >= 1) gemm_acc<Pt::F, Pt::F, kB>(DP, DP, strd(sZ, LD), strd(sX, LD), accE);
    }
    for_acc(kB, DP, accK, [&](int m, int n, float val) {
        if (n < D) dKr[blk_c * kB * D + m * D + n] = scale * val;
    });
    for_acc(kB, DP, accV, [&](int m, int n, float val) {
        if (n < D && c * kB + m < L) dv[(base + c * kB + m) * D + n] = from_f32<T>(val);
    });
    for_acc(DP, DP, accE, [&](int m, int n, float val) {
        if (m < D && n < D) dEm[blk_c * D * D + m * D + n] = -val;
    });
    __syncthreads();
    if (tid < kB) colsum[blk_c * kB + tid] = sCol[tid];
}

// ---------------------------------------------------------------------------
// precond_bwd: per block, (dQl, dKr, dE, dDg) back through
//   G = strictLower(diag(beta) W W^T), T = (I + G)^{-1}, U = T diag(beta),
//   X = lower(Q W^T), P = X U, Ql = Q - P W, M = strictLower(W K^T), R = U M,
//   Kr = K - R^T W, Y = U^T W, E = W^T Y, Dg = lower(Q K^T) - P M
// [Notes s2.6, s2.7]; intermediate B x B and B x d products live in a per-block
// scratch area of the workspace (kScr tiles of 64 x 64 floats, row stride 64).
constexpr int kScr = 17;
enum { sU_, sX_, sM_, sY_, sP_, sR_, sdP_, sdR_, sdY_, sdM_, sdU_, sdX_, sTmp_, sdG_, sWW_,
       sdT_, sAA_ };

template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
bwd_precond_kernel(int L, int nb, int slice0, const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ w, const float* __restrict__ beta,
                   const float* __restrict__ dQl, const float* __restrict__ dKr,
                   const float* __restrict__ dEm, const float* __restrict__ dDg,
                   float* __restrict__ scr, T* __restrict__ dq, T* __restrict__ dk,
                   T* __restrict__ dw, float* __restrict__ dbeta) {
    using Dm = Dims<D>;
    using Pt = Parts<T, PARTS>;
    // q, k, w tiles in their own (exact) element type: bf16 data halves the
    // LDS, which lets two workgroups share a CU
    using E = typename std::conditional<sizeof(T) == 2, __bf16, float>::type;
    constexpr int DP = Dm::DP, F = Pt::F, XP = Pt::X;
    constexpr int LD = sizeof(T) == 2 ? DP + 8 : Dm::LD;
    __shared__ __attribute__((aligned(16))) E sQ[kB * LD], sK[kB * LD], sW[kB * LD];
    __shared__ __attribute__((aligned(16))) float sT[kB * kLdB], sG[kB * kLdB];
    __shared__ float sBeta[kB], sdB[kB];
    const int tid = threadIdx.x;
    const int c = (int)(blockIdx.x % nb), sl = (int)(blockIdx.x / nb);
    const size_t slice = (size_t)slice0 + sl, blk = slice * nb + c, base = slice * L;
    float* S = scr + (size_t)blockIdx.x * kScr * kB * kB;
    auto g = [&](int t) { return S + (size_t)t * kB * kB; };
    auto gc = [&](int t) { return cont(g(t), kB); };    // (i, k) = tile[i][k]
    auto gs = [&](int t) { return strd(g(t), kB); };    // (i, k) = tile[k][i]
    const float* dql = dQl + blk * kB * D;
    const float* dkr = dKr + blk * kB * D;
    const float* dem = dEm + blk * D * D;
    const float* ddg = dDg + blk * kB * kB;

    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP, pos = c * kB + r;
        const bool in = x < D && pos < L;
        const size_t gi = (base + pos) * D + x;
        sQ[r * LD + x] = (E)(in ? to_f32(q[gi]) : 0.f);
        sK[r * LD + x] = (E)(in ? to_f32(k[gi]) : 0.f);
        sW[r * LD + x] = (E)(in ? to_f32(w[gi]) : 0.f);
    }
    if (tid < kB) {
        const int pos = c * kB + tid;
        sBeta[tid] = pos < L ? beta[base + pos] : 0.f;
        sdB[tid] = 0.f;
    }
    __syncthreads();
    // G and W W^T (inputs are exact in their dtype)
    gemm<XP, XP, DP>(kB, kB, contv(sW, LD), contv(sW, LD), [&](int m, int n, float val) {
        sG[m * kLdB + n] = n < m ? sBeta[m] * val : 0.f;
        g(sWW_)[m * kB + n] = val;
    });
    __syncthreads();
    // T = (I + G)^{-1}: T_jj = 1, T_ij = -sum_{k=j}^{i-1} G_ik T_kj.  A lane of the
    // first wave per column, the column in registers; the sum runs over all
    // k < i for every lane (T_kj = 0 for k < j), so the loops are uniform and
    // unrolled, and every lane reads the same G entries (LDS broadcasts).
    if (tid < kB) {
        const int j = tid;
        float t[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc -= sG[i * kLdB + kk] * t[kk];
            t[i] = i == j ? 1.f : (i < j ? 0.f : acc);
        }
#pragma unroll
        for (int i = 0; i < kB; ++i) sT[i * kLdB + j] = t[i];
    }
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) g(sU_)[e] = sT[(e / kB) * kLdB + e % kB] * sBeta[e % kB];
    // forward products X, M (exact inputs), then Y = U^T W
    gemm<XP, XP, DP>(kB, kB, contv(sQ, LD), contv(sW, LD),
                 [&](int m, int n, float val) { g(sX_)[m * kB + n] = n <= m ? val : 0.f; });
    gemm<XP, XP, DP>(kB, kB, contv(sW, LD), contv(sK, LD),
                 [&](int m, int n, float val) { g(sM_)[m * kB + n] = n < m ? val : 0.f; });
    __syncthreads();
    gemm<F, XP, kB>(kB, DP, gs(sU_), strdv(sW, LD),
                [&](int m, int n, float val) { g(sY_)[m * kB + n] = val; });
    // P = X U, R = U M
    gemm<F, F, kB>(kB, kB, gc(sX_), gs(sU_),
               [&](int m, int n, float val) { g(sP_)[m * kB + n] = val; });
    gemm<F, F, kB>(kB, kB, gc(sU_), gs(sM_),
               [&](int m, int n, float val) { g(sR_)[m * kB + n] = val; });
    __syncthreads();
    // dP = -dDg M^T - dQl W^T;  dR = -W dKr^T;  dY = W dE
    gemm<F, F, kB>(kB, kB, cont(ddg, kB), gc(sM_),
               [&](int m, int n, float val) { g(sdP_)[m * kB + n] = -val; });
    gemm<F, XP, DP>(kB, kB, cont(dql, D, kB, D), contv(sW, LD),
                [&](int m, int n, float val) { g(sdP_)[m * kB + n] -= val; });
    gemm<XP, F, DP>(kB, kB, contv(sW, LD), cont(dkr, D, kB, D),
                [&](int m, int n, float val) { g(sdR_)[m * kB + n] = -val; });
    gemm<XP, F, DP>(kB, DP, contv(sW, LD), strd(dem, D, D, D),
                [&](int m, int n, float val) { g(sdY_)[m * kB + n] = val; });
    __syncthreads();
    // dM = strictLower(-P^T dDg + U^T dR);  dU = lower(X^T dP + dR M^T + W dY^T)
    gemm<F, F, kB>(kB, kB, gs(sP_), strd(ddg, kB),
               [&](int m, int n, float val) { g(sdM_)[m * kB + n] = -val; });
    gemm<F, F, kB>(kB, kB, gs(sU_), gs(sdR_), [&](int m, int n, float val) {
        g(sdM_)[m * kB + n] = n < m ? g(sdM_)[m * kB + n] + val : 0.f;
    });
    gemm<F, F, kB>(kB, kB, gc(sdR_), gc(sM_),
               [&](int m, int n, float val) { g(sdU_)[m * kB + n] = val; });
    gemm<XP, F, DP>(kB, kB, contv(sW, LD), gc(sdY_),
                [&](int m, int n, float val) { g(sdU_)[m * kB + n] += val; });
    // (the last term also takes U = T diag(beta) into dbeta: dbeta_j += sum_a T_aj dU_aj)
    gemm<F, F, kB>(kB, kB, gs(sX_), gs(sdP_), [&](int m, int n, float val) {
        g(sdU_)[m * kB + n] = n <= m ? g(sdU_)[m * kB + n] + val : 0.f;
    });
    // dX = lower(dP U^T)
    gemm<F, F, kB>(kB, kB, gc(sdP_), gc(sU_),
               [&](int m, int n, float val) { g(sdX_)[m * kB + n] = n <= m ? val : 0.f; });
    __syncthreads();
    // dbeta_n = sum_m T_mn dU_mn, one thread per n summing in row order (a
    // fixed order, so the result does not depend on how waves are scheduled)
    if (tid < kB) {
        float acc = 0.f;
#pragma unroll 1
        for (int m = tid; m < kB; ++m) acc += sT[m * kLdB + tid] * g(sdU_)[m * kB + tid];
        sdB[tid] = acc;
    }
    // dT = dU diag(beta)
    for (int e = tid; e < kB * kB; e += 256) g(sdT_)[e] = g(sdU_)[e] * sBeta[e % kB];
    __syncthreads();
    // dG = strictLower(-T^T dT T^T): Tmp = dT T^T, then -T^T Tmp
    gemm<F, F, kB>(kB, kB, gc(sdT_), cont(sT, kLdB),
               [&](int m, int n, float val) { g(sTmp_)[m * kB + n] = val; });
    __syncthreads();
    // (G_ij = beta_i (w_i . w_j), i > j: dbeta_i += sum_j dG_ij (W W^T)_ij)
    gemm<F, F, kB>(kB, kB, strd(sT, kLdB), gs(sTmp_), [&](int m, int n, float val) {
        g(sdG_)[m * kB + n] = n < m ? -val : 0.f;
    });
    __syncthreads();
    // dbeta_m += sum_{n<m} dG_mn (W W^T)_mn, one thread per m in column order
    if (tid < kB) {
        float acc = 0.f;
#pragma unroll 1
        for (int n = 0; n < tid; ++n) acc += g(sdG_)[tid * kB + n] * g(sWW_)[tid * kB + n];
        sdB[tid] += acc;
    }
    // the symmetric weight A + A^T, A = diag(beta) dG, for dW
    for (int e = tid; e < kB * kB; e += 256) {
        const int m = e / kB, n = e % kB;
        g(sAA_)[e] = sBeta[m] * g(sdG_)[m * kB + n] + sBeta[n] * g(sdG_)[n * kB + m];
    }
    // dW = -P^T dQl - R dKr + dX^T Q + dM K + Y dE^T + U dY + (A + A^T) W;
    // dQ = dQl + dDg K + dX W;  dK = dKr + dDg^T Q + dM^T W -- matrix-core
    // accumulators in registers (a wave per output tile)
    __syncthreads();
    f32x16 aW = zero16(), aQ = zero16(), aK = zero16();
    gemm_acc<F, F, kB>(kB, DP, gs(sP_), strd(dql, D, D, kB), aW);
    for (int e = 0; e < 16; ++e) aW[e] = -aW[e];
    {
        f32x16 t = zero16();
        gemm_acc<F, F, kB>(kB, DP, gc(sR_), strd(dkr, D, D, kB), t);
        for (int e = 0; e < 16; ++e) aW[e] -= t[e];
    }
    gemm_acc<F, XP, kB>(kB, DP, gs(sdX_), strdv(sQ, LD), aW);
    gemm_acc<F, XP, kB>(kB, DP, gc(sdM_), strdv(sK, LD), aW);
    gemm_acc<F, F, DP>(kB, DP, gc(sY_), cont(dem, D, D, D), aW);
    gemm_acc<F, F, kB>(kB, DP, gc(sU_), gs(sdY_), aW);
    gemm_acc<F, XP, kB>(kB, DP, gc(sAA_), strdv(sW, LD), aW);
    gemm_acc<F, XP, kB>(kB, DP, cont(ddg, kB), strdv(sK, LD), aQ);
    gemm_acc<F, XP, kB>(kB, DP, gc(sdX_), strdv(sW, LD), aQ);
    gemm_acc<F, XP, kB>(kB, DP, strd(ddg, kB), strdv(sQ, LD), aK);
    gemm_acc<F, XP, kB>(kB, DP, gs(sdM_), strdv(sW, LD), aK);
    for_acc(kB, DP, aW, [&](int m, int n, float val) {
        const int pos = c * kB + m;
        if (n < D && pos < L) dw[(base + pos) * D + n] = from_f32<T>(val);
    });
    for_acc(kB, DP, aQ, [&](int m, int n, float val) {
        const int pos = c * kB + m;
        if (n < D && pos < L) dq[(base + pos) * D + n] = from_f32<T>(val + dql[m * D + n]);
    });
    for_acc(kB, DP, aK, [&](int m, int n, float val) {
        const int pos = c * kB + m;
        if (n < D && pos < L) dk[(base + pos) * D + n] = from_f32<T>(val + dkr[m * D + n]);
    });
    __syncthreads();
    if (tid < kB && c * kB + tid < L) dbeta[base + c * kB + tid] = sdB[tid];
}

// ---------------------------------------------------------------------------
// gate_bwd: per slice, dC_t = rowsum_t - colsum_t and dlogf_s = sum_{t >= s} dC_t
// for s >= 1; dlogf_0 = 0.  A suffix sum over 256 contiguous chunks.
__global__ void __launch_bounds__(256)
bwd_gate_kernel(int L, int nb, const float* __restrict__ rowsum,
                const float* __restrict__ colsum, float* __restrict__ dlogf) {
    __shared__ float part[256];
    const int tid = threadIdx.x;
    const size_t slice = blockIdx.x, base = slice * L, bb = slice * nb * kB;
    const int per = (L + 255) / 256, t0 = tid * per, t1 = min(L, t0 + per);
    float s = 0.f;
    for (int t = t0; t < t1; ++t) s += rowsum[bb + t] - colsum[bb + t];
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {   // exclusive suffix sums of the chunk totals
        float run = 0.f;
        for (int u = 255; u >= 0; --u) {
            const float x = part[u];
            part[u] = run;
            run += x;
        }
    }
    __syncthreads();
    float run = part[tid];
    for (int t = t1 - 1; t >= t0; --t) {
        run += rowsum[bb + t] - colsum[bb + t];
        dlogf[base + t] = t == 0 ? 0.f : run;
    }
}

// ---------------------------------------------------------------------------
// bf16 pair kernels (d in {32, 64}).  Every operand tile is held in LDS as
// bf16 parts -- one for the caller's exact bf16 data (V, dO), hi + lo for fp32
// intermediates -- in the orientation its products read it, so a fragment is
// one or two 16-byte loads and nothing is converted inside a product.

// An R x C fp32 matrix as P bf16 parts, rows padded to C + 8 elements (16-byte
// multiples; consecutive rows start in different bank groups).
template <int R, int C, int P>
struct BTile {
    static constexpr int LDE = C + 8;
    __bf16 v[P][R * LDE];
    __device__ void put(int r, int c, float x) {
        const __bf16 h = (__bf16)x;
        v[0][r * LDE + c] = h;
        if constexpr (P == 2) v[1][r * LDE + c] = (__bf16)(x - (float)h);
    }
    __device__ void put4(int r, int c0, const f32x4& x) {
        bf16x4_t h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = (__bf16)x[e];
            l[e] = (__bf16)(x[e] - (float)h[e]);
        }
        *reinterpret_cast<bf16x4_t*>(&v[0][r * LDE + c0]) = h;
        if constexpr (P == 2) *reinterpret_cast<bf16x4_t*>(&v[1][r * LDE + c0]) = l;
    }
    __device__ float get(int r, int c) const {
        float x = (float)v[0][r * LDE + c];
        if constexpr (P == 2) x += (float)v[1][r * LDE + c];
        return x;
    }
    __device__ f32x4 get4(int r, int c0) const {
        const bf16x4_t h = *reinterpret_cast<const bf16x4_t*>(&v[0][r * LDE + c0]);
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)h[e];
        if constexpr (P == 2) {
            const bf16x4_t l = *reinterpret_cast<const bf16x4_t*>(&v[1][r * LDE + c0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] += (float)l[e];
        }
        return x;
    }
};
// operand view of a tile: (i, k) = row i, column k
struct BV {
    const __bf16* p0;
    const __bf16* p1;
    int ld;
};
template <typename Tile>
__device__ inline BV bview(const Tile& t) {
    return BV{t.v[0], t.v[sizeof(t.v) / sizeof(t.v[0]) - 1], Tile::LDE};
}
template <int P>
__device__ inline void bparts(const BV& a, int i, int k0, bf16x8 (&o)[3]) {
    o[0] = *reinterpret_cast<const bf16x8*>(a.p0 + i * a.ld + k0);
    if constexpr (P == 2) o[1] = *reinterpret_cast<const bf16x8*>(a.p1 + i * a.ld + k0);
}
// One 32 x 32 tile of sum_k A(m0 + ., k) B(n0 + ., k).
template <int PA, int PB, int K>
__device__ inline f32x16 tile_b(const BV& A, const BV& Bv, int m0, int n0, int r, int h) {
    f32x16 c = zero16();
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        bf16x8 ap[3], bp[3];
        bparts<PA>(A, m0 + r, k0 + 8 * h, ap);
        bparts<PB>(Bv, n0 + r, k0 + 8 * h, bp);
        c = mma<PA, PB>(ap, bp, c);
    }
    return c;
}
// All 32 x 32 tiles of an M x N product dealt to the workgroup's waves, the
// epilogue called once per group of four consecutive product rows of a lane:
// out4(n, m, v) receives rows m .. m+3 of column n
template <int PA, int PB, int K, typename FO>
__device__ inline void gemm_b4(int M, int N, const BV& A, const BV& Bv, FO out4) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32, nt = (M / 32) * tn;
    for (int t = wave; t < nt; t += nw) {
        const int m0 = (t / tn) * 32, n0 = (t % tn) * 32;
        const f32x16 c = tile_b<PA, PB, K>(A, Bv, m0, n0, r, h);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out4(n0 + r, m0 + 8 * i + 4 * h, f32x4{c[4 * i], c[4 * i + 1], c[4 * i + 2], c[4 * i + 3]});
    }
}
template <int PA, int PB, int K>
__device__ inline void gemm_b_acc(int M, int N, const BV& A, const BV& Bv, f32x16& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32;
    if (wave >= (M / 32) * tn) return;
    const int m0 = (wave / tn) * 32, n0 = (wave % tn) * 32;
    const f32x16 c = tile_b<PA, PB, K>(A, Bv, m0, n0, r, h);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += c[e];
}

// A fragment read down the columns of a bf16 LDS matrix of row stride ld:
// the 8 consecutive rows k0 .. k0+7 of column i, through gfx950's transposing
// LDS load.  In each group of 16 lanes (16 consecutive columns i, one k0),
// lane j names 4 consecutive elements of row k0 + j/4 starting at column
// c0 + 4 (j mod 4), and lane i receives column c0 + i of those 4 rows; a
// second load covers rows k0+gap .. k0+gap+3 (gap 4: the next four rows; gap 8
// pairs with the column order of the tile images).  Every lane of the wave must
// take part.
typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
__device__ inline bf16x8 frag_col(const __bf16* t, int ld, int i, int k0, int gap = 4) {
    const int j = threadIdx.x & 15;
    const __bf16* p = t + (k0 + (j >> 2)) * ld + (i - j) + 4 * (j & 3);
    typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
    const bf16x4v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
    const bf16x4v b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + gap * ld));
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[e + 4] = b[e];
    }
    return x;
}
// as gemm_b_acc (one part each), CA / CB: the operand is read down the columns
// of its stored matrix (the product contracts the matrix's rows)
template <bool CA, bool CB, int K>
__device__ inline void gemm_bc_acc(int M, int N, const BV& A, const BV& Bv, f32x16& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32;
    if (wave >= (M / 32) * tn) return;
    const int m0 = (wave / tn) * 32, n0 = (wave % tn) * 32;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const bf16x8 a = CA ? frag_col(A.p0, A.ld, m0 + r, k0 + 8 * h)
                            : *reinterpret_cast<const bf16x8*>(A.p0 + (m0 + r) * A.ld + k0 + 8 * h);
        const bf16x8 b = CB ? frag_col(Bv.p0, Bv.ld, n0 + r, k0 + 8 * h)
                            : *reinterpret_cast<const bf16x8*>(Bv.p0 + (n0 + r) * Bv.ld + k0 + 8 * h);
        acc = mfma32(a, b, acc);
    }
}

// Work order of the bf16 pair kernels: workgroup = (slice, rank), rank 0 the
// block with the most partner blocks.  Slices are taken kPairGroup at a time
// and, inside a group, ranks in order with the group's slices interleaved, so
// the workgroups resident at once cover a few slices and the key-block tiles
// (query kernel) and dO tiles (key kernel) they all stream are hit in L2.  The
// grid goes to the XCDs round-robin and kPairGroup is a multiple of 8, so all
// workgroups of a slice share one XCD's L2.  At the LM-layer shape this cuts
// the query kernel's HBM reads from ~29 to ~13 KB per block pair.
constexpr int kPairGroup = 16;

__device__ inline void pair_order(int nb, int nsc, int& rank, int& sl) {
    const int span = kPairGroup * nb, g = (int)blockIdx.x / span, r = (int)blockIdx.x % span;
    const int sz = min(kPairGroup, nsc - g * kPairGroup);
    rank = r / sz;
    sl = g * kPairGroup + r % sz;
}

// key, bf16: for key block c, over the query blocks b >= c.  The logits are
// formed query-major (S = X Kr^T) and written transposed, four queries of a
// key at a time, so P^T and dS^T are key-major operands of dV = P^T dO and
// dKr = dS^T X; X, Z and dO come in as 16-byte pieces of their rows, and the
// products that contract over the queries read them down their columns with
// the transposing LDS load.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
bwd_key_b16_kernel(int L, int nb, int nsc, int slice0, float scale, int fox,
                   const bf16* __restrict__ v, const bf16* __restrict__ dout,
                   const float* __restrict__ lse, const float* __restrict__ delta, FwdWs fw,
                   const float* __restrict__ X, const float* __restrict__ Z,
                   float* __restrict__ dKr, float* __restrict__ dEm, bf16* __restrict__ dv,
                   float* __restrict__ colsum) {
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sK;     // Kr_c [key][d]
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sV;     // V_c [key][d]
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sX;     // X_bc [query][d]
    // dO_b [query][d], then A_{c-1} [query][d] once dP is formed (five tiles,
    // so that three workgroups share a CU)
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sdO;
    BTile<kB, D, 1>& sZ = sdO;
    __shared__ __attribute__((aligned(16))) BTile<kB, kB, 1> sPT;   // P^T, then dS^T [key][query] (bf16)
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB];
    __shared__ float sColW[4][32];   // per (wave, lane) column sums of dS
    // log2-unit logit terms of the off-diagonal steps: per query row
    // (gate, shift, -lse; -inf past the sequence end) and per key (-gate)
    __shared__ __attribute__((aligned(16))) float sRow2[kB];
    __shared__ float sCol2[kB];
    float shift = 0.f;              // sum of the gate totals of blocks c .. b-1
    const int tid = threadIdx.x;
    int c, sl;
    pair_order(nb, nsc, c, sl);
    const size_t slice = (size_t)slice0 + sl, blk_c = slice * nb + c, base = slice * L;
    const size_t npairs = (size_t)nb * (nb - 1) / 2;
    // the carried queries and the gradient chain, bf16 [pair][kB][D]
    const __bf16* Xs = reinterpret_cast<const __bf16*>(X) + (size_t)sl * npairs * kB * D;
    const __bf16* Zs = reinterpret_cast<const __bf16*>(Z) + (size_t)sl * npairs * kB * D;

    {   // resident: scale * Kr_c (bf16 rows from the preconditioning), V_c
        // (every load in flight before the first LDS write)
        const __bf16* krc = static_cast<const __bf16*>(fw.kr) + blk_c * kB * D;
        // (rows past the sequence end read its last row, zeroed at the write)
        constexpr int NV8 = kB * D / 8 / 256;
        static_assert(NV8 * 256 == kB * D / 8, "whole V pieces per thread");
        u32x4 kq[NV8];
        u32x4 vq[NV8];
#pragma unroll
        for (int it = 0; it < NV8; ++it) {
            const int e = tid + 256 * it, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            kq[it] = *reinterpret_cast<const u32x4*>(krc + (size_t)r * D + c0);
        }
#pragma unroll
        for (int it = 0; it < NV8; ++it) {
            const int e = tid + 256 * it, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int pos = min(c * kB + r, L - 1);
            vq[it] = *reinterpret_cast<const u32x4*>(v + (base + pos) * D + c0);
        }
        const float gc = fw.gl[blk_c * kB + (tid % kB)];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < NV8; ++it) {
            const int e = tid + 256 * it, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            *reinterpret_cast<u32x4*>(&sK.v[0][r * sK.LDE + c0]) = kq[it];
        }
#pragma unroll
        for (int it = 0; it < NV8; ++it) {
            const int e = tid + 256 * it, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            *reinterpret_cast<u32x4*>(&sV.v[0][r * sV.LDE + c0]) =
                c * kB + r < L ? vq[it] : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < kB) {
            sGc[tid] = fox ? gc : 0.f;
            sCol2[tid] = -(fox ? gc : 0.f) * kLog2e;
        }
    }
    // prefetch of query block b's X_bc, Z_bc, dO (16-byte pieces of their
    // rows) and row terms
    constexpr int UB = kB * D / 8 / 256;
    u32x4 pX[UB], pZ[UB], pO[UB];
    float pLse = 0.f, pDel = 0.f, pGb = 0.f, pTot = 0.f;   // pTot: the gate total of block b - 1
    auto prefetch = [&](int b) {
        const size_t blk_b = slice * nb + b;
        pTot = fox && b >= 1 ? fw.tot[blk_b - 1] : 0.f;
        if (b > c) {
            const __bf16* xb = Xs + pair_index(b, c) * kB * D;
#pragma unroll
            for (int i = 0; i < UB; ++i) {
                const int e = tid + 256 * i;
                pX[i] = *reinterpret_cast<const u32x4*>(xb + (size_t)8 * e);
            }
        }
        // rows past the sequence end are loaded from its last row and masked
        // at the commit: a register written before a load it may overlap
        // would make the compiler wait for every load in flight
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int pos = min(b * kB + r, L - 1);
            pO[i] = *reinterpret_cast<const u32x4*>(dout + (base + pos) * D + c0);
        }
        if (tid < kB) {
            pLse = lse[base + min(b * kB + tid, L - 1)];
            pDel = delta[blk_b * kB + tid];
            pGb = fw.gl[blk_b * kB + tid];
        }
    };
    auto commit = [&](int b) {
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            if (b > c) *reinterpret_cast<u32x4*>(&sX.v[0][r * sX.LDE + c0]) = pX[i];
            *reinterpret_cast<u32x4*>(&sdO.v[0][r * sdO.LDE + c0]) =
                b * kB + r < L ? pO[i] : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < kB) {
            const bool in = b * kB + tid < L;
            const float gb = fox ? pGb : 0.f;
            sLse[tid] = in ? pLse : 0.f;
            sDel[tid] = pDel;
            sGb[tid] = gb;
            sRow2[tid] = in ? (gb + shift - pLse) * kLog2e : -INFINITY;
        }
    };
    // A_{c-1} of pair (b, c) is fetched a pair ahead, once the previous pair
    // has written its copy, and written over dO's tile after dP is formed
    auto load_z = [&](int b) {
        const __bf16* zb = Zs + pair_index(b, c) * kB * D;
#pragma unroll
        for (int i = 0; i < UB; ++i) pZ[i] = *reinterpret_cast<const u32x4*>(zb + (size_t)8 * (tid + 256 * i));
    };
    auto commit_z = [&] {
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            *reinterpret_cast<u32x4*>(&sZ.v[0][r * sZ.LDE + c0]) = pZ[i];
        }
    };
    f32x16 accV = zero16(), accK = zero16(), accE = zero16();
    float colAcc = 0.f;   // the lane's key column (fixed by the tiling): dS summed over queries
    // dV += P^T dO;  then dS = P (dO V^T - Delta), written back transposed
    auto backprop = [&]() {
        __syncthreads();   // P^T complete
        gemm_bc_acc<false, true, kB>(kB, D, bview(sPT), bview(sdO), accV);
        __syncthreads();   // every read of P^T done
        gemm_b4<1, 1, D>(kB, kB, bview(sdO), bview(sV), [&](int n, int m, f32x4 dp) {
            // queries m .. m+3, key n
            const f32x4 p = sPT.get4(n, m);
            f32x4 ds;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ds[e] = p[e] * (dp[e] - sDel[m + e]);
                colAcc += ds[e];
            }
            sPT.put4(n, m, ds);
        });
        __syncthreads();   // dS^T complete
    };

    // diagonal tile (b = c): P^T[j][i] = exp(scale Dg[i][j] + bias - lse_i), j <= i
    prefetch(c);
    commit(c);
    __syncthreads();
    {
        constexpr int NIT = kB * kB / 4 / 256;
        float dgv[NIT][4];   // every load in flight before the first use
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + 256 * it, j = e / (kB / 4), i0 = 4 * (e % (kB / 4));
#pragma unroll
            for (int q = 0; q < 4; ++q) dgv[it][q] = fw.dg[blk_c * kB * kB + (i0 + q) * kB + j];
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + 256 * it, j = e / (kB / 4), i0 = 4 * (e % (kB / 4));   // key j, queries i0 .. i0+3
            f32x4 p;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = i0 + q;
                // formed for every entry, then selected: a branch around it
                // would pull the entry's load in and wait on it there
                const float x = __expf(scale * dgv[it][q] + (sGc[i] - sGc[j]) - sLse[i]);
                p[q] = j <= i && c * kB + i < L ? x : 0.f;
            }
            sPT.put4(j, i0, p);
        }
    }
    if (c + 1 < nb) prefetch(c + 1);
    if (c >= 1 && c + 1 < nb) load_z(c + 1);
    backprop();

    for (int b = c + 1; b < nb; ++b) {
        shift += pTot;   // block b - 1's total, fetched by prefetch(b)
        commit(b);
        __syncthreads();
        if (b + 1 < nb) prefetch(b + 1);
        // P = exp(X (scale Kr)^T + bias - lse), queries m .. m+3 of key n, into P^T
        gemm_b4<1, 1, D>(kB, kB, bview(sX), bview(sK), [&](int n, int m, f32x4 sv) {
            const f32x4 rw = *reinterpret_cast<const f32x4*>(sRow2 + m);
            const float cl = sCol2[n];
            f32x4 p;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(kLog2e, sv[e], rw[e] + cl));
            sPT.put4(n, m, p);
        });
        backprop();
        if (c >= 1) {       // dO's tile is free (dS^T complete): A_{c-1} over it
            commit_z();
            __syncthreads();
            if (b + 1 < nb) load_z(b + 1);
        }
        // dKr += dS^T X (scaled at the end);  dE -= A_{c-1}^T X
        gemm_bc_acc<false, true, kB>(kB, D, bview(sPT), bview(sX), accK);
        if (c >= 1) gemm_bc_acc<true, true, kB>(D, D, bview(sZ), bview(sX), accE);
        __syncthreads();   // the pair's tiles may be replaced
    }
    for_acc(kB, D, accK, [&](int m, int n, float val) {
        dKr[blk_c * kB * D + m * D + n] = scale * val;
    });
    for_acc(kB, D, accV, [&](int m, int n, float val) {
        if (c * kB + m < L) dv[(base + c * kB + m) * D + n] = from_f32<bf16>(val);
    });
    for_acc(D, D, accE, [&](int m, int n, float val) { dEm[blk_c * D * D + m * D + n] = -val; });
    {   // the lane's key column of the (query x key) dS tiles: the column's
        // two lane halves, then its two waves, are added pairwise (a + b =
        // b + a), so the sum does not depend on the order the waves run in
        const int lane = tid & 63, wave = tid >> 6;
        const float both = colAcc + __shfl_xor(colAcc, 32, 64);
        if (lane < 32) sColW[wave][lane] = both;
    }
    __syncthreads();
    if (tid < kB) colsum[blk_c * kB + tid] = sColW[tid / 32][tid % 32] + sColW[tid / 32 + 2][tid % 32];
}

// query, bf16: for query block b, left to right over the key blocks c < b.
// The logits are formed key-major (S^T = Kr X^T) and written back query-major,
// four keys of a query at a time; the chain is carried transposed
// (A^T = scale Kr^T dS^T + A^T - E^T A^T), a lane owning one query's four
// consecutive d values per register group, so the operand copy of A in LDS
// and the stores of A go out as vectors.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
bwd_query_b16_kernel(int L, int nb, int nsc, int slice0, float scale, int fox,
                     const bf16* __restrict__ v, const bf16* __restrict__ o,
                     const bf16* __restrict__ dout, const float* __restrict__ lse, FwdWs fw,
                     const float* __restrict__ X, float* __restrict__ Z,
                     float* __restrict__ dQl, float* __restrict__ dDg,
                     float* __restrict__ rowsum, float* __restrict__ delta) {
    // Five tiles, so that three workgroups share a CU: X's tile takes P (then
    // dS) once the logits are formed, and V's takes -E once dP is formed.
    using TX = BTile<kB, D, 1>;
    using TS = BTile<kB, kB, 1>;
    using TE = BTile<D, D, 1>;
    constexpr int XS_BYTES = sizeof(TX) > sizeof(TS) ? sizeof(TX) : sizeof(TS);
    constexpr int VE_BYTES = sizeof(TX) > sizeof(TE) ? sizeof(TX) : sizeof(TE);
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sdO;    // dO_b [query][d]
    __shared__ __attribute__((aligned(16))) char sVE[VE_BYTES];     // V_c [key][d], then -E_c [d][d]
    __shared__ __attribute__((aligned(16))) char sXS[XS_BYTES];     // X_bc [query][d], then P, dS [query][key]
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sK;     // scale Kr_c [key][d]
    __shared__ __attribute__((aligned(16))) BTile<kB, D, 1> sA;     // A_{c-1} [query][d]
    TX& sV = *reinterpret_cast<TX*>(sVE);
    TE& sE = *reinterpret_cast<TE*>(sVE);
    TX& sX = *reinterpret_cast<TX*>(sXS);
    TS& sS = *reinterpret_cast<TS*>(sXS);
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB];
    __shared__ float sRowW[4][32];   // per (wave, lane) row sums of dS
    // log2-unit logit terms of the off-diagonal steps: per query row (gate,
    // -lse; -inf past the sequence end) and per key of the current block (-gate)
    __shared__ float sRowB[kB];
    __shared__ __attribute__((aligned(16))) float sCol2[kB];
    __shared__ float sTw[4];   // per-wave parts of the gate totals before block b
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int b, sl;
    pair_order(nb, nsc, b, sl);
    b = nb - 1 - b;
    const size_t slice = (size_t)slice0 + sl, blk_b = slice * nb + b, base = slice * L;
    const size_t npairs = (size_t)nb * (nb - 1) / 2;
    // the carried queries and the gradient chain, bf16 [pair][kB][D]
    const __bf16* Xs = reinterpret_cast<const __bf16*>(X) + (size_t)sl * npairs * kB * D;
    __bf16* Zs = reinterpret_cast<__bf16*>(Z) + (size_t)sl * npairs * kB * D;
    // scale * Kr and -E as bf16 rows (from the preconditioning)
    const __bf16* kr = static_cast<const __bf16*>(fw.kr);
    const __bf16* em = static_cast<const __bf16*>(fw.em);
    constexpr int UB = kB * D / 8 / 256;
    // 16-byte pieces of the D x D transition: D * D / 8 of them, at most one per thread
    constexpr int NEU = D * D / 8;
    static_assert(NEU <= 256 || NEU == 512, "E pieces per thread");
    constexpr int UE = NEU > 256 ? 2 : 1;

    // resident: dO_b; Delta = dO . o per row: each thread the dot of its
    // 8-element piece of a row (loaded with the row), then the D / 8 threads
    // of the row combined by an xor butterfly, in a fixed order. The setup's
    // loads are all issued first, rows past the sequence end reading its last
    // row (masked below), so that they overlap.
    u32x4 ud[UB], uo[UB];
#pragma unroll
    for (int i = 0; i < UB; ++i) {
        const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
        const size_t gi = (base + min(b * kB + r, L - 1)) * D + c0;
        ud[i] = *reinterpret_cast<const u32x4*>(dout + gi);
        uo[i] = *reinterpret_cast<const u32x4*>(o + gi);
    }
    const float rLse = lse[base + min(b * kB + (tid % kB), L - 1)];
    const float rGb = fw.gl[blk_b * kB + (tid % kB)];
    // the gate totals of blocks 0 .. b-1 (the first 256 read here, any more
    // in the loop below)
    const float tot0 = fw.tot[slice * nb + min(tid, nb - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < UB; ++i) {
        const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
        const bool in = b * kB + r < L;
        const u32x4 u = in ? ud[i] : u32x4{0u, 0u, 0u, 0u}, w = in ? uo[i] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&sdO.v[0][r * sdO.LDE + c0]) = u;
        float dl = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            dl += __uint_as_float(u[q] << 16) * __uint_as_float(w[q] << 16);
            dl += __uint_as_float(u[q] & 0xffff0000u) * __uint_as_float(w[q] & 0xffff0000u);
        }
#pragma unroll
        for (int off = 1; off < D / 8; off <<= 1) dl += __shfl_xor(dl, off, 64);
        if (e % (D / 8) == 0) {
            sDel[r] = dl;
            delta[blk_b * kB + r] = dl;
        }
    }
    if (tid < kB) {
        const bool in = b * kB + tid < L;
        const float gb = fox ? rGb : 0.f, ls = in ? rLse : 0.f;
        sLse[tid] = ls;
        sGb[tid] = gb;
        sRowB[tid] = in ? (gb - ls) * kLog2e : -INFINITY;
    }
    // the gate totals of blocks 0 .. b-1, summed by all threads (fixed order)
    if (fox) {
        float part = tid < b ? tot0 : 0.f;
        for (int cc = tid + 256; cc < b; cc += 256) part += fw.tot[slice * nb + cc];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off, 64);
        if (lane == 0) sTw[wave] = part;
    }
    // prefetch of key block c's V, scale * Kr, X_bc, -E (16-byte pieces)
    u32x4 pV[UB], pX[UB], pK[UB], pE[UE];
    float pGc = 0.f, pTot = 0.f;   // pTot: the gate total of block c - 1
    auto prefetch = [&](int c) {
        const size_t blk_c = slice * nb + c;
        pTot = fox && c >= 1 ? fw.tot[blk_c - 1] : 0.f;
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            // rows past the sequence end: the last row, masked at the commit (a
            // register written before a load it may overlap would make the
            // compiler wait for every load in flight)
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            const int pos = min(c * kB + r, L - 1);
            pV[i] = *reinterpret_cast<const u32x4*>(v + (base + pos) * D + c0);
        }
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i;
            pK[i] = *reinterpret_cast<const u32x4*>(kr + blk_c * kB * D + (size_t)8 * e);
        }
        if (c < b)
#pragma unroll
            for (int i = 0; i < UB; ++i) {
                const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
                pX[i] = *reinterpret_cast<const u32x4*>(Xs + pair_index(b, c) * kB * D +
                                                         (size_t)r * D + c0);
            }
        if (tid < kB) pGc = fw.gl[blk_c * kB + tid];
    };
    // -E_c is fetched a pair ahead, once the previous pair has written its
    // copy, and written over V's tile after dP is formed
    auto load_e = [&](int c) {
        const size_t blk_c = slice * nb + c;
#pragma unroll
        for (int i = 0; i < UE; ++i) {
            const int e = tid + 256 * i;
            if (e < NEU) pE[i] = *reinterpret_cast<const u32x4*>(em + blk_c * D * D + (size_t)8 * e);
        }
    };
    auto commit_e = [&] {
#pragma unroll
        for (int i = 0; i < UE; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            if (e < NEU) *reinterpret_cast<u32x4*>(&sE.v[0][r * sE.LDE + c0]) = pE[i];
        }
    };
    auto commit = [&](int c) {
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            *reinterpret_cast<u32x4*>(&sV.v[0][r * sV.LDE + c0]) =
                c * kB + r < L ? pV[i] : u32x4{0u, 0u, 0u, 0u};
        }
        // Kr enters both of its products scaled (S^T = scale Kr X^T in the
        // exponent, scale Kr^T dS^T in the chain), and E negated, so the chain
        // accumulates straight into A^T
#pragma unroll
        for (int i = 0; i < UB; ++i) {
            const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
            *reinterpret_cast<u32x4*>(&sK.v[0][r * sK.LDE + c0]) = pK[i];
        }
        if (c < b)
#pragma unroll
            for (int i = 0; i < UB; ++i) {
                const int e = tid + 256 * i, r = e / (D / 8), c0 = 8 * (e % (D / 8));
                *reinterpret_cast<u32x4*>(&sX.v[0][r * sX.LDE + c0]) = pX[i];
            }
        if (tid < kB) {
            const float gc = fox ? pGc : 0.f;
            sGc[tid] = gc;
            sCol2[tid] = -gc * kLog2e;
        }
    };
    float rowAcc = 0.f;   // the lane's query column (fixed by the tiling): dS summed over keys
    // dS = P (dO V^T - Delta), formed key-major (dP^T = V dO^T) and written back
    auto backprop = [&](bool diag) {
        gemm_b4<1, 1, D>(kB, kB, bview(sV), bview(sdO), [&](int n, int m, f32x4 dp) {
            // keys m .. m+3, query n
            const f32x4 p = sS.get4(n, m);
            f32x4 ds;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ds[e] = p[e] * (dp[e] - sDel[n]);
                rowAcc += ds[e];
            }
            sS.put4(n, m, ds);
            if (diag)
                *reinterpret_cast<f32x4*>(dDg + blk_b * kB * kB + n * kB + m) =
                    f32x4{scale * ds[0], scale * ds[1], scale * ds[2], scale * ds[3]};
        });
        __syncthreads();   // dS complete
    };

    // diagonal tile: P from the in-block logits
    prefetch(b);   // V_b only is used here
    commit(b);
    __syncthreads();
    {
        constexpr int NIT = kB * kB / 4 / 256;
        f32x4 dg4[NIT];   // every load in flight before the first use
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + 256 * it, i = e / (kB / 4), j0 = 4 * (e % (kB / 4));
            dg4[it] = *reinterpret_cast<const f32x4*>(fw.dg + blk_b * kB * kB + i * kB + j0);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int e = tid + 256 * it, i = e / (kB / 4), j0 = 4 * (e % (kB / 4));   // query i, keys j0 .. j0+3
            f32x4 p;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                p[q] = j <= i && b * kB + i < L
                    ? __expf(scale * dg4[it][q] + (sGb[i] - sGb[j]) - sLse[i])
                    : 0.f;
            }
            sS.put4(i, j0, p);
        }
    }
    if (b > 0) prefetch(0);
    __syncthreads();
    backprop(true);

    // the chain, transposed: a wave owns a (32 d) x (32 queries) tile of A^T
    f32x16 At = zero16();
    float Tc = 0.f;                 // sum of the gate totals of blocks before c
    const int tq = kB / 32, mA = (wave / tq) * 32, nA = (wave % tq) * 32, h = lane >> 5;
    const bool owner = wave < (D / 32) * tq;
    const int qcol = nA + (lane & 31);   // the lane's query
    for (int c = 0; c < b; ++c) {
        commit(c);
        __syncthreads();
        if (c + 1 < b) prefetch(c + 1);
        if (c >= 1) {   // Z = A_{c-1}, bf16 rows [q][d], from its LDS copy: whole rows per wave
            constexpr int CPR = D / 8, RPP = 256 / CPR;
            __bf16* zo = Zs + pair_index(b, c) * kB * D;
#pragma unroll
            for (int u = 0; u < kB / RPP; ++u) {
                const int q = u * RPP + tid / CPR, d0 = 8 * (tid % CPR);
                *reinterpret_cast<bf16x8*>(zo + (size_t)q * D + d0) =
                    *reinterpret_cast<const bf16x8*>(&sA.v[0][q * sA.LDE + d0]);
            }
        }
        const float shift = fox ? ((sTw[0] + sTw[1]) + (sTw[2] + sTw[3])) - Tc : 0.f;   // totals of blocks c .. b-1
        // S^T = (scale Kr) X^T, a 32 x 32 tile per wave: keys m .. m+3 of query
        // n, written to the query-major P over X's tile once every wave has
        // read X
        const float shift2 = shift * kLog2e;
        {
            const int r = lane & 31, hh = lane >> 5, m0 = (wave >> 1) * 32, n0 = (wave & 1) * 32;
            const f32x16 sv = tile_b<1, 1, D>(bview(sK), bview(sX), m0, n0, r, hh);
            __syncthreads();   // X's tile is free
            const int n = n0 + r;
            const float rw = sRowB[n] + shift2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + 8 * i + 4 * hh;
                const f32x4 cl = *reinterpret_cast<const f32x4*>(sCol2 + m);
                f32x4 p;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(kLog2e, sv[4 * i + e], rw + cl[e]));
                sS.put4(n, m, p);
            }
        }
        backprop(false);
        if (c >= 1) {       // V's tile is free (dS complete): -E_c over it
            commit_e();
            __syncthreads();
        }
        // A^T <- A^T + (scale Kr)^T dS^T + (-E)^T A^T, accumulated in place
        gemm_bc_acc<true, false, kB>(D, kB, bview(sK), bview(sS), At);
        if (c >= 1) gemm_bc_acc<true, false, D>(D, kB, bview(sE), bview(sA), At);
        if (c + 1 < b && c + 1 >= 1) load_e(c + 1);
        __syncthreads();   // every read of A_{c-1} and of the pair's tiles is done
        if (owner)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sA.put4(qcol, mA + 8 * i + 4 * h,
                        f32x4{At[4 * i], At[4 * i + 1], At[4 * i + 2], At[4 * i + 3]});
        Tc += pTot;   // block c's total, fetched by prefetch(c + 1) (unused after the last c)
    }
    if (owner) {
        float* qo = dQl + blk_b * kB * D + (size_t)qcol * D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(qo + mA + 8 * i + 4 * h) =
                f32x4{At[4 * i], At[4 * i + 1], At[4 * i + 2], At[4 * i + 3]};
    }
    {   // the lane's query column: lane halves, then the two waves of the
        // column, added pairwise (order-independent, as for the key pass)
        const float both = rowAcc + __shfl_xor(rowAcc, 32, 64);
        if (lane < 32) sRowW[wave][lane] = both;
    }
    __syncthreads();
    if (tid < kB) rowsum[blk_b * kB + tid] = sRowW[tid / 32][tid % 32] + sRowW[tid / 32 + 2][tid % 32];
}

// ---------------------------------------------------------------------------
// chain for bf16 inputs at d in {32, 64}: the carried queries stay in
// registers, a 32 x 32 tile of Qw per wave in the matrix-core C layout (lane:
// column d, registers: rows q), as the forward's scan keeps them.  Each step
// writes the tile to LDS once as bf16 Qw^T; from there the pair's X_bc rows
// go to memory as 16-byte chunks (read down Qw^T's columns by the transposing
// load) and the transition Qw <- Qw - Qw E_c^T takes its Qw operand the same
// way, accumulating into the registers.  -E_c comes from the block's tile
// image (bf16, the values the forward's scan uses), read straight from memory
// as the other operand; its columns sit in the image's swap23 order, so the Qw
// fragment pairs rows k0+4h .. +3 with rows k0+8+4h .. +3 to match.
template <int D>
__global__ void __launch_bounds__(256)
bwd_chain_b16_kernel(int nb, int nsc, int slice0, const float* __restrict__ ql,
                     const char* __restrict__ img, float* __restrict__ X) {
    using I = Img<D>;
    constexpr int TN = D / 32, NT = (kB / 32) * TN;        // Qw tiles
    constexpr int LQ = kB + 8;                              // LDS row stride (bf16)
    constexpr int LR = D + 8;
    __shared__ __attribute__((aligned(16))) __bf16 sQt[D * LQ];   // Qw^T [d][q]
    // Qw [q][d] as well, for the stores: a lane then takes 16 bytes along a
    // row and the lanes of a wave write whole rows, contiguous in memory
    __shared__ __attribute__((aligned(16))) __bf16 sQr[kB * LR];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 31, h = lane >> 5;
    const int b = nb - 1 - (int)(blockIdx.x / nsc), sl = (int)(blockIdx.x % nsc);
    const size_t slice = (size_t)slice0 + sl, npairs = (size_t)nb * (nb - 1) / 2;
    __bf16* Xs = reinterpret_cast<__bf16*>(X) + (size_t)sl * npairs * kB * D;
    const bool owner = wave < NT;
    const int m0 = (wave / TN) * 32, n0 = (wave % TN) * 32;   // q rows, d columns of the tile
    f32x16 qw = zero16();
    if (owner) {
        const float* qlb = ql + (slice * nb + b) * kB * D;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) qw[4 * i + j] = qlb[(m0 + 8 * i + 4 * h + j) * D + n0 + r];
    }
    // the lane's -E_c operand: row d = n0 + r of the image's -E, one 16-byte
    // unit per 16 columns (the lane half's 8 columns)
    bf16x8 ef[D / 16];
    auto loadE = [&](int c) {
        const char* ie = img + (slice * nb + c) * I::BYTES + I::OFF_E + (n0 + r) * I::RB_E;
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc)
            ef[kc] = *reinterpret_cast<const bf16x8*>(ie + swz_unit(n0 + r, 2 * kc + h, I::RB_E) * 16);
    };
    if (owner && b - 1 >= 1) loadE(b - 1);
    // the X_bc chunk a lane stores: 16 consecutive q per group of 16 lanes, 8 d
    constexpr int XP = (kB * D / 8) / 256;                    // fragment passes per wave
    for (int c = b - 1; c >= 0; --c) {
        if (owner)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x4_t x4{(__bf16)qw[4 * i], (__bf16)qw[4 * i + 1], (__bf16)qw[4 * i + 2],
                                  (__bf16)qw[4 * i + 3]};
                *reinterpret_cast<bf16x4_t*>(sQt + (n0 + r) * LQ + m0 + 8 * i + 4 * h) = x4;
#pragma unroll
                for (int j = 0; j < 4; ++j) sQr[(m0 + 8 * i + 4 * h + j) * LR + n0 + r] = x4[j];
            }
        __syncthreads();   // Qw^T and Qw in LDS
        {   // X_bc = Qw as bf16 rows [q][d]: D / 8 lanes per row
            constexpr int CPR = D / 8, RPW = 64 / CPR;
            __bf16* xo = Xs + pair_index(b, c) * kB * D;
#pragma unroll
            for (int u = 0; u < XP; ++u) {
                const int q = (u * 4 + wave) * RPW + lane / CPR, d0 = 8 * (lane % CPR);
                *reinterpret_cast<bf16x8*>(xo + (size_t)q * D + d0) =
                    *reinterpret_cast<const bf16x8*>(sQr + q * LR + d0);
            }
        }
        if (c > 0 && owner) {
            // Qw(q, d) += sum_k Qw(q, k) (-E_c(d, k))
#pragma unroll
            for (int kc = 0; kc < D / 16; ++kc) {
                const bf16x8 a = frag_col(sQt, LQ, m0 + r, 16 * kc + 4 * h, 8);
                qw = mfma32(a, ef[kc], qw);
            }
            if (c - 1 >= 1) loadE(c - 1);
        }
        __syncthreads();   // every read of this step's LDS done
    }
}

// ---------------------------------------------------------------------------
// precond_bwd for bf16 inputs at d in {32, 64}: the same products as
// bwd_precond_kernel, every operand and intermediate held in LDS as one bf16
// part (the precision the pair kernels work in), so no product waits on a
// round trip to global memory.  One 512-thread workgroup per block; its two
// four-wave halves run independent products side by side.  Seventeen tile
// slots of 64 x 72 bf16 hold the live matrices; a slot is reused once its
// matrix is dead, and the fp32 G of the UT solve and the fp32 dG for the
// symmetric weight each take two adjacent free slots.
constexpr int kLT = 72;                        // row stride of a slot (bf16)
constexpr int kSlot = kB * kLT;                // elements per slot
constexpr int kSlots = 17;

// fragment of a slot-resident bf16 matrix: 8 consecutive contraction indices
// of operand row i, read along a row (C) or down a column (S)
__device__ inline bf16x8 fragC(const __bf16* t, int i, int k0) {
    return *reinterpret_cast<const bf16x8*>(t + i * kLT + k0);
}
__device__ inline bf16x8 fragS(const __bf16* t, int i, int k0) { return frag_col(t, kLT, i, k0); }
// One 32 x 32 tile of sum_k A(m0 + ., k) B(n0 + ., k); SA / SB: the operand is
// read down the stored matrix's columns (the product contracts its rows).
template <bool SA, bool SB, int K>
__device__ inline f32x16 tprod(const __bf16* A, const __bf16* B, int m0, int n0, f32x16 c) {
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const bf16x8 a = SA ? fragS(A, m0 + r, k0 + 8 * h) : fragC(A, m0 + r, k0 + 8 * h);
        const bf16x8 b = SB ? fragS(B, n0 + r, k0 + 8 * h) : fragC(B, n0 + r, k0 + 8 * h);
        c = mfma32(a, b, c);
    }
    return c;
}
// The output tiles of an M x N product dealt to the four waves of half g
// (waves 4g .. 4g+3); the wave's own tile index, or -1
__device__ inline int half_tile(int g, int M, int N, int k) {
    const int wave = threadIdx.x >> 6;
    if ((wave >> 2) != g) return -1;
    const int t = (wave & 3) + 4 * k;
    return t < (M / 32) * (N / 32) ? t : -1;
}
// element visitor of a tile in the matrix-core C layout
template <typename F>
__device__ inline void for_tile(int t, int N, const f32x16& c, F f) {
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int m0 = (t / (N / 32)) * 32, n0 = (t % (N / 32)) * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) f(m0 + 8 * i + 4 * h + j, n0 + r, c[4 * i + j]);
}
// C = A B (as tprod) over all output tiles, on half g, written through f
template <bool SA, bool SB, int K, typename F>
__device__ inline void hprod(int g, int M, int N, const __bf16* A, const __bf16* B, F f) {
    for (int k = 0;; ++k) {
        const int t = half_tile(g, M, N, k);
        if (t < 0) return;
        const int m0 = (t / (N / 32)) * 32, n0 = (t % (N / 32)) * 32;
        for_tile(t, N, tprod<SA, SB, K>(A, B, m0, n0, zero16()), f);
    }
}
__device__ inline void put_bf(__bf16* t, int m, int n, float v) { t[m * kLT + n] = (__bf16)v; }

template <int D>
__global__ void __launch_bounds__(512)
bwd_precond_b16_kernel(int L, int nb, int slice0, const bf16* __restrict__ q,
                       const bf16* __restrict__ k, const bf16* __restrict__ w,
                       const float* __restrict__ beta, const float* __restrict__ dQl,
                       const float* __restrict__ dKr, const float* __restrict__ dEm,
                       const float* __restrict__ dDg, bf16* __restrict__ dq,
                       bf16* __restrict__ dk, bf16* __restrict__ dw,
                       float* __restrict__ dbeta) {
    static_assert(D == 32 || D == 64, "bf16 tiles");
    __shared__ __attribute__((aligned(16))) __bf16 sl[kSlots * kSlot];
    __shared__ float sBeta[kB];
    // dbeta partials: per (tile row, column) of the dU term and per (tile
    // column, row) of the dG term, summed in a fixed order at the end
    __shared__ float sDbU[2][kB], sDbG[2][kB];
    const int tid = threadIdx.x;
    const int c = (int)(blockIdx.x % nb), sli = (int)(blockIdx.x / nb);
    const size_t slice = (size_t)slice0 + sli, blk = slice * nb + c, base = slice * L;
    auto S = [&](int i) { return sl + i * kSlot; };
    // slot map (a slot is reused once its matrix is dead)
    __bf16 *sW = S(0), *sQ = S(1), *sK = S(2), *sDg = S(3), *sDq = S(4), *sDk = S(5),
           *sDe = S(6), *sX = S(7), *sM = S(8), *sDr = S(9), *sT = S(10), *sU = S(11),
           *sDy = S(12), *sDp = S(13), *sDm = S(14), *sP = S(15), *sR = S(16);
    __bf16 *sY = S(15), *sDx = S(16), *sDt = S(4), *sTmp = S(5), *sAA = S(6);
    float* fG = reinterpret_cast<float*>(S(15));   // slots 15-16, phases 1-3
    float* fdG = reinterpret_cast<float*>(S(7));   // slots 7-8, phases 9-10
    static_assert(kB * kLdB * 4 <= 2 * kSlot * 2, "fp32 matrix in two slots");
    const float* dql = dQl + blk * kB * D;
    const float* dkr = dKr + blk * kB * D;
    const float* dem = dEm + blk * D * D;
    const float* ddg = dDg + blk * kB * kB;

    // ---- 0. inputs: q, k, w (exact), the incoming gradients rounded to bf16.
    //         Every global load is issued before the first LDS write, rows past
    //         the sequence end read its last row (masked at the write), so the
    //         loads overlap instead of waiting one by one.
    constexpr int nI = kB * D / 8, nA = kB * D / 4, nE = D * D / 4, nG = kB * kB / 4;
    constexpr int RI = (nI + 511) / 512, RA = (nA + 511) / 512, RE = (nE + 511) / 512,
                  RG = (nG + 511) / 512;
    u32x4 uq[RI], uk[RI], uw[RI];
    f32x4 fq[RA], fk[RA], fe[RE], fg[RG];
#pragma unroll
    for (int i = 0; i < RI; ++i) {
        const int e = (tid + 512 * i) % nI, r = e / (D / 8), x0 = 8 * (e % (D / 8));
        const size_t gi = (base + min(c * kB + r, L - 1)) * D + x0;
        uq[i] = *reinterpret_cast<const u32x4*>(q + gi);
        uk[i] = *reinterpret_cast<const u32x4*>(k + gi);
        uw[i] = *reinterpret_cast<const u32x4*>(w + gi);
    }
#pragma unroll
    for (int i = 0; i < RA; ++i) {
        const int e = (tid + 512 * i) % nA;
        fq[i] = *reinterpret_cast<const f32x4*>(dql + 4 * e);
        fk[i] = *reinterpret_cast<const f32x4*>(dkr + 4 * e);
    }
#pragma unroll
    for (int i = 0; i < RE; ++i)
        fe[i] = *reinterpret_cast<const f32x4*>(dem + 4 * ((tid + 512 * i) % nE));
#pragma unroll
    for (int i = 0; i < RG; ++i)
        fg[i] = *reinterpret_cast<const f32x4*>(ddg + 4 * ((tid + 512 * i) % nG));
    const float bt = beta[base + min(c * kB + (tid % kB), L - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < RI; ++i) {
        const int e = tid + 512 * i, r = (e % nI) / (D / 8), x0 = 8 * (e % (D / 8));
        if (e < nI) {
            const bool in = c * kB + r < L;
            *reinterpret_cast<u32x4*>(sQ + r * kLT + x0) = in ? uq[i] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(sK + r * kLT + x0) = in ? uk[i] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(sW + r * kLT + x0) = in ? uw[i] : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // an fp32 piece e of a row-major rows x cols matrix, rounded into a slot
    auto put4 = [&](__bf16* dst, int cols, int e, const f32x4& v) {
        const int r = e / (cols / 4), x0 = 4 * (e % (cols / 4));
        *reinterpret_cast<bf16x4_t*>(dst + r * kLT + x0) =
            bf16x4_t{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    };
#pragma unroll
    for (int i = 0; i < RA; ++i)
        if (tid + 512 * i < nA) {
            put4(sDq, D, tid + 512 * i, fq[i]);
            put4(sDk, D, tid + 512 * i, fk[i]);
        }
#pragma unroll
    for (int i = 0; i < RE; ++i)
        if (tid + 512 * i < nE) put4(sDe, D, tid + 512 * i, fe[i]);
#pragma unroll
    for (int i = 0; i < RG; ++i)
        if (tid + 512 * i < nG) put4(sDg, kB, tid + 512 * i, fg[i]);
    if (tid < kB) sBeta[tid] = c * kB + tid < L ? bt : 0.f;
    __syncthreads();

    // ---- 1. G = diag(beta) strictLower(W W^T) (fp32, for the solve) | X = lower(Q W^T)
    hprod<false, false, D>(0, kB, kB, sW, sW, [&](int m, int n, float v) {
        fG[m * kLdB + n] = n < m ? sBeta[m] * v : 0.f;
    });
    hprod<false, false, D>(1, kB, kB, sQ, sW,
                           [&](int m, int n, float v) { put_bf(sX, m, n, n <= m ? v : 0.f); });
    __syncthreads();
    // ---- 2. M = strictLower(W K^T) | dR = -W dKr^T
    hprod<false, false, D>(0, kB, kB, sW, sK,
                           [&](int m, int n, float v) { put_bf(sM, m, n, n < m ? v : 0.f); });
    hprod<false, false, D>(1, kB, kB, sW, sDk, [&](int m, int n, float v) { put_bf(sDr, m, n, -v); });
    __syncthreads();
    // ---- 3. T = (I + G)^{-1} and U = T diag(beta), a column per lane of wave 0
    //         (uniform unrolled substitution, G read as LDS broadcasts) |
    //         dY = W dE, dP = -dQl W^T - dDg M^T, dQ += dDg K, dK += dDg^T Q
    if (tid < kB) {
        const int j = tid;
        float t[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc -= fG[i * kLdB + kk] * t[kk];
            t[i] = i == j ? 1.f : (i < j ? 0.f : acc);
        }
        const float bj = sBeta[j];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            put_bf(sT, i, j, t[i]);
            put_bf(sU, i, j, t[i] * bj);
        }
    }
    hprod<false, true, D>(1, kB, D, sW, sDe, [&](int m, int n, float v) { put_bf(sDy, m, n, v); });
    for (int kq = 0;; ++kq) {
        const int t = half_tile(1, kB, kB, kq);
        if (t < 0) break;
        const int m0 = (t / 2) * 32, n0 = (t % 2) * 32;
        f32x16 acc = tprod<false, false, D>(sDq, sW, m0, n0, zero16());
        acc = tprod<false, false, kB>(sDg, sM, m0, n0, acc);
        for_tile(t, kB, acc, [&](int m, int n, float v) { put_bf(sDp, m, n, -v); });
    }
    // dQ, dK accumulators (half 1, a tile of each per wave), their input-only
    // terms while the solve runs: dDg K, dDg^T Q
    const int qt = half_tile(1, kB, D, 0);
    const int qm0 = qt >= 0 ? (qt / (D / 32)) * 32 : 0, qn0 = qt >= 0 ? (qt % (D / 32)) * 32 : 0;
    f32x16 aQ = zero16(), aK = zero16();
    // the tile's dQl and dKr terms of the outputs, fetched now (in the tile's
    // C layout) so that the final stores do not wait on them one by one
    f32x16 dqv = zero16(), dkv = zero16();
    if (qt >= 0) {
        const int r = threadIdx.x & 31, h = (threadIdx.x >> 5) & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = qm0 + 8 * i + 4 * h + j, n = qn0 + r;
                dqv[4 * i + j] = dql[m * D + n];
                dkv[4 * i + j] = dkr[m * D + n];
            }
        aQ = tprod<false, true, kB>(sDg, sK, qm0, qn0, aQ);
        aK = tprod<true, true, kB>(sDg, sQ, qm0, qn0, aK);
    }
    __syncthreads();
    // ---- 4. P = X U | R = U M
    hprod<false, true, kB>(0, kB, kB, sX, sU, [&](int m, int n, float v) { put_bf(sP, m, n, v); });
    hprod<false, true, kB>(1, kB, kB, sU, sM, [&](int m, int n, float v) { put_bf(sR, m, n, v); });
    __syncthreads();
    // ---- 5. dW accumulators (half 0, a tile per wave): -P^T dQl - R dKr |
    //         dM = strictLower(-P^T dDg + U^T dR)
    const int wt = half_tile(0, kB, D, 0);          // this wave's dW tile (half 0)
    const int wm0 = wt >= 0 ? (wt / (D / 32)) * 32 : 0, wn0 = wt >= 0 ? (wt % (D / 32)) * 32 : 0;
    f32x16 aW = zero16();
    if (wt >= 0) {
        aW = tprod<true, true, kB>(sP, sDq, wm0, wn0, aW);
        aW = tprod<false, true, kB>(sR, sDk, wm0, wn0, aW);
#pragma unroll
        for (int e = 0; e < 16; ++e) aW[e] = -aW[e];
    }
    for (int kq = 0;; ++kq) {
        const int t = half_tile(1, kB, kB, kq);
        if (t < 0) break;
        const int m0 = (t / 2) * 32, n0 = (t % 2) * 32;
        f32x16 acc = tprod<true, true, kB>(sP, sDg, m0, n0, zero16());
        f32x16 acc2 = tprod<true, true, kB>(sU, sDr, m0, n0, zero16());
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = acc2[e] - acc[e];
        for_tile(t, kB, acc, [&](int m, int n, float v) { put_bf(sDm, m, n, n < m ? v : 0.f); });
    }
    __syncthreads();
    // ---- 6. Y = U^T W | dX = lower(dP U^T)
    hprod<true, true, kB>(0, kB, D, sU, sW, [&](int m, int n, float v) { put_bf(sY, m, n, v); });
    hprod<false, false, kB>(1, kB, kB, sDp, sU,
                            [&](int m, int n, float v) { put_bf(sDx, m, n, n <= m ? v : 0.f); });
    __syncthreads();
    // ---- 7. dW += Y dE^T + U dY |
    //         dU = lower(X^T dP + dR M^T + W dY^T) -> dT = dU diag(beta), and
    //         U = T diag(beta) gives dbeta_n += sum_m T_mn dU_mn
    if (wt >= 0) {
        aW = tprod<false, false, D>(sY, sDe, wm0, wn0, aW);
        aW = tprod<false, true, kB>(sU, sDy, wm0, wn0, aW);
    }
    for (int kq = 0;; ++kq) {
        const int t = half_tile(1, kB, kB, kq);
        if (t < 0) break;
        const int m0 = (t / 2) * 32, n0 = (t % 2) * 32;
        f32x16 acc = tprod<true, true, kB>(sX, sDp, m0, n0, zero16());
        acc = tprod<false, false, kB>(sDr, sM, m0, n0, acc);
        acc = tprod<false, false, D>(sW, sDy, m0, n0, acc);
        // dbeta_n: the lane sums its 16 rows of column n in a fixed order,
        // the two lane halves of the column are added (a + b = b + a), and
        // the tile's partial goes to its own slot: no order-dependent atomics
        float part = 0.f;
        for_tile(t, kB, acc, [&](int m, int n, float v) {
            const float du = n <= m ? v : 0.f;
            put_bf(sDt, m, n, du * sBeta[n]);
            part += (float)sT[m * kLT + n] * du;
        });
        part += __shfl_xor(part, 32, 64);
        if ((threadIdx.x & 63) < 32) sDbU[t / 2][(t % 2) * 32 + (threadIdx.x & 31)] = part;
    }
    __syncthreads();
    // ---- 8. Tmp = dT T^T
    hprod<false, false, kB>(0, kB, kB, sDt, sT, [&](int m, int n, float v) { put_bf(sTmp, m, n, v); });
    __syncthreads();
    // ---- 9. dG = strictLower(-T^T Tmp) (fp32), with G_mn = beta_m (W W^T)_mn
    //         giving dbeta_m += sum_n dG_mn (W W^T)_mn | dQ += dX W, dK += dM^T W
    for (int kq = 0;; ++kq) {
        const int t = half_tile(0, kB, kB, kq);
        if (t < 0) break;
        const int m0 = (t / 2) * 32, n0 = (t % 2) * 32;
        const f32x16 g = tprod<true, true, kB>(sT, sTmp, m0, n0, zero16());
        const f32x16 ww = tprod<false, false, D>(sW, sW, m0, n0, zero16());
        f32x16 dgv;
#pragma unroll
        for (int e = 0; e < 16; ++e) dgv[e] = -g[e];
        int e = 0;
        f32x16 prod;
        for_tile(t, kB, dgv, [&](int m, int n, float v) {
            const float dg = n < m ? v : 0.f;
            fdG[m * kLdB + n] = dg;
            prod[e] = dg * ww[e];
            ++e;
        });
        // dbeta_m: each of the lane's 16 rows summed over the tile's 32 columns
        // by an xor butterfly (every lane ends with the same, order-fixed sum)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float r = prod[i];
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) r += __shfl_xor(r, off, 64);
            prod[i] = r;
        }
        const int lane = threadIdx.x & 63;
        if ((lane & 31) == 0) {
            const int m0 = (t / 2) * 32, h = lane >> 5;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) sDbG[t % 2][m0 + 8 * i + 4 * h + j] = prod[4 * i + j];
        }
    }
    if (qt >= 0) {
        aQ = tprod<false, true, kB>(sDx, sW, qm0, qn0, aQ);
        aK = tprod<true, true, kB>(sDm, sW, qm0, qn0, aK);
    }
    __syncthreads();
    // ---- 10. the symmetric weight A + A^T, A = diag(beta) dG, of dW's last term
    for (int e = tid; e < kB * kB; e += 512) {
        const int m = e / kB, n = e % kB;
        put_bf(sAA, m, n, sBeta[m] * fdG[m * kLdB + n] + sBeta[n] * fdG[n * kLdB + m]);
    }
    __syncthreads();
    // ---- 11. dW += dX^T Q + dM K + (A + A^T) W; then every output
    if (wt >= 0) {
        aW = tprod<true, true, kB>(sDx, sQ, wm0, wn0, aW);
        aW = tprod<false, true, kB>(sDm, sK, wm0, wn0, aW);
        aW = tprod<false, true, kB>(sAA, sW, wm0, wn0, aW);
        for_tile(wt, D, aW, [&](int m, int n, float v) {
            const int pos = c * kB + m;
            if (pos < L) dw[(base + pos) * D + n] = from_f32<bf16>(v);
        });
    }
    if (qt >= 0) {
        int e = 0;
        for_tile(qt, D, aQ, [&](int m, int n, float v) {
            const int pos = c * kB + m;
            if (pos < L) dq[(base + pos) * D + n] = from_f32<bf16>(v + dqv[e]);
            ++e;
        });
        e = 0;
        for_tile(qt, D, aK, [&](int m, int n, float v) {
            const int pos = c * kB + m;
            if (pos < L) dk[(base + pos) * D + n] = from_f32<bf16>(v + dkv[e]);
            ++e;
        });
    }
    __syncthreads();
    if (tid < kB && c * kB + tid < L)
        dbeta[base + c * kB + tid] = (sDbU[0][tid] + sDbU[1][tid]) + (sDbG[0][tid] + sDbG[1][tid]);
}

template <typename T, int D, int PARTS>
hipError_t bwd_t(const BwdArgs& a, hipStream_t st) {
    const int nb = (a.L + kB - 1) / kB, ns = a.N * a.H;
    const int fox = a.logf ? 1 : 0;
    FwdArgs f{};
    f.N = a.N; f.H = a.H; f.L = a.L; f.d = a.d; f.block = kB; f.bf16 = sizeof(T) == 2;
    f.q = a.q; f.k = a.k; f.w = a.w; f.beta = a.beta; f.logf = a.logf;
    f.ws = a.fw;
    f.v = a.v;
    f.scale = a.scale;
    hipError_t e;
    if (a.img) {   // bf16, d in {32, 64}: the matrix-core preconditioning
        f.ws.img = a.img;
        // the pair kernels take scale * Kright and -E as bf16 rows, in the
        // (fp32-sized) kr and em areas
        f.ws.kb16 = a.fw.kr;
        f.ws.eb16 = a.fw.em;
        e = launch_precond_bf16(f, st);
    } else {
        e = launch_precond_f32(f, st);
    }
    if (e != hipSuccess) return e;
    for (int s0 = 0; s0 < ns; s0 += a.chunk) {
        const int nsc = std::min(a.chunk, ns - s0);
        if (nb > 1) {
            if constexpr (sizeof(T) == 2 && D >= 32)
                hipLaunchKernelGGL((bwd_chain_b16_kernel<D>), dim3(nsc * (nb - 1)), dim3(256), 0,
                                   st, nb, nsc, s0, a.fw.ql, (const char*)a.img, a.X);
            else
                hipLaunchKernelGGL((bwd_chain_kernel<D, PARTS>), dim3(nsc * (nb - 1)),
                                   dim3(256), 0, st, nb, nsc, s0, a.fw.ql, (const float*)a.fw.em,
                                   a.X);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if constexpr (sizeof(T) == 2 && D >= 32) {
            hipLaunchKernelGGL((bwd_query_b16_kernel<D>), dim3(nsc * nb), dim3(256), 0, st, a.L,
                               nb, nsc, s0, a.scale, fox, (const bf16*)a.v, (const bf16*)a.o,
                               (const bf16*)a.dout, a.lse, a.fw, a.X, a.Z, a.dQl, a.dDg,
                               a.rowsum, a.delta);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL((bwd_key_b16_kernel<D>), dim3(nsc * nb), dim3(256), 0, st, a.L, nb,
                               nsc, s0, a.scale, fox, (const bf16*)a.v, (const bf16*)a.dout,
                               a.lse, a.delta, a.fw, a.X, a.Z, a.dKr, a.dEm, (bf16*)a.dv,
                               a.colsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL((bwd_query_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0, st,
                               a.L, nb, nsc, s0, a.scale, fox, (const T*)a.v, (const T*)a.o,
                               (const T*)a.dout, a.lse, a.fw, a.X, a.Z, a.dQl, a.dDg, a.rowsum,
                               a.delta);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            hipLaunchKernelGGL((bwd_key_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0, st,
                               a.L, nb, nsc, s0, a.scale, fox, (const T*)a.v, (const T*)a.dout,
                               a.lse, a.delta, a.fw, a.X, a.Z, a.dKr, a.dEm, (T*)a.dv, a.colsum);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if constexpr (sizeof(T) == 2 && D >= 32) {
            hipLaunchKernelGGL((bwd_precond_b16_kernel<D>), dim3(nsc * nb), dim3(512), 0, st,
                               a.L, nb, s0, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.w,
                               a.beta, a.dQl, a.dKr, a.dEm, a.dDg, (bf16*)a.dq, (bf16*)a.dk,
                               (bf16*)a.dw, a.dbeta);
        } else {
            hipLaunchKernelGGL((bwd_precond_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0,
                               st, a.L, nb, s0, (const T*)a.q, (const T*)a.k, (const T*)a.w,
                               a.beta, a.dQl, a.dKr, a.dEm, a.dDg, a.scr, (T*)a.dq, (T*)a.dk,
                               (T*)a.dw, a.dbeta);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (fox) {
        hipLaunchKernelGGL(bwd_gate_kernel, dim3(ns), dim3(256), 0, st, a.L, nb, a.rowsum,
                           a.colsum, a.dlogf);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T, int PARTS>
hipError_t bwd_d(const BwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 16: return bwd_t<T, 16, PARTS>(a, st);
        case 32: return bwd_t<T, 32, PARTS>(a, st);
        case 64: return bwd_t<T, 64, PARTS>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// workspace pieces of the backward for a chunk of `chunk` slices (floats)
size_t bwd_pair_floats(int L, int d, int chunk) {
    const size_t nb = (L + kB - 1) / kB;
    return (size_t)chunk * (nb * (nb - 1) / 2) * kB * d;
}
size_t bwd_scratch_floats(int L, int chunk) {
    const size_t nb = (L + kB - 1) / kB;
    return (size_t)chunk * nb * kScr * kB * kB;
}
int bwd_block() { return kB; }

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    return a.bf16 ? bwd_d<bf16, 2>(a, st) : bwd_d<float, 3>(a, st);
}

}  // namespace pa
