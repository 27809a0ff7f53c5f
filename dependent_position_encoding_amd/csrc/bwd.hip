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

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace pa {

namespace {

constexpr int kB = 64;          // block size
constexpr int kLdB = kB + 4;    // LDS row stride of a B x B tile (floats)

template <int D>
struct Dims {
    static constexpr int DP = D < 32 ? 32 : D;   // head dim padded to the 32-wide tiles
    static constexpr int LD = DP + 4;            // LDS row stride of a B x DP / DP x DP tile
};

// 8 fp32 values as bf16 operand parts: hi + lo (2) or hi + mid + lo (3)
template <int PARTS>
__device__ inline void parts8(const float (&v)[8], bf16x8 (&o)[3]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[0][e] = (__bf16)v[e];
        const float r = v[e] - (float)o[0][e];
        o[1][e] = (__bf16)r;
        if constexpr (PARTS == 3) o[2][e] = (__bf16)(r - (float)o[1][e]);
    }
}
// acc += A B over the partial products that matter, smallest first
template <int PARTS>
__device__ inline f32x16 mma(const bf16x8 (&a)[3], const bf16x8 (&b)[3], f32x16 c) {
    if constexpr (PARTS == 3) {
        c = mfma32(a[1], b[1], c);
        c = mfma32(a[2], b[0], c);
        c = mfma32(a[0], b[2], c);
    }
    c = mfma32(a[1], b[0], c);
    c = mfma32(a[0], b[1], c);
    return mfma32(a[0], b[0], c);
}

// C (M x N) = sum_k A(m, k) B(k, n) on the matrix cores; the 32 x 32 output
// tiles are dealt to the workgroup's waves and out(m, n, value) receives each
// element (exactly one lane per element).  M, N multiples of 32, K of 16.
template <int PARTS, typename FA, typename FB, typename FO>
__device__ inline void gemm(int M, int N, int K, FA A, FB Bm, FO out) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int r = lane & 31, h = lane >> 5;
    const int tn = N / 32, nt = (M / 32) * tn;
    for (int t = wave; t < nt; t += nw) {
        const int m0 = (t / tn) * 32, n0 = (t % tn) * 32;
        f32x16 c = zero16();
        for (int k0 = 0; k0 < K; k0 += 16) {
            float av[8], bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                av[e] = A(m0 + r, k0 + 8 * h + e);
                bv[e] = Bm(k0 + 8 * h + e, n0 + r);
            }
            bf16x8 ap[3], bp[3];
            parts8<PARTS>(av, ap);
            parts8<PARTS>(bv, bp);
            c = mma<PARTS>(ap, bp, c);
        }
        // C layout: lane -> column n0 + r, register 4i + j -> row m0 + 8i + 4h + j
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) out(m0 + 8 * i + 4 * h + j, n0 + r, c[4 * i + j]);
    }
}

__device__ inline size_t pair_index(int b, int c) { return (size_t)b * (b - 1) / 2 + c; }

// ---------------------------------------------------------------------------
// chain: for query block b >= 1 of a slice, the queries Qw_c used against every
// key block c < b, carried right to left as in the forward scan; stored per
// block pair in X [slice][pair][B][d].
template <int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_chain_kernel(int nb, int slice0, const float* __restrict__ ql,
                 const float* __restrict__ em, float* __restrict__ X) {
    using Dm = Dims<D>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ float sQ[kB * LD], sT[kB * LD], sE[DP * LD];
    const int tid = threadIdx.x;
    const int b = 1 + (int)(blockIdx.x % (nb - 1)), sl = (int)(blockIdx.x / (nb - 1));
    const size_t slice = (size_t)slice0 + sl, npairs = (size_t)nb * (nb - 1) / 2;
    float* Xs = X + (size_t)sl * npairs * kB * D;
    const float* qlb = ql + (slice * nb + b) * kB * D;
    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP;
        sQ[r * LD + x] = x < D ? qlb[r * D + x] : 0.f;
    }
    for (int e = tid; e < DP * LD; e += 256) sE[e] = 0.f;   // the padding stays zero
    for (int c = b - 1; c >= 0; --c) {
        __syncthreads();
        float* xo = Xs + pair_index(b, c) * kB * D;
        for (int e = tid; e < kB * D; e += 256) xo[e] = sQ[(e / D) * LD + e % D];
        if (c == 0) break;
        const float* ec = em + (slice * nb + c) * D * D;
        for (int e = tid; e < D * D; e += 256) sE[(e / D) * LD + e % D] = ec[e];
        __syncthreads();
        // Qw_{c-1} = Qw_c - Qw_c E_c^T
        gemm<PARTS>(kB, DP, DP, [&](int m, int k) { return sQ[m * LD + k]; },
                    [&](int k, int n) { return sE[n * LD + k]; },
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
// the rows' dS sums and Delta.
template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_query_kernel(int L, int nb, int slice0, float scale, int fox, const T* __restrict__ v,
                 const T* __restrict__ o, const T* __restrict__ dout,
                 const float* __restrict__ lse, FwdWs fw, const float* __restrict__ X,
                 float* __restrict__ Z, float* __restrict__ dQl, float* __restrict__ dDg,
                 float* __restrict__ rowsum, float* __restrict__ delta) {
    using Dm = Dims<D>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ float sdO[kB * LD], sV[kB * LD], sA[kB * LD], sG[kB * LD];
    __shared__ float sS[kB * kLdB], sP[kB * kLdB];
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB], sRow[kB];
    __shared__ float sTb;
    const int tid = threadIdx.x;
    const int b = (int)(blockIdx.x % nb), sl = (int)(blockIdx.x / nb);
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
    // sS holds logits -> P; then dP -> sP and dS = P (dP - Delta) -> sS, rows summed
    auto backprop_softmax = [&]() {
        for (int e = tid; e < kB * kB; e += 256) {
            const int i = e / kB, j = e % kB;
            const float s = sS[i * kLdB + j];
            sS[i * kLdB + j] = b * kB + i < L ? __expf(s - sLse[i]) : 0.f;
        }
        gemm<PARTS>(kB, kB, DP, [&](int m, int k) { return sdO[m * LD + k]; },
                    [&](int k, int n) { return sV[n * LD + k]; },
                    [&](int m, int n, float val) { sP[m * kLdB + n] = val; });
        __syncthreads();
        for (int e = tid; e < kB * kB; e += 256) {
            const int i = e / kB, j = e % kB;
            sS[i * kLdB + j] *= sP[i * kLdB + j] - sDel[i];
        }
        __syncthreads();
        if (tid < kB) {
            float s = 0.f;
            for (int j = 0; j < kB; ++j) s += sS[tid * kLdB + j];
            sRow[tid] += s;
        }
    };

    // diagonal tile
    load_v(b);
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) {
        const int i = e / kB, j = e % kB;
        sS[i * kLdB + j] = j <= i ? scale * fw.dg[blk_b * kB * kB + e] + (sGb[i] - sGb[j])
                                  : -INFINITY;
    }
    __syncthreads();
    backprop_softmax();
    for (int e = tid; e < kB * kB; e += 256)
        dDg[blk_b * kB * kB + e] = scale * sS[(e / kB) * kLdB + e % kB];
    for (int e = tid; e < kB * DP; e += 256) sA[(e / DP) * LD + e % DP] = 0.f;

    float Tc = 0.f;                 // sum of the gate totals of blocks before c
    for (int c = 0; c < b; ++c) {
        const size_t blk_c = slice * nb + c;
        __syncthreads();
        if (tid < kB) sGc[tid] = fox ? fw.gl[blk_c * kB + tid] : 0.f;
        load_v(c);
        __syncthreads();
        const float shift = fox ? sTb - Tc : 0.f;   // sum of the totals of blocks c .. b-1
        const float* xbc = Xs + pair_index(b, c) * kB * D;
        const float* krc = kr + blk_c * kB * D;
        const float* ec = em + blk_c * D * D;
        gemm<PARTS>(kB, kB, DP, [&](int m, int k) { return k < D ? xbc[m * D + k] : 0.f; },
                    [&](int k, int n) { return k < D ? krc[n * D + k] : 0.f; },
                    [&](int m, int n, float val) {
                        sS[m * kLdB + n] = scale * val + (sGb[m] + shift - sGc[n]);
                    });
        __syncthreads();
        backprop_softmax();
        // G = scale dS Kr_c
        gemm<PARTS>(kB, DP, kB, [&](int m, int k) { return sS[m * kLdB + k]; },
                    [&](int k, int n) { return n < D ? krc[k * D + n] : 0.f; },
                    [&](int m, int n, float val) { sG[m * LD + n] = scale * val; });
        if (c >= 1) {
            float* zo = Zs + pair_index(b, c) * kB * D;
            for (int e = tid; e < kB * D; e += 256) zo[e] = sA[(e / D) * LD + e % D];
            // A_c = G + A_{c-1} - A_{c-1} E_c  (A E_c into sP)
            gemm<PARTS>(kB, DP, DP, [&](int m, int k) { return sA[m * LD + k]; },
                        [&](int k, int n) { return k < D && n < D ? ec[k * D + n] : 0.f; },
                        [&](int m, int n, float val) { sP[m * LD + n] = val; });
            __syncthreads();
            for (int e = tid; e < kB * DP; e += 256) {
                const int r = e / DP, x = e % DP;
                sA[r * LD + x] += sG[r * LD + x] - sP[r * LD + x];
            }
        } else {
            __syncthreads();
            for (int e = tid; e < kB * DP; e += 256) {
                const int r = e / DP, x = e % DP;
                sA[r * LD + x] = sG[r * LD + x];
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
// dE_c and the keys' dS column sums, accumulated in LDS.
template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_key_kernel(int L, int nb, int slice0, float scale, int fox, const T* __restrict__ v,
               const T* __restrict__ dout, const float* __restrict__ lse,
               const float* __restrict__ delta, FwdWs fw, const float* __restrict__ X,
               const float* __restrict__ Z, float* __restrict__ dKr, float* __restrict__ dEm,
               T* __restrict__ dv, float* __restrict__ colsum) {
    using Dm = Dims<D>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ float sV[kB * LD], sK[kB * LD], sdV[kB * LD], sdK[kB * LD], sdE[DP * LD];
    __shared__ float sdO[kB * LD], sS[kB * kLdB], sP[kB * kLdB];
    __shared__ float sLse[kB], sDel[kB], sGb[kB], sGc[kB], sCol[kB];
    const int tid = threadIdx.x;
    const int c = (int)(blockIdx.x % nb), sl = (int)(blockIdx.x / nb);
    const size_t slice = (size_t)slice0 + sl, blk_c = slice * nb + c, base = slice * L;
    const size_t npairs = (size_t)nb * (nb - 1) / 2;
    const float* Xs = X + (size_t)sl * npairs * kB * D;
    const float* Zs = Z + (size_t)sl * npairs * kB * D;
    const float* krc = static_cast<const float*>(fw.kr) + blk_c * kB * D;

    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP, pos = c * kB + r;
        sV[r * LD + x] = x < D && pos < L ? to_f32(v[(base + pos) * D + x]) : 0.f;
        sK[r * LD + x] = x < D ? krc[r * D + x] : 0.f;
        sdK[r * LD + x] = 0.f;
    }
    for (int e = tid; e < DP * LD; e += 256) sdE[e] = 0.f;
    if (tid < kB) {
        sGc[tid] = fox ? fw.gl[blk_c * kB + tid] : 0.f;
        sCol[tid] = 0.f;
    }
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
    // sS: logits -> P; dV += P^T dO; dP -> sP; dS -> sS; columns summed
    auto backprop = [&](int b, bool first) {
        __syncthreads();   // the logits tile is complete
        for (int e = tid; e < kB * kB; e += 256) {
            const int i = e / kB, j = e % kB;
            const float s = sS[i * kLdB + j];
            sS[i * kLdB + j] = b * kB + i < L ? __expf(s - sLse[i]) : 0.f;
        }
        __syncthreads();
        gemm<PARTS>(kB, DP, kB, [&](int m, int k) { return sS[k * kLdB + m]; },
                    [&](int k, int n) { return sdO[k * LD + n]; },
                    [&](int m, int n, float val) {
                        sdV[m * LD + n] = first ? val : sdV[m * LD + n] + val;
                    });
        gemm<PARTS>(kB, kB, DP, [&](int m, int k) { return sdO[m * LD + k]; },
                    [&](int k, int n) { return sV[n * LD + k]; },
                    [&](int m, int n, float val) { sP[m * kLdB + n] = val; });
        __syncthreads();
        for (int e = tid; e < kB * kB; e += 256) {
            const int i = e / kB, j = e % kB;
            sS[i * kLdB + j] *= sP[i * kLdB + j] - sDel[i];
        }
        __syncthreads();
        if (tid < kB) {
            float s = 0.f;
            for (int i = 0; i < kB; ++i) s += sS[i * kLdB + tid];
            sCol[tid] += s;
        }
    };

    // diagonal tile (b = c)
    load_rows(c);
    __syncthreads();
    for (int e = tid; e < kB * kB; e += 256) {
        const int i = e / kB, j = e % kB;
        sS[i * kLdB + j] = j <= i ? scale * fw.dg[blk_c * kB * kB + e] + (sGc[i] - sGc[j])
                                  : -INFINITY;
    }
    backprop(c, true);

    float shift = 0.f;              // sum of the gate totals of blocks c .. b-1
    for (int b = c + 1; b < nb; ++b) {
        if (fox) shift += fw.tot[slice * nb + b - 1];
        __syncthreads();
        load_rows(b);
        __syncthreads();
        const float* xbc = Xs + pair_index(b, c) * kB * D;
        gemm<PARTS>(kB, kB, DP, [&](int m, int k) { return k < D ? xbc[m * D + k] : 0.f; },
                    [&](int k, int n) { return sK[n * LD + k]; },
                    [&](int m, int n, float val) {
                        sS[m * kLdB + n] = scale * val + (sGb[m] + shift - sGc[n]);
                    });
        backprop(b, false);
        // dKr += scale dS^T Qw_c;  dE -= A_{c-1}^T Qw_c
        gemm<PARTS>(kB, DP, kB, [&](int m, int k) { return sS[k * kLdB + m]; },
                    [&](int k, int n) { return n < D ? xbc[k * D + n] : 0.f; },
                    [&](int m, int n, float val) { sdK[m * LD + n] += scale * val; });
        if (c >= 1) {
            const float* zbc = Zs + pair_index(b, c) * kB * D;
            gemm<PARTS>(DP, DP, kB, [&](int m, int k) { return m < D ? zbc[k * D + m] : 0.f; },
                        [&](int k, int n) { return n < D ? xbc[k * D + n] : 0.f; },
                        [&](int m, int n, float val) { sdE[m * LD + n] -= val; });
        }
    }
    __syncthreads();
    for (int e = tid; e < kB * D; e += 256) {
        const int r = e / D, x = e % D, pos = c * kB + r;
        dKr[blk_c * kB * D + e] = sdK[r * LD + x];
        if (pos < L) dv[(base + pos) * D + x] = from_f32<T>(sdV[r * LD + x]);
    }
    for (int e = tid; e < D * D; e += 256) dEm[blk_c * D * D + e] = sdE[(e / D) * LD + e % D];
    if (tid < kB) colsum[blk_c * kB + tid] = sCol[tid];
}

// ---------------------------------------------------------------------------
// precond_bwd: per block, (dQl, dKr, dE, dDg) back through
//   G = strictLower(diag(beta) W W^T), T = (I + G)^{-1}, U = T diag(beta),
//   X = lower(Q W^T), P = X U, Ql = Q - P W, M = strictLower(W K^T), R = U M,
//   Kr = K - R^T W, Y = U^T W, E = W^T Y, Dg = lower(Q K^T) - P M
// [Notes s2.6, s2.7]; intermediate B x B and B x d products live in a per-block
// scratch area of the workspace (kScr tiles of 64 x 64 floats).
constexpr int kScr = 15;
enum { sU_, sX_, sM_, sY_, sP_, sR_, sdP_, sdR_, sdY_, sdM_, sdU_, sdX_, sTmp_, sdG_, sWW_ };

template <typename T, int D, int PARTS>
__global__ void __launch_bounds__(256)
bwd_precond_kernel(int L, int nb, int slice0, const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ w, const float* __restrict__ beta,
                   const float* __restrict__ dQl, const float* __restrict__ dKr,
                   const float* __restrict__ dEm, const float* __restrict__ dDg,
                   float* __restrict__ scr, T* __restrict__ dq, T* __restrict__ dk,
                   T* __restrict__ dw, float* __restrict__ dbeta) {
    using Dm = Dims<D>;
    constexpr int DP = Dm::DP, LD = Dm::LD;
    __shared__ float sQ[kB * LD], sK[kB * LD], sW[kB * LD];
    __shared__ float sT[kB * kLdB], sG[kB * kLdB], oQ[kB * LD], oK[kB * LD];
    __shared__ float sBeta[kB], sdB[kB];
    const int tid = threadIdx.x;
    const int c = (int)(blockIdx.x % nb), sl = (int)(blockIdx.x / nb);
    const size_t slice = (size_t)slice0 + sl, blk = slice * nb + c, base = slice * L;
    float* S = scr + (size_t)blockIdx.x * kScr * kB * kB;
    auto g = [&](int t) { return S + (size_t)t * kB * kB; };   // 64 x 64, row stride 64
    const float* dql = dQl + blk * kB * D;
    const float* dkr = dKr + blk * kB * D;
    const float* dem = dEm + blk * D * D;
    const float* ddg = dDg + blk * kB * kB;

    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP, pos = c * kB + r;
        const bool in = x < D && pos < L;
        const size_t gi = (base + pos) * D + x;
        sQ[r * LD + x] = in ? to_f32(q[gi]) : 0.f;
        sK[r * LD + x] = in ? to_f32(k[gi]) : 0.f;
        sW[r * LD + x] = in ? to_f32(w[gi]) : 0.f;
    }
    if (tid < kB) {
        const int pos = c * kB + tid;
        sBeta[tid] = pos < L ? beta[base + pos] : 0.f;
        sdB[tid] = 0.f;
    }
    __syncthreads();
    auto Wm = [&](int m, int kk) { return sW[m * LD + kk]; };        // W (m, k)
    auto WT = [&](int kk, int n) { return sW[n * LD + kk]; };        // W^T as the right operand
    auto Um = [&](int a, int j) { return sT[a * kLdB + j] * sBeta[j]; };
    // G and W W^T
    gemm<PARTS>(kB, kB, DP, Wm, WT, [&](int m, int n, float val) {
        sG[m * kLdB + n] = n < m ? sBeta[m] * val : 0.f;
        g(sWW_)[m * kB + n] = val;
    });
    __syncthreads();
    // T = (I + G)^{-1}: T_jj = 1, T_ij = -sum_{k=j}^{i-1} G_ik T_kj, a column per thread
    if (tid < kB) {
        const int j = tid;
        for (int i = 0; i < kB; ++i) {
            float t = i == j ? 1.f : 0.f;
            if (i > j)
                for (int kk = j; kk < i; ++kk) t -= sG[i * kLdB + kk] * sT[kk * kLdB + j];
            sT[i * kLdB + j] = t;
        }
    }
    __syncthreads();
    // forward products: X, M, Y, U; then P, R
    gemm<PARTS>(kB, kB, DP, [&](int m, int kk) { return sQ[m * LD + kk]; }, WT,
                [&](int m, int n, float val) { g(sX_)[m * kB + n] = n <= m ? val : 0.f; });
    gemm<PARTS>(kB, kB, DP, Wm, [&](int kk, int n) { return sK[n * LD + kk]; },
                [&](int m, int n, float val) { g(sM_)[m * kB + n] = n < m ? val : 0.f; });
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return Um(kk, m); },
                [&](int kk, int n) { return sW[kk * LD + n]; },
                [&](int m, int n, float val) { g(sY_)[m * kB + n] = val; });
    for (int e = tid; e < kB * kB; e += 256) g(sU_)[e] = Um(e / kB, e % kB);
    __syncthreads();
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sX_)[m * kB + kk]; }, Um,
                [&](int m, int n, float val) { g(sP_)[m * kB + n] = val; });
    gemm<PARTS>(kB, kB, kB, Um, [&](int kk, int n) { return g(sM_)[kk * kB + n]; },
                [&](int m, int n, float val) { g(sR_)[m * kB + n] = val; });
    __syncthreads();
    // dP = -dDg M^T - dQl W^T;  dR = -W dKr^T;  dY = W dE
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return ddg[m * kB + kk]; },
                [&](int kk, int n) { return g(sM_)[n * kB + kk]; },
                [&](int m, int n, float val) { g(sdP_)[m * kB + n] = -val; });
    gemm<PARTS>(kB, kB, DP, Wm, [&](int kk, int n) { return kk < D ? dkr[n * D + kk] : 0.f; },
                [&](int m, int n, float val) { g(sdR_)[m * kB + n] = -val; });
    gemm<PARTS>(kB, DP, DP, Wm,
                [&](int kk, int n) { return kk < D && n < D ? dem[kk * D + n] : 0.f; },
                [&](int m, int n, float val) { g(sdY_)[m * kB + n] = val; });
    __syncthreads();
    gemm<PARTS>(kB, kB, DP, [&](int m, int kk) { return kk < D ? dql[m * D + kk] : 0.f; }, WT,
                [&](int m, int n, float val) { g(sdP_)[m * kB + n] -= val; });
    // dM = strictLower(-P^T dDg + U^T dR)
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sP_)[kk * kB + m]; },
                [&](int kk, int n) { return ddg[kk * kB + n]; },
                [&](int m, int n, float val) { g(sdM_)[m * kB + n] = -val; });
    // dU = lower(X^T dP + dR M^T + W dY^T), first term after dP is complete
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sdR_)[m * kB + kk]; },
                [&](int kk, int n) { return g(sM_)[n * kB + kk]; },
                [&](int m, int n, float val) { g(sdU_)[m * kB + n] = val; });
    __syncthreads();
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return Um(kk, m); },
                [&](int kk, int n) { return g(sdR_)[kk * kB + n]; },
                [&](int m, int n, float val) {
                    g(sdM_)[m * kB + n] = n < m ? g(sdM_)[m * kB + n] + val : 0.f;
                });
    gemm<PARTS>(kB, kB, DP, Wm, [&](int kk, int n) { return g(sdY_)[n * kB + kk]; },
                [&](int m, int n, float val) { g(sdU_)[m * kB + n] += val; });
    // dX = lower(dP U^T)
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sdP_)[m * kB + kk]; },
                [&](int kk, int n) { return Um(n, kk); },
                [&](int m, int n, float val) { g(sdX_)[m * kB + n] = n <= m ? val : 0.f; });
    __syncthreads();
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sX_)[kk * kB + m]; },
                [&](int kk, int n) { return g(sdP_)[kk * kB + n]; },
                [&](int m, int n, float val) {
                    g(sdU_)[m * kB + n] = n <= m ? g(sdU_)[m * kB + n] + val : 0.f;
                });
    __syncthreads();
    // U = T diag(beta): dbeta_j += sum_a T_aj dU_aj;  dT = dU diag(beta)
    // dG = strictLower(-T^T dT T^T): Tmp = dT T^T, then -T^T Tmp
    if (tid < kB) {
        float s = 0.f;
        for (int a = tid; a < kB; ++a) s += sT[a * kLdB + tid] * g(sdU_)[a * kB + tid];
        sdB[tid] += s;
    }
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return g(sdU_)[m * kB + kk] * sBeta[kk]; },
                [&](int kk, int n) { return sT[n * kLdB + kk]; },
                [&](int m, int n, float val) { g(sTmp_)[m * kB + n] = val; });
    __syncthreads();
    gemm<PARTS>(kB, kB, kB, [&](int m, int kk) { return sT[kk * kLdB + m]; },
                [&](int kk, int n) { return g(sTmp_)[kk * kB + n]; },
                [&](int m, int n, float val) { g(sdG_)[m * kB + n] = n < m ? -val : 0.f; });
    __syncthreads();
    // G_ij = beta_i (w_i . w_j), i > j: dbeta_i += sum_j dG_ij (W W^T)_ij
    if (tid < kB) {
        float s = 0.f;
        for (int j = 0; j < tid; ++j) s += g(sdG_)[tid * kB + j] * g(sWW_)[tid * kB + j];
        sdB[tid] += s;
    }
    // dW = -P^T dQl - R dKr + dX^T Q + dM K + Y dE^T + U dY + (A + A^T) W,
    // A = diag(beta) dG; accumulated in sG (free now)
    auto acc = [&](int m, int n, float val) { sG[m * kLdB + n] += val; };
    for (int e = tid; e < kB * kLdB; e += 256) sG[e] = 0.f;
    __syncthreads();
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return -g(sP_)[kk * kB + m]; },
                [&](int kk, int n) { return n < D ? dql[kk * D + n] : 0.f; }, acc);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return -g(sR_)[m * kB + kk]; },
                [&](int kk, int n) { return n < D ? dkr[kk * D + n] : 0.f; }, acc);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return g(sdX_)[kk * kB + m]; },
                [&](int kk, int n) { return sQ[kk * LD + n]; }, acc);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return g(sdM_)[m * kB + kk]; },
                [&](int kk, int n) { return sK[kk * LD + n]; }, acc);
    gemm<PARTS>(kB, DP, DP, [&](int m, int kk) { return g(sY_)[m * kB + kk]; },
                [&](int kk, int n) { return kk < D && n < D ? dem[n * D + kk] : 0.f; }, acc);
    gemm<PARTS>(kB, DP, kB, Um, [&](int kk, int n) { return g(sdY_)[kk * kB + n]; }, acc);
    gemm<PARTS>(kB, DP, kB,
                [&](int m, int kk) {
                    return sBeta[m] * g(sdG_)[m * kB + kk] + sBeta[kk] * g(sdG_)[kk * kB + m];
                },
                [&](int kk, int n) { return sW[kk * LD + n]; }, acc);
    // dQ = dQl + dDg K + dX W;  dK = dKr + dDg^T Q + dM^T W
    for (int e = tid; e < kB * DP; e += 256) {
        const int r = e / DP, x = e % DP;
        oQ[r * LD + x] = x < D ? dql[r * D + x] : 0.f;
        oK[r * LD + x] = x < D ? dkr[r * D + x] : 0.f;
    }
    __syncthreads();
    auto accQ = [&](int m, int n, float val) { oQ[m * LD + n] += val; };
    auto accK = [&](int m, int n, float val) { oK[m * LD + n] += val; };
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return ddg[m * kB + kk]; },
                [&](int kk, int n) { return sK[kk * LD + n]; }, accQ);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return g(sdX_)[m * kB + kk]; },
                [&](int kk, int n) { return sW[kk * LD + n]; }, accQ);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return ddg[kk * kB + m]; },
                [&](int kk, int n) { return sQ[kk * LD + n]; }, accK);
    gemm<PARTS>(kB, DP, kB, [&](int m, int kk) { return g(sdM_)[kk * kB + m]; },
                [&](int kk, int n) { return sW[kk * LD + n]; }, accK);
    __syncthreads();
    for (int e = tid; e < kB * D; e += 256) {
        const int r = e / D, x = e % D, pos = c * kB + r;
        if (pos < L) {
            const size_t gi = (base + pos) * D + x;
            dq[gi] = from_f32<T>(oQ[r * LD + x]);
            dk[gi] = from_f32<T>(oK[r * LD + x]);
            dw[gi] = from_f32<T>(sG[r * kLdB + x]);
        }
    }
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

template <typename T, int D, int PARTS>
hipError_t bwd_t(const BwdArgs& a, hipStream_t st) {
    const int nb = (a.L + kB - 1) / kB, ns = a.N * a.H;
    const int fox = a.logf ? 1 : 0;
    FwdArgs f{};
    f.N = a.N; f.H = a.H; f.L = a.L; f.d = a.d; f.block = kB; f.bf16 = sizeof(T) == 2;
    f.q = a.q; f.k = a.k; f.w = a.w; f.beta = a.beta; f.logf = a.logf;
    f.ws = a.fw;
    hipError_t e = launch_precond_f32(f, st);
    if (e != hipSuccess) return e;
    for (int s0 = 0; s0 < ns; s0 += a.chunk) {
        const int nsc = std::min(a.chunk, ns - s0);
        if (nb > 1) {
            hipLaunchKernelGGL((bwd_chain_kernel<D, PARTS>), dim3(nsc * (nb - 1)), dim3(256), 0,
                               st, nb, s0, a.fw.ql, (const float*)a.fw.em, a.X);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((bwd_query_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0, st,
                           a.L, nb, s0, a.scale, fox, (const T*)a.v, (const T*)a.o,
                           (const T*)a.dout, a.lse, a.fw, a.X, a.Z, a.dQl, a.dDg, a.rowsum,
                           a.delta);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_key_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0, st,
                           a.L, nb, s0, a.scale, fox, (const T*)a.v, (const T*)a.dout, a.lse,
                           a.delta, a.fw, a.X, a.Z, a.dKr, a.dEm, (T*)a.dv, a.colsum);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_precond_kernel<T, D, PARTS>), dim3(nsc * nb), dim3(256), 0, st,
                           a.L, nb, s0, (const T*)a.q, (const T*)a.k, (const T*)a.w, a.beta,
                           a.dQl, a.dKr, a.dEm, a.dDg, a.scr, (T*)a.dq, (T*)a.dk, (T*)a.dw,
                           a.dbeta);
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
