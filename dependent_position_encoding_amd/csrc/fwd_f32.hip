// fwd_f32.hip -- float32 blockwise PaTH forward on the vector ALUs.
//
// Citations: [Notes s2.x] = reading-notes page "PaTH Attention:通过累积
// Householder 变换编码位置" (cc.laoqi.cc), section 2.x.
//
// This is the float32 path (and the generic fallback for head sizes the
// matrix-core path does not take).  It runs the same block algorithm as the
// bf16 path: a per-block UT solve and boundary preconditioning, then a
// right-to-left scan with an online softmax [Notes s2.6, s2.7], all in fp32
// with operands staged in LDS.  One workgroup of 256 threads per block.
#include "common.hpp"
#include "kernels.hpp"

namespace pa {

// Per block c of one (n,h) slice, rows r = 0..B-1 at positions c*B + r:
//   G = strictLower(diag(beta) W W^T),  T = (I + G)^{-1},  U = T diag(beta)
//   P = lower(Q W^T) U,            Qleft  = Q - P W        (q moved to the
//                                                           block's left edge)
//   M = strictLower(W K^T),        Kright = K - (U M)^T W  (k moved to the
//                                                           block's right edge)
//   E = W^T U^T W                  (block transition H_first...H_last = I - E)
//   Dg = lower(Q K^T) - P M        (in-block logits, unscaled)
//   gl = in-block inclusive cumsum of log f, tot = its last element.
// [Notes s2.6: UT form, full-matrix logits; s2.7: Qleft, Kright, F_b.]
// Rows past the sequence end are zero with beta = 0 (H = I): they change
// nothing and are masked by causality.
template <typename T, int B, int D>
__global__ void __launch_bounds__(256)
precond_f32_kernel(const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ w, const float* __restrict__ beta,
                   const float* __restrict__ logf, int L, int nb,
                   FwdWs ws) {
    __shared__ float sW[B][D + 1], sQ[B][D + 1], sK[B][D + 1];
    __shared__ float sU[B][B + 1], sX[B][B + 1], sP[B][B + 1], sM[B][B + 1];
    __shared__ float sY[B][D + 1];
    __shared__ float sBeta[B];

    const int blk = blockIdx.x;              // slice * nb + c
    const int slice = blk / nb, c = blk % nb;
    const int tid = threadIdx.x;
    const size_t base = (size_t)slice * L;
    const int row0 = c * B;

    for (int e = tid; e < B * D; e += 256) {
        int r = e / D, x = e % D, pos = row0 + r;
        bool in = pos < L;
        size_t g = (base + pos) * D + x;
        sW[r][x] = in ? to_f32(w[g]) : 0.f;
        sQ[r][x] = in ? to_f32(q[g]) : 0.f;
        sK[r][x] = in ? to_f32(k[g]) : 0.f;
    }
    if (tid < B) {
        int pos = row0 + tid;
        sBeta[tid] = pos < L ? beta[base + pos] : 0.f;
    }
    __syncthreads();

    // G (strictly lower) into sX
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        float s = 0.f;
        if (i > j) {
            for (int x = 0; x < D; ++x) s += sW[i][x] * sW[j][x];
            s *= sBeta[i];
        }
        sX[i][j] = s;
    }
    __syncthreads();
    // T = (I + G)^{-1} by forward substitution, one column per thread,
    //   T_jj = 1,  T_ij = -sum_{k=j}^{i-1} G_ik T_kj  (i > j),
    // with the column in registers: t = e_j, then for k = 0, 1, ... every
    // t_i (i > k) takes its term -G_ik t_k (terms with k < j add exact zeros),
    // so each entry sees the same operations in the same order as the sum.
    if (tid < B) {
        const int j = tid;
        float t[B];
#pragma unroll
        for (int i = 0; i < B; ++i) t[i] = i == j ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < B - 1; ++kk)
#pragma unroll
            for (int i = kk + 1; i < B; ++i) t[i] -= sX[i][kk] * t[kk];
#pragma unroll
        for (int i = 0; i < B; ++i) sU[i][j] = t[i];
    }
    __syncthreads();
    // U = T diag(beta)
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        sU[i][j] *= sBeta[j];
    }
    // lower(Q W^T) into sX, strictLower(W K^T) into sM
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        float a = 0.f, m = 0.f;
        if (j <= i) for (int x = 0; x < D; ++x) a += sQ[i][x] * sW[j][x];
        if (i > j) for (int x = 0; x < D; ++x) m += sW[i][x] * sK[j][x];
        sX[i][j] = a;
        sM[i][j] = m;
    }
    __syncthreads();
    // P = lower(QW^T) U
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        float s = 0.f;
        for (int a = j; a <= i; ++a) s += sX[i][a] * sU[a][j];
        sP[i][j] = s;
    }
    __syncthreads();
    // R = U M into sX (R[a][j] = sum_b U[a][b] M[b][j], b in (j, a])
    for (int e = tid; e < B * B; e += 256) {
        int a = e / B, j = e % B;
        float s = 0.f;
        for (int b = j + 1; b <= a; ++b) s += sU[a][b] * sM[b][j];
        sX[a][j] = s;
    }
    // Y = U^T W  (Y[cc][y] = sum_a U[a][cc] W[a][y])
    for (int e = tid; e < B * D; e += 256) {
        int cc = e / D, y = e % D;
        float s = 0.f;
        for (int a = cc; a < B; ++a) s += sU[a][cc] * sW[a][y];
        sY[cc][y] = s;
    }
    __syncthreads();

    const size_t bq = (size_t)blk * B * D;
    float* kr = reinterpret_cast<float*>(ws.kr);
    for (int e = tid; e < B * D; e += 256) {
        int r = e / D, x = e % D;
        float sq = sQ[r][x], sk = sK[r][x];
        for (int j = 0; j <= r; ++j) sq -= sP[r][j] * sW[j][x];        // Q - P W
        for (int a = r + 1; a < B; ++a) sk -= sX[a][r] * sW[a][x];     // K - R^T W
        ws.ql[bq + e] = sq;
        kr[bq + e] = sk;
        if (ws.k32) ws.k32[bq + e] = sk;
    }
    float* em = reinterpret_cast<float*>(ws.em);
    const size_t be = (size_t)blk * D * D;
    for (int e = tid; e < D * D; e += 256) {
        int x = e / D, y = e % D;
        float s = 0.f;
        for (int cc = 0; cc < B; ++cc) s += sW[cc][x] * sY[cc][y];
        em[be + e] = s;
        if (ws.e32) ws.e32[be + e] = s;
    }
    const size_t bd = (size_t)blk * B * B;
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        float s = 0.f;
        if (j <= i) {
            for (int x = 0; x < D; ++x) s += sQ[i][x] * sK[j][x];
            for (int b = j + 1; b <= i; ++b) s -= sP[i][b] * sM[b][j];
        }
        ws.dg[bd + e] = s;
    }
    if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < B; ++r) {
            int pos = row0 + r;
            if (logf && pos < L) acc += logf[base + pos];
            ws.gl[(size_t)blk * B + r] = acc;
        }
        ws.tot[blk] = acc;
    }
}

// Right-to-left scan for query block b [Notes s2.7]: the diagonal block from
// its in-block logits, then for c = b-1 .. 0: logits Qwork . Kright_c^T (plus
// the gate bias), online-softmax update, value accumulation, and
// Qwork <- Qwork (I - E_c)^T to carry the queries across block c.
template <typename T, int B, int D>
__global__ void __launch_bounds__(256)
scan_f32_kernel(const T* __restrict__ v, int L, int nb, float scale, int fox,
                FwdWs ws, T* __restrict__ o, float* __restrict__ lse) {
    __shared__ float sQw[B][D + 1], sO[B][D + 1], sS[B][B + 1];
    __shared__ float sK[B][D + 1], sV[B][D + 1], sE[D][D + 1];
    __shared__ float sM[B], sL[B], sGb[B], sGc[B];

    // heaviest query blocks first
    const int nslice = gridDim.x / nb;
    const int b = nb - 1 - (int)(blockIdx.x / nslice);
    const int slice = blockIdx.x % nslice;
    const int tid = threadIdx.x;
    const size_t base = (size_t)slice * L;
    const size_t blk_b = (size_t)slice * nb + b;
    const float* kr = reinterpret_cast<const float*>(ws.kr);
    const float* em = reinterpret_cast<const float*>(ws.em);

    if (tid < B) sGb[tid] = fox ? ws.gl[blk_b * B + tid] : 0.f;
    for (int e = tid; e < B * D; e += 256) {
        int r = e / D, x = e % D, pos = b * B + r;
        sV[r][x] = pos < L ? to_f32(v[(base + pos) * D + x]) : 0.f;
        sQw[r][x] = ws.ql[blk_b * B * D + e];
    }
    __syncthreads();
    // diagonal block
    for (int e = tid; e < B * B; e += 256) {
        int i = e / B, j = e % B;
        sS[i][j] = (j <= i) ? scale * ws.dg[blk_b * B * B + e] + (sGb[i] - sGb[j])
                            : -INFINITY;
    }
    __syncthreads();
    if (tid < B) {
        float m = -INFINITY;
        for (int j = 0; j < B; ++j) m = fmaxf(m, sS[tid][j]);
        float l = 0.f;
        for (int j = 0; j < B; ++j) {
            float p = __expf(sS[tid][j] - m);
            sS[tid][j] = p;
            l += p;
        }
        sM[tid] = m;
        sL[tid] = l;
    }
    __syncthreads();
    for (int e = tid; e < B * D; e += 256) {
        int i = e / D, x = e % D;
        float s = 0.f;
        for (int j = 0; j < B; ++j) s += sS[i][j] * sV[j][x];
        sO[i][x] = s;
    }
    float grun = 0.f;
    for (int c = b - 1; c >= 0; --c) {
        const size_t blk_c = (size_t)slice * nb + c;
        __syncthreads();
        grun += fox ? ws.tot[blk_c] : 0.f;
        for (int e = tid; e < B * D; e += 256) {
            int r = e / D, x = e % D;
            sK[r][x] = kr[blk_c * B * D + e];
            sV[r][x] = to_f32(v[(base + c * B + r) * D + x]);
        }
        for (int e = tid; e < D * D; e += 256) sE[e / D][e % D] = em[blk_c * D * D + e];
        if (tid < B) sGc[tid] = fox ? ws.gl[blk_c * B + tid] : 0.f;
        __syncthreads();
        for (int e = tid; e < B * B; e += 256) {
            int i = e / B, j = e % B;
            float s = 0.f;
            for (int x = 0; x < D; ++x) s += sQw[i][x] * sK[j][x];
            sS[i][j] = scale * s + (sGb[i] + grun - sGc[j]);
        }
        __syncthreads();
        if (tid < B) {
            float mo = sM[tid], m = mo;
            for (int j = 0; j < B; ++j) m = fmaxf(m, sS[tid][j]);
            float l = 0.f;
            for (int j = 0; j < B; ++j) {
                float p = __expf(sS[tid][j] - m);
                sS[tid][j] = p;
                l += p;
            }
            float alpha = __expf(mo - m);
            sM[tid] = m;
            sL[tid] = sL[tid] * alpha + l;
            sGc[tid] = alpha;          // reuse as the row rescale factor
        }
        __syncthreads();
        for (int e = tid; e < B * D; e += 256) {
            int i = e / D, x = e % D;
            float s = 0.f;
            for (int j = 0; j < B; ++j) s += sS[i][j] * sV[j][x];
            sO[i][x] = sO[i][x] * sGc[i] + s;
        }
        if (c > 0) {
            // Qwork <- Qwork - Qwork E_c^T; new rows into sK (free now)
            for (int e = tid; e < B * D; e += 256) {
                int i = e / D, x = e % D;
                float s = 0.f;
                for (int y = 0; y < D; ++y) s += sQw[i][y] * sE[x][y];
                sK[i][x] = sQw[i][x] - s;
            }
            __syncthreads();
            for (int e = tid; e < B * D; e += 256) sQw[e / D][e % D] = sK[e / D][e % D];
        }
    }
    __syncthreads();
    for (int e = tid; e < B * D; e += 256) {
        int i = e / D, x = e % D, pos = b * B + i;
        if (pos < L) o[(base + pos) * D + x] = from_f32<T>(sO[i][x] / sL[i]);
    }
    if (tid < B && lse) {
        int pos = b * B + tid;
        if (pos < L) lse[base + pos] = sM[tid] + logf(sL[tid]);
    }
}

template <typename T, int B, int D>
static hipError_t launch_fwd_f32_t(const FwdArgs& a, hipStream_t st) {
    const int nb = (a.L + B - 1) / B;
    const int nblk = a.N * a.H * nb;
    hipLaunchKernelGGL((precond_f32_kernel<T, B, D>), dim3(nblk), dim3(256), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.w, a.beta, a.logf,
                       a.L, nb, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[1], st)) != hipSuccess) return e;
    hipLaunchKernelGGL((scan_f32_kernel<T, B, D>), dim3(nblk), dim3(256), 0, st,
                       (const T*)a.v, a.L, nb, a.scale, a.logf ? 1 : 0, a.ws,
                       (T*)a.o, a.lse);
    return hipGetLastError();
}

template <typename T, int B>
static hipError_t launch_fwd_f32_d(const FwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 16: return launch_fwd_f32_t<T, B, 16>(a, st);
        case 32: return launch_fwd_f32_t<T, B, 32>(a, st);
        case 64: return launch_fwd_f32_t<T, B, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_fwd_f32_b(const FwdArgs& a, hipStream_t st) {
    switch (a.block) {
        case 16: return launch_fwd_f32_d<T, 16>(a, st);
        case 32: return launch_fwd_f32_d<T, 32>(a, st);
        case 64: return launch_fwd_f32_d<T, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

// The preconditioning step alone (block 64), for the backward pass, which
// differentiates through these per-block products.
template <typename T, int D>
static hipError_t launch_precond_t(const FwdArgs& a, hipStream_t st) {
    const int nb = (a.L + 63) / 64;
    hipLaunchKernelGGL((precond_f32_kernel<T, 64, D>), dim3(a.N * a.H * nb), dim3(256), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.w, a.beta, a.logf, a.L, nb,
                       a.ws);
    return hipGetLastError();
}
template <typename T>
static hipError_t launch_precond_d(const FwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 16: return launch_precond_t<T, 16>(a, st);
        case 32: return launch_precond_t<T, 32>(a, st);
        case 64: return launch_precond_t<T, 64>(a, st);
    }
    return hipErrorInvalidValue;
}
hipError_t launch_precond_f32(const FwdArgs& a, hipStream_t st) {
    return a.bf16 ? launch_precond_d<bf16>(a, st) : launch_precond_d<float>(a, st);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
    return a.bf16 ? launch_fwd_f32_b<bf16>(a, st) : launch_fwd_f32_b<float>(a, st);
}

}  // namespace pa
