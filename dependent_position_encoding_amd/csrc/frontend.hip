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
// Two kernels, both on the matrix cores:
//   project: P = x [Wd; ub; uf]^T, one GEMM over the input width Dm, fp32
//            [N*L, Rp] in the workspace (Rp = R + H (+ H) rounded up to 32).
//   finish:  per (token tile of 32, head): c^T = sum_(tau, r) A[ch][(tau, r)]
//            P[t - tau][r] with A[ch][(tau, r)] = kc[ch][tau] Wu[ch][r] -- the
//            convolution folded into the contraction, so the three shifted
//            rows of P are just more k-steps -- then the norm over the head's
//            channels (a lane owns one token: a sum over its registers and one
//            exchange with the other lane half), beta and log f from P's gate
//            columns.
// Products are formed transposed (weights as the A operand) so that a lane
// ends up owning one token and stores four consecutive outputs at a time.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace pa {

namespace {

// 8 consecutive inputs as bf16 operand parts: bf16 data is exact (one part),
// fp32 data is split three ways (hi + mid + lo) for fp32 accuracy.
__device__ inline void ld8_parts(const bf16* p, bool ok, bf16x8 (&o)[3]) {
    if (ok) {
        o[0] = *reinterpret_cast<const bf16x8*>(p);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[0][e] = (__bf16)0.f;
    }
}
__device__ inline void ld8_parts(const float* p, bool ok, bf16x8 (&o)[3]) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (ok) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a[e] : b[e - 4];
        o[0][e] = (__bf16)x;
        const float r = x - (float)o[0][e];
        o[1][e] = (__bf16)r;
        o[2][e] = (__bf16)(r - (float)o[1][e]);
    }
}

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

// P^T tile (32 columns of [Wd; ub; uf] x 32 tokens) per wave, contracted
// over Dm in steps of 16.
template <typename T>
__global__ void __launch_bounds__(256)
param_project_kernel(const T* __restrict__ x, const T* __restrict__ Wd, const T* __restrict__ ub,
                     const T* __restrict__ uf, int M, int Dm, int R, int H, int Rp,
                     float* __restrict__ P) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
    const int ntn = Rp / 32, ntt = (M + 31) / 32;
    const int tile = blockIdx.x * 4 + wave;
    if (tile >= ntt * ntn) return;
    const int tt = tile / ntn, jt = tile % ntn;
    const int j = 32 * jt + c, t = 32 * tt + c;
    const T* wrow = j < R                   ? Wd + (size_t)j * Dm
                    : j < R + H             ? ub + (size_t)(j - R) * Dm
                    : (uf && j < R + 2 * H) ? uf + (size_t)(j - R - H) * Dm
                                            : nullptr;
    const T* xrow = x + (size_t)(t < M ? t : 0) * Dm;
    const bool wok = wrow != nullptr, xok = t < M;
    f32x16 acc = zero16();
#pragma unroll 4
    for (int k0 = 0; k0 < Dm; k0 += 16) {
        bf16x8 a[3], b[3];
        ld8_parts(wrow + k0 + 8 * h, wok, a);
        ld8_parts(xrow + k0 + 8 * h, xok, b);
        acc = mfma_parts<T>(a, b, acc);
    }
    if (t < M) {
        float* out = P + (size_t)t * Rp + 32 * jt + 4 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<f32x4*>(out + 8 * i) =
                f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    }
}

// 8 consecutive values as float (16- or 32-byte aligned loads)
__device__ inline void ld8f(const bf16* p, float (&v)[8]) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}
__device__ inline void ld8f(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[e + 4] = b[e];
    }
}

__device__ inline float sigmoid2(float z) { return 2.f / (1.f + __expf(-z)); }
__device__ inline float log_sigmoid(float z) {
    return z >= 0.f ? -log1pf(__expf(-z)) : z - log1pf(__expf(z));
}

// One wave per (sequence n, 32 tokens, head): c^T (D channels x 32 tokens).
template <typename T, int D>
__global__ void __launch_bounds__(256)
param_finish_kernel(const float* __restrict__ P, const T* __restrict__ Wu,
                    const float* __restrict__ kc, const float* __restrict__ bb,
                    const float* __restrict__ bf, int N, int L, int R, int H, int Rp,
                    T* __restrict__ w, float* __restrict__ beta, float* __restrict__ logf) {
    constexpr int CT = D < 32 ? 1 : D / 32;   // 32-channel tiles per head
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
    const int ntt = (L + 31) / 32;
    const int job = blockIdx.x * 4 + wave;
    if (job >= N * ntt * H) return;
    const int hh = job % H, tt = (job / H) % ntt, n = job / (H * ntt);
    const int t = 32 * tt + c;                 // this lane's token (B-operand column)
    const size_t row = (size_t)n * L + t;
    f32x16 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = zero16();
    for (int tau = 0; tau < 3; ++tau) {
        const bool pok = t < L && t - tau >= 0;
        const float* prow = P + (pok ? row - tau : 0) * Rp;
        for (int r0 = 0; r0 < R; r0 += 16) {
            bf16x8 bh, bl;
            {
                f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
                if (pok) {
                    a = *reinterpret_cast<const f32x4*>(prow + r0 + 8 * h);
                    b = *reinterpret_cast<const f32x4*>(prow + r0 + 8 * h + 4);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = e < 4 ? a[e] : b[e - 4];
                    bh[e] = (__bf16)v;
                    bl[e] = (__bf16)(v - (float)bh[e]);
                }
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const int chl = 32 * ct + c;              // channel within the head
                const bool cok = chl < D;
                const int ch = hh * D + (cok ? chl : 0);
                const float k = cok ? kc[(size_t)ch * 3 + tau] : 0.f;
                float wv[8];
                ld8f(Wu + (size_t)ch * R + r0 + 8 * h, wv);
                bf16x8 ah, al;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = k * wv[e];
                    ah[e] = (__bf16)v;
                    al[e] = (__bf16)(v - (float)ah[e]);
                }
                acc[ct] = mfma_split(ah, al, bh, bl, acc[ct]);
            }
        }
    }
    // lane: token t; registers 4i..4i+3 of tile ct: channels 32ct + 8i + 4h + j
    float ss = 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss += acc[ct][r] * acc[ct][r];
    ss = pair_sum(ss);
    const float inv = ss > 0.f ? rsqrtf(ss) : 0.f;
    if (t < L) {
        T* wo = w + (((size_t)n * H + hh) * L + t) * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * ct + 8 * i + 4 * h;
                if (ch0 < D) {
                    if constexpr (sizeof(T) == 2) {
                        typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                        bf16x4 pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(acc[ct][4 * i + e] * inv);
                        *reinterpret_cast<bf16x4*>(wo + ch0) = pk;
                    } else {
                        f32x4 pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pk[e] = acc[ct][4 * i + e] * inv;
                        *reinterpret_cast<f32x4*>(wo + ch0) = pk;
                    }
                }
            }
        if (h == 0) {
            const size_t o = ((size_t)n * H + hh) * L + t;
            beta[o] = sigmoid2(P[row * Rp + R + hh] + bb[hh]);
            if (logf) logf[o] = log_sigmoid(P[row * Rp + R + H + hh] + bf[hh]);
        }
    }
}

template <typename T, int D>
hipError_t finish_t(const ParamArgs& a, hipStream_t st) {
    const int ntt = (a.L + 31) / 32;
    const long jobs = (long)a.N * ntt * a.H;
    hipLaunchKernelGGL((param_finish_kernel<T, D>), dim3((unsigned)((jobs + 3) / 4)), dim3(256), 0,
                       st, a.P, (const T*)a.Wu, a.kc, a.bb, a.bf, a.N, a.L, a.R, a.H, a.Rp,
                       (T*)a.w, a.beta, a.logf);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_param_t(const ParamArgs& a, hipStream_t st) {
    const long M = (long)a.N * a.L;
    const long tiles = ((M + 31) / 32) * (a.Rp / 32);
    hipLaunchKernelGGL((param_project_kernel<T>), dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
                       st, (const T*)a.x, (const T*)a.Wd, (const T*)a.ub, (const T*)a.uf,
                       (int)M, a.Dm, a.R, a.H, a.Rp, a.P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (a.d) {
        case 16: return finish_t<T, 16>(a, st);
        case 32: return finish_t<T, 32>(a, st);
        case 64: return finish_t<T, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int param_columns(int R, int H, bool gate) { return (R + H * (gate ? 2 : 1) + 31) / 32 * 32; }

hipError_t launch_param(const ParamArgs& a, hipStream_t st) {
    return a.bf16 ? launch_param_t<bf16>(a, st) : launch_param_t<float>(a, st);
}

}  // namespace pa
