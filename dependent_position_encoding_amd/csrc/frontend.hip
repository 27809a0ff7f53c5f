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

// The projection GEMM.  One 128-thread workgroup (2 waves) per 64 tokens and
// up to kProjTiles column tiles.  The input width Dm is walked in chunks of
// 64: both operands' chunks are loaded with consecutive lanes along a row
// (rows of x and of the weights lie Dm elements apart, so a lane-per-row
// pattern would put every lane of an instruction on the same memory channel)
// into LDS, double-buffered, the next chunk held in registers meanwhile.
// Each wave forms 32 tokens x (32 kProjTiles) columns of P^T, one x fragment
// serving all its column tiles.
constexpr int kProjTiles = 4;
constexpr int kProjK = 64;                  // chunk of the contraction

template <typename T>
struct ProjLds {
    static constexpr int RS = kProjK * (int)sizeof(T) + 16;    // row stride, bytes (padded)
    static constexpr int XB = 64 * RS;                          // x chunk: 64 tokens
    static constexpr int WB = 32 * kProjTiles * RS;             // weight chunk
    static constexpr int STAGE = XB + WB;
    static constexpr int UPR = kProjK * (int)sizeof(T) / 16;   // 16-byte units per row
};

template <typename T>
__global__ void __launch_bounds__(128)
param_project_kernel(const T* __restrict__ x, const T* __restrict__ Wd, const T* __restrict__ ub,
                     const T* __restrict__ uf, int M, int Dm, int R, int H, int Rp,
                     float* __restrict__ P) {
    using S = ProjLds<T>;
    __shared__ __attribute__((aligned(16))) char lds[2][S::STAGE];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
    const int ntn = Rp / 32, ngroups = (ntn + kProjTiles - 1) / kProjTiles;
    const int tb = blockIdx.x / ngroups, jg = blockIdx.x % ngroups;
    const int t0 = 64 * tb, jt0 = jg * kProjTiles, nt = min(kProjTiles, ntn - jt0);
    const int nrows_w = 32 * nt;
    // row pointers of the weights behind P's columns (NULL rows are padding)
    auto wrow_of = [&](int j) -> const T* {
        if (j < R) return Wd + (size_t)j * Dm;
        if (j < R + H) return ub + (size_t)(j - R) * Dm;
        if (uf && j < R + 2 * H) return uf + (size_t)(j - R - H) * Dm;
        return nullptr;
    };
    // this thread's 16-byte units of a chunk: x first (64 rows), then weights
    constexpr int UPR = S::UPR;
    const int xunits = 64 * UPR, units = xunits + nrows_w * UPR;
    constexpr int MAXU = (64 + 32 * kProjTiles) * UPR / 128 + 1;
    const char* src[MAXU];
    int dst[MAXU];
    bool live[MAXU];
#pragma unroll
    for (int i = 0; i < MAXU; ++i) {
        const int u = tid + 128 * i;
        live[i] = u < units;
        const int uu = live[i] ? u : 0;
        const bool isx = uu < xunits;
        const int rr = isx ? uu / UPR : (uu - xunits) / UPR, ux = uu % UPR;
        const T* base = nullptr;
        if (isx) {
            base = t0 + rr < M ? x + (size_t)(t0 + rr) * Dm : nullptr;
        } else {
            base = wrow_of(32 * jt0 + rr);
        }
        src[i] = base ? reinterpret_cast<const char*>(base) + 16 * ux : nullptr;
        dst[i] = (isx ? 0 : S::XB) + rr * S::RS + 16 * ux;
    }
    u32x4 pre[MAXU];
    const int nchunks = Dm / kProjK + (Dm % kProjK ? 1 : 0);
    auto fetch = [&](int kc) {
        const int kbytes = kc * kProjK * (int)sizeof(T);
#pragma unroll
        for (int i = 0; i < MAXU; ++i) {
            const bool ok = live[i] && src[i] && kbytes + (dst[i] % S::RS) < Dm * (int)sizeof(T);
            pre[i] = ok ? *reinterpret_cast<const u32x4*>(src[i] + kbytes) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < MAXU; ++i)
            if (live[i]) *reinterpret_cast<u32x4*>(lds[buf] + dst[i]) = pre[i];
    };
    f32x16 acc[kProjTiles];
#pragma unroll
    for (int q = 0; q < kProjTiles; ++q) acc[q] = zero16();
    fetch(0);
    stash(0);
    __syncthreads();
    for (int kc = 0; kc < nchunks; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nchunks) fetch(kc + 1);
        const char* xs = lds[buf] + (32 * wave + c) * S::RS;
#pragma unroll
        for (int ks = 0; ks < kProjK / 16; ++ks) {
            const int kb = (16 * ks + 8 * h) * (int)sizeof(T);
            bf16x8 b[3];
            ld8_parts(reinterpret_cast<const T*>(xs + kb), true, b);
#pragma unroll
            for (int q = 0; q < kProjTiles; ++q) {
                if (q < nt) {
                    bf16x8 a[3];
                    ld8_parts(reinterpret_cast<const T*>(lds[buf] + S::XB + (32 * q + c) * S::RS + kb),
                              true, a);
                    acc[q] = mfma_parts<T>(a, b, acc[q]);
                }
            }
        }
        if (kc + 1 < nchunks) stash(buf ^ 1);
        __syncthreads();
    }
    const int t = t0 + 32 * wave + c;
    if (t < M) {
        // lane: token t; registers 4i..4i+3 of tile q: columns 32(jt0+q) + 8i + 4h
#pragma unroll
        for (int q = 0; q < kProjTiles; ++q) {
            if (q < nt) {
                float* out = P + (size_t)t * Rp + 32 * (jt0 + q) + 4 * h;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<f32x4*>(out + 8 * i) =
                        f32x4{acc[q][4 * i], acc[q][4 * i + 1], acc[q][4 * i + 2], acc[q][4 * i + 3]};
            }
        }
    }
}

__device__ inline float sigmoid2(float z) { return 2.f / (1.f + __expf(-z)); }
__device__ inline float log_sigmoid(float z) {
    return z >= 0.f ? -log1pf(__expf(-z)) : z - log1pf(__expf(z));
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

// One workgroup per (sequence n, 32 tokens, group of kHeadsPerGroup heads):
// the tile's rows of P (two more before it for the convolution) are split
// once into bf16 hi + lo in LDS; the four waves then take the group's heads
// in turn, each forming c^T (D channels x 32 tokens) = sum over taps tau and
// rank steps of (kc[:, tau] Wu) P_{t - tau}^T.  One load of a Wu fragment
// serves the three taps, a head's taps are loaded before its products, and
// the next rank step's Wu fragment is in flight while the current one is used.
constexpr int kHeadsPerGroup = 8;
constexpr int kOutPad = 8;    // LDS row padding (elements) of a wave's output tile

// Dynamic LDS of the finish kernel: the staged P rows (hi and lo, 34 rows of
// R + 8 bf16) and four per-wave output tiles (32 rows of D + kOutPad).
template <typename T, int D>
struct FinishLds {
    __host__ __device__ static size_t out_offset(int R) { return ((size_t)2 * 34 * (R + 8) * 2 + 15) / 16 * 16; }
    __host__ __device__ static size_t bytes(int R) { return out_offset(R) + (size_t)4 * 32 * (D + kOutPad) * sizeof(T); }
};

template <typename T, int D>
__global__ void __launch_bounds__(256)
param_finish_kernel(const float* __restrict__ P, const T* __restrict__ Wu,
                    const float* __restrict__ kc, const float* __restrict__ bb,
                    const float* __restrict__ bf, int N, int L, int R, int H, int Rp,
                    T* __restrict__ w, float* __restrict__ beta, float* __restrict__ logf) {
    constexpr int CT = D < 32 ? 1 : D / 32;   // 32-channel tiles per head
    // dynamic LDS, sized for R at launch (FinishLds)
    extern __shared__ __attribute__((aligned(16))) char dyn[];
    const int PS = R + 8;                      // row stride (bf16) of the staged P
    __bf16* sPh = reinterpret_cast<__bf16*>(dyn);
    __bf16* sPl = sPh + 34 * PS;
    T* sOutAll = reinterpret_cast<T*>(dyn + FinishLds<T, D>::out_offset(R));
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5, c = lane & 31;
    const int ntt = (L + 31) / 32, nhg = (H + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const int hg = blockIdx.x % nhg, tt = (blockIdx.x / nhg) % ntt, n = blockIdx.x / (nhg * ntt);
    const int t0 = 32 * tt;
    const int h_end = min(H, (hg + 1) * kHeadsPerGroup);
    // stage P rows t0-2 .. t0+31 (zero outside [0, L)), split into hi + lo
    const int upr = R / 4;
    for (int u = tid; u < 34 * upr; u += 256) {
        const int rr = u / upr, c4 = (u % upr) * 4, t = t0 - 2 + rr;
        const bool tok = t >= 0 && t < L;
        // unconditional load (clamped row), zeroed after: static wait counts
        f32x4 v = *reinterpret_cast<const f32x4*>(P + ((size_t)n * L + (tok ? t : 0)) * Rp + c4);
        if (!tok) v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 hi = (__bf16)v[e];
            sPh[rr * PS + c4 + e] = hi;
            sPl[rr * PS + c4 + e] = (__bf16)(v[e] - (float)hi);
        }
    }
    __syncthreads();
    // bf16 weights: the group's taps, transposed to [tau][channel], for the
    // combination after the products
    __shared__ __attribute__((aligned(16))) float sKc[3][kHeadsPerGroup * D];
    if constexpr (sizeof(T) == 2) {
        const int hg0 = hg * kHeadsPerGroup;
        for (int e = tid; e < 3 * kHeadsPerGroup * D; e += 256) {
            const int tau = e / (kHeadsPerGroup * D), cl = e % (kHeadsPerGroup * D);
            const int chg = hg0 * D + cl;
            sKc[tau][cl] = chg < H * D ? kc[(size_t)chg * 3 + tau] : 0.f;
        }
        __syncthreads();
    }
    const int t = t0 + c;                      // this lane's token (B-operand column)
    const size_t row = (size_t)n * L + t;
    for (int hh = hg * kHeadsPerGroup + wave; hh < h_end; hh += 4) {
        f32x16 acc[CT];
        if constexpr (sizeof(T) == 2) {
            // y_tau = Wu P_{t-tau}^T with the exact bf16 Wu as the A operand
            // (P split hi + lo), then c = sum_tau kc[:, tau] * y_tau
            f32x16 y[3][CT];
#pragma unroll
            for (int tau = 0; tau < 3; ++tau)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) y[tau][ct] = zero16();
            for (int r0 = 0; r0 < R; r0 += 16) {
                bf16x8 wa[CT];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const int chl = 32 * ct + c;
                    wa[ct] = *reinterpret_cast<const bf16x8*>(
                        Wu + (size_t)(hh * D + (chl < D ? chl : 0)) * R + r0 + 8 * h);
                    if (chl >= D) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) wa[ct][e] = (__bf16)0.f;
                    }
                }
#pragma unroll
                for (int tau = 0; tau < 3; ++tau) {
                    const int pr = (c + 2 - tau) * PS + r0 + 8 * h;   // row t - tau
                    const bf16x8 bh = *reinterpret_cast<const bf16x8*>(sPh + pr);
                    const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sPl + pr);
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        y[tau][ct] = mfma32(wa[ct], bl, y[tau][ct]);
                        y[tau][ct] = mfma32(wa[ct], bh, y[tau][ct]);
                    }
                }
            }
            const int cl0 = (hh - hg * kHeadsPerGroup) * D;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch0 = 32 * ct + 8 * i + 4 * h;
                    f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, k2 = k0;
                    if (ch0 < D) {
                        k0 = *reinterpret_cast<const f32x4*>(&sKc[0][cl0 + ch0]);
                        k1 = *reinterpret_cast<const f32x4*>(&sKc[1][cl0 + ch0]);
                        k2 = *reinterpret_cast<const f32x4*>(&sKc[2][cl0 + ch0]);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[ct][4 * i + j] = k0[j] * y[0][ct][4 * i + j] + k1[j] * y[1][ct][4 * i + j] +
                                             k2[j] * y[2][ct][4 * i + j];
                }
            }
        } else {
        int ch[CT];
        float kt[CT][3], wnext[CT][8];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            acc[ct] = zero16();
            const int chl = 32 * ct + c;              // channel within the head
            const bool cok = chl < D;
            ch[ct] = hh * D + (cok ? chl : 0);
#pragma unroll
            for (int tau = 0; tau < 3; ++tau) {
                const float kv = kc[(size_t)ch[ct] * 3 + tau];
                kt[ct][tau] = cok ? kv : 0.f;
            }
            ld8f(Wu + (size_t)ch[ct] * R + 8 * h, wnext[ct]);
        }
        for (int r0 = 0; r0 < R; r0 += 16) {
            float wcur[CT][8];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int e = 0; e < 8; ++e) wcur[ct][e] = wnext[ct][e];
            {
                // the next rank step's fragment (the last step reloads its own)
                const int rn = r0 + 16 < R ? r0 + 16 : r0;
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) ld8f(Wu + (size_t)ch[ct] * R + rn + 8 * h, wnext[ct]);
            }
#pragma unroll
            for (int tau = 0; tau < 3; ++tau) {
                const int pr = (c + 2 - tau) * PS + r0 + 8 * h;   // row t - tau
                const bf16x8 bh = *reinterpret_cast<const bf16x8*>(sPh + pr);
                const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sPl + pr);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    bf16x8 ah, al;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float v = kt[ct][tau] * wcur[ct][e];
                        ah[e] = (__bf16)v;
                        al[e] = (__bf16)(v - (float)ah[e]);
                    }
                    acc[ct] = mfma_split(ah, al, bh, bl, acc[ct]);
                }
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
        // the 32 x D tile of w goes out through this wave's LDS tile, so that
        // the stores write whole rows (16 bytes per lane along a row)
        T* sOut = sOutAll + wave * 32 * (D + kOutPad);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch0 = 32 * ct + 8 * i + 4 * h;
                if (ch0 < D) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sOut[c * (D + kOutPad) + ch0 + e] = from_f32<T>(acc[ct][4 * i + e] * inv);
                }
            }
        __builtin_amdgcn_wave_barrier();
        {
            constexpr int UPR = D * (int)sizeof(T) / 16;          // 16-byte units per row
            const int nrows = min(32, L - t0);
            T* wbase = w + (((size_t)n * H + hh) * L + t0) * D;
            for (int u = lane; u < nrows * UPR; u += 64) {
                const int rr = u / UPR, x = u % UPR;
                const unsigned* src = reinterpret_cast<const unsigned*>(
                    reinterpret_cast<const char*>(sOut + rr * (D + kOutPad)) + 16 * x);
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = src[e];
                reinterpret_cast<u32x4*>(wbase + (size_t)rr * D)[x] = v;
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (t < L) {
            if (h == 0) {
                const size_t o = ((size_t)n * H + hh) * L + t;
                beta[o] = sigmoid2(P[row * Rp + R + hh] + bb[hh]);
                if (logf) logf[o] = log_sigmoid(P[row * Rp + R + H + hh] + bf[hh]);
            }
        }
    }
}

template <typename T, int D>
hipError_t finish_t(const ParamArgs& a, hipStream_t st) {
    const int ntt = (a.L + 31) / 32, nhg = (a.H + kHeadsPerGroup - 1) / kHeadsPerGroup;
    const size_t lds = FinishLds<T, D>::bytes(a.R);
    if (lds > 65536) {   // beyond the default dynamic LDS limit (fp32 with a large rank)
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&param_finish_kernel<T, D>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((param_finish_kernel<T, D>), dim3((unsigned)((long)a.N * ntt * nhg)),
                       dim3(256), lds, st, a.P, (const T*)a.Wu, a.kc,
                       a.bb, a.bf, a.N, a.L, a.R, a.H, a.Rp, (T*)a.w, a.beta, a.logf);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_param_t(const ParamArgs& a, hipStream_t st) {
    const long M = (long)a.N * a.L;
    const long ngroups = (a.Rp / 32 + kProjTiles - 1) / kProjTiles;
    hipLaunchKernelGGL((param_project_kernel<T>), dim3((unsigned)(((M + 63) / 64) * ngroups)),
                       dim3(128), 0,
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
