// fwd_bf16.hip -- matrix-core PaTH forward for bf16 inputs (head dim 32, 64).
//
// Citations: [Notes s2.x] = reading-notes page "PaTH Attention:通过累积
// Householder 变换编码位置" (cc.laoqi.cc), section 2.x.
//
// Two kernels per call:
//   precond (one 512-thread workgroup per 64-token block, operands staged in
//   LDS once by direct HBM -> LDS loads): UT solve
//     U = (I + strictLower(diag(beta) W W^T))^{-1} diag(beta)   [Notes s2.6]
//     and the block products of [Notes s2.7]:
//       P = lower(Q W^T) U,  Qleft = Q - P W,  M = strictLower(W K^T),
//       Kright = K - (U M)^T W,  E = W^T U^T W (block transition I - E),
//       Dg = lower(Q K^T) - P M  (in-block logits),
//     on bf16 MFMA with fp32 accumulation; fp32 intermediates are split into
//     bf16 hi + lo parts so these products keep close to fp32 accuracy.
//   scan (one 256-thread workgroup = 4 waves per pair of 64-query blocks,
//     heaviest pairs first): the diagonal block from Dg, then for c = b-1 .. 0
//     the right-to-left scan of [Notes s2.7] with an online softmax.  Each key
//     block's operands (Kright pre-scaled by scale*log2(e), V^T, -E, the gate
//     cumsum) are written by precond as one contiguous "tile image" that is
//     byte-for-byte the LDS layout the scan reads (16-byte units swizzled
//     against bank conflicts), so the scan streams it with direct
//     global->LDS loads, double-buffered.  Everything is kept transposed so
//     that no operand needs a register transpose:
//       S^T     = Kright_c . Qwork^T           (keys x queries)
//       O^T    += V_c^T . P^T                  (d x queries)
//       Qwork^T += (-E_c) . Qwork^T            (d x queries, fp32 state)
//     Each wave owns 32 queries = one C-tile column, so a lane owns a single
//     query: the online-softmax rescale is a per-lane scalar and the row max
//     needs one exchange between the two lane halves.
#include "common.hpp"
#include "kernels.hpp"
#include "img.hpp"
#include "mfma.hpp"

namespace pa {

namespace {

constexpr int kB = 64;       // block size

// Writes a C tile through f(row, col, value).
template <typename F>
__device__ inline void for_tile(const f32x16& acc, int m0, int n0, int lane, F f) {
    const int h = lane >> 5, col = n0 + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) f(m0 + crow(r, h), col, acc[r]);
}

// A C tile of a transposed product, read back row-wise: lane (tile column
// c) holds row n0 + c of the wanted matrix, and registers 4i .. 4i+3 hold its
// columns m0 + 8i + 4h .. +3, handed to f(row, col0, four values) together
// so that they can be stored as one vector.
template <typename F>
__device__ inline void for_tile4(const f32x16& acc, int m0, int n0, int lane, F f) {
    const int h = lane >> 5, row = n0 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        f(row, m0 + 8 * i + 4 * h, f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]});
}
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

// Wait for this wave's outstanding vector-memory loads (including direct
// HBM -> LDS copies); the caller synchronises before reading the LDS.
__device__ inline void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// LDS layout of the preconditioning: no padding; every 16-byte unit of a row
// sits at a row-dependent XOR position so that a row fragment (16 consecutive
// rows, one unit each, per quarter-wave) and a transposed fragment (4 rows x
// 2 adjacent units) both hit 16 distinct 16-byte bank groups.  For 128-byte
// rows the pair index r / 2 is rotated by one bit first: rows r and r + 2
// then differ in the upper unit bits, which a plain r / 2 would not give the
// transposed read.  Byte offsets of element (r, c):
//   natural bf16 tiles [64][D] (rows of RB = 2 D bytes): pb<RB>(r, c);
//   bf16 64 x 64 matrices (one part of a split matrix, 128-byte rows): pb<128>;
//   float 64 x 64 matrices (256-byte rows): pf(r, c).
template <int RB>
__device__ __forceinline__ int psw(int r, int u) {
    if constexpr (RB == 128) {
        const int s = (r >> 1) & 7;
        return u ^ (((s & 1) << 2) | (s >> 1));
    } else if constexpr (RB == 64) {
        return u ^ ((r >> 2) & 3);
    } else {
        return u ^ (r & 15);
    }
}
template <int RB>
__device__ __forceinline__ int pb(int r, int c) {
    return r * RB + (psw<RB>(r, c >> 3) << 4) + ((c & 7) << 1);
}
__device__ __forceinline__ int pf(int r, int c) {
    return r * 256 + (psw<256>(r, c >> 2) << 4) + ((c & 3) << 2);
}
__device__ __forceinline__ float& fat(char* s, int r, int c) {
    return *reinterpret_cast<float*>(s + pf(r, c));
}
constexpr int kSlot = 64 * 64 * 4;          // one float 64 x 64 matrix, or a split one
constexpr int kPart = kSlot / 2;            // the lo part of a split matrix starts here

// Row fragment of a bf16 LDS matrix with RB-byte rows: row r, columns k .. k+7.
template <int RB>
__device__ __forceinline__ bf16x8 frow(const char* t, int r, int k) {
    return *reinterpret_cast<const bf16x8*>(t + pb<RB>(r, k));
}
// Column fragment: rows k .. k+3 and k+GAP .. k+GAP+3 of column c (the lane's
// column; the 16 lanes of a group hold 16 consecutive columns), through
// gfx950's transposing LDS load: in each group of 16 lanes, lane j names 4
// consecutive elements of row k + j/4 starting at column c0 + 4 (j mod 4) (c0
// the group's first column), and lane i receives column c0 + i of those 4
// rows.  GAP = 4 gives rows k .. k+7; GAP = 8 gives the key order of a C tile
// reused as an operand (rows k .. k+3 then k+8 .. k+11).  Every lane of the
// wave must take part.
template <int RB, int GAP = 4>
__device__ __forceinline__ bf16x8 fcol(const char* t, int c, int k) {
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;
    const int j = threadIdx.x & 15, r = k + (j >> 2), c4 = c - j + 4 * (j & 3);
    const bf16x4v a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + pb<RB>(r, c4)));
    const bf16x4v b =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(t + pb<RB>(r + GAP, c4)));
    bf16x8 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[e + 4] = b[e];
    }
    return x;
}
// Eight floats of row r of a float matrix as a bf16 hi + lo operand pair:
// columns c0 + 8h .. +7, or with PERM the columns c0 + swap23(8h + e) that
// match a C tile reused as the other operand; zero when !ok.
template <bool PERM>
__device__ inline void fsplit8(const char* s, int r, int c0, int h, bool ok, bf16x8& hi,
                               bf16x8& lo) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (ok) {
        a = *reinterpret_cast<const f32x4*>(s + pf(r, c0 + (PERM ? 4 * h : 8 * h)));
        b = *reinterpret_cast<const f32x4*>(s + pf(r, c0 + (PERM ? 8 + 4 * h : 8 * h + 4)));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a[e] : b[e - 4];
        hi[e] = (__bf16)x;
        lo[e] = (__bf16)(x - (float)hi[e]);
    }
}
// Four floats as bf16 hi and lo parts of a split 64 x 64 matrix in slot s.
__device__ inline void sput4(char* s, int r, int c, f32x4 v) {
    bf16x4 hi, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
    }
    *reinterpret_cast<bf16x4*>(s + pb<128>(r, c)) = hi;
    *reinterpret_cast<bf16x4*>(s + kPart + pb<128>(r, c)) = lo;
}
// acc += A[m0:+32, kb:ke] B[n0:+32, kb:ke]^T for two split matrices in slots
// (row fragments, hi and lo of both; lo * lo dropped).  [kb, ke) (multiples
// of 16, uniform in the wave) is where both operands can be nonzero: the
// block matrices here are triangular, so whole k-steps are exact zeros.
__device__ inline void mm_ss(f32x16& acc, const char* A, const char* Bn, int m0, int n0, int lane,
                             int kb = 0, int ke = kB) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < kB; k0 += 16) {
        if (k0 < kb || k0 >= ke) continue;
        const int k = k0 + 8 * h;
        const bf16x8 ah = frow<128>(A, m0 + r, k), bh = frow<128>(Bn, n0 + r, k);
        acc = mfma32(ah, frow<128>(Bn + kPart, n0 + r, k), acc);
        acc = mfma32(frow<128>(A + kPart, m0 + r, k), bh, acc);
        acc = mfma32(ah, bh, acc);
    }
}
// acc += A[m0:+32, kb:ke] B[kb:ke, n0:+32] for a split matrix A in a slot and
// the natural [64][D] tile B read down its columns (exact bf16); [kb, ke) as
// for mm_ss.
template <int RB>
__device__ inline void mm_sc(f32x16& acc, const char* A, const char* Bt, int m0, int n0, int lane,
                             int kb = 0, int ke = kB) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < kB; k0 += 16) {
        if (k0 < kb || k0 >= ke) continue;
        const int k = k0 + 8 * h;
        const bf16x8 b = fcol<RB>(Bt, n0 + r, k);
        acc = mfma32(frow<128>(A + kPart, m0 + r, k), b, acc);
        acc = mfma32(frow<128>(A, m0 + r, k), b, acc);
    }
}
// acc += A[m0:+32, 0:D] B[n0:+32, 0:D]^T for two natural [64][D] tiles
// (row fragments, exact bf16).
template <int D>
__device__ inline void mm_nn(f32x16& acc, const char* A, const char* Bn, int m0, int n0, int lane) {
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int k0 = 0; k0 < D; k0 += 16)
        acc = mfma32(frow<2 * D>(A, m0 + r, k0 + 8 * h), frow<2 * D>(Bn, n0 + r, k0 + 8 * h), acc);
}

// Direct HBM -> LDS copy of the block's rows [row0, row0 + 64) of one [L][D]
// bf16 slice into a natural swizzled tile.  A wave fills 1 KB of LDS
// contiguously (16 bytes a lane); each lane fetches the unit that belongs at
// its LDS position.  The buffer resource spans the slice, so rows past its end
// (a ragged last block) read as zeros.
template <int D, int NTH = 512>
__device__ inline void stage_rows(const __bf16* slice_base, int L, int row0, char* dst, int tid) {
    constexpr int RB = 2 * D, UPR = RB / 16, NU = 64 * UPR;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(slice_base), 0, (uint32_t)L * RB, 0x00020000);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
#pragma unroll
    for (int u0 = 0; u0 < NU; u0 += NTH) {
        if (u0 + wave * 64 < NU) {
            const int U = u0 + wave * 64 + lane, r = U / UPR;
            const uint32_t src = (uint32_t)(row0 + r) * RB + psw<RB>(r, U % UPR) * 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(dst + (u0 + wave * 64) * 16), 16, src,
                0, 0, 0);
        }
    }
}

// One 512-thread workgroup (8 waves) per 64-token block.  The block's Q, K,
// W and V rows are copied into LDS once, at the start, with direct
// HBM -> LDS loads; every product then reads its operands from LDS, so a
// workgroup waits on HBM once.  72 KB of LDS (Q, K, W and three 64 x 64
// slots, each a float matrix or a split one) and <= 128 VGPRs let two
// workgroups share a CU and overlap each other's waits.
template <int D>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
precond_mfma_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                    const __bf16* __restrict__ v, const __bf16* __restrict__ w,
                    const float* __restrict__ beta, const float* __restrict__ logf,
                    int L, int nb, float kscale, FwdWs ws) {
    constexpr int B = kB, RB = 2 * D, NTH = 512, DT = D / 32;
    using I = Img<D>;
    // Q, K, W rows (natural) and three slots, each a float or a split matrix:
    //   s0 : G (float)        -> X1 (split)    -> P (split)
    //   s1 : T (float)        -> U^T (split)   -> Y^T (split)
    //   s2 : V (natural bf16) -> T^T (float)   -> M^T (split)
    __shared__ __attribute__((aligned(16))) char sQ[B * RB], sK[B * RB], sW[B * RB];
    __shared__ __attribute__((aligned(16))) char s0[kSlot], s1[kSlot], s2[kSlot];
    __shared__ __attribute__((aligned(16))) float sBeta[B];

    const int blk = blockIdx.x, slice = blk / nb, c = blk % nb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t base = (size_t)slice * L;
    const int row0 = c * B, nvalid = min(B, L - row0);
    char* img = static_cast<char*>(ws.img) + (size_t)blk * I::BYTES;

    // ---- 0. Q, K, W, V rows into LDS (one wait); beta; T = 0; gate cumsum
    stage_rows<D>(q + base * D, L, row0, sQ, tid);
    stage_rows<D>(k + base * D, L, row0, sK, tid);
    stage_rows<D>(w + base * D, L, row0, sW, tid);
    stage_rows<D>(v + base * D, L, row0, s2, tid);
    for (int e = tid; e < B * B / 4; e += NTH)
        *reinterpret_cast<f32x4*>(s1 + 16 * e) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave == 7) {
        sBeta[lane] = lane < nvalid ? beta[base + row0 + lane] : 0.f;
        // in-block inclusive prefix sum of log f (one lane per token)
        float acc = (logf && lane < nvalid) ? logf[base + row0 + lane] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float up = __shfl_up(acc, off, 64);
            if (lane >= off) acc += up;
        }
        ws.gl[(size_t)blk * B + lane] = acc;
        reinterpret_cast<float*>(img + I::OFF_G)[lane] = acc;
        if (lane == 63) ws.tot[blk] = acc;
    }
    wait_loads();
    __syncthreads();

    // ---- 1. V^T with keys in operand order; G = diag(beta) strictLower(WW^T).
    //         Image unit (x, 8 sg) holds keys swap23(8 sg + e): rows 16 (sg/2)
    //         + 4 (sg%2) + {0..3} and those + 8, two transposing reads of V.
    //         Inside each diagonal 16 x 16 block the upper triangle holds G
    //         transposed (entry (k, i), k < i, is G[i][k] = beta_i (w_i . w_k),
    //         WW^T being symmetric), so the forward substitution reads a column
    //         of G as one row; nothing else reads that triangle.
    if (tid < D * 8) {
        const int g = tid >> 4, cg = g % (D / 16), sg = g / (D / 16);
        const int x = 16 * cg + (tid & 15);
        const bf16x8 pk = fcol<RB, 8>(s2, x, 16 * (sg >> 1) + 4 * (sg & 1));
        *reinterpret_cast<bf16x8*>(img + I::OFF_V + img_off(x, 8 * sg, I::RB_V)) = pk;
    }
    if (wave < 3) {
        const int gmt = wave == 0 ? 0 : 1, gnt = wave == 2 ? 1 : 0;   // G's lower tiles
        f32x16 acc = zero16();
        mm_nn<D>(acc, sW, sW, 32 * gnt, 32 * gmt, lane);   // (W W^T)^T tile: lane = row i of G
        for_tile4(acc, 32 * gnt, 32 * gmt, lane, [&](int i, int j0, f32x4 v) {
            const float bi = sBeta[i];
            const bool dblk = (i >> 4) == (j0 >> 4);   // j0 .. j0 + 3 share a 16-block
            const f32x4 bj = *reinterpret_cast<const f32x4*>(sBeta + j0);
            f32x4 g;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                g[e] = i > j0 + e ? bi * v[e] : (dblk && j0 + e > i ? bj[e] * v[e] : 0.f);
            *reinterpret_cast<f32x4*>(s0 + pf(i, j0)) = g;
        });
    }
    __syncthreads();

    // ---- 2. T = (I + G)^{-1}.  Diagonal 16 x 16 blocks by forward
    //         substitution (one column per lane), then the off-diagonal blocks
    //         by doubling on the matrix cores: the inverse of a lower
    //         block-triangular [[A, 0], [C, B]] has off-diagonal block
    //         -B^{-1} C A^{-1}.  Wave w (w = 0, 1) solves diagonal blocks 2w and
    //         2w + 1 (lanes 0-15 and 16-31) and then the 16 -> 32 step of rows
    //         and columns [32 w, 32 w + 32), which needs nothing but its own
    //         results; wave 0 then forms X = G[32:64, 0:32] T[0:32, 0:32] of the
    //         32 -> 64 step.  After the barrier wave 0 finishes with
    //         -T[32:64, 32:64] X.  T is kept in both layouts (T in s1, T^T in s2)
    //         so that every operand is read along LDS rows.  Meanwhile waves 4-7
    //         form X1 = lower(Q W^T) and M^T (M = strictLower(W K^T)) in
    //         registers.
    const int xt = wave - 4, xmt = xt >> 1, xnt = xt & 1;
    const int mrow = lane & 31, hh = lane >> 5;
    f32x16 x1r = zero16(), mtr = zero16(), x32 = zero16();
    if (wave < 2) {
        if (lane < 32) {
            const int o = 16 * (2 * wave + (lane >> 4)), cl = lane & 15;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = i == cl ? 1.f : 0.f;
            // right-looking: once t[kk] is final, t[i] -= G[i][kk] t[kk] for
            // i > kk, with G[o + i][o + kk] read as row kk of the block's upper
            // triangle, 16 bytes (four i) at a time
#pragma unroll
            for (int kk = 0; kk < 15; ++kk)
#pragma unroll
                for (int u = (kk + 1) >> 2; u < 4; ++u) {
                    const f32x4 g4 = *reinterpret_cast<const f32x4*>(s0 + pf(o + kk, o + 4 * u));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * u + e > kk) t[4 * u + e] -= g4[e] * t[kk];
                }
#pragma unroll
            for (int i = 0; i < 16; ++i) fat(s1, o + i, o + cl) = t[i];
            const int tr = o + cl;
            for (int c4 = 0; c4 < o; c4 += 4)
                *reinterpret_cast<f32x4*>(s2 + pf(tr, c4)) = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c4 = 0; c4 < 16; c4 += 4)
                *reinterpret_cast<f32x4*>(s2 + pf(tr, o + c4)) =
                    f32x4{t[c4], t[c4 + 1], t[c4 + 2], t[c4 + 3]};
        }
        // the wave's own LDS writes above are read back below by other lanes:
        // keep the compiler from moving those reads ahead of the writes
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            // 16 -> 32 inside rows/columns [o2, o2 + 32): X = G_10 T_00, Y = -T_11 X
            const int o2 = 32 * wave;
            const bool ok = mrow < 16;
            bf16x8 ah, al, bh, bl;
            fsplit8<false>(s0, o2 + 16 + mrow, o2, hh, ok, ah, al);
            fsplit8<false>(s2, o2 + mrow, o2, hh, ok, bh, bl);
            const f32x16 x = mfma_split(ah, al, bh, bl, zero16());
            // X's C tile (rows 0-15 in registers 0-7) is the B operand of T_11 X
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bh[e] = (__bf16)x[e];
                bl[e] = (__bf16)(x[e] - (float)bh[e]);
            }
            fsplit8<true>(s1, o2 + 16 + mrow, o2 + 16, hh, ok, ah, al);
            const f32x16 y = mfma_split(ah, al, bh, bl, zero16());
            if (ok) {
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int row = crow(r, hh);
                    fat(s1, o2 + 16 + row, o2 + mrow) = -y[r];
                    fat(s2, o2 + mrow, o2 + 16 + row) = -y[r];
                }
            }
        }
        if (wave == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // 32 -> 64, first product: X = G[32:64, 0:32] T[0:32, 0:32]
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 ah, al, bh, bl;
                fsplit8<false>(s0, 32 + mrow, 16 * ks, hh, true, ah, al);
                fsplit8<false>(s2, mrow, 16 * ks, hh, true, bh, bl);
                x32 = mfma_split(ah, al, bh, bl, x32);
            }
        }
    } else if (wave >= 4) {
        if (!(xmt == 0 && xnt == 1))
            mm_nn<D>(x1r, sW, sQ, 32 * xnt, 32 * xmt, lane);     // (Q W^T)^T: lane = row of X1
        if (!(xmt == 1 && xnt == 0))
            mm_nn<D>(mtr, sW, sK, 32 * xnt, 32 * xmt, lane);     // M^T[j][b] = k_j . w_b, lane = j
    }
    __syncthreads();
    if (wave == 0) {
        // 32 -> 64, second product: Y = -T[32:64, 32:64] X
        f32x16 y = zero16();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 ah, al, bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bh[e] = (__bf16)x32[8 * ks + e];
                bl[e] = (__bf16)(x32[8 * ks + e] - (float)bh[e]);
            }
            fsplit8<true>(s1, 32 + mrow, 32 + 16 * ks, hh, true, ah, al);
            y = mfma_split(ah, al, bh, bl, y);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = crow(r, hh);
            fat(s1, 32 + row, mrow) = -y[r];
            fat(s2, mrow, 32 + row) = -y[r];
        }
    }
    __syncthreads();

    // ---- 3. U^T = (T diag(beta))^T from T^T, row by row (over T); X1 to
    //         LDS over G (waves 4-7)
    {
        const int j = tid / 8, c0 = (tid % 8) * 8;
        const float bj = sBeta[j];
        const f32x4 a = *reinterpret_cast<const f32x4*>(s2 + pf(j, c0));
        const f32x4 b = *reinterpret_cast<const f32x4*>(s2 + pf(j, c0 + 4));
        sput4(s1, j, c0, a * bj);
        sput4(s1, j, c0 + 4, b * bj);
    }
    if (wave >= 4)
        for_tile4(x1r, 32 * xnt, 32 * xmt, lane, [&](int i, int j0, f32x4 v) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = j0 + e <= i ? v[e] : 0.f;
            sput4(s0, i, j0, v);
        });
    __syncthreads();

    // ---- 4. M^T to LDS over T^T (waves 4-7); P = X1 U (waves 0-3) and
    //         Y^T (Y = U^T W) on waves 4 .. 4 + 2 DT - 1, both as transposed
    //         products; Kright = K - (U M)^T W = K - M^T Y and E = W^T Y below.
    {
        if (wave >= 4)
            for_tile4(mtr, 32 * xnt, 32 * xmt, lane, [&](int j, int b0, f32x4 v) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = b0 + e > j ? v[e] : 0.f;
                sput4(s2, j, b0, v);
            });
        f32x16 acc = zero16();
        const int mt = wave < 4 ? wave >> 1 : (wave - 4) / 2;
        const int nt = wave < 4 ? wave & 1 : (wave - 4) % 2;
        if (wave < 4) {
            // P^T[a][i] = sum_k U^T[a][k] X1[i][k]
            // X1 lower (c <= i) and U lower (c >= a): c in [32 nt, 32 (mt + 1))
            if (!(mt == 0 && nt == 1)) mm_ss(acc, s1, s0, 32 * nt, 32 * mt, lane, 32 * nt, 32 * (mt + 1));
        } else if (wave < 4 + 2 * DT) {
            // Y[cc][y] = sum_a U^T[cc][a] W[a][y]  (U lower: a >= cc)
            mm_sc<RB>(acc, s1, sW, 32 * nt, 32 * mt, lane, 32 * nt, kB);
        }
        __syncthreads();
        if (wave < 4)
            for_tile4(acc, 32 * nt, 32 * mt, lane, [&](int i, int a0, f32x4 v) { sput4(s0, i, a0, v); });
        else if (wave < 4 + 2 * DT)
            for_tile4(acc, 32 * nt, 32 * mt, lane, [&](int y, int c0, f32x4 v) { sput4(s1, y, c0, v); });
    }
    __syncthreads();

    // ---- 5. outputs, stored straight to HBM, heaviest jobs first:
    //         Dg = lower(Q K^T) - P M (in-block logits), Kright = K - M^T Y
    //         (image, scaled, and its fp32 copy), Qleft = Q - P W,
    //         -E = -W^T Y (image, and E in fp32)
    constexpr int ND = 3, NK = 2 * DT, NQ = 2 * DT, NE = DT * DT, NJ = ND + NK + NQ + NE;
    auto job = [&](int j) {
        f32x16 acc = zero16();
        if (j < ND) {
            const int mt = j == 0 ? 0 : 1, nt = j == 2 ? 1 : 0;
            f32x16 qk = zero16();
            mm_nn<D>(qk, sQ, sK, 32 * mt, 32 * nt, lane);
            // P lower (a <= i), M strictly lower (a > j): a in [32 nt, 32 (mt + 1))
            mm_ss(acc, s0, s2, 32 * mt, 32 * nt, lane, 32 * nt, 32 * (mt + 1));
            float* dg = ws.dg + (size_t)blk * B * B;
            const int h = lane >> 5, jj = 32 * nt + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = 32 * mt + crow(r, h);
                dg[i * B + jj] = jj <= i ? qk[r] - acc[r] : 0.f;
            }
        } else if (j < ND + NK) {
            // transposed: (M^T Y)^T[x][r] = sum_a Y^T[x][a] M^T[r][a], lane = key r
            const int t = j - ND, mt = t / DT, nt = t % DT;
            mm_ss(acc, s1, s2, 32 * nt, 32 * mt, lane, 32 * mt, kB);   // M^T[r][a]: a > r
            float* k32 = ws.k32 ? ws.k32 + (size_t)blk * B * D : nullptr;
            __bf16* kb16 = ws.kb16 ? static_cast<__bf16*>(ws.kb16) + (size_t)blk * B * D : nullptr;
            const float qscale = kscale * kLn2;   // the score scale itself
            for_tile4(acc, 32 * nt, 32 * mt, lane, [&](int r, int x0, f32x4 a) {
                const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(sK + pb<RB>(r, x0));
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = (float)k4[e] - a[e];
                bf16x4 ks;
#pragma unroll
                for (int e = 0; e < 4; ++e) ks[e] = (__bf16)(val[e] * kscale);
                // four consecutive columns stay consecutive under swap23
                *reinterpret_cast<bf16x4*>(img + I::OFF_K + img_off(r, swap23(x0), I::RB_K)) = ks;
                if (k32) *reinterpret_cast<f32x4*>(k32 + r * D + x0) = val;
                if (kb16) {
                    bf16x4 kq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) kq[e] = (__bf16)(val[e] * qscale);
                    *reinterpret_cast<bf16x4*>(kb16 + r * D + x0) = kq;
                }
            });
        } else if (j < ND + NK + NQ) {
            // (P W)[i][x] = sum_a P[i][a] W[a][x]
            const int t = j - ND - NK, mt = t / DT, nt = t % DT;
            mm_sc<RB>(acc, s0, sW, 32 * mt, 32 * nt, lane, 0, 32 * (mt + 1));   // P lower: a <= i
            float* ql = ws.ql + (size_t)blk * B * D;
            for_tile(acc, 32 * mt, 32 * nt, lane, [&](int i, int x, float a) {
                ql[i * D + x] = (float)*reinterpret_cast<const __bf16*>(sQ + pb<RB>(i, x)) - a;
            });
        } else {
            // transposed: E^T[y][x] = sum_a Y^T[y][a] W[a][x], lane = row x of E
            const int t = j - ND - NK - NQ, mt = t / DT, nt = t % DT;
            mm_sc<RB>(acc, s1, sW, 32 * nt, 32 * mt, lane);
            float* e32 = ws.e32 ? ws.e32 + (size_t)blk * D * D : nullptr;
            __bf16* eb16 = ws.eb16 ? static_cast<__bf16*>(ws.eb16) + (size_t)blk * D * D : nullptr;
            for_tile4(acc, 32 * nt, 32 * mt, lane, [&](int x, int y0, f32x4 a) {
                bf16x4 es;
#pragma unroll
                for (int e = 0; e < 4; ++e) es[e] = (__bf16)(-a[e]);
                *reinterpret_cast<bf16x4*>(img + I::OFF_E + img_off(x, swap23(y0), I::RB_E)) = es;
                if (e32) *reinterpret_cast<f32x4*>(e32 + x * D + y0) = a;
                if (eb16) *reinterpret_cast<bf16x4*>(eb16 + x * D + y0) = es;
            });
        }
    };
    for (int j = wave; j < NJ; j += 8) job(j);
}

// ---------------------------------------------------------------------------
// Work order of the scan-shaped kernels: one workgroup per (slice, pair of
// query blocks), pair p covering blocks nb-1-2p and nb-2-2p, so lower p means
// more key blocks.  Slices are taken sg at a time and, inside a group, pairs
// heaviest first with the group's slices interleaved:
//  - the workgroups resident at once share a few slices, so a key block's
//    tile image, streamed by every pair to its left, is read from HBM about
//    once and then hit in cache;
//  - workgroups go to the XCDs round-robin and sg is a multiple of 8, so all
//    workgroups of a slice sit on one XCD and share its L2;
//  - the long pairs start first and the short ones fill the tail.
// Groups of 32 slices balance the short sequences best; from 128 pairs per
// slice on, the scan does better with groups of 8 (fewer slices' images in
// each L2 at a time; measured 3 % at L = 32768, 2-8 % slower below 16384).
constexpr int kSliceGroup = 32;
inline int scan_slice_group(int nb) { return (nb + 1) / 2 >= 128 ? 8 : kSliceGroup; }

__device__ inline void pair_of(int nb, int sg, int& pair, int& slice) {
    const int np = (nb + 1) / 2, nh = gridDim.x / np, span = sg * np;
    const int g = blockIdx.x / span, r = blockIdx.x % span;
    const int sz = min(sg, nh - g * sg);
    pair = r / sz;
    slice = g * sg + r % sz;
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS copy of one tile image through a buffer resource: the
// lanes of a wave fill 1 KB of LDS contiguously (16 bytes each), the image
// offset travels in a scalar register and the lane offset is one VGPR, so the
// stream costs the scan almost no registers.  The caller waits on vmcnt and
// synchronises before reading.
template <int BYTES>
__device__ inline void load_image(__amdgpu_buffer_rsrc_t rsrc, uint32_t src_off, char* dst,
                                  int tid) {
    constexpr int UNITS = BYTES / 16, FULL = UNITS / 256, REM = UNITS % 256;
    // the wave index is uniform; saying so keeps the offsets in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    auto one = [&](int u0) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(dst + u0 * 16), 16,
            (uint32_t)lane * 16, src_off + (uint32_t)u0 * 16, 0, 0);
    };
#pragma unroll
    for (int it = 0; it < FULL; ++it) one((it * 4 + wave) * 64);
    if constexpr (REM > 0) {
        const int u0 = FULL * 256 + wave * 64;
        if (u0 + lane < UNITS) one(u0);
    }
}


template <int D, bool FOX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
scan_mfma_kernel(int L, int nb, int sg, float scale2, FwdWs ws, __bf16* __restrict__ o,
                 float* __restrict__ lse) {
    using I = Img<D>;
    constexpr int B = kB, NT = D / 32, NKC = D / 16;
    // lazy rescale: keep a stale max while every weight stays within 2^8
    constexpr float kSumTau = 256.f;
    __shared__ __attribute__((aligned(16))) char sImg[2][I::BYTES];

    int pair, slice;
    pair_of(nb, sg, pair, slice);
    const int bA = nb - 1 - 2 * pair, bB = bA - 1;          // bB may be -1
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int col = lane & 31;
    const int myb = wave < 2 ? bA : bB;
    const int qloc = 32 * (wave & 1) + col;
    const size_t blk0 = (size_t)slice * nb;
    // this slice's images: nb * I::BYTES bytes (the host keeps that below 4 GiB)
    const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(ws.img) + blk0 * I::BYTES, 0, nb * I::BYTES, 0x00020000);

    load_image<I::BYTES>(irs, (uint32_t)bA * I::BYTES, sImg[0], tid);
    if (bB >= 0) load_image<I::BYTES>(irs, (uint32_t)bB * I::BYTES, sImg[1], tid);

    f32x16 Qw[NT], Ot[NT], S[2];
    float m = 0.f, l = 0.f, gq = 0.f, grun = 0.f;
    // the lane's row of the diagonal tile's in-block logits, fetched with the
    // queries (before the first wait) so that the diagonal step does not wait
    // on HBM a second time
    f32x4 dgr[8];
    if (myb >= 0) {
        const size_t bq = blk0 + myb;
        const float* dgp = ws.dg + (bq * B + qloc) * B;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dgr[4 * mt + i] = *reinterpret_cast<const f32x4*>(dgp + 32 * mt + 8 * i + 4 * h);
    }
    if (myb >= 0) {
        const size_t bq = blk0 + myb;
        const float* qlp = ws.ql + (bq * B + qloc) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            Ot[t] = zero16();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(qlp + 32 * t + 8 * i + 4 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j) Qw[t][4 * i + j] = v4[j];
            }
        }
        if (FOX) gq = ws.gl[bq * B + qloc] * kLog2e;
    }

    // P = 2^S as bf16 operands (keys in the k-slots), S left as it is;
    // returns this lane's share of the row sum of that bf16 P
    auto probs = [&](bf16x8 (&Pb)[4]) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Pb[kc][e] = (__bf16)__builtin_amdgcn_exp2f(S[kc >> 1][8 * (kc & 1) + e]);
        return sum_bf16x32(Pb);
    };
    // O^T += V^T P^T from the V^T image
    auto pv = [&](const char* im, const bf16x8 (&Pb)[4]) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int row = 32 * t + col;
            bf16x8 va[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                va[kc] = *reinterpret_cast<const bf16x8*>(
                    im + I::OFF_V + row * I::RB_V + swz_unit(row, 2 * kc + h, I::RB_V) * 16);
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Ot[t] = mfma32(va[kc], Pb[kc], Ot[t]);
        }
    };

    auto diag = [&](const char* im) {
        const float* gimg = reinterpret_cast<const float*>(im + I::OFF_G);
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k0 = 32 * mt + 8 * i + 4 * h;
                const f32x4 d4 = dgr[4 * mt + i];
                f32x4 g4 = {0.f, 0.f, 0.f, 0.f};
                if (FOX) g4 = *reinterpret_cast<const f32x4*>(gimg + k0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float sv = (k0 + j <= qloc)
                                         ? d4[j] * scale2 + (FOX ? gq - g4[j] * kLog2e : 0.f)
                                         : -INFINITY;
                    S[mt][4 * i + j] = sv;
                    mx = fmaxf(mx, sv);
                }
            }
        mx = pair_max(mx);
        m = mx;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[mt][r] -= m;
        bf16x8 Pb[4];
        l = probs(Pb);   // this half's keys only; the halves are added at the end
        pv(im, Pb);
    };

    // one scan step against key block c (image in buf)
    auto step = [&](const char* im, int c) {
        (void)c;
        const float* gimg = reinterpret_cast<const float*>(im + I::OFF_G);
        // the block's log-f total is its last in-block cumsum entry
        if (FOX) grun += gimg[B - 1];
        const float rowb = gq + grun * kLog2e;
        bf16x8 Qb[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) Qb[kc][e] = (__bf16)Qw[kc >> 1][8 * (kc & 1) + e];
        // S'^T = Kright_c . Qwork^T - m_ref (log2 units), where one more
        // contraction group adds the gate's per-key term -gl_c * log2(e)
        // (hi + lo against ones) and the per-query reference
        // -(m - rowb) (hi + mid + lo, exact to fp32, against ones on the key
        // side), so the softmax needs no per-score subtraction.  Both lane
        // halves (k-slots 0-7 and 8-15) carry the same group with the query
        // side halved (an exact scaling), so the lanes need no half select.
        // The last step (c = 0) also carries the queries across block 0,
        // which is unused but cheaper than a branch.
        const float nref = 0.5f * (rowb - m);
        const __bf16 zb = (__bf16)0.f, ob = (__bf16)1.f, hb = (__bf16)0.5f;
        bf16x8 qside;
        {
            const __bf16 r0 = (__bf16)nref;
            const float t1 = nref - (float)r0;
            const __bf16 r1 = (__bf16)t1;
            const __bf16 r2 = (__bf16)(t1 - (float)r1);
#pragma unroll
            for (int e = 0; e < 8; ++e) qside[e] = zb;
            qside[0] = hb;
            qside[1] = hb;
            qside[2] = r0;
            qside[3] = r1;
            qside[4] = r2;
        }
        // the step's matrix-core phases run at a raised wave priority and its
        // softmax at the normal one, so that a SIMD's arbiter issues the
        // products of one wave while the others do their vector work; P.V,
        // which ends the step, one level above the scores, so that a wave
        // finishing its step goes before one starting the next
        __builtin_amdgcn_s_setprio(1);
        bf16x8 ka[2][NKC];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const int row = 32 * mt + col;
                ka[mt][kc] = *reinterpret_cast<const bf16x8*>(
                    im + I::OFF_K + row * I::RB_K + swz_unit(row, 2 * kc + h, I::RB_K) * 16);
            }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            S[mt] = zero16();
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) S[mt] = mfma32(ka[mt][kc], Qb[kc], S[mt]);
            float gb = 0.f;
            if (FOX) gb = -gimg[32 * mt + col] * kLog2e;
            const __bf16 ghi = (__bf16)gb, glo = (__bf16)(gb - (float)ghi);
            bf16x8 a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = zb;
            a[0] = ghi;
            a[1] = glo;
            a[2] = ob;
            a[3] = ob;
            a[4] = ob;
            S[mt] = mfma32(a, qside, S[mt]);
        }
        // Qwork^T += (-E_c) Qwork^T: carry the queries across block c.  It
        // needs only the bf16 Qwork already formed, so it is issued before the
        // softmax and the matrix cores work while the vector ALUs do exp.
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int row = 32 * t + col;
            bf16x8 ea[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                ea[kc] = *reinterpret_cast<const bf16x8*>(
                    im + I::OFF_E + row * I::RB_E + swz_unit(row, 2 * kc + h, I::RB_E) * 16);
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) Qw[t] = mfma32(ea[kc], Qb[kc], Qw[t]);
        }
        __builtin_amdgcn_s_setprio(0);
        // online softmax with a lazily updated reference max: S' is already
        // relative to m, and the weights are formed against it first.  Their
        // bf16 sum over the lane's keys bounds every weight, so while it stays
        // within kSumTau no weight exceeds it (an overflow shows as inf, and a
        // NaN fails the test too); otherwise the row's max is taken and the
        // reference moved up to it, as a max-first update would do.
        bf16x8 Pb[4];
        float ps = probs(Pb);
        if (__any(!(ps <= kSumTau))) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[mt][r]);
            mx = pair_max(mx);
            const float up = fmaxf(mx, 0.f);
            const float alpha = __builtin_amdgcn_exp2f(-up);
            l *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) Ot[t][r] *= alpha;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[mt][r] -= up;
            m += up;
            ps = probs(Pb);
        }
        l += ps;
        __builtin_amdgcn_s_setprio(2);
        pv(im, Pb);
        __builtin_amdgcn_s_setprio(0);
    };

    wait_loads();
    __syncthreads();
    // phase 1: diagonal of the upper block (waves 0-1)
    if (wave < 2) diag(sImg[0]);
    __syncthreads();
    if (bB >= 0) {
        if (bB > 0) load_image<I::BYTES>(irs, (uint32_t)(bB - 1) * I::BYTES, sImg[0], tid);
        // phase 2: key block bB -- a scan step for the upper block, the
        // diagonal for the lower one
        if (wave < 2) step(sImg[1], bB);
        else diag(sImg[1]);
        wait_loads();
        __syncthreads();
        // two steps per trip, so that each names its buffer statically (the
        // first, key block bA - 2, is in buffer 0) and the operand addresses
        // are fixed offsets
        for (int c = bB - 1; c >= 0; c -= 2) {
            if (c > 0) load_image<I::BYTES>(irs, (uint32_t)(c - 1) * I::BYTES, sImg[1], tid);
            step(sImg[0], c);
            wait_loads();
            __syncthreads();
            if (c == 0) break;
            if (c > 1) load_image<I::BYTES>(irs, (uint32_t)(c - 2) * I::BYTES, sImg[0], tid);
            step(sImg[1], c - 1);
            wait_loads();
            __syncthreads();
        }
    }

    l = pair_sum(l);   // both halves' keys (all lanes take part in the exchange)
    const int pos = myb * B + qloc;
    if (myb >= 0 && pos < L) {
        const float inv = 1.f / l;
        __bf16* op = o + ((size_t)slice * L + pos) * D;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                bf16x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = (__bf16)(Ot[t][4 * i + j] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * t + 8 * i + 4 * h) = pk;
            }
        if (lse && h == 0) lse[(size_t)slice * L + pos] = (m + __log2f(l)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Plain causal softmax attention (every beta = 0, no gate): the baseline the
// PaTH kernels are measured against.  Same workgroup shape, launch order,
// matrix-core formulation and online softmax as scan_mfma_kernel, minus the
// preconditioning and the Qwork transition.  A key block's K and V rows are
// copied HBM -> LDS by direct buffer loads into natural tiles (rows
// XOR-swizzled, double-buffered, 32 KB at d = 64); S^T = K Q^T reads K rows
// along LDS rows against the lane's exact query row, and O^T += V^T P^T reads
// V^T down the tile's columns with the transposing LDS load, in the key order
// of the P operand.  The score scale enters the exponent's fma.
template <int D>
__global__ void __launch_bounds__(256)
causal_mfma_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                   const __bf16* __restrict__ v, int L, int nb, float scale2,
                   __bf16* __restrict__ o, float* __restrict__ lse) {
    constexpr int B = kB, NT = D / 32, NKC = D / 16, RB = 2 * D, TILE = B * RB;
    constexpr float kSumTau = 256.f;   // lazy rescale, as in the scan
    __shared__ __attribute__((aligned(16))) char sKV[2][2 * TILE];   // [buf][K tile | V tile]

    int pair, slice;
    pair_of(nb, kSliceGroup, pair, slice);
    const int bA = nb - 1 - 2 * pair, bB = bA - 1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
    const int col = lane & 31;
    const int myb = wave < 2 ? bA : bB;
    const int qloc = 32 * (wave & 1) + col;
    const size_t sbase = (size_t)slice * L;
    auto load_kv = [&](int c, char* dst) {
        stage_rows<D, 256>(k + sbase * D, L, c * B, dst, tid);
        stage_rows<D, 256>(v + sbase * D, L, c * B, dst + TILE, tid);
    };

    load_kv(bA, sKV[0]);
    if (bB >= 0) load_kv(bB, sKV[1]);

    // the lane's query row, exact (k-slots 8h .. 8h+7 of group kc are
    // elements 16 kc + 8h .. +7, the order the K row fragments take)
    f32x16 Ot[NT], S[2];
    bf16x8 Qb[NKC];
    float m = 0.f, l = 0.f;
    {
        const int pos = myb >= 0 ? min(myb * B + qloc, L - 1) : 0;
        const __bf16* qp = q + (sbase + pos) * D;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) Qb[kc] = *reinterpret_cast<const bf16x8*>(qp + 16 * kc + 8 * h);
#pragma unroll
        for (int t = 0; t < NT; ++t) Ot[t] = zero16();
    }

    auto scores = [&](const char* t) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            S[mt] = zero16();
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                S[mt] = mfma32(frow<RB>(t, 32 * mt + col, 16 * kc + 8 * h), Qb[kc], S[mt]);
        }
    };
    // P = 2^(scale2 S - m) as bf16 operands, S left as it is; returns this
    // lane's share of the row sum of that bf16 P
    auto probs = [&](bf16x8 (&Pb)[4]) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                Pb[kc][e] = (__bf16)__builtin_amdgcn_exp2f(
                    __builtin_fmaf(S[kc >> 1][8 * (kc & 1) + e], scale2, -m));
        return sum_bf16x32(Pb);
    };
    // O^T += V^T P^T; the P operand's k-slots of group kc hold keys
    // 16 kc + 4h .. +3 and 16 kc + 8 + 4h .. +3 (the C tile's row order)
    auto pv = [&](const char* t, const bf16x8 (&Pb)[4]) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                Ot[tt] = mfma32(fcol<RB, 8>(t + TILE, 32 * tt + col, 16 * kc + 4 * h), Pb[kc], Ot[tt]);
    };
    auto row_max = [&]() {
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[mt][r]);
        return pair_max(mx) * scale2;
    };
    auto diag = [&](const char* t) {
        scores(t);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (32 * mt + crow(r, h) > qloc) S[mt][r] = -INFINITY;
        m = row_max();
        bf16x8 Pb[4];
        l = probs(Pb);   // this half's keys only; the halves are added at the end
        pv(t, Pb);
    };
    // the weights against the stale reference first; the row's max is taken
    // only when their bf16 sum over the lane's keys exceeds kSumTau (which
    // bounds every weight; an overflow shows as inf)
    auto step = [&](const char* t) {
        scores(t);
        bf16x8 Pb[4];
        float ps = probs(Pb);
        if (__any(!(ps <= kSumTau))) {
            const float mn = fmaxf(m, row_max());
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            l *= alpha;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int r = 0; r < 16; ++r) Ot[tt][r] *= alpha;
            m = mn;
            ps = probs(Pb);
        }
        l += ps;
        pv(t, Pb);
    };

    wait_loads();
    __syncthreads();
    if (wave < 2) diag(sKV[0]);
    __syncthreads();
    if (bB >= 0) {
        if (bB > 0) load_kv(bB - 1, sKV[0]);
        if (wave < 2) step(sKV[1]);
        else diag(sKV[1]);
        wait_loads();
        __syncthreads();
        // two steps per trip: the first, key block bA - 2, is in buffer 0
        for (int c = bB - 1; c >= 0; c -= 2) {
            if (c > 0) load_kv(c - 1, sKV[1]);
            step(sKV[0]);
            wait_loads();
            __syncthreads();
            if (c == 0) break;
            if (c > 1) load_kv(c - 2, sKV[0]);
            step(sKV[1]);
            wait_loads();
            __syncthreads();
        }
    }

    l = pair_sum(l);   // both halves' keys (all lanes take part in the exchange)
    const int pos = myb * B + qloc;
    if (myb >= 0 && pos < L) {
        const float inv = 1.f / l;
        __bf16* op = o + (sbase + pos) * D;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
                bf16x4 pk;
#pragma unroll
                for (int j = 0; j < 4; ++j) pk[j] = (__bf16)(Ot[tt][4 * i + j] * inv);
                *reinterpret_cast<bf16x4*>(op + 32 * tt + 8 * i + 4 * h) = pk;
            }
        if (lse && h == 0) lse[sbase + pos] = (m + __log2f(l)) * kLn2;
    }
}

template <int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
    const int nb = (a.L + kB - 1) / kB;
    const int nblk = a.N * a.H * nb;
    const float scale2 = a.scale * kLog2e;
    hipLaunchKernelGGL((precond_mfma_kernel<D>), dim3(nblk), dim3(512), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.w, a.beta, a.logf, a.L, nb, scale2, a.ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[1], st)) != hipSuccess) return e;
    const int ngrid = a.N * a.H * ((nb + 1) / 2);
    if (a.logf)
        hipLaunchKernelGGL((scan_mfma_kernel<D, true>), dim3(ngrid), dim3(256), 0, st, a.L, nb,
                           scan_slice_group(nb),
                           scale2, a.ws, (__bf16*)a.o, a.lse);
    else
        hipLaunchKernelGGL((scan_mfma_kernel<D, false>), dim3(ngrid), dim3(256), 0, st, a.L, nb,
                           scan_slice_group(nb),
                           scale2, a.ws, (__bf16*)a.o, a.lse);
    return hipGetLastError();
}

}  // namespace

bool fwd_bf16_supported(int d, int block) { return (d == 32 || d == 64) && block == 64; }

size_t fwd_bf16_image_bytes(int d) { return d == 32 ? Img<32>::BYTES : Img<64>::BYTES; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
    switch (a.d) {
        case 32: return launch_t<32>(a, st);
        case 64: return launch_t<64>(a, st);
    }
    return hipErrorInvalidValue;
}

// The preconditioning alone, for the backward pass: besides the images it
// writes ql, dg, gl, tot and, with ws.k32 / ws.e32 set, Kright and E in fp32.
hipError_t launch_precond_bf16(const FwdArgs& a, hipStream_t st) {
    const int nb = (a.L + kB - 1) / kB, nblk = a.N * a.H * nb;
    const float scale2 = a.scale * kLog2e;
    switch (a.d) {
        case 32:
            hipLaunchKernelGGL((precond_mfma_kernel<32>), dim3(nblk), dim3(512), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                               (const __bf16*)a.w, a.beta, a.logf, a.L, nb, scale2, a.ws);
            break;
        case 64:
            hipLaunchKernelGGL((precond_mfma_kernel<64>), dim3(nblk), dim3(512), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                               (const __bf16*)a.w, a.beta, a.logf, a.L, nb, scale2, a.ws);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool causal_supported(int d, bool bf16) { return bf16 && (d == 32 || d == 64); }

hipError_t launch_causal(const FwdArgs& a, hipStream_t st) {
    const int nb = (a.L + kB - 1) / kB;
    const int ngrid = a.N * a.H * ((nb + 1) / 2);
    const float scale2 = a.scale * kLog2e;
    switch (a.d) {
        case 32:
            hipLaunchKernelGGL((causal_mfma_kernel<32>), dim3(ngrid), dim3(256), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.L,
                               nb, scale2, (__bf16*)a.o, a.lse);
            break;
        case 64:
            hipLaunchKernelGGL((causal_mfma_kernel<64>), dim3(ngrid), dim3(256), 0, st,
                               (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.L,
                               nb, scale2, (__bf16*)a.o, a.lse);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
