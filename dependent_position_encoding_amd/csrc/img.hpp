// img.hpp -- layout of the per-block tile image written by the matrix-core
// preconditioning and read by the forward scan (as its LDS image) and by the
// backward's carried-query chain (its -E operand).  Internal; not in the ABI.
#pragma once
#include <hip/hip_runtime.h>

namespace pa {

// Tile image of one 64-token key block (bytes), identical in HBM and in LDS:
//   [Kright: 64 rows (keys) x D bf16][V^T: D rows x 64 bf16]
//   [-E: D rows (d_out) x D bf16 (d_in)][gate cumsum: 64 float]
// Within a 16-column group every bf16 row stores its columns in MFMA operand
// order (swap23: columns 0-3 and 8-11 in the first 16-byte unit, 4-7 and
// 12-15 in the second).  A row's 16-byte units are XOR-swizzled by row so
// that the 32 rows one operand read touches fall on distinct LDS banks.
template <int D>
struct Img {
    static constexpr int B = 64;
    static constexpr int RB_K = 2 * D, RB_V = 2 * B, RB_E = 2 * D;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = OFF_K + B * RB_K;
    static constexpr int OFF_E = OFF_V + D * RB_V;
    static constexpr int OFF_G = OFF_E + D * RB_E;
    static constexpr int BYTES = OFF_G + B * 4;
};

// Position of 16-byte unit u of row r in a tile with rb-byte rows.
__host__ __device__ constexpr int swz_unit(int r, int u, int rb) {
    return u ^ ((r / (256 / rb > 1 ? 256 / rb : 1)) % (rb / 16));
}
// Byte offset of bf16 column e of row r.
__host__ __device__ constexpr int img_off(int r, int e, int rb) {
    return r * rb + swz_unit(r, e >> 3, rb) * 16 + (e & 7) * 2;
}

}  // namespace pa
