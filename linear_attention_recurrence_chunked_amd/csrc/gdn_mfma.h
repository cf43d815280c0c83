// gdn_mfma.h -- 16x16 matrix-core (MFMA) tile helpers for gfx950.
//
// Every product in the chunk kernel is built from 16x16 output tiles. Both
// operands are read from LDS buffers stored "contraction-contiguous": the A
// operand as A[m][k] and the B operand as Bt[n][k] (k contiguous), so one
// fragment loader serves both sides.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (and of the fp32 16x16x4 form with
// one element per lane), lane l = 0..63:
//   A fragment: row (l % 16), contraction elements KPL*(l/16) .. +KPL-1
//   B fragment: column (l % 16), the same contraction elements
//   C/D tile:   4 floats, rows 4*(l/16) + e (e = 0..3), column (l % 16)
// Any permutation of the contraction index that is the same for A and B gives
// the same product, so only the row/column and C placements matter.
#pragma once

#include "gdn_common.h"

namespace gdn {

template <typename E> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int KPL = 8;   // operand elements per lane
    static constexpr int KS = 32;   // contraction length of one instruction
    static constexpr int PAD = 8;   // LDS row padding (elements): 16-byte rows, no bank conflicts
    typedef bf16x8 frag;
    __device__ __forceinline__ static frag ld(const bf16* base, int ldm, int r0, int k0) {
        const int l = lane_id();
        return *(const bf16x8*)(base + (r0 + (l & 15)) * ldm + k0 + 8 * (l >> 4));
    }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static constexpr int KPL = 1;
    static constexpr int KS = 4;
    static constexpr int PAD = 4;   // row stride = 4 (mod 64) words: (row, k) -> distinct banks
    typedef float frag;
    __device__ __forceinline__ static frag ld(const float* base, int ldm, int r0, int k0) {
        const int l = lane_id();
        return base[(r0 + (l & 15)) * ldm + k0 + (l >> 4)];
    }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// fp32 B operand read from a row-major B[k][n] buffer (used by the fp32
// triangular-inverse merges, where no transposed copy exists).
__device__ __forceinline__ float ld_b_rowmajor(const float* base, int ldm, int k0, int n0) {
    const int l = lane_id();
    return base[(k0 + (l >> 4)) * ldm + n0 + (l & 15)];
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace gdn
