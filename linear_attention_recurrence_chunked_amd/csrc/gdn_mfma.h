// gdn_mfma.h -- matrix-core (MFMA) operand helpers for gfx950.
//
// All products are built from 16x16 fp32 output tiles contracted 32 deep. In
// a 32-deep step lane l (group g = l/16) supplies eight contraction indices,
// and any assignment works as long as both operands use the same one. Two
// assignments are used:
//
//  * token contractions (T R, P U, K^T U): lane group g supplies k =
//    {4g .. 4g+3} and {16+4g .. 16+4g+3}, exactly the rows a lane holds in
//    a pair of 16x16 accumulator tiles (rows 4g + e, e = 0..3, column l%16),
//    so computed tiles feed the next product straight from registers. The
//    LDS side (T, P) is stored with its columns permuted (tpos) so that the
//    eight values a lane needs are contiguous: one 16-byte read.
//  * key-dimension contractions (K S, Q S, K K^T, Q K^T): lane group g
//    supplies k = 8g .. 8g+7 of the 32-deep step, a contiguous 16-byte piece
//    of a K or Q row. The state tiles kept in registers are produced with
//    their rows permuted (spos) so that a pair of them supplies exactly those
//    rows as the state operand.
//
// 16-byte fragment reads replace pairs of 8-byte reads: the compiler would
// merge such a pair into one ds_read2_b64, which runs about four times slower
// than two plain reads on gfx950 for these lane patterns.
//
// bf16: one v_mfma_f32_16x16x32_bf16 per step; computed operands are carried
//       as a pair hi = bf16(x), lo = bf16(x - hi) and a product of pairs is
//       hi*hi + hi*lo + lo*hi (about 16 significant bits).
// fp32: eight v_mfma_f32_16x16x4f32 per step, one k value per lane each.
//
// Accumulator layout of a 16x16 tile (lane l, element e): row 4*(l/16) + e,
// column l % 16.
#pragma once

#include "gdn_common.h"

namespace gdn {

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Stored column of token s (0..31) in a T or P row: the values lane group g
// needs, s = 4g..4g+3 and 16+4g..16+4g+3, sit at columns 8g .. 8g+7.
__host__ __device__ constexpr int tpos(int s) { return 8 * ((s & 15) >> 2) + 4 * (s >> 4) + (s & 3); }

// Key row held by element e of lane group g in state tile kt: the tile pair
// (2m, 2m+1) holds rows 32m + 8g + 0..7, the contiguous slice lane group g
// supplies in key-dimension contractions.
__host__ __device__ constexpr int spos(int kt, int g, int e) { return 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + e; }

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed LDS read: lanes j of a 16-lane group give the address of 4
// consecutive elements of row j/4 (columns 4*(j%4)..+3) of a 4x16 block; lane
// i receives column i of the block (rows 0..3).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(const_cast<bf16*>(p)));
    return __builtin_bit_cast(bf16x4, r);
}

typedef __attribute__((address_space(3))) char lds_char;

// 32-bit LDS byte address of a generic pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_char*)p;
}

// Hides the value of a per-lane LDS base address from the optimiser, so that
// reads at base + compile-time constant keep the constant in the
// instruction's immediate offset instead of hoisting one base + constant
// register per read out of the enclosing loop.
__device__ __forceinline__ uint32_t opaque_base(uint32_t a) {
    asm volatile("" : "+v"(a));
    return a;
}

// Typed LDS pointer at a 32-bit byte address.
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint32_t a) {
    return (__attribute__((address_space(3))) T*)(lds_char*)(uintptr_t)a;
}

// Wave-local ordering of LDS accesses (no cross-wave barrier).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// hi/lo bf16 pair of two floats: hi = bf16(a), bf16(b) packed (round to
// nearest even) and lo = bf16(a - hi_a), bf16(b - hi_b). The fp32 values of
// the hi parts are read off the packed bits (a shift and a mask), so a pair
// costs two conversions, two bit operations and two subtractions.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    const float ha = __builtin_bit_cast(float, h << 16);
    const float hb = __builtin_bit_cast(float, h & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
    hi = h;
}

// The same pair for values that die here: each difference is one bf16 dot
// product x + (-1) hi_x + 0 hi_y accumulated into x's own register, which is
// exact (x - bf16(x) is representable in fp32), so a pair costs two
// conversions and two dot products. (For a value that stays live the
// compiler would add a copy per dot product; split2 is cheaper there.)
// m0 = 0x0000bf80 and m1 = 0xbf800000 are the packed factors (-1, 0) and
// (0, -1). The caller passes them in registers, opaque to the compiler: the
// compiler would otherwise encode (-1, 0) as the inline constant -1.0, which
// this instruction reads as the fp32 bit pattern, i.e. as (0, -1).
constexpr uint32_t kDotNegLo = 0x0000bf80u, kDotNegHi = 0xbf800000u;
__device__ __forceinline__ void split2_last(float a, float b, uint32_t& hi, uint32_t& lo,
                                            uint32_t m0, uint32_t m1) {
    const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
    const float la = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m0), a, false);
    const float lb = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, m1), b, false);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{la, lb}, bf16x2));
    hi = __builtin_bit_cast(uint32_t, h);
}

template <typename E> struct Op;

template <> struct Op<bf16> {
    static constexpr bool SPLIT = true;
    typedef bf16x8 F;   // one 32-deep operand fragment

    // A[r0 + l%16][k0 + 8g .. k0 + 8g + 7]: one 16-byte read from row-major A.
    __device__ __forceinline__ static F ldc(const bf16* A, int ld, int r0, int k0) {
        const int l = lane_id();
        return *(const F*)(A + (r0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
    }
    // Transposed state-update operand for state tile kt: row i of the result
    // is key index spos(kt, i/4, i%4) = 32(kt/2) + 8(i/4) + 4(kt%2) + i%4,
    // contraction over the tokens k0 + {4g.., 16+4g..} of row-major X[t][dk].
    // Lane j of a 16-lane group points the transpose read at row 4g + j/4,
    // key columns 32(kt/2) + 8(j%4) + 4(kt%2) .. +3.
    __device__ __forceinline__ static F ldt(const bf16* X, int ld, int kt, int k0) {
        const int l = lane_id(), g = l >> 4, j = l & 15;
        const bf16* p = X + (k0 + 4 * g + (j >> 2)) * ld + 32 * (kt >> 1) + 4 * (kt & 1) + 8 * (j & 3);
        const bf16x4 a = lds_read_tr(p);
        const bf16x4 b = lds_read_tr(p + 16 * ld);
        return F{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
    // ldc in two parts: the lane's byte offset, and the read of the fragment
    // at rows r0.., columns k0.. from base = buffer address + that offset.
    __device__ __forceinline__ static uint32_t ldc_lane(int ld) {
        const int l = lane_id();
        return (uint32_t)(((l & 15) * ld + 8 * (l >> 4)) * 2);
    }
    __device__ __forceinline__ static F ldc_at(uint32_t base, int ld, int r0, int k0) {
        return *lds_ptr<const F>(base + (uint32_t)((r0 * ld + k0) * 2));
    }
    // ldt in two parts: the lane's byte offset (the same for every tile kt),
    // and the read of tile kt at base = buffer address + that offset.
    __device__ __forceinline__ static uint32_t ldt_lane(int ld, int k0) {
        const int l = lane_id(), g = l >> 4, j = l & 15;
        return (uint32_t)(((k0 + 4 * g + (j >> 2)) * ld + 8 * (j & 3)) * 2);
    }
    __device__ __forceinline__ static F ldt_at(uint32_t base, int ld, int kt) {
        const lds_char* p = (const lds_char*)(uintptr_t)base + (32 * (kt >> 1) + 4 * (kt & 1)) * 2;
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
        const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p + 16 * ld * 2));
        const bf16x4 x = __builtin_bit_cast(bf16x4, a), y = __builtin_bit_cast(bf16x4, b);
        return F{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
    // B fragment from two accumulator tiles (k block 0 = x0 rows, block 1 = x1
    // rows); LAST: the tiles die here (split2_last, with its factors m0, m1).
    template <bool LAST = false>
    __device__ __forceinline__ static void split(f32x4 x0, f32x4 x1, F& hi, F& lo,
                                                 uint32_t m0 = 0, uint32_t m1 = 0) {
        uint32_t h0, h1, h2, h3, w0, w1, w2, w3;
        auto s2 = [&](float a, float b, uint32_t& h, uint32_t& w) {
            if constexpr (LAST) split2_last(a, b, h, w, m0, m1); else split2(a, b, h, w);
        };
        s2(x0[0], x0[1], h0, w0);
        s2(x0[2], x0[3], h1, w1);
        s2(x1[0], x1[1], h2, w2);
        s2(x1[2], x1[3], h3, w3);
        hi = __builtin_bit_cast(F, u32x4{h0, h1, h2, h3});
        lo = __builtin_bit_cast(F, u32x4{w0, w1, w2, w3});
    }
    __device__ __forceinline__ static f32x4 mma(F a, F b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

struct F8 { float v[8]; };

template <> struct Op<float> {
    static constexpr bool SPLIT = false;
    typedef F8 F;

    __device__ __forceinline__ static F ldc(const float* A, int ld, int r0, int k0) {
        const int l = lane_id();
        const float* p = A + (r0 + (l & 15)) * ld + k0 + 8 * (l >> 4);
        const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
        F r;
#pragma unroll
        for (int e = 0; e < 4; ++e) { r.v[e] = a[e]; r.v[4 + e] = b[e]; }
        return r;
    }
    __device__ __forceinline__ static F ldt(const float* X, int ld, int kt, int k0) {
        const int l = lane_id(), j = l & 15;
        const float* p = X + (k0 + 4 * (l >> 4)) * ld + 32 * (kt >> 1) + 8 * (j >> 2) + 4 * (kt & 1) + (j & 3);
        F a;
#pragma unroll
        for (int e = 0; e < 4; ++e) { a.v[e] = p[e * ld]; a.v[4 + e] = p[(16 + e) * ld]; }
        return a;
    }
    __device__ __forceinline__ static uint32_t ldc_lane(int ld) {
        const int l = lane_id();
        return (uint32_t)(((l & 15) * ld + 8 * (l >> 4)) * 4);
    }
    __device__ __forceinline__ static F ldc_at(uint32_t base, int ld, int r0, int k0) {
        const __attribute__((address_space(3))) float* p =
            lds_ptr<const float>(base + (uint32_t)((r0 * ld + k0) * 4));
        const f32x4 a = *(const __attribute__((address_space(3))) f32x4*)p;
        const f32x4 b = *(const __attribute__((address_space(3))) f32x4*)(p + 4);
        F r;
#pragma unroll
        for (int e = 0; e < 4; ++e) { r.v[e] = a[e]; r.v[4 + e] = b[e]; }
        return r;
    }
    __device__ __forceinline__ static uint32_t ldt_lane(int ld, int k0) {
        const int l = lane_id(), j = l & 15;
        return (uint32_t)(((k0 + 4 * (l >> 4)) * ld + 8 * (j >> 2) + (j & 3)) * 4);
    }
    __device__ __forceinline__ static F ldt_at(uint32_t base, int ld, int kt) {
        const __attribute__((address_space(3))) float* p =
            (const __attribute__((address_space(3))) float*)((const lds_char*)(uintptr_t)base)
            + 32 * (kt >> 1) + 4 * (kt & 1);
        F a;
#pragma unroll
        for (int e = 0; e < 4; ++e) { a.v[e] = p[e * ld]; a.v[4 + e] = p[(16 + e) * ld]; }
        return a;
    }
    template <bool LAST = false>
    __device__ __forceinline__ static void split(f32x4 x0, f32x4 x1, F& hi, F& lo,
                                                 uint32_t = 0, uint32_t = 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) { hi.v[e] = x0[e]; hi.v[4 + e] = x1[e]; }
        lo = hi;  // unused on the fp32 path
    }
    __device__ __forceinline__ static f32x4 mma(const F& a, const F& b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
        return c;
    }
};

// fp32 16x16x4 MFMA with both operands read from row-major fp32 LDS buffers:
// A[r0 + l%16][k0 + l/16], B[k0 + l/16][n0 + l%16].
__device__ __forceinline__ f32x4 mma_f32_rm(f32x4 c, const float* A, int lda, int r0,
                                            const float* B, int ldb, int n0, int k0) {
    const int l = lane_id();
    return __builtin_amdgcn_mfma_f32_16x16x4f32(A[(r0 + (l & 15)) * lda + k0 + (l >> 4)],
                                                B[(k0 + (l >> 4)) * ldb + n0 + (l & 15)], c,
                                                0, 0, 0);
}

// As mma_f32_rm with A given transposed: A[r][k] = At[k][r].
__device__ __forceinline__ f32x4 mma_f32_tm(f32x4 c, const float* At, int lda, int r0,
                                            const float* B, int ldb, int n0, int k0) {
    const int l = lane_id();
    return __builtin_amdgcn_mfma_f32_16x16x4f32(At[(k0 + (l >> 4)) * lda + r0 + (l & 15)],
                                                B[(k0 + (l >> 4)) * ldb + n0 + (l & 15)], c,
                                                0, 0, 0);
}

}  // namespace gdn
