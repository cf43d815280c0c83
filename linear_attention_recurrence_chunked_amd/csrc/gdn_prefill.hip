// gdn_prefill.hip -- chunk-parallel gated delta-rule prefill on gfx950.
//
// The chunked form that the "GDN CTE Kernel API Reference" page describes in
// its introduction (work inside a chunk is parallel and goes through a
// unit-lower-triangular inverse; a recurrence carries the state across
// chunks). For one head and a chunk of C tokens with start state S0 and
// gamma = within-chunk inclusive cumulative sum of g_log:
//
//   A  = diag(beta) (K K^T) (.) Mstrict     Mstrict[r,s] = e^{gamma_r-gamma_s}, s < r
//   T  = (I + A)^{-1}                       unit lower triangular, fp32
//   R  = diag(beta) V - diag(beta e^gamma) K S0
//   U  = T R                                the per-token updates u_t
//   O  = scale (diag(e^gamma) Q S0 + P U),  P = Q K^T (.) Mincl  (s <= r)
//   S1 = e^{gamma_C} S0 + K^T diag(e^{gamma_C - gamma}) U
//
// derived from the token recurrence S_t = e^{g_t} S_{t-1} + beta_t k_t
// (v_t - e^{g_t} S_{t-1}^T k_t)^T, o_t = scale S_t^T q_t: unrolling the chunk
// gives (I + A) U = diag(beta) V - diag(beta e^gamma) K S0. The right-hand side
// R is formed in fp32 before anything is rounded, so the cancellation between
// new values and the state's prediction happens at full precision.
//
// Design (one fused kernel, no HBM intermediates): one workgroup of NW waves
// owns one (batch, value head, BV-wide slice of Dv) and walks the chunks of
// its sequence in order, holding its [Dk x BV] slice of the fp32 state in
// MFMA accumulator registers throughout. Per chunk only q, k, v, g, beta are
// read and out is written, so HBM traffic is the algorithmic minimum. The
// state-independent work (gamma, A, T, the masked Q K^T) is recomputed by each
// Dv slice; BV is chosen per launch so the grid fills the 256 compute units.
// Products are 16x16-tile MFMAs from LDS. On the bf16 path every operand that
// is not an exact input (S, T, R, P, U) is carried as a pair of bf16 numbers
// hi + lo (hi = bf16(x), lo = bf16(x - hi)), and a product of two such values
// is hi*hi + hi*lo + lo*hi, so results keep about 16 significant bits; q, k, v
// are exact in bf16 and need one term. The triangular inverse is fp32: 16x16
// diagonal blocks by forward substitution (one lane per column), then
// doubling merges T21 = -T22 (A21 T11) on fp32 MFMA.
#include "gdn_common.h"
#include "gdn_launch.h"
#include "gdn_mfma.h"

namespace gdn {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename E> struct Vec16;  // one 16-byte vector of E
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

// Writes 4 consecutive values as the operand type. With SPLIT the low parts
// (x - hi) go to p + lo_off.
template <bool SPLIT>
__device__ __forceinline__ void store4(bf16* p, int lo_off, f32x4 x) {
    bf16x4 hi = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    *(bf16x4*)p = hi;
    if constexpr (SPLIT) {
        bf16x4 lo = {(bf16)(x[0] - (float)hi[0]), (bf16)(x[1] - (float)hi[1]),
                     (bf16)(x[2] - (float)hi[2]), (bf16)(x[3] - (float)hi[3])};
        *(bf16x4*)(p + lo_off) = lo;
    }
}
template <bool SPLIT>
__device__ __forceinline__ void store4(float* p, int, f32x4 x) { *(f32x4*)p = x; }

template <bool SPLIT>
__device__ __forceinline__ void store1(bf16* p, int lo_off, float x) {
    const bf16 hi = (bf16)x;
    p[0] = hi;
    if constexpr (SPLIT) p[lo_off] = (bf16)(x - (float)hi);
}
template <bool SPLIT>
__device__ __forceinline__ void store1(float* p, int, float x) { p[0] = x; }

// Linear index of a lower-triangular 16x16 tile (row-major over i >= j) -> (i, j).
__device__ __forceinline__ void tri_index(int lt, int& i, int& j) {
    i = 0;
    while (lt > i) { lt -= i + 1; ++i; }
    j = lt;
}

template <typename E, int C, int DK, int BV, int NW>
struct PrefillCfg {
    using M = Mfma<E>;
    static constexpr bool SPLIT = sizeof(E) == 2;   // hi/lo operand pairs on the bf16 path
    static constexpr int NP = SPLIT ? 2 : 1;        // parts per pair buffer row
    static constexpr int ES = (int)sizeof(E);
    static constexpr int VE = Vec16<E>::N;
    static constexpr int PAD = M::PAD;
    static constexpr int LDK = DK + PAD;            // K, Q rows [t][dk]
    static constexpr int LDKT = C + PAD;            // Kt rows [dk][t]
    static constexpr int LDV = BV + PAD;            // V rows [t][v]
    static constexpr int LDS2 = NP * DK + PAD;      // St pair rows [v][hi dk | lo dk]
    static constexpr int LDC2 = NP * C + PAD;       // P, T, Rt, Ut, Ud pair rows [x][hi t | lo t]
    static constexpr int LDF = C + 4;               // fp32 [t][s] rows (A, Tf)
    static constexpr int NT = C / 16;
    static constexpr int NKT = DK / 16;
    static constexpr int NVT = BV / 16;
    static constexpr int NLT = NT * (NT + 1) / 2;
    static constexpr int NO = NT * NVT;             // out / U / R tiles
    static constexpr int NS = NKT * NVT;            // state tiles
    static constexpr int THREADS = NW * 64;
    static constexpr int OPW = (NO + NW - 1) / NW;
    static constexpr int SPW = (NS + NW - 1) / NW;
    static constexpr int JPW = (2 * NLT + NW - 1) / NW;
    // Buffer sizes (bytes)
    static constexpr int SZ_K = C * LDK * ES;
    static constexpr int SZ_KT = DK * LDKT * ES;
    static constexpr int SZ_V = C * LDV * ES;
    static constexpr int SZ_ST = BV * LDS2 * ES;
    static constexpr int SZ_PC = C * LDC2 * ES;     // C-row pair buffer (P, T)
    static constexpr int SZ_PV = BV * LDC2 * ES;    // BV-row pair buffer (Rt, Ut, Ud)
    static constexpr int SZ_F = C * LDF * 4;
    static constexpr int SZ_X = (C / 2) * (C / 2 + 4) * 4;
    static constexpr int SZ_SC = 8 * C * 4;
    // Regions; buffers sharing a region have disjoint lifetimes within a chunk:
    //   R1: K, Q (staging .. K S0 / Q S0)     -> T pair, Rt pair
    //   R2: A, Tf (K K^T .. merges)           -> Ut pair, Ud pair
    static constexpr int SZ_R1 = cmax(2 * SZ_K, SZ_PC + SZ_PV);
    static constexpr int SZ_R2 = cmax(2 * SZ_F, 2 * SZ_PV);
    static constexpr int OFF_R1 = 0;
    static constexpr int OFF_R2 = OFF_R1 + SZ_R1;
    static constexpr int OFF_KT = OFF_R2 + SZ_R2;
    static constexpr int OFF_V = OFF_KT + SZ_KT;
    static constexpr int OFF_ST = OFF_V + SZ_V;
    static constexpr int OFF_P = OFF_ST + SZ_ST;
    static constexpr int OFF_X = OFF_P + SZ_PC;
    static constexpr int OFF_SC = OFF_X + SZ_X;
    static constexpr int LDS_BYTES = OFF_SC + SZ_SC;
    static_assert(LDS_BYTES <= 160 * 1024, "chunk tiles exceed the 160 KiB LDS of a CU");
    static_assert(C % M::KS == 0 && DK % M::KS == 0, "tile sizes must match the MFMA depth");
    static_assert(C == 32 || C == 64, "chunk must be 32 or 64");
    static_assert((SZ_K | SZ_KT | SZ_V | SZ_ST | SZ_PC | SZ_PV | SZ_F | SZ_X) % 16 == 0,
                  "LDS buffers must stay 16-byte aligned");
};

// acc += A B over contraction range [k0, k1), both operands contraction-
// contiguous in LDS. A pair operand has its low part at +lo_off elements in
// the same row. Terms: hi*hi (+ hi*lo if B is a pair) (+ lo*hi if A is a pair).
template <typename E, bool PA, bool PB>
__device__ __forceinline__ f32x4 mma_range(f32x4 acc, const E* A, int lda, int ra, int alo,
                                           const E* B, int ldb, int rb, int blo, int k0, int k1)
{
    using M = Mfma<E>;
    for (int k = k0; k < k1; k += M::KS) {
        const auto ah = M::ld(A, lda, ra, k);
        const auto bh = M::ld(B, ldb, rb, k);
        if constexpr (PB) acc = M::mma(ah, M::ld(B, ldb, rb, k + blo), acc);
        if constexpr (PA) acc = M::mma(M::ld(A, lda, ra, k + alo), bh, acc);
        acc = M::mma(ah, bh, acc);
    }
    return acc;
}

template <typename E, int C, int DK, int BV, int NW>
__global__ __launch_bounds__(NW * 64) void gdn_prefill_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ g_log, const float* __restrict__ beta, float scale,
    float* __restrict__ state, E* __restrict__ out,
    int Hk, int Hv, int S, int Dk, int Dv, int nvt)
{
    using Cf = PrefillCfg<E, C, DK, BV, NW>;
    using M = Mfma<E>;
    using VecE = typename Vec16<E>::type;
    constexpr bool SP = Cf::SPLIT;
    constexpr int VE = Cf::VE, LDK = Cf::LDK, LDKT = Cf::LDKT, LDV = Cf::LDV;
    constexpr int LDS2 = Cf::LDS2, LDC2 = Cf::LDC2, LDF = Cf::LDF, NW_ = NW;
    constexpr int THREADS = Cf::THREADS, KS = M::KS;
    constexpr int LO_C = C, LO_DK = DK;             // offsets of the low parts in pair rows

    __shared__ __attribute__((aligned(16))) char smem[Cf::LDS_BYTES];
    E* sK = (E*)(smem + Cf::OFF_R1);
    E* sQ = (E*)(smem + Cf::OFF_R1 + Cf::SZ_K);
    E* sT = (E*)(smem + Cf::OFF_R1);                       // after K/Q are dead
    E* sRt = (E*)(smem + Cf::OFF_R1 + Cf::SZ_PC);
    float* sA = (float*)(smem + Cf::OFF_R2);
    float* sTf = (float*)(smem + Cf::OFF_R2 + Cf::SZ_F);
    E* sUt = (E*)(smem + Cf::OFF_R2);                      // after A/Tf are dead
    E* sUd = (E*)(smem + Cf::OFF_R2 + Cf::SZ_PV);
    E* sKt = (E*)(smem + Cf::OFF_KT);
    E* sV = (E*)(smem + Cf::OFF_V);
    E* sSt = (E*)(smem + Cf::OFF_ST);
    E* sP = (E*)(smem + Cf::OFF_P);
    float* sX = (float*)(smem + Cf::OFF_X);
    float* sc = (float*)(smem + Cf::OFF_SC);
    float* sc_b = sc;              // beta
    float* sc_eg = sc + C;         // e^gamma
    float* sc_gam = sc + 2 * C;    // gamma
    float* sc_bk = sc + 3 * C;     // beta e^gamma
    float* sc_dl = sc + 4 * C;     // e^{gamma_C - gamma}
    float* sc_misc = sc + 5 * C;   // [0] = e^{gamma_C}

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int l = tid & 63;
    const int lc = l & 15;          // column of this lane in a 16x16 C tile
    const int lr = 4 * (l >> 4);    // first of its 4 rows

    // blockIdx -> (v slice, value head, batch)
    int bid = blockIdx.x;
    const int vt = bid % nvt; bid /= nvt;
    const int h = bid % Hv;
    const int b = bid / Hv;
    const int j = h / (Hv / Hk);
    const int v0 = vt * BV;
    const int vcols = min(BV, Dv - v0);
    const size_t bh = (size_t)b * Hv + h;
    const E* kb = k + ((size_t)b * Hk + j) * (size_t)S * Dk;
    const E* qb = q + ((size_t)b * Hk + j) * (size_t)S * Dk;
    const E* vb = v + bh * (size_t)S * Dv + v0;
    const float* gb = g_log + bh * (size_t)S;
    const float* bb = beta + bh * (size_t)S;
    E* ob = out + bh * (size_t)S * Dv + v0;
    float* sb = state + bh * (size_t)Dk * Dv + v0;

    // ---- initial state: fp32 accumulators + LDS copy St[v][dk] (hi | lo)
    f32x4 accS[Cf::SPW];
#pragma unroll
    for (int m = 0; m < Cf::SPW; ++m) {
        const int id = wave + NW_ * m;
        accS[m] = zero4();
        if (id < Cf::NS) {
            const int tk = id / Cf::NVT, vj = id % Cf::NVT;
            const int col = 16 * vj + lc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 16 * tk + lr + e;
                accS[m][e] = (dk < Dk && col < vcols) ? sb[(size_t)dk * Dv + col] : 0.f;
            }
            store4<SP>(sSt + col * LDS2 + 16 * tk + lr, LO_DK, accS[m]);
        }
    }

    for (int c0 = 0; c0 < S; c0 += C) {
        __syncthreads();  // previous chunk (or the initial St) complete

        // ---- P0: stage K (row-major + transposed), Q, V; wave 0 also does
        //      gamma = inclusive cumsum of g over the chunk and the scalars.
        for (int id = tid; id < C * DK / VE; id += THREADS) {
            const int t = id % C, d0 = (id / C) * VE;
            VecE x = {};
            if (d0 < Dk) x = *(const VecE*)(kb + (size_t)(c0 + t) * Dk + d0);
            *(VecE*)(sK + t * LDK + d0) = x;
#pragma unroll
            for (int e = 0; e < VE; ++e) sKt[(d0 + e) * LDKT + t] = x[e];
        }
        for (int id = tid; id < C * DK / VE; id += THREADS) {
            const int d0 = (id % (DK / VE)) * VE, t = id / (DK / VE);
            VecE x = {};
            if (d0 < Dk) x = *(const VecE*)(qb + (size_t)(c0 + t) * Dk + d0);
            *(VecE*)(sQ + t * LDK + d0) = x;
        }
        for (int id = tid; id < C * BV / VE; id += THREADS) {
            const int d0 = (id % (BV / VE)) * VE, t = id / (BV / VE);
            VecE x = {};
            if (d0 < vcols) x = *(const VecE*)(vb + (size_t)(c0 + t) * Dv + d0);
            *(VecE*)(sV + t * LDV + d0) = x;
        }
        if (wave == 0) {
            float x = (l < C) ? gb[c0 + l] : 0.f;
            const float bt = (l < C) ? bb[c0 + l] : 0.f;
#pragma unroll
            for (int off = 1; off < C; off <<= 1) {
                const float y = __shfl_up(x, off);
                if (l >= off) x += y;
            }
            const float gC = __shfl(x, C - 1);
            if (l < C) {
                const float eg = __expf(x);
                sc_b[l] = bt;
                sc_gam[l] = x;
                sc_eg[l] = eg;
                sc_bk[l] = bt * eg;
                sc_dl[l] = __expf(gC - x);   // gC <= x: never overflows
            }
            if (l == 0) sc_misc[0] = __expf(gC);
        }
        __syncthreads();

        // ---- P1: A = masked beta K K^T (fp32), P = masked Q K^T (pair),
        //      and, for owned tiles, K S0 and Q S0 (S0 as a pair).
        //      Decay factors e^{gamma_r - gamma_s} are only used where s <= r
        //      (a select, never a product with a masked value).
#pragma unroll
        for (int m = 0; m < Cf::JPW; ++m) {
            const int job = wave + NW_ * m;
            if (job < 2 * Cf::NLT) {
                const bool isQ = job >= Cf::NLT;
                int ti, tj;
                tri_index(isQ ? job - Cf::NLT : job, ti, tj);
                const E* Ab = isQ ? sQ : sK;
                f32x4 acc = mma_range<E, false, false>(zero4(), Ab, LDK, 16 * ti, 0, sK, LDK,
                                                       16 * tj, 0, 0, DK);
                const int s = 16 * tj + lc;
                const float gs = sc_gam[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * ti + lr + e;
                    const float dec = __expf(sc_gam[r] - gs);
                    if (!isQ) sA[r * LDF + s] = (s < r) ? sc_b[r] * dec * acc[e] : 0.f;
                    else store1<SP>(sP + r * LDC2 + s, LO_C, (s <= r) ? dec * acc[e] : 0.f);
                }
            }
        }
        for (int id = tid; id < C * C; id += THREADS) {   // zero the strictly-upper tiles of P
            const int r = id / C, s = id % C;
            if ((s >> 4) > (r >> 4)) store1<SP>(sP + r * LDC2 + s, LO_C, 0.f);
        }
        f32x4 accO[Cf::OPW], accR[Cf::OPW];
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            accO[m] = zero4();
            accR[m] = zero4();
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
                accR[m] = mma_range<E, false, SP>(accR[m], sK, LDK, 16 * ti, 0, sSt, LDS2,
                                                  16 * vj, LO_DK, 0, DK);
                accO[m] = mma_range<E, false, SP>(accO[m], sQ, LDK, 16 * ti, 0, sSt, LDS2,
                                                  16 * vj, LO_DK, 0, DK);
            }
        }
        __syncthreads();

        // ---- P2a: 16x16 diagonal blocks of T by forward substitution (wave 0),
        //      R = beta V - beta e^gamma (K S0) -> Rt pair (owners).
        if (wave == 0) {
            const int d = l >> 4, jc = l & 15;
            if (d < Cf::NT) {
                const float* Ad = sA + (16 * d) * LDF + 16 * d;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = (r == jc) ? 1.f : 0.f;
#pragma unroll
                    for (int s = 0; s < r; ++s) acc -= Ad[r * LDF + s] * x[s];
                    x[r] = acc;
                }
                float* Td = sTf + (16 * d) * LDF + 16 * d;
#pragma unroll
                for (int r = 0; r < 16; ++r) Td[r * LDF + jc] = x[r];
            }
        }
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
                const int vl = 16 * vj + lc, t0 = 16 * ti + lr;
                f32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r[e] = sc_b[t0 + e] * to_f32(sV[(t0 + e) * LDV + vl]) -
                           sc_bk[t0 + e] * accR[m][e];
                store4<SP>(sRt + vl * LDC2 + t0, LO_C, r);
            }
        }
        __syncthreads();

        // ---- P2b: doubling merges, T21 = -T22 (A21 T11), fp32 MFMA
#pragma unroll
        for (int mb = 16; mb < C; mb *= 2) {
            const int nblk = C / (2 * mb);
            const int tpr = mb / 16;
            const int tpb = tpr * tpr;
            const int LDX = mb + 4;
            for (int job = wave; job < nblk * tpb; job += NW_) {     // X = A21 T11
                const int bk = job / tpb, tt = job % tpb, ti = tt / tpr, tj = tt % tpr;
                const int base = 2 * mb * bk;
                f32x4 acc = zero4();
                for (int kk = 16 * tj; kk < mb; kk += 4)
                    acc = Mfma<float>::mma(Mfma<float>::ld(sA, LDF, base + mb + 16 * ti, base + kk),
                                           ld_b_rowmajor(sTf, LDF, base + kk, base + 16 * tj), acc);
                float* Xb = sX + bk * mb * LDX;
#pragma unroll
                for (int e = 0; e < 4; ++e) Xb[(16 * ti + lr + e) * LDX + 16 * tj + lc] = acc[e];
            }
            __syncthreads();
            for (int job = wave; job < nblk * tpb; job += NW_) {     // T21 = -T22 X
                const int bk = job / tpb, tt = job % tpb, ti = tt / tpr, tj = tt % tpr;
                const int base = 2 * mb * bk;
                const float* Xb = sX + bk * mb * LDX;
                f32x4 acc = zero4();
                for (int kk = 0; kk < 16 * (ti + 1); kk += 4)
                    acc = Mfma<float>::mma(Mfma<float>::ld(sTf, LDF, base + mb + 16 * ti, base + mb + kk),
                                           ld_b_rowmajor(Xb, LDX, kk, 16 * tj), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTf[(base + mb + 16 * ti + lr + e) * LDF + base + 16 * tj + lc] = -acc[e];
            }
            __syncthreads();
        }

        // ---- P2c: T -> pair buffer in the operand type (upper triangle zero)
        for (int id = tid; id < C * C; id += THREADS) {
            const int r = id / C, s = id % C;
            store1<SP>(sT + r * LDC2 + s, LO_C, (s <= r) ? sTf[r * LDF + s] : 0.f);
        }
        __syncthreads();

        // ---- P3: U = T R (owners) -> Ut pair, Ud = diag(e^{gamma_C-gamma}) U pair
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
                const int kend = ((16 * (ti + 1) + KS - 1) / KS) * KS;
                const f32x4 u = mma_range<E, SP, SP>(zero4(), sT, LDC2, 16 * ti, LO_C, sRt, LDC2,
                                                     16 * vj, LO_C, 0, kend);
                const int vl = 16 * vj + lc, t0 = 16 * ti + lr;
                store4<SP>(sUt + vl * LDC2 + t0, LO_C, u);
                f32x4 ud;
#pragma unroll
                for (int e = 0; e < 4; ++e) ud[e] = u[e] * sc_dl[t0 + e];
                store4<SP>(sUd + vl * LDC2 + t0, LO_C, ud);
            }
        }
        __syncthreads();

        // ---- P4: O = scale (e^gamma Q S0 + P U) -> out; S = e^{gamma_C} S0 + K^T Ud
#pragma unroll
        for (int m = 0; m < Cf::OPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NO) {
                const int ti = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int e = 0; e < 4; ++e) accO[m][e] *= sc_eg[16 * ti + lr + e];
                const int kend = ((16 * (ti + 1) + KS - 1) / KS) * KS;
                accO[m] = mma_range<E, SP, SP>(accO[m], sP, LDC2, 16 * ti, LO_C, sUt, LDC2,
                                               16 * vj, LO_C, 0, kend);
                const int col = 16 * vj + lc;
                if (col < vcols) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ob[(size_t)(c0 + 16 * ti + lr + e) * Dv + col] =
                            from_f32<E>(scale * accO[m][e]);
                }
            }
        }
        const float egC = sc_misc[0];
#pragma unroll
        for (int m = 0; m < Cf::SPW; ++m) {
            const int id = wave + NW_ * m;
            if (id < Cf::NS) {
                const int tk = id / Cf::NVT, vj = id % Cf::NVT;
#pragma unroll
                for (int e = 0; e < 4; ++e) accS[m][e] *= egC;
                accS[m] = mma_range<E, false, SP>(accS[m], sKt, LDKT, 16 * tk, 0, sUd, LDC2,
                                                  16 * vj, LO_C, 0, C);
                store4<SP>(sSt + (16 * vj + lc) * LDS2 + 16 * tk + lr, LO_DK, accS[m]);
            }
        }
    }

    // ---- final state
#pragma unroll
    for (int m = 0; m < Cf::SPW; ++m) {
        const int id = wave + NW_ * m;
        if (id < Cf::NS) {
            const int tk = id / Cf::NVT, vj = id % Cf::NVT;
            const int col = 16 * vj + lc;
            if (col < vcols) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int dk = 16 * tk + lr + e;
                    if (dk < Dk) sb[(size_t)dk * Dv + col] = accS[m][e];
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch

template <typename E, int C, int DK, int BV>
static hipError_t launch_cfg(const PrefillArgs& a, hipStream_t stream)
{
    constexpr int NW = 8;
    const int nvt = (a.Dv + BV - 1) / BV;
    const long long blocks = (long long)nvt * a.Hv * a.B;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gdn_prefill_kernel<E, C, DK, BV, NW>), dim3((unsigned)blocks),
                       dim3(NW * 64), 0, stream,
                       (const E*)a.q, (const E*)a.k, (const E*)a.v, a.g_log, a.beta, a.scale,
                       a.state, (E*)a.out, a.Hk, a.Hv, a.S, a.Dk, a.Dv, nvt);
    return hipGetLastError();
}

// Value-slice width: the widest of {max_bv, .., 16} that still gives at least
// one workgroup per compute unit (256 on MI355X); narrower slices repeat the
// state-independent chunk work, so wider is better once the chip is full.
static int pick_bv(const PrefillArgs& a, int max_bv)
{
    const long long units = (long long)a.B * a.Hv;
    for (int bv = max_bv; bv > 16; bv /= 2)
        if (a.Dv > bv / 2 && units * ((a.Dv + bv - 1) / bv) >= 256) return bv;
    return 16;
}

template <typename E, int C, int DK>
static hipError_t launch_dk(const PrefillArgs& a, int max_bv, hipStream_t stream)
{
    switch (pick_bv(a, max_bv)) {
        case 64: if constexpr (sizeof(E) == 2) return launch_cfg<E, C, DK, 64>(a, stream);
                 [[fallthrough]];
        case 32: return launch_cfg<E, C, DK, 32>(a, stream);
        default: return launch_cfg<E, C, DK, 16>(a, stream);
    }
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, hipStream_t stream)
{
    if (dtype == 1) {   // bf16 operands: 64-token chunks
        return a.Dk <= 64 ? launch_dk<bf16, 64, 64>(a, 64, stream)
                          : launch_dk<bf16, 64, 128>(a, 64, stream);
    }
    // fp32 operands: 32-token chunks keep the fp32 tiles inside LDS
    return a.Dk <= 64 ? launch_dk<float, 32, 64>(a, 32, stream)
                      : launch_dk<float, 32, 128>(a, 32, stream);
}

}  // namespace gdn
