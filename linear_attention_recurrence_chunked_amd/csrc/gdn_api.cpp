// gdn_api.cpp -- the C ABI of libgdn (include/gdn.h): host-side validation
// and dispatch to the HIP launchers. Validation runs entirely on the host and
// before any HIP call, so every error path can be exercised without a GPU and
// leaves all buffers untouched.
#include "gdn.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gdn_launch.h"

namespace {

constexpr int kMaxConvTaps = 8;   // conv1d window width the kernels support
constexpr int kMaxHeadDim = 128;  // Dk, Dv upper bound ("GDN CTE", Notes)
// Token counts of the conv1d and RMSNormGated streams: the kernels round a
// count up to whole tiles (at most 8192 tokens) in 32-bit arithmetic, so a
// count is accepted only with that much headroom below INT32_MAX.
constexpr int64_t kMaxStreamTokens = INT32_MAX - 65536;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// a * b * ... in uint64 with overflow detection; returns false on overflow.
bool mul_ok(uint64_t& acc, uint64_t x) {
    if (x != 0 && acc > UINT64_MAX / x) return false;
    acc *= x;
    return true;
}

bool extent(const void* p, std::initializer_list<uint64_t> dims, uint64_t elem, Range& r) {
    uint64_t n = elem;
    for (uint64_t d : dims)
        if (!mul_ok(n, d)) return false;
    const uintptr_t lo = (uintptr_t)p;
    if (n > UINTPTR_MAX - lo) return false;
    r = Range{lo, lo + (uintptr_t)n};
    return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Common {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta; float* state; void* out;
    int B, Hk, Hv, S, Dk, Dv, dtype;
};

// Shared checks for prefill (S = sequence length) and decode (S = 1).
gdn_status validate(const Common& c, bool prefill) {
    if (!c.q || !c.k || !c.v || !c.g || !c.beta || !c.state || !c.out) return GDN_ERR_NULL;
    if (c.dtype != GDN_F32 && c.dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (c.B < 1 || c.Hk < 1 || c.Hv < 1 || c.S < 1) return GDN_ERR_SHAPE;
    if (c.Hv % c.Hk != 0) return GDN_ERR_SHAPE;
    if ((int64_t)c.B * c.Hv > INT32_MAX) return GDN_ERR_SHAPE;
    // the prefill addresses one (batch, head) stream of S rows with 32-bit
    // byte offsets: S * max(Dk, Dv) elements (plus a chunk) must fit
    if (prefill && ((int64_t)c.S + 64) * 128 * 4 > INT32_MAX) return GDN_ERR_SHAPE;
    if (c.Dk < 16 || c.Dk > kMaxHeadDim || c.Dk % 16 != 0) return GDN_ERR_UNSUPPORTED;
    if (c.Dv < 16 || c.Dv > kMaxHeadDim || c.Dv % 16 != 0) return GDN_ERR_UNSUPPORTED;
    const void* ptrs[] = {c.q, c.k, c.v, c.g, c.beta, c.state, c.out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;

    const uint64_t es = c.dtype == GDN_BF16 ? 2 : 4;
    const uint64_t B = c.B, Hk = c.Hk, Hv = c.Hv, S = c.S, Dk = c.Dk, Dv = c.Dv;
    Range rq, rk, rv, rg, rb, rs, ro;
    if (!extent(c.q, {B, Hk, S, Dk}, es, rq) || !extent(c.k, {B, Hk, S, Dk}, es, rk) ||
        !extent(c.v, {B, Hv, S, Dv}, es, rv) || !extent(c.g, {B, Hv, S}, 4, rg) ||
        !extent(c.beta, {B, Hv, S}, 4, rb) || !extent(c.state, {B, Hv, Dk, Dv}, 4, rs) ||
        !extent(c.out, {B, Hv, S, Dv}, es, ro))
        return GDN_ERR_SHAPE;
    // Written buffers may not overlap each other or anything read.
    const Range reads[] = {rq, rk, rv, rg, rb};
    for (const Range& r : reads)
        if (overlaps(ro, r) || overlaps(rs, r)) return GDN_ERR_ALIAS;
    if (overlaps(ro, rs)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

// Extra checks of the gated entry points: A_log and dt_bias [Hv] fp32, 4-byte
// aligned, not overlapping what the call writes; l2_eps finite and >= 0.
gdn_status validate_gates(const Common& c, const float* A_log, const float* dt_bias,
                          float l2_eps) {
    if (!A_log || !dt_bias) return GDN_ERR_NULL;
    if (!(l2_eps >= 0.0f) || !isfinite(l2_eps)) return GDN_ERR_VALUE;
    if (((uintptr_t)A_log & 3u) || ((uintptr_t)dt_bias & 3u)) return GDN_ERR_ALIGN;
    const uint64_t es = c.dtype == GDN_BF16 ? 2 : 4;
    const uint64_t B = c.B, Hv = c.Hv, S = c.S, Dk = c.Dk, Dv = c.Dv;
    Range ra, rd, rs, ro;
    if (!extent(A_log, {Hv}, 4, ra) || !extent(dt_bias, {Hv}, 4, rd) ||
        !extent(c.state, {B, Hv, Dk, Dv}, 4, rs) || !extent(c.out, {B, Hv, S, Dv}, es, ro))
        return GDN_ERR_SHAPE;
    if (overlaps(ra, rs) || overlaps(ra, ro) || overlaps(rd, rs) || overlaps(rd, ro))
        return GDN_ERR_ALIAS;
    return GDN_OK;
}

gdn_status prefill_common(const Common& c, bool gated, const float* A_log, const float* dt_bias,
                          float l2_eps, float scale, void* workspace, size_t workspace_bytes,
                          gdn_stream stream, int inverse = GDN_INV_SUBSTITUTION) {
    gdn_status st = validate(c, /*prefill=*/true);
    if (st == GDN_OK && gated) st = validate_gates(c, A_log, dt_bias, l2_eps);
    if (st != GDN_OK) return st;
    const size_t need = gdn_chunked_prefill_workspace_bytes(c.B, c.Hk, c.Hv, c.S, c.Dk, c.Dv,
                                                            c.dtype);
    if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return GDN_ERR_WORKSPACE;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    const gdn::PrefillArgs a{c.q, c.k, c.v, c.g, c.beta, scale, c.state, c.out,
                             c.B, c.Hk, c.Hv, c.S, c.Dk, c.Dv, gated, A_log, dt_bias, l2_eps,
                             inverse};
    return gdn::launch_prefill(a, c.dtype, (hipStream_t)stream) == hipSuccess ? GDN_OK
                                                                               : GDN_ERR_HIP;
}

gdn_status decode_common(const Common& c, bool gated, const float* A_log, const float* dt_bias,
                         float l2_eps, float scale, gdn_stream stream) {
    gdn_status st = validate(c, /*prefill=*/false);
    if (st == GDN_OK && gated) st = validate_gates(c, A_log, dt_bias, l2_eps);
    if (st != GDN_OK) return st;
    (void)hipGetLastError();
    const gdn::DecodeArgs a{c.q, c.k, c.v, c.g, c.beta, scale, c.state, c.out,
                            c.B, c.Hk, c.Hv, c.Dk, c.Dv, gated, A_log, dt_bias, l2_eps};
    return gdn::launch_decode(a, c.dtype, (hipStream_t)stream) == hipSuccess ? GDN_OK
                                                                             : GDN_ERR_HIP;
}

// conv1d checks: prefill (T tokens) or decode (T = 1, x [B, C]).
gdn_status validate_conv(const void* x, const float* w, const void* state, const void* out,
                         int B, int C, int T, int K, int dtype) {
    if (!x || !w || !state || !out) return GDN_ERR_NULL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (B < 1 || C < 1 || T < 1 || K < 1) return GDN_ERR_SHAPE;
    if (K > kMaxConvTaps) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)T > kMaxStreamTokens) return GDN_ERR_SHAPE;
    const int64_t tiles = ((int64_t)T + 2047) / 2048;  // at least the kernel's tile count
    if ((int64_t)B * C * tiles > INT32_MAX) return GDN_ERR_SHAPE;
    const void* ptrs[] = {x, w, state, out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    const uint64_t es = dtype == GDN_BF16 ? 2 : 4;
    Range rx, rw, rs, ro;
    if (!extent(x, {(uint64_t)B, (uint64_t)C, (uint64_t)T}, es, rx) ||
        !extent(w, {(uint64_t)C, (uint64_t)K}, 4, rw) ||
        !extent(state, {(uint64_t)B, (uint64_t)C, (uint64_t)K}, es, rs) ||
        !extent(out, {(uint64_t)B, (uint64_t)C, (uint64_t)T}, es, ro))
        return GDN_ERR_SHAPE;
    if (overlaps(ro, rx) || overlaps(ro, rw) || overlaps(rs, rx) || overlaps(rs, rw) ||
        overlaps(ro, rs))
        return GDN_ERR_ALIAS;
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_chunked_prefill_workspace_bytes(int B, int Hk, int Hv, int S, int Dk, int Dv,
                                           int dtype) {
    (void)B; (void)Hk; (void)Hv; (void)S; (void)Dk; (void)Dv; (void)dtype;
    return 0;  // the fused chunk kernel keeps every intermediate on chip
}

gdn_status gdn_chunked_prefill(const void* q, const void* k, const void* v,
                               const float* g_log, const float* beta, float scale,
                               float* state_inout, void* out,
                               int B, int Hk, int Hv, int S, int Dk, int Dv,
                               int dtype, void* workspace, size_t workspace_bytes,
                               gdn_stream stream) {
    const Common c{q, k, v, g_log, beta, state_inout, out, B, Hk, Hv, S, Dk, Dv, dtype};
    return prefill_common(c, false, nullptr, nullptr, 0.0f, scale, workspace, workspace_bytes,
                          stream);
}

gdn_status gdn_chunked_prefill_inverse(const void* q, const void* k, const void* v,
                                       const float* g_log, const float* beta, float scale,
                                       float* state_inout, void* out,
                                       int B, int Hk, int Hv, int S, int Dk, int Dv,
                                       int dtype, int inverse, void* workspace,
                                       size_t workspace_bytes, gdn_stream stream) {
    const Common c{q, k, v, g_log, beta, state_inout, out, B, Hk, Hv, S, Dk, Dv, dtype};
    const gdn_status st = validate(c, /*prefill=*/true);
    if (st != GDN_OK) return st;
    if (inverse != GDN_INV_SUBSTITUTION && inverse != GDN_INV_NEUMANN) return GDN_ERR_VALUE;
    return prefill_common(c, false, nullptr, nullptr, 0.0f, scale, workspace, workspace_bytes,
                          stream, inverse);
}

gdn_status gdn_chunked_prefill_gated(const void* q, const void* k, const void* v,
                                     const float* a, const float* b,
                                     const float* A_log, const float* dt_bias,
                                     float scale, float l2_eps,
                                     float* state_inout, void* out,
                                     int B, int Hk, int Hv, int S, int Dk, int Dv,
                                     int dtype, void* workspace, size_t workspace_bytes,
                                     gdn_stream stream) {
    const Common c{q, k, v, a, b, state_inout, out, B, Hk, Hv, S, Dk, Dv, dtype};
    return prefill_common(c, true, A_log, dt_bias, l2_eps, scale, workspace, workspace_bytes,
                          stream);
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const float* g_log, const float* beta, float scale,
                           float* state_inout, void* out,
                           int B, int Hk, int Hv, int Dk, int Dv, int dtype,
                           gdn_stream stream) {
    const Common c{q, k, v, g_log, beta, state_inout, out, B, Hk, Hv, 1, Dk, Dv, dtype};
    return decode_common(c, false, nullptr, nullptr, 0.0f, scale, stream);
}

gdn_status gdn_decode_step_gated(const void* q, const void* k, const void* v,
                                 const float* a, const float* b,
                                 const float* A_log, const float* dt_bias,
                                 float scale, float l2_eps,
                                 float* state_inout, void* out,
                                 int B, int Hk, int Hv, int Dk, int Dv, int dtype,
                                 gdn_stream stream) {
    const Common c{q, k, v, a, b, state_inout, out, B, Hk, Hv, 1, Dk, Dv, dtype};
    return decode_common(c, true, A_log, dt_bias, l2_eps, scale, stream);
}

gdn_status gdn_conv1d_prefill(const void* mixed, const float* conv_weight, void* out,
                              void* conv_state_out, int B, int C, int T, int K, int dtype,
                              gdn_stream stream) {
    const gdn_status st = validate_conv(mixed, conv_weight, conv_state_out, out, B, C, T, K, dtype);
    if (st != GDN_OK) return st;
    (void)hipGetLastError();
    const gdn::ConvArgs a{mixed, conv_weight, out, conv_state_out, B, C, T, K};
    return gdn::launch_conv1d(a, dtype, false, (hipStream_t)stream) == hipSuccess ? GDN_OK
                                                                                  : GDN_ERR_HIP;
}

gdn_status gdn_conv1d_decode(const void* x, const float* conv_weight, void* conv_state_inout,
                             void* out, int B, int C, int K, int dtype, gdn_stream stream) {
    const gdn_status st = validate_conv(x, conv_weight, conv_state_inout, out, B, C, 1, K, dtype);
    if (st != GDN_OK) return st;
    (void)hipGetLastError();
    const gdn::ConvArgs a{x, conv_weight, out, conv_state_inout, B, C, 1, K};
    return gdn::launch_conv1d(a, dtype, true, (hipStream_t)stream) == hipSuccess ? GDN_OK
                                                                                 : GDN_ERR_HIP;
}

gdn_status gdn_decode_block(const void* mixed, const void* z, const float* a, const float* b,
                            const void* conv_state_in, void* conv_state_out,
                            const float* conv_weight, const float* A_log, const float* dt_bias,
                            const float* norm_weight, float scale, float l2_eps, float norm_eps,
                            float* state_inout, void* out,
                            int B, int Hk, int Hv, int Dk, int Dv, int K, int dtype,
                            gdn_stream stream) {
    if (!mixed || !z || !a || !b || !conv_state_in || !conv_state_out || !conv_weight ||
        !A_log || !dt_bias || !norm_weight || !state_inout || !out)
        return GDN_ERR_NULL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (B < 1 || Hk < 1 || Hv < 1 || K < 1 || Hv % Hk != 0) return GDN_ERR_SHAPE;
    if ((int64_t)B * Hv > INT32_MAX) return GDN_ERR_SHAPE;
    if (Dk < 16 || Dk > kMaxHeadDim || Dk % 16 != 0) return GDN_ERR_UNSUPPORTED;
    if (Dv < 16 || Dv > kMaxHeadDim || Dv % 16 != 0) return GDN_ERR_UNSUPPORTED;
    if (K > kMaxConvTaps) return GDN_ERR_UNSUPPORTED;
    if (!(l2_eps >= 0.0f) || !isfinite(l2_eps) || !(norm_eps >= 0.0f) || !isfinite(norm_eps))
        return GDN_ERR_VALUE;
    const void* ptrs[] = {mixed, z, a, b, conv_state_in, conv_state_out, conv_weight, A_log,
                          dt_bias, norm_weight, state_inout, out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    const uint64_t es = dtype == GDN_BF16 ? 2 : 4;
    const uint64_t C = 2 * (uint64_t)Hk * Dk + (uint64_t)Hv * Dv;
    if (C > INT32_MAX) return GDN_ERR_SHAPE;
    const uint64_t uB = B, uHv = Hv, uK = K;
    Range rmx, rz, ra, rb, rci, rco, rw, ral, rdt, rnw, rs, ro;
    if (!extent(mixed, {uB, C}, es, rmx) || !extent(z, {uB, uHv * Dv}, es, rz) ||
        !extent(a, {uB, uHv}, 4, ra) || !extent(b, {uB, uHv}, 4, rb) ||
        !extent(conv_state_in, {uB, C, uK}, es, rci) ||
        !extent(conv_state_out, {uB, C, uK}, es, rco) || !extent(conv_weight, {C, uK}, 4, rw) ||
        !extent(A_log, {uHv}, 4, ral) || !extent(dt_bias, {uHv}, 4, rdt) ||
        !extent(norm_weight, {(uint64_t)Dv}, 4, rnw) ||
        !extent(state_inout, {uB, uHv, (uint64_t)Dk, (uint64_t)Dv}, 4, rs) ||
        !extent(out, {uB, uHv * Dv}, es, ro))
        return GDN_ERR_SHAPE;
    const Range reads[] = {rmx, rz, ra, rb, rci, rw, ral, rdt, rnw};
    const Range writes[] = {rco, rs, ro};
    for (const Range& w : writes)
        for (const Range& r : reads)
            if (overlaps(w, r)) return GDN_ERR_ALIAS;
    if (overlaps(rco, rs) || overlaps(rco, ro) || overlaps(rs, ro)) return GDN_ERR_ALIAS;
    (void)hipGetLastError();
    const gdn::DecodeArgs da{nullptr, nullptr, nullptr, a, b, scale, state_inout, out,
                             B, Hk, Hv, Dk, Dv, true, A_log, dt_bias, l2_eps};
    const gdn::BlockArgs blk{mixed, z, conv_state_in, conv_state_out, conv_weight, norm_weight,
                             norm_eps, K};
    return gdn::launch_decode_block(da, blk, dtype, (hipStream_t)stream) == hipSuccess
               ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_rmsnorm_gated(const void* o, const void* z, const float* norm_weight, float eps,
                             void* out, int B, int Hv, int S, int Dv, int dtype,
                             gdn_stream stream) {
    if (!o || !z || !norm_weight || !out) return GDN_ERR_NULL;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (B < 1 || Hv < 1 || S < 1) return GDN_ERR_SHAPE;
    if ((int64_t)S > kMaxStreamTokens) return GDN_ERR_SHAPE;
    if (Dv < 16 || Dv > kMaxHeadDim || Dv % 16 != 0) return GDN_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f) || !isfinite(eps)) return GDN_ERR_VALUE;
    const void* ptrs[] = {o, z, norm_weight, out};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDN_ERR_ALIGN;
    const uint64_t es = dtype == GDN_BF16 ? 2 : 4;
    Range ro, rz, rw, rout;
    if (!extent(o, {(uint64_t)B, (uint64_t)Hv, (uint64_t)S, (uint64_t)Dv}, es, ro) ||
        !extent(z, {(uint64_t)B, (uint64_t)S, (uint64_t)Hv, (uint64_t)Dv}, es, rz) ||
        !extent(norm_weight, {(uint64_t)Dv}, 4, rw) ||
        !extent(out, {(uint64_t)B, (uint64_t)S, (uint64_t)Hv, (uint64_t)Dv}, es, rout))
        return GDN_ERR_SHAPE;
    if (overlaps(rout, ro) || overlaps(rout, rz) || overlaps(rout, rw)) return GDN_ERR_ALIAS;
    (void)hipGetLastError();
    const gdn::NormArgs na{o, z, norm_weight, eps, out, B, Hv, S, Dv};
    return gdn::launch_rmsnorm_gated(na, dtype, (hipStream_t)stream) == hipSuccess ? GDN_OK
                                                                                   : GDN_ERR_HIP;
}

const char* gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid shape (sizes < 1, Hv % Hk != 0, or overflow)";
        case GDN_ERR_UNSUPPORTED: return "unsupported size (Dk, Dv must be multiples of 16 in [16, 128]; conv taps K <= 8)";
        case GDN_ERR_DTYPE: return "invalid dtype";
        case GDN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case GDN_ERR_ALIAS: return "out or state_inout overlaps another tensor argument";
        case GDN_ERR_WORKSPACE: return "workspace too small";
        case GDN_ERR_HIP: return "HIP launch failed";
        case GDN_ERR_VALUE: return "invalid scalar argument (an epsilon is negative or not finite, or an unknown inverse method)";
        default: return "unknown status";
    }
}

int gdn_version(void) { return 200; }

}  // extern "C"
