// api_driver.cpp -- drives every entry point of the C ABI (include/gdn.h)
// through valid and invalid arguments with fake, never-dereferenced device
// addresses, under AddressSanitizer and UBSan (built with the launcher stubs
// of launch_stub.cpp). It checks each status code and that exactly the valid
// calls reached a launcher; any sanitizer report aborts the run.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <cmath>
#include <initializer_list>
#include <limits>

#include "gdn.h"

extern int g_launches;

static int g_fail = 0;

#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const int got_ = (int)(call);                                               \
        if (got_ != (int)(want)) {                                                  \
            fprintf(stderr, "%s:%d: %s = %d, want %d\n", __FILE__, __LINE__, #call,  \
                    got_, (int)(want));                                             \
            ++g_fail;                                                               \
        }                                                                           \
    } while (0)

// distinct 1 TiB-spaced fake device addresses, 16-byte aligned
static void* fake(int i, uintptr_t off = 0) {
    return (void*)((uintptr_t)(i + 1) * ((uintptr_t)1 << 40) + off);
}
static float* ff(int i, uintptr_t off = 0) { return (float*)fake(i, off); }

static gdn_status prefill(int B, int Hk, int Hv, int S, int Dk, int Dv, int dtype,
                          void* out = nullptr, float* st = nullptr, const void* q = nullptr) {
    return gdn_chunked_prefill(q ? q : fake(0), fake(1), fake(2), ff(3), ff(4), 0.125f,
                               st ? st : ff(5), out ? out : fake(6), B, Hk, Hv, S, Dk, Dv,
                               dtype, nullptr, 0, nullptr);
}

int main() {
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const float inf = std::numeric_limits<float>::infinity();
    int valid = 0;

    // --- prefill: valid calls at several shapes and both dtypes
    EXPECT(prefill(4, 16, 32, 8192, 128, 128, GDN_BF16), GDN_OK); ++valid;
    EXPECT(prefill(1, 2, 2, 1, 16, 16, GDN_F32), GDN_OK); ++valid;
    EXPECT(prefill(3, 3, 3, 37, 80, 48, GDN_BF16), GDN_OK); ++valid;
    EXPECT(prefill(1, 1, 1, 4194239, 128, 128, GDN_F32), GDN_OK); ++valid;   // longest S
    // invalid shapes, dims, dtypes, overflow, alignment, aliasing, nulls
    EXPECT(prefill(0, 1, 1, 64, 64, 64, GDN_BF16), GDN_ERR_SHAPE);
    EXPECT(prefill(1, 2, 3, 64, 64, 64, GDN_BF16), GDN_ERR_SHAPE);
    EXPECT(prefill(1, 1, 1, -5, 64, 64, GDN_BF16), GDN_ERR_SHAPE);
    EXPECT(prefill(1, 1, 1, 4194240, 128, 128, GDN_F32), GDN_ERR_SHAPE);
    EXPECT(prefill(1 << 30, 1, 2, 1 << 22, 128, 128, GDN_F32), GDN_ERR_SHAPE);
    EXPECT(prefill(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 128, 128, GDN_F32), GDN_ERR_SHAPE);
    EXPECT(prefill(1, 1, 1, 64, 136, 64, GDN_BF16), GDN_ERR_UNSUPPORTED);
    EXPECT(prefill(1, 1, 1, 64, 64, 24, GDN_BF16), GDN_ERR_UNSUPPORTED);
    EXPECT(prefill(1, 1, 1, 64, 64, 64, 7), GDN_ERR_DTYPE);
    EXPECT(prefill(1, 1, 1, 64, 64, 64, GDN_BF16, fake(6, 8)), GDN_ERR_ALIGN);
    EXPECT(prefill(1, 1, 1, 64, 64, 64, GDN_BF16, fake(0, 16)), GDN_ERR_ALIAS);
    EXPECT(prefill(1, 1, 1, 64, 64, 64, GDN_BF16, nullptr, ff(2)), GDN_ERR_ALIAS);
    EXPECT(gdn_chunked_prefill(nullptr, fake(1), fake(2), ff(3), ff(4), 1.f, ff(5), fake(6),
                               1, 1, 1, 64, 64, 64, GDN_BF16, nullptr, 0, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_chunked_prefill_inverse(fake(0), fake(1), fake(2), ff(3), ff(4), 1.f, ff(5),
                                       fake(6), 2, 2, 4, 512, 128, 128, GDN_BF16,
                                       GDN_INV_NEUMANN, nullptr, 0, nullptr), GDN_OK); ++valid;
    EXPECT(gdn_chunked_prefill_inverse(fake(0), fake(1), fake(2), ff(3), ff(4), 1.f, ff(5),
                                       fake(6), 2, 2, 4, 512, 128, 128, GDN_BF16, 9, nullptr, 0,
                                       nullptr), GDN_ERR_VALUE);
    EXPECT(gdn_chunked_prefill_workspace_bytes(INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, 128,
                                               128, GDN_BF16), 0);
    // gated prefill: eps and head parameters
    EXPECT(gdn_chunked_prefill_gated(fake(0), fake(1), fake(2), ff(3), ff(4), ff(7), ff(8), 0.1f,
                                     1e-6f, ff(5), fake(6), 2, 2, 4, 100, 64, 64, GDN_BF16,
                                     nullptr, 0, nullptr), GDN_OK); ++valid;
    for (float eps : {-1.f, nan, inf})
        EXPECT(gdn_chunked_prefill_gated(fake(0), fake(1), fake(2), ff(3), ff(4), ff(7), ff(8),
                                         0.1f, eps, ff(5), fake(6), 2, 2, 4, 100, 64, 64,
                                         GDN_BF16, nullptr, 0, nullptr), GDN_ERR_VALUE);
    EXPECT(gdn_chunked_prefill_gated(fake(0), fake(1), fake(2), ff(3), ff(4), ff(7), ff(5, 64), 0.1f,
                                     1e-6f, ff(5), fake(6), 2, 2, 4, 100, 64, 64, GDN_BF16,
                                     nullptr, 0, nullptr), GDN_ERR_ALIAS);

    // --- decode (gated and plain)
    EXPECT(gdn_decode_step(fake(0), fake(1), fake(2), ff(3), ff(4), 0.1f, ff(5), fake(6), 256, 16,
                           32, 128, 128, GDN_BF16, nullptr), GDN_OK); ++valid;
    EXPECT(gdn_decode_step(fake(0), fake(1), fake(2), ff(3), ff(4), 0.1f, ff(5), fake(6),
                           INT32_MAX, 1, INT32_MAX, 128, 128, GDN_BF16, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_decode_step_gated(fake(0), fake(1), fake(2), ff(3), ff(4), ff(7), ff(8), 0.1f,
                                 0.f, ff(5), fake(6), 8, 2, 4, 64, 64, GDN_F32, nullptr), GDN_OK);
    ++valid;

    // --- conv1d
    EXPECT(gdn_conv1d_prefill(fake(0), ff(1), fake(2), fake(3), 4, 8192, 8192, 4, GDN_BF16,
                              nullptr), GDN_OK); ++valid;
    for (int T : {INT32_MAX, INT32_MAX - 8191, INT32_MAX - 65535})
        EXPECT(gdn_conv1d_prefill(fake(0), ff(1), fake(2), fake(3), 1, 1, T, 4, GDN_BF16,
                                  nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_conv1d_prefill(fake(0), ff(1), fake(2), fake(3), 1 << 20, 1 << 12, 4096, 4,
                              GDN_BF16, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_conv1d_prefill(fake(0), ff(1), fake(2), fake(3), 2, 16, 100, 9, GDN_BF16,
                              nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_conv1d_decode(fake(0), ff(1), fake(2), fake(3), 256, 8192, 4, GDN_BF16, nullptr),
           GDN_OK); ++valid;
    EXPECT(gdn_conv1d_decode(fake(0), ff(1), fake(2), fake(0, 16), 2, 16, 4, GDN_BF16, nullptr),
           GDN_ERR_ALIAS);

    // --- RMSNormGated
    EXPECT(gdn_rmsnorm_gated(fake(0), fake(1), ff(2), 1e-6f, fake(3), 4, 32, 8192, 128, GDN_BF16,
                             nullptr), GDN_OK); ++valid;
    for (int S : {INT32_MAX, INT32_MAX - 511, INT32_MAX - 65535})
        EXPECT(gdn_rmsnorm_gated(fake(0), fake(1), ff(2), 1e-6f, fake(3), 1, 1, S, 128, GDN_BF16,
                                 nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_rmsnorm_gated(fake(0), fake(1), ff(2), nan, fake(3), 1, 1, 8, 128, GDN_BF16,
                             nullptr), GDN_ERR_VALUE);

    // --- decode block
    EXPECT(gdn_decode_block(fake(0), fake(1), ff(2), ff(3), fake(4), fake(5), ff(6), ff(7), ff(8),
                            ff(9), 0.1f, 1e-6f, 1e-6f, ff(10), fake(11), 256, 16, 32, 128, 128, 4,
                            GDN_BF16, nullptr), GDN_OK); ++valid;
    EXPECT(gdn_decode_block(fake(0), fake(1), ff(2), ff(3), fake(4), fake(4, 32), ff(6), ff(7),
                            ff(8), ff(9), 0.1f, 1e-6f, 1e-6f, ff(10), fake(11), 2, 2, 4, 64, 64, 4,
                            GDN_BF16, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_decode_block(fake(0), fake(1), ff(2), ff(3), fake(4), fake(5), ff(6), ff(7), ff(8),
                            ff(9), 0.1f, 1e-6f, 1e-6f, ff(10), fake(11), INT32_MAX, 16, INT32_MAX,
                            128, 128, 4, GDN_BF16, nullptr), GDN_ERR_SHAPE);

    for (int code = -1; code <= 10; ++code)
        if (!gdn_status_string(code)) ++g_fail;
    if (gdn_version() < 100) ++g_fail;
    if (g_launches != valid) {
        fprintf(stderr, "launches %d, valid calls %d\n", g_launches, valid);
        ++g_fail;
    }
    printf("api driver: %d valid calls launched, %d failures\n", g_launches, g_fail);
    return g_fail ? 1 : 0;
}
