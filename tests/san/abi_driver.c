/*
 * Host sanitizer driver for the C ABI (include/gdn.h): linked with the real
 * front end (gdn_api.cpp, host_layout.cpp) and a launcher stub, all built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py.  Every entry point is called with valid
 * arguments (fake, never dereferenced device addresses) and with each kind of
 * invalid argument, including sizes at the limits the front end accepts; the
 * expected status of every call is checked.  Written in C, so the header is
 * also checked to be plain C.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn.h"

int gdn_stub_launches(void);

static int failures = 0;
#define EXPECT(call, want)                                                                 \
    do {                                                                                   \
        const int got_ = (int)(call);                                                      \
        if (got_ != (int)(want)) {                                                         \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
                    (int)(want));                                                          \
            failures++;                                                                    \
        }                                                                                  \
    } while (0)

/* 256-byte aligned fake device addresses, 16 MiB apart */
#define F(i) ((void*)(uintptr_t)(0x10000000ull + (uint64_t)(i) * 0x1000000ull))

static gdn_problem prob(int32_t n, int64_t t, int32_t hk, int32_t hv, int32_t d) {
    gdn_problem p;
    memset(&p, 0, sizeof p);
    p.num_seqs = n; p.total_tokens = t; p.h_k = hk; p.h_v = hv; p.d_k = d; p.d_v = d;
    p.qkv_dtype = GDN_BF16; p.out_dtype = GDN_F32; p.qk_l2norm = 1; p.conv_width = 4;
    return p;
}

static gdn_status pre(const gdn_problem* p, void* o, void* ws, size_t wsb) {
    return gdn_prefill_varlen(p, F(1), F(2), F(3), F(4), F(5), F(6), F(9), NULL, NULL, NULL, NULL, o, F(10),
                              ws, wsb, NULL);
}

int main(void) {
    gdn_problem p = prob(2, 100, 2, 4, 128);
    const size_t need = gdn_prefill_workspace_bytes(&p);
    int launches = 0;

    /* valid calls reach the launcher */
    EXPECT(pre(&p, F(7), F(8), need), GDN_OK);
    launches++;
    p.d_v = 64;
    EXPECT(pre(&p, F(7), F(8), gdn_prefill_workspace_bytes(&p)), GDN_OK);
    launches++;
    p = prob(2, 100, 2, 4, 128);
    EXPECT(gdn_prefill_varlen_noalloc(&p, F(1), F(2), F(3), F(4), F(5), F(6), F(9), NULL, NULL, NULL, NULL, F(7),
                                      F(10), NULL), GDN_OK);
    launches++;
    EXPECT(gdn_prefill_varlen_pooled(&p, F(1), F(2), F(3), F(4), F(5), F(6), F(9), NULL, F(11), F(12), NULL, NULL,
                                     F(7), F(8), need, NULL), GDN_OK);
    launches++;
    gdn_problem b = p;
    b.segment_chunks = 4;
    EXPECT(pre(&b, F(7), F(8), gdn_prefill_workspace_bytes(&b)), GDN_OK);
    launches++;
    EXPECT(gdn_prefill_workspace_bytes(&b) > need, 1);
    EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_WORKSPACE);
    b.segment_chunks = -1;
    EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    gdn_problem dp = prob(4, 4, 2, 4, 128);
    EXPECT(gdn_decode_step(&dp, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), NULL, F(7), NULL), GDN_OK);
    launches++;
    gdn_problem mp = prob(4, 12, 2, 4, 64);
    EXPECT(gdn_decode_multi(&mp, 3, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), F(13), F(14), F(7),
                            NULL), GDN_OK);
    launches++;

    /* null problem and pointers */
    EXPECT(gdn_prefill_varlen(NULL, F(1), F(2), F(3), F(4), F(5), F(6), NULL, NULL, NULL, NULL, NULL, F(7), NULL,
                              F(8), need, NULL), GDN_ERR_NULL);
    EXPECT(gdn_prefill_varlen_noalloc(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                      NULL, NULL), GDN_ERR_NULL);
    EXPECT(gdn_decode_step(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
           GDN_ERR_NULL);
    EXPECT(pre(&p, NULL, F(8), need), GDN_ERR_NULL);
    EXPECT(gdn_prefill_workspace_bytes(NULL), 0);

    /* problem checks */
    b = p; b.h_v = 3;               EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.qkv_dtype = 9;                     EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_DTYPE);
    b = p; b.d_k = 96; b.d_v = 96;              EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_UNSUPPORTED);
    b = p; b.conv_width = 3;                    EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_UNSUPPORTED);
    b = p; b.l2_eps = -1.0f;                    EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.scale = 1.0f / 0.0f;               EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.total_tokens = (int64_t)1 << 40;   EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.num_seqs = 1 << 30;                EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.h_k = b.h_v = 0x7fffffff;          EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.d_k = b.d_v = 0x7fffffff;          EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.num_seqs = -1;                     EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.num_seqs = 0;                      EXPECT(pre(&b, F(7), F(8), need), GDN_ERR_SHAPE);
    b = p; b.num_seqs = 0; b.total_tokens = 0;  EXPECT(pre(&b, F(7), F(8), need), GDN_OK);
    /* workspace sizes never overflow inside the accepted ranges */
    b = prob(1 << 24, (int64_t)1 << 31, 4096, 4096, 128);
    EXPECT(gdn_prefill_workspace_bytes(&b) > ((size_t)1 << 40), 1);
    b.d_k = b.d_v = 0x7fffffff;
    EXPECT(gdn_prefill_workspace_bytes(&b), 0);

    /* workspace, alignment and aliasing */
    EXPECT(pre(&p, F(7), F(8), need - 1), GDN_ERR_WORKSPACE);
    EXPECT(pre(&p, F(7), NULL, need), GDN_ERR_WORKSPACE);
    EXPECT(pre(&p, (char*)F(7) + 4, F(8), need), GDN_ERR_UNSUPPORTED);
    EXPECT(pre(&p, F(1), F(8), need), GDN_ERR_ALIAS);
    EXPECT(pre(&p, F(7), F(3), need), GDN_ERR_ALIAS);
    EXPECT(gdn_prefill_varlen_noalloc(&p, F(1), F(2), F(3), F(4), F(5), F(6), F(9), NULL, NULL, NULL, NULL, F(1),
                                      F(10), NULL), GDN_ERR_ALIAS);
    b = prob(4, 4 * 4096, 16, 32, 128);
    b.conv_width = 0;
    EXPECT(gdn_prefill_varlen_noalloc(&b, F(1), F(2), F(3), F(4), F(5), F(6), NULL, NULL, NULL, NULL, NULL, F(7),
                                      F(10), NULL), GDN_ERR_SCRATCH);

    /* decode */
    b = dp; b.total_tokens = 5;                 EXPECT(gdn_decode_step(&b, F(1), F(2), F(3), F(4), F(5), F(9), NULL,
                                                                   F(11), F(12), NULL, F(7), NULL), GDN_ERR_SHAPE);
    EXPECT(gdn_decode_step(&dp, F(1), F(2), F(3), F(4), F(5), NULL, NULL, F(11), F(12), NULL, F(7), NULL),
           GDN_ERR_NULL);
    EXPECT(gdn_decode_step(&dp, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), NULL, F(12), NULL),
           GDN_ERR_ALIAS);
    EXPECT(gdn_decode_multi(&mp, 9, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), NULL, NULL, F(7), NULL),
           GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_decode_multi(&mp, 0, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), NULL, NULL, F(7), NULL),
           GDN_ERR_SHAPE);
    b = prob(1 << 24, 1 << 24, 4096, 4096, 128);
    EXPECT(gdn_decode_step(&b, F(1), F(2), F(3), F(4), F(5), F(9), NULL, F(11), F(12), NULL, F(7), NULL),
           GDN_ERR_SHAPE);

    /* stream copy helper validation (no launch reached) */
    EXPECT(gdn_stream_copy(F(1), F(1), 4096, 8, NULL), GDN_ERR_ALIAS);
    EXPECT(gdn_stream_copy(F(1), F(2), 4095, 8, NULL), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_stream_copy(F(1), F(2), 4096, 0, NULL), GDN_ERR_SHAPE);

    for (int s = -8; s <= 0; s++)
        if (!gdn_status_string((gdn_status)s) || strcmp(gdn_status_string((gdn_status)s), "unknown status") == 0)
            failures++;
    EXPECT(gdn_stub_launches(), launches);
    printf(failures ? "abi driver: %d FAILED\n" : "abi driver: ok\n", failures);
    return failures != 0;
}
