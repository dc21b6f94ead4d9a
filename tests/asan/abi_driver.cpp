// Host-only driver for the sanitizer build of the C ABI: calls every entry
// point of include/ulysses_sp.h with invalid, extreme and boundary arguments
// and checks the status each returns.  No call gets past argument
// validation, so no GPU is needed; AddressSanitizer and UndefinedBehavior-
// Sanitizer watch the validation code (size arithmetic on huge inputs,
// status-string lookups, pointer checks).  Exit status 0: every expectation
// held and no sanitizer report.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ulysses_sp.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
    if (got != want) {
        printf("FAIL %s: got %d, want %d\n", what, got, want);
        ++failures;
    }
}

static void expect_zero(const char *what, size_t got) {
    if (got != 0) {
        printf("FAIL %s: got %zu, want 0\n", what, got);
        ++failures;
    }
}

int main(void) {
    // fake device addresses: never dereferenced, because validation fails first
    void *a = (void *)(uintptr_t)0x10000, *mis = (void *)(uintptr_t)0x10002;
    const int64_t *pos = (const int64_t *)a;
    float *fa = (float *)a;
    const int64_t big = INT64_MAX, huge = INT64_MAX / 2 + 1;

    for (int s = -3; s < 20; ++s) {
        const char *m = sp_status_string(s);
        if (!m || !strlen(m)) {
            printf("FAIL status string %d\n", s);
            ++failures;
        }
    }
    expect("abi version", sp_abi_version(), 1);

    // relayout
    expect("s2h null", ulysses_seq_to_head(NULL, NULL, 4, 1024, 3, 8, 64, -1, NULL), SP_E_NULL);
    expect("s2h P=0", ulysses_seq_to_head(a, a, 0, 1024, 3, 8, 64, -1, NULL), SP_E_SHAPE);
    expect("s2h N%P", ulysses_seq_to_head(a, a, 4, 1023, 3, 8, 64, -1, NULL), SP_E_NOT_DIVISIBLE);
    expect("s2h H%P", ulysses_seq_to_head(a, a, 4, 1024, 3, 6, 64, -1, NULL), SP_E_NOT_DIVISIBLE);
    expect("s2h rank", ulysses_seq_to_head(a, a, 4, 1024, 3, 8, 64, 4, NULL), SP_E_RANK);
    expect("s2h rank<-1", ulysses_seq_to_head(a, a, 4, 1024, 3, 8, 64, -2, NULL), SP_E_RANK);
    expect("s2h align", ulysses_seq_to_head(mis, a, 4, 1024, 3, 8, 64, -1, NULL), SP_E_ALIGN);
    expect("s2h huge N", ulysses_seq_to_head(a, a, 4, huge, 3, 8, 64, -1, NULL), SP_E_SHAPE);
    expect("s2h max N", ulysses_seq_to_head(a, a, 1, big, 3, 8, 64, -1, NULL), SP_E_SHAPE);
    expect("s2h huge G", ulysses_seq_to_head(a, a, 4, 1024, INT32_MAX, INT32_MAX / 8 * 8, 64, -1, NULL),
           SP_E_SHAPE);
    expect("s2h N=0", ulysses_seq_to_head(NULL, NULL, 4, 0, 3, 8, 64, -1, NULL), SP_OK);
    expect("h2s piece", ulysses_head_to_seq(a, a, 4, 1024, 1, 4, 3, -1, NULL), SP_E_SHAPE);
    expect("h2s negative", ulysses_head_to_seq(a, a, 4, -4, 1, 8, 64, -1, NULL), SP_E_SHAPE);
    expect("kv H,P", ulysses_seq_to_head_kv(a, a, 4, 1024, 2, 3, 64, -1, NULL), SP_E_NOT_DIVISIBLE);
    expect("kv huge", ulysses_seq_to_head_kv(a, a, 16, huge, 2, 8, 128, -1, NULL), SP_E_SHAPE);
    expect("kv grad dtype", ulysses_head_to_seq_kv_grad(a, a, 16, 1024, 2, 8, 128, 7, -1, NULL),
           SP_E_DTYPE);
    expect("kv grad null", ulysses_head_to_seq_kv_grad(NULL, a, 16, 1024, 2, 8, 128, 1, -1, NULL),
           SP_E_NULL);

    // attention workspace sizes: invalid or overflowing sizes give 0
    expect_zero("ws max N", sp_attn_workspace_bytes(big, 4, 1, 128));
    expect_zero("ws huge N", sp_attn_workspace_bytes(huge, 1, 1, 64));
    expect_zero("ws max heads", sp_attn_workspace_bytes(1024, INT32_MAX, 1, 128));
    expect_zero("ws hq%hkv", sp_attn_workspace_bytes(1024, 4, 3, 128));
    expect_zero("ws d", sp_attn_workspace_bytes(1024, 4, 1, 96));
    expect_zero("ws negative", sp_attn_workspace_bytes(-1, 4, 1, 128));

    // attention forward / backward
    expect("fwd null", sp_attn_fwd(NULL, NULL, NULL, NULL, 256, 4, 1, 128, 0.f, NULL, NULL, NULL, 0, NULL),
           SP_E_NULL);
    expect("fwd d", sp_attn_fwd(a, a, a, pos, 256, 4, 1, 96, 0.f, a, fa, a, 1 << 20, NULL), SP_E_SHAPE);
    expect("fwd hq%hkv", sp_attn_fwd(a, a, a, pos, 256, 6, 4, 128, 0.f, a, fa, a, 1 << 20, NULL),
           SP_E_NOT_DIVISIBLE);
    expect("fwd nan scale", sp_attn_fwd(a, a, a, pos, 256, 4, 1, 128, NAN, a, fa, a, 1 << 20, NULL),
           SP_E_SHAPE);
    expect("fwd max N", sp_attn_fwd(a, a, a, pos, big, 4, 1, 128, 0.f, a, fa, a, 1 << 20, NULL), SP_E_SHAPE);
    expect("fwd huge N", sp_attn_fwd(a, a, a, pos, huge, 1, 1, 64, 0.f, a, fa, a, 1 << 20, NULL), SP_E_SHAPE);
    expect("fwd max heads", sp_attn_fwd(a, a, a, pos, 1024, INT32_MAX, 1, 64, 0.f, a, fa, a, 1 << 20, NULL),
           SP_E_SHAPE);
    expect("fwd ws", sp_attn_fwd(a, a, a, pos, 256, 4, 1, 128, 0.f, a, fa, a, 16, NULL), SP_E_WORKSPACE);
    expect("fwd align", sp_attn_fwd(mis, a, a, pos, 256, 4, 1, 128, 0.f, a, fa, a, 1 << 20, NULL),
           SP_E_ALIGN);
    expect("fwd N=0", sp_attn_fwd(NULL, NULL, NULL, NULL, 0, 4, 1, 128, 0.f, NULL, NULL, NULL, 0, NULL),
           SP_OK);
    expect("fwd stride small", sp_attn_fwd_strided(a, 256, a, a, 128, pos, 256, 4, 1, 128, 0.f, a, 512, fa,
                                                   a, 1 << 20, NULL), SP_E_SHAPE);
    expect("fwd stride huge", sp_attn_fwd_strided(a, big, a, a, 128, pos, 256, 4, 1, 128, 0.f, a, 512, fa,
                                                  a, 1 << 20, NULL), SP_E_SHAPE);
    expect("fwd stride neg", sp_attn_fwd_strided(a, -512, a, a, 128, pos, 256, 4, 1, 128, 0.f, a, 512, fa,
                                                 a, 1 << 20, NULL), SP_E_SHAPE);
    expect("bwd dtype", sp_attn_bwd(a, a, a, a, a, fa, pos, 256, 4, 1, 128, 0.f, 9, a, a, a, a, 1 << 20,
                                    NULL), SP_E_DTYPE);
    expect("bwd null", sp_attn_bwd(a, a, a, a, NULL, fa, pos, 256, 4, 1, 128, 0.f, 1, a, a, a, a, 1 << 20,
                                   NULL), SP_E_NULL);
    expect("bwd max N", sp_attn_bwd(a, a, a, a, a, fa, pos, big, 4, 1, 128, 0.f, 1, a, a, a, a, 1 << 20,
                                    NULL), SP_E_SHAPE);
    expect("bwd strided dk stride", sp_attn_bwd_strided(a, 512, a, a, 128, a, 512, a, 512, fa, pos, 256, 4,
                                                        1, 128, 0.f, 1, a, 512, a, 8, a, 128, a, 1 << 20,
                                                        NULL), SP_E_SHAPE);
    expect("noalloc oversize", sp_attn_bwd_noalloc(a, a, a, a, a, fa, pos, (int64_t)1 << 20, 8, 1, 64, 0.f,
                                                   1, a, a, a, NULL), SP_E_SCRATCH);
    expect("noalloc max N", sp_attn_bwd_noalloc(a, a, a, a, a, fa, pos, big, 8, 1, 64, 0.f, 1, a, a, a,
                                                NULL), SP_E_SHAPE);
    expect("noalloc null", sp_attn_bwd_noalloc(a, a, a, a, a, NULL, pos, 1024, 4, 1, 64, 0.f, 1, a, a, a,
                                               NULL), SP_E_NULL);

    // fused cross-entropy
    expect_zero("lce ws max vocab", sp_linear_ce_workspace_bytes(big, 64));
    expect_zero("lce ws vocab limit", sp_linear_ce_workspace_bytes(8421377, 64));
    expect_zero("lce ws max chunk", sp_linear_ce_workspace_bytes(1000, big / 64 * 64));
    expect_zero("lce ws chunk", sp_linear_ce_workspace_bytes(1000, 100));
    expect("lce hidden", sp_linear_ce(a, a, pos, -100, fa, 300, 1000, 200, 1, fa, fa, a, fa, 128, a, 1 << 30,
                                      NULL), SP_E_SHAPE);
    expect("lce max vocab", sp_linear_ce(a, a, pos, -100, fa, 300, big, 256, 1, fa, fa, a, fa, 128, a,
                                         1 << 30, NULL), SP_E_SHAPE);
    expect("lce max tokens", sp_linear_ce(a, a, pos, -100, fa, big, 1000, 256, 1, fa, fa, a, fa, 128, a,
                                          1 << 30, NULL), SP_E_SHAPE);
    expect("lce max hidden", sp_linear_ce(a, a, pos, -100, fa, 300, 1000, big / 256 * 256, 1, fa, fa, a, fa,
                                          128, a, 1 << 30, NULL), SP_E_SHAPE);
    expect("lce ws", sp_linear_ce(a, a, pos, -100, fa, 300, 1000, 256, 1, fa, fa, a, fa, 128, a, 16, NULL),
           SP_E_WORKSPACE);
    expect("lce dtype", sp_linear_ce(a, a, pos, -100, fa, 300, 1000, 256, 4, fa, fa, a, fa, 128, a, 1 << 30,
                                     NULL), SP_E_DTYPE);

    // token-weighted loss
    expect("loss P=0", sp_weighted_loss(fa, pos, 0, 1024, -100, fa, fa, (int64_t *)a, fa, NULL), SP_E_SHAPE);
    expect("loss N%P", sp_weighted_loss(fa, pos, 3, 1024, -100, fa, fa, (int64_t *)a, fa, NULL),
           SP_E_NOT_DIVISIBLE);
    expect("loss null", sp_weighted_loss(fa, pos, 4, 1024, -100, NULL, fa, (int64_t *)a, fa, NULL),
           SP_E_NULL);
    expect("loss align", sp_weighted_loss(fa, (const int64_t *)mis, 4, 1024, -100, fa, fa, (int64_t *)a,
                                          fa, NULL), SP_E_ALIGN);
    expect("loss max N", sp_weighted_loss(fa, pos, 1, big, -100, fa, fa, (int64_t *)a, fa, NULL),
           SP_E_SHAPE);

    if (failures) {
        printf("%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("abi driver: all expectations held\n");
    return 0;
}
