/* Plain C use of libgdn's ABI (no torch, no C++): version, status strings, and argument
 * validation, which runs before any device work, so this needs no GPU.  Built and run by
 * tests/test_c_abi.py; prints one line per check and exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdn.h"

static int fails = 0;
#define CHECK(cond, what)                                              \
    do {                                                               \
        if (cond) printf("ok   %s\n", what);                           \
        else { printf("FAIL %s\n", what); ++fails; }                   \
    } while (0)

int main(void) {
    float buf[4096];
    memset(buf, 0, sizeof buf);
    CHECK(gdn_version() >= 200, "version");
    CHECK(strcmp(gdn_status_str(GDN_OK), "ok") == 0, "status string");
    /* decode: HV not a multiple of HQK */
    gdn_status s = gdn_decode_step(buf, buf, buf, buf, buf, buf, buf, 1, 3, 4, 32, 32, GDN_F32, 1.0f, 0);
    CHECK(s == GDN_ERR_SHAPE && strlen(gdn_last_error()) > 0, "decode rejects HV % HQK != 0");
    /* prefill: head dim 48 unsupported */
    int32_t cu[2] = {0, 4};
    s = gdn_prefill(buf, buf, buf, buf, buf, cu, cu, 1, 4, NULL, buf, NULL, 1, 1, 48, 32, GDN_F32, 1.0f, NULL, 0, 0);
    CHECK(s == GDN_ERR_UNSUPPORTED, "prefill rejects dk = 48");
    /* prefill: host lengths that do not reach total_T */
    s = gdn_prefill(buf, buf, buf, buf, buf, cu, cu, 1, 5, NULL, buf, NULL, 1, 1, 32, 32, GDN_F32, 1.0f, NULL, 0, 0);
    CHECK(s == GDN_ERR_SEQLENS, "prefill rejects cu_seqlens[N] != total_T");
    /* an empty batch is a valid no-op */
    int32_t cu0[1] = {0};
    s = gdn_prefill(NULL, NULL, NULL, NULL, NULL, cu0, cu0, 0, 0, NULL, NULL, NULL, 1, 1, 32, 32, GDN_F32, 1.0f, NULL, 0, 0);
    CHECK(s == GDN_OK, "empty prefill");
    /* block parts: norm eps < 0 */
    s = gdn_gated_rmsnorm(buf, buf + 1024, buf + 2048, -1.0f, buf, 4, 32, GDN_F32, 0);
    CHECK(s == GDN_ERR_VALUE, "gated norm rejects eps < 0");
    /* the split plan: one 8192-token sequence with 16 heads takes the split path */
    CHECK(strcmp(gdn_prefill_kernel_name(1, 8192, NULL, 16, 16, 128, 128, GDN_BF16), "prefill_chunked_split") == 0,
          "kernel name of a split batch");
    printf("%s\n", fails ? "FAILED" : "all ok");
    return fails ? 1 : 0;
}
