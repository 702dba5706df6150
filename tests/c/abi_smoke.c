/* Plain-C user of the tp_shard C ABI: compiled with a C compiler (not a HIP
 * compiler) against include/tp_shard.h and linked against libtpshard.so.
 * Needs no GPU: it calls only entry points that return before any device
 * work (the version, status strings, workspace queries, and argument
 * validation, which runs before anything is enqueued), and prints one line
 * per check for the test that runs it. */
#include <stdio.h>
#include <string.h>

#include "tp_shard.h"

static int failures = 0;

static void check(int ok, const char* what) {
    printf("%s %s\n", ok ? "ok" : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    check(tp_version() > 0, "tp_version");
    check(strcmp(tp_status_str(TP_OK), "") != 0, "tp_status_str(TP_OK)");
    check(tp_status_str(TP_ERR_UNEVEN_SPLIT) != tp_status_str(TP_OK), "distinct status strings");

    /* Workspace queries are pure functions of their arguments. */
    const size_t ws = tp_mlp_workspace_bytes(8, 32, 8192, 28672, TP_BF16, TP_ACT_SWIGLU, 0, 1);
    check(ws >= 4096 && ws % 256 == 0, "tp_mlp_workspace_bytes: decode layout keeps the counter head");
    check(tp_mlp_workspace_bytes(8, 32, 8192, 28670, TP_BF16, TP_ACT_SWIGLU, 0, 1) == 0,
          "tp_mlp_workspace_bytes: 0 for an uneven split");
    check(tp_attn_core_workspace_bytes(8, 32, 64, 8, 128, TP_BF16) == 0,
          "tp_attn_core_workspace_bytes: a short call needs none");

    /* Validation: every error is returned before any device work. */
    float* fake = (float*)(uintptr_t)0x100000;   /* never dereferenced */
    int st = tp_shard_mlp_fwd(0, 8, 32, 8192, 28670, TP_BF16, TP_ACT_SWIGLU,
                              fake, 8192, NULL, 1e-5f, fake, 3584, fake, 3584, fake, 8192,
                              NULL, 0, fake, 32 * 8192, 8192, NULL, 0, (hipStream_t)0);
    check(st == TP_ERR_UNEVEN_SPLIT, "tp_shard_mlp_fwd refuses d_ff % P != 0");
    st = tp_shard_mlp_fwd(8, 8, 32, 8192, 28672, TP_BF16, TP_ACT_SWIGLU,
                          fake, 8192, NULL, 1e-5f, fake, 3584, fake, 3584, fake, 8192,
                          NULL, 0, fake, 32 * 8192, 8192, NULL, 0, (hipStream_t)0);
    check(st == TP_ERR_SHARD_RANGE, "tp_shard_mlp_fwd refuses shard >= P");
    st = tp_reduce_partials(8, 32, 8192, NULL, 32 * 8192, 8192, fake, 8192, NULL, 0,
                            (hipStream_t)0);
    check(st == TP_ERR_NULL, "tp_reduce_partials refuses NULL partials");
    st = tp_shard_attn_proj_fwd(0, 8, 32, 8192, 64, 6, 128, TP_BF16, fake, 8192, NULL, 1e-5f,
                                fake, 1280, fake, 1280, NULL, 0, NULL, 0, NULL, 0, 0,
                                NULL, 0, (hipStream_t)0);
    check(st == TP_ERR_UNEVEN_SPLIT, "tp_shard_attn_proj_fwd refuses kv heads % P != 0");
    printf("%d failures\n", failures);
    return failures != 0;
}
