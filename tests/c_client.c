/* A C99 caller of the library's C ABI (include/attn.h), linked against
 * libattn.so.  It uses only entry points that make no HIP call: the ring plan
 * (host bookkeeping) and argument validation, which happens before any HIP
 * call, so it runs on a machine without a GPU. */
#include <stdio.h>
#include <stddef.h>
#include "attn.h"

int main(void) {
    attn_ring_call plan[32];
    int i, n, rc, merges = 0;
    /* the 128K zigzag share of rank 0 of 8: 17 live sub-calls, 15 of them
       merging into the late chunk's partial */
    n = attn_ring_plan(131072, 8, 0, 1, 1, plan, 32);
    for (i = 0; i < n; ++i) merges += plan[i].accumulate;
    printf("plan %d merges %d first_block %d last_kv_pos0 %lld\n", n, merges, plan[0].block,
           n > 0 ? plan[n - 1].kv_pos0 : -1LL);
    /* an unsupported head dim is rejected before any HIP call */
    rc = attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 16, 96, 0, 0, 1, NULL, NULL, 0.0, ATTN_BF16, 0, NULL);
    printf("rc %d unsupported %d\n", rc, rc == ATTN_ERR_UNSUPPORTED);
    printf("message %s\n", attn_last_error());
    printf("version %d\n", attn_version());
    return 0;
}
