/* Plain C caller of liblgn.so: include/lgn.h compiles as C99 and the
 * library's host helpers and argument checks answer without a GPU (every call
 * below returns before any HIP call).  Prints "ok" and exits 0, or names the
 * first failed check and exits 1. */
#include <stdio.h>
#include <string.h>

#include "lgn.h"

#define CHECK(cond)                                        \
    do {                                                   \
        if (!(cond)) {                                     \
            printf("failed: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                      \
        }                                                  \
    } while (0)

int main(void) {
    CHECK(lgn_version() != NULL && strlen(lgn_version()) > 0);
    CHECK(strcmp(lgn_status_string(LGN_OK), lgn_status_string(LGN_ERR_INVALID_ARG)) != 0);
    CHECK(lgn_twopass_workspace_bytes(1024, 4096) == (size_t)1024 * 4096 * 4);
    CHECK(lgn_wide_workspace_bytes(16384, 16384) == LGN_WIDE_NOALLOC_SCRATCH_BYTES);
    CHECK(lgn_fused_supported(0, 32768, 1024, 4096, 64) == 1);   /* 64 channels per group */
    CHECK(lgn_fused_supported(1, 32768, 1024, 4096, 64) == 1);
    CHECK(lgn_fused_supported(0, 64, 32, 4096, 1) == 0);         /* 4096 channels per group */
    /* null pointers with a non-empty problem: rejected before any HIP call */
    CHECK(lgn_forward_f32(NULL, NULL, NULL, NULL, NULL, NULL, 64, 32, 128, 8, 1e-5f, NULL,
                          (hipStream_t)0) == LGN_ERR_INVALID_ARG);
    CHECK(lgn_forward_bf16(NULL, NULL, NULL, NULL, NULL, NULL, 64, 32, 128, 8, 1e-5f, NULL,
                           (hipStream_t)0) == LGN_ERR_INVALID_ARG);
    CHECK(lgn_linear_lse_f32(NULL, NULL, NULL, 4, 32, 128, NULL, NULL, 0, (hipStream_t)0) ==
          LGN_ERR_INVALID_ARG);
    printf("ok\n");
    return 0;
}
