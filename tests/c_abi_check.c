/* Calls the library from plain C (gcc, no HIP compiler): argument validation,
 * status strings, workspace sizes and the shape-only plan, none of which touch
 * a GPU.  Exits 0 when every check holds, else prints the failing line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bi.h"

#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            return 1;                                            \
        }                                                        \
    } while (0)

int main(void) {
    void *fake = (void *)(uintptr_t)(12345 * 4096); /* never dereferenced */
    int64_t chunk = 0;

    CHECK(strncmp(bi_status_string(BI_OK), "BI_OK", 5) == 0);
    CHECK(strncmp(bi_status_string(BI_ERR_WORKSPACE), "BI_ERR_WORKSPACE", 16) == 0);
    /* validation happens before any HIP call */
    CHECK(bi_forward(NULL, fake, fake, NULL, 4, 8, 8, BI_BF16, NULL, 1) == BI_ERR_NULL);
    CHECK(bi_forward(fake, fake, fake, NULL, 4, 8, 8, 9, NULL, 1) == BI_ERR_DTYPE);
    CHECK(bi_forward(fake, fake, fake, NULL, -1, 8, 8, BI_BF16, NULL, 1) == BI_ERR_SHAPE);
    CHECK(bi_forward(NULL, NULL, NULL, NULL, 0, 8, 8, BI_BF16, NULL, 1) == BI_OK);
    CHECK(bi_backward_dx(fake, NULL, fake, 4, 8, 8, BI_F16, NULL, 1) == BI_ERR_NULL);
    CHECK(bi_backward_dw(fake, fake, fake, 4096, 768, 48, BI_BF16, NULL, 0, NULL, 1) ==
          BI_ERR_WORKSPACE);
    CHECK(bi_backward_dw_workspace_bytes(4096, 768, 48, BI_BF16, 1) > 0);
    CHECK(bi_bias_grad_workspace_bytes(256, 100, BI_BF16) == 0);
    CHECK(bi_bias_grad_workspace_bytes(1000, 100, BI_BF16) == 4u * 100u * 4u);
    CHECK(bi_fp8_mm(fake, fake, fake, NULL, fake, 4, 64, 64, NULL, 1) == BI_ERR_NULL);
    CHECK(bi_fp8_quantize(fake, fake, fake, NULL, 16, 7, NULL) == BI_ERR_DTYPE);
    CHECK(bi_grouped_nt(fake, fake, fake, fake, fake, 4, 0, 8, 2, BI_BF16, NULL, 1) ==
          BI_ERR_SHAPE);
    /* tc = 2 where the automatic choice would fall back to the scalar tier */
    CHECK(bi_forward(fake, fake, fake, NULL, 4, 128, 48, BI_BF16, NULL, 2) == BI_ERR_UNSUPPORTED);
    /* the plan depends on (op, dtype, tc, k, n) only */
    CHECK(bi_plan(0, BI_BF16, 1, 768, 3072, &chunk) > 0);
    CHECK(bi_plan(0, BI_BF16, 0, 768, 3072, &chunk) == 0);
    CHECK(bi_plan(0, BI_F32, 1, 768, 3072, &chunk) == 0);
    printf("c abi ok\n");
    return 0;
}
