/* A C99 caller of libqhead: the header compiles as plain C (-pedantic) and
 * the host-side entry points answer without a GPU. Built and run by
 * tests/test_abi_cpu.py. */
#include "qhead.h"

#include <stdio.h>
#include <string.h>

int main(void) {
    int32_t chunks[8];
    int fails = 0;
    if (qhead_plan_chunks(QHEAD_FMT_FP8, 40, chunks, 8) != 3) fails++;
    if (chunks[0] != 16 || chunks[1] != 16 || chunks[2] != 8) fails++;
    if (qhead_plan_chunks(QHEAD_FMT_W8A8, 300, chunks, 8) != 3 || chunks[2] != 44) fails++;
    if (qhead_max_rows_per_launch(QHEAD_FMT_Q6K) != 8) fails++;
    if (qhead_w8a8_workspace_bytes(7168) % 256 != 0) fails++;
    if (strcmp(qhead_status_string(QHEAD_OK), qhead_status_string(QHEAD_ERR_SHAPE)) == 0) fails++;
    /* rows == 0 succeeds without looking at the pointers; a bad shape fails first */
    if (qhead_fp8_rowscale(NULL, NULL, NULL, 0, 16, 8, NULL, NULL) != QHEAD_OK) fails++;
    if (qhead_nvfp4(NULL, NULL, NULL, 1, 48, 8, NULL, 1.0f, NULL) != QHEAD_ERR_SHAPE) fails++;
    if (qhead_q6k_gemv(NULL, NULL, 0, 512, 8, NULL, NULL) != QHEAD_OK) fails++;
    printf("c abi smoke: %d failure(s)\n", fails);
    return fails;
}
