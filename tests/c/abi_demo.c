/*
 * The C ABI used from plain C (every library call made from C, not through
 * the Python binding): calibrate -> weight
 * ranges -> plan -> quantize -> dual GEMM on a small synthetic layer, with
 * the HIP runtime for device memory.  Every input and artefact is copied back
 * and written to a file of named blobs; tests/test_gpu_c_abi.py checks them
 * against the CPU oracle.
 *
 *   abi_demo OUT_FILE
 *
 * Built twice: as that executable, and (with ABI_DEMO_LIB) as a shared object
 * exporting abi_demo_run(), which the test calls in its own process.
 * Blob format: 16-byte zero-padded name, uint64 byte count, bytes.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mixed_gemm.h"

#define CK(x)                                                                          \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)
#define MG(x)                                                                          \
    do {                                                                               \
        int e_ = (x);                                                                  \
        if (e_ != MG_OK) {                                                             \
            fprintf(stderr, "mg error %d at line %d: %s\n", e_, __LINE__, mg_last_error()); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

enum { M = 300, K = 512, N = 192, KOUT = 12 };

static uint32_t rng_state = 12345u;
static float unit(void) {            /* uniform in [-1, 1): input recipe only */
    rng_state = rng_state * 1664525u + 1013904223u;
    return (float)(rng_state >> 8) * (2.0f / 16777216.0f) - 1.0f;
}
static uint16_t to_bf16(float f) {   /* round to nearest even: input recipe only */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static FILE* out;
static int blob(const char* name, const void* dev_or_host, size_t bytes, int on_device) {
    char tag[16] = {0};
    uint64_t n = bytes;
    void* h = malloc(bytes ? bytes : 1);
    if (!h) return 1;
    if (on_device && bytes) {
        if (hipMemcpy(h, dev_or_host, bytes, hipMemcpyDeviceToHost) != hipSuccess) return 1;
    } else if (bytes) {
        memcpy(h, dev_or_host, bytes);
    }
    strncpy(tag, name, 15);
    fwrite(tag, 1, 16, out);
    fwrite(&n, 8, 1, out);
    fwrite(h, 1, bytes, out);
    free(h);
    return 0;
}

int abi_demo_run(const char* path) {
    rng_state = 12345u;
    printf("mixed_gemm C ABI version %d\n", mg_version());

    /* host inputs: X ~ U(-0.25, 0.25) with every 37th channel x25; W ~ U(-0.02, 0.02) */
    static uint16_t X[M * K], W[N * K];
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < K; ++j) {
            float v = 0.25f * unit();
            if (j % 37 == 5) v *= 25.0f;
            X[m * K + j] = to_bf16(v);
        }
    X[7 * K + 3] = 0x8000u;          /* a negative zero */
    for (int i = 0; i < N * K; ++i) W[i] = to_bf16(0.02f * unit());

    hipStream_t st;
    CK(hipStreamCreate(&st));
    uint16_t *dX, *dW, *dY;
    float *act_max, *w_max, *dY32;
    CK(hipMalloc((void**)&dX, sizeof X));
    CK(hipMalloc((void**)&dW, sizeof W));
    CK(hipMalloc((void**)&act_max, K * sizeof(float)));
    CK(hipMalloc((void**)&w_max, K * sizeof(float)));
    CK(hipMalloc((void**)&dY, (size_t)M * N * 2));
    CK(hipMalloc((void**)&dY32, (size_t)M * N * 4));
    CK(hipMemcpy(dX, X, sizeof X, hipMemcpyHostToDevice));
    CK(hipMemcpy(dW, W, sizeof W, hipMemcpyHostToDevice));

    /* an invalid call fails on the host with a message and touches nothing */
    if (mg_calib_act(dX, MG_BF16, M, 60, act_max, st) != MG_ERR_SHAPE || mg_last_error()[0] == 0) {
        fprintf(stderr, "expected MG_ERR_SHAPE for K = 60\n");
        return 1;
    }

    /* plan and activation buffers, sized by the library */
    mg_plan_desc d = {K, N, KOUT, MG_W_1X32, 1, MG_SCORE_MAX, 0.6};
    size_t pb[8], ab[3];
    MG(mg_plan_bytes(&d, pb));
    MG(mg_act_bytes(&d, M, ab));
    void* pbuf[8] = {0};
    for (int i = 0; i < 8; ++i)
        if (pb[i]) CK(hipMalloc(&pbuf[i], pb[i]));
    void* abuf[3] = {0};
    for (int i = 0; i < 3; ++i)
        if (ab[i]) CK(hipMalloc(&abuf[i], ab[i]));
    mg_plan p = {d, (float*)pbuf[0], (float*)pbuf[1], (int32_t*)pbuf[2], (int32_t*)pbuf[3],
                 (uint8_t*)pbuf[4], (uint8_t*)pbuf[5], (uint8_t*)pbuf[6], (uint16_t*)pbuf[7]};
    mg_act a = {(uint8_t*)abuf[0], (uint8_t*)abuf[1], (uint16_t*)abuf[2]};

    /* calibrate (two batches) -> weight ranges -> plan -> forward (bf16 and f32 outputs) */
    MG(mg_calib_reset(act_max, K, st));
    MG(mg_calib_act(dX, MG_BF16, 100, K, act_max, st));
    MG(mg_calib_act(dX + 100 * K, MG_BF16, M - 100, K, act_max, st));
    MG(mg_weight_range(dW, MG_BF16, N, K, w_max, st));
    MG(mg_plan_build(&p, act_max, w_max, dW, MG_BF16, st));
    MG(mg_forward(&p, dX, MG_BF16, M, &a, dY, MG_BF16, st));
    MG(mg_dual_gemm(&p, &a, M, dY32, MG_F32, st));
    CK(hipStreamSynchronize(st));

    out = fopen(path, "wb");
    if (!out) {
        perror(path);
        return 1;
    }
    int32_t dims[4] = {M, K, N, KOUT};
    int bad = blob("dims", dims, sizeof dims, 0) || blob("X", dX, sizeof X, 1) || blob("W", dW, sizeof W, 1) ||
              blob("act_max", act_max, K * 4, 1) || blob("w_max", w_max, K * 4, 1);
    const char* pn[8] = {"s", "rcp", "O", "pos", "Wq", "Ws", "Wst", "WO"};
    for (int i = 0; i < 8; ++i) bad = bad || blob(pn[i], pbuf[i], pb[i], 1);
    const char* an[3] = {"Aq", "As", "XO"};
    for (int i = 0; i < 3; ++i) bad = bad || blob(an[i], abuf[i], ab[i], 1);
    bad = bad || blob("Y", dY, (size_t)M * N * 2, 1) || blob("Y32", dY32, (size_t)M * N * 4, 1);
    fclose(out);
    if (bad) {
        fprintf(stderr, "writing %s failed\n", path);
        return 1;
    }
    for (int i = 0; i < 8; ++i)
        if (pbuf[i]) CK(hipFree(pbuf[i]));
    for (int i = 0; i < 3; ++i)
        if (abuf[i]) CK(hipFree(abuf[i]));
    CK(hipFree(dX));
    CK(hipFree(dW));
    CK(hipFree(act_max));
    CK(hipFree(w_max));
    CK(hipFree(dY));
    CK(hipFree(dY32));
    CK(hipStreamDestroy(st));
    printf("ok\n");
    return 0;
}

#ifndef ABI_DEMO_LIB
int main(int argc, char** argv) {
    if (argc != 2) {
        fprintf(stderr, "usage: %s OUT_FILE\n", argv[0]);
        return 2;
    }
    return abi_demo_run(argv[1]);
}
#endif
