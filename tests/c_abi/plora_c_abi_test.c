/*
 * plora_c_abi_test.c -- the packed multi-LoRA operator driven from plain C
 * through include/plora.h: device buffers from the HIP runtime, the three
 * entry points on the null stream, results checked against the fp64 oracle
 * (oracle/plora_oracle.c, linked in: this program is test infrastructure).
 *
 * Problem: d_in 256, d_out 384 (pipelined kernels both ways), three adapters
 * of ranks 8, 16 and 64 over 70, 0 and 130 tokens, bf16 inputs drawn from a
 * fixed linear congruential generator.  Checks, per output and in relative
 * Frobenius norm: Y and dX (bf16) within 2e-2, H, G, dA and dB (fp32) within
 * 1e-4, against the oracle run on the same bf16-rounded inputs.  Prints PASS
 * and returns 0, or prints what failed and returns 1.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "plora.h"

int oracle_packed_lora(int n, int64_t T, const int64_t* off, const int32_t* ranks, const double* alphas, int64_t d_in,
                       int64_t d_out, const double* X, const double* dY, const double* W, const double* A,
                       const double* B, double* Y, double* H, double* dX, double* G, double* dA, double* dB);

static uint64_t g_state = 0x2545F4914F6CDD1Dull;
static double uniform(void) { /* Knuth's MMIX LCG, top 53 bits */
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(g_state >> 11) / 9007199254740992.0;
}
static double normal(void) { /* Box-Muller */
    const double u = uniform() + 1e-300, v = uniform();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
/* fp32 -> bf16, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

#define CHECK_HIP(x)                                                            \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            printf("FAIL: %s: %s\n", #x, hipGetErrorString(e_));                \
            return 1;                                                           \
        }                                                                       \
    } while (0)
#define CHECK_PLORA(x)                                                          \
    do {                                                                        \
        int r_ = (x);                                                           \
        if (r_ != PLORA_OK) {                                                   \
            printf("FAIL: %s: %s\n", #x, plora_last_error());                   \
            return 1;                                                           \
        }                                                                       \
    } while (0)

/* bf16 tensor: host draws (scaled normal), rounded, uploaded; the rounded
 * values as doubles for the oracle */
static int make_bf16(size_t n, double scale, double** host, void** dev) {
    uint16_t* h = (uint16_t*)malloc(n * 2);
    *host = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        h[i] = to_bf16((float)(scale * normal()));
        (*host)[i] = from_bf16(h[i]);
    }
    if (hipMalloc(dev, n * 2 > 0 ? n * 2 : 16) != hipSuccess) return 1;
    if (n && hipMemcpy(*dev, h, n * 2, hipMemcpyHostToDevice) != hipSuccess) return 1;
    free(h);
    return 0;
}

static double rel_err_bf16(const uint16_t* got, const double* ref, size_t n) {
    double num = 0, den = 0;
    for (size_t i = 0; i < n; ++i) {
        const double d = from_bf16(got[i]) - ref[i];
        num += d * d;
        den += ref[i] * ref[i];
    }
    return den > 0 ? sqrt(num / den) : sqrt(num);
}
static double rel_err_f32(const float* got, const double* ref, size_t n) {
    double num = 0, den = 0;
    for (size_t i = 0; i < n; ++i) {
        const double d = (double)got[i] - ref[i];
        num += d * d;
        den += ref[i] * ref[i];
    }
    return den > 0 ? sqrt(num / den) : sqrt(num);
}

int main(void) {
    const int n = 3;
    const int64_t off[4] = {0, 70, 70, 200};
    const int32_t ranks[3] = {8, 16, 64};
    const float alphas[3] = {16.0f, 8.0f, 128.0f};
    const double alphas_d[3] = {16.0, 8.0, 128.0};
    const int64_t T = 200, d_in = 256, d_out = 384, R = 8 + 16 + 64;
    plora_desc d = {n, PLORA_BF16, T, d_in, d_out, off, ranks, alphas};
    CHECK_PLORA(plora_validate(&d));
    const size_t he = plora_h_elems(&d), ws_bytes = plora_workspace_bytes(&d);

    double *hX, *hW, *hA, *hB, *hdY;
    void *X, *W, *A, *B, *dY;
    if (make_bf16((size_t)(T * d_in), 1.0, &hX, &X) || make_bf16((size_t)(d_out * d_in), 1.0 / 16.0, &hW, &W) ||
        make_bf16((size_t)(R * d_in), 0.125, &hA, &A) || make_bf16((size_t)(R * d_out), 0.02, &hB, &B) ||
        make_bf16((size_t)(T * d_out), 1.0, &hdY, &dY)) {
        printf("FAIL: device allocation or upload\n");
        return 1;
    }
    void *Y, *dX, *ws = NULL;
    float *H, *G, *dA, *dB;
    CHECK_HIP(hipMalloc(&Y, (size_t)(T * d_out) * 2));
    CHECK_HIP(hipMalloc(&dX, (size_t)(T * d_in) * 2));
    CHECK_HIP(hipMalloc((void**)&H, he * 4));
    CHECK_HIP(hipMalloc((void**)&G, he * 4));
    CHECK_HIP(hipMalloc((void**)&dA, (size_t)(R * d_in) * 4));
    CHECK_HIP(hipMalloc((void**)&dB, (size_t)(R * d_out) * 4));
    if (ws_bytes) CHECK_HIP(hipMalloc(&ws, ws_bytes));

    CHECK_PLORA(plora_forward(&d, X, W, A, B, Y, H, NULL));
    CHECK_PLORA(plora_backward_dx(&d, dY, W, A, B, dX, G, NULL));
    CHECK_PLORA(plora_backward_dAdB(&d, X, dY, H, G, dA, dB, ws, ws_bytes, NULL));
    CHECK_HIP(hipDeviceSynchronize());

    uint16_t* gY = (uint16_t*)malloc((size_t)(T * d_out) * 2);
    uint16_t* gdX = (uint16_t*)malloc((size_t)(T * d_in) * 2);
    float* gH = (float*)malloc(he * 4);
    float* gG = (float*)malloc(he * 4);
    float* gdA = (float*)malloc((size_t)(R * d_in) * 4);
    float* gdB = (float*)malloc((size_t)(R * d_out) * 4);
    CHECK_HIP(hipMemcpy(gY, Y, (size_t)(T * d_out) * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdX, dX, (size_t)(T * d_in) * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gH, H, he * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gG, G, he * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdA, dA, (size_t)(R * d_in) * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gdB, dB, (size_t)(R * d_out) * 4, hipMemcpyDeviceToHost));

    double* rY = (double*)malloc((size_t)(T * d_out) * sizeof(double));
    double* rdX = (double*)malloc((size_t)(T * d_in) * sizeof(double));
    double* rH = (double*)malloc(he * sizeof(double));
    double* rG = (double*)malloc(he * sizeof(double));
    double* rdA = (double*)malloc((size_t)(R * d_in) * sizeof(double));
    double* rdB = (double*)malloc((size_t)(R * d_out) * sizeof(double));
    if (oracle_packed_lora(n, T, off, ranks, alphas_d, d_in, d_out, hX, hdY, hW, hA, hB, rY, rH, rdX, rG, rdA, rdB)) {
        printf("FAIL: oracle\n");
        return 1;
    }
    /* the oracle's scale is alpha / r in double; the library's in fp32: both exact here */
    const double eY = rel_err_bf16(gY, rY, (size_t)(T * d_out)), edX = rel_err_bf16(gdX, rdX, (size_t)(T * d_in));
    const double eH = rel_err_f32(gH, rH, he), eG = rel_err_f32(gG, rG, he);
    const double edA = rel_err_f32(gdA, rdA, (size_t)(R * d_in)), edB = rel_err_f32(gdB, rdB, (size_t)(R * d_out));
    printf("library %s (ABI %d); relative Frobenius errors: Y %.3e dX %.3e H %.3e G %.3e dA %.3e dB %.3e\n",
           plora_source_hash(), plora_version(), eY, edX, eH, eG, edA, edB);
    const int ok = eY <= 2e-2 && edX <= 2e-2 && eH <= 1e-4 && eG <= 1e-4 && edA <= 1e-4 && edB <= 1e-4;
    /* the empty adapter's gradient rows are written as zeros */
    int zero_ok = 1;
    for (int64_t j = 8 * d_in; j < 24 * d_in; ++j) zero_ok &= gdA[j] == 0.0f;
    printf("%s\n", ok && zero_ok ? "PASS" : "FAIL: outside the tolerances or the empty adapter's dA not zero");
    return ok && zero_ok ? 0 : 1;
}
