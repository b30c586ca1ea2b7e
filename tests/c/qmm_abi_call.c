/*
 * qmm_abi_call.c -- drives the C ABI (include/qmm.h) from C, with no Python
 * or torch in the process: reads x, Q, scales and (optionally) zeros from
 * files, makes one qmm_gemv call, writes y (fp32) to a file, then times
 * eager calls -- the host-side cost of one call (steady clock around the
 * call itself) and the device time per call (HIP events around the batch).
 *
 *   qmm_abi_call M N K w_bit group_size x_dtype x.bin Q.bin S.bin Z.bin|- y.bin calls
 *
 * Prints one JSON line.  Exit status 0 on success, 1 on any failed call.
 */
#define _POSIX_C_SOURCE 200809L
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <time.h>

#include "qmm.h"

static void* read_file(const char* path, size_t* n) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    fseek(f, 0, SEEK_END);
    long len = ftell(f);
    fseek(f, 0, SEEK_SET);
    void* buf = malloc(len > 0 ? (size_t)len : 1);
    if (buf && fread(buf, 1, (size_t)len, f) != (size_t)len) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    *n = (size_t)len;
    return buf;
}

static void* to_device(const char* path, size_t* n) {
    void* h = read_file(path, n);
    if (!h) return NULL;
    void* d = NULL;
    if (hipMalloc(&d, *n ? *n : 16) != hipSuccess || hipMemcpy(d, h, *n, hipMemcpyHostToDevice) != hipSuccess)
        d = NULL;
    free(h);
    return d;
}

static double now_us(void) {
    struct timespec t;
    clock_gettime(CLOCK_MONOTONIC, &t);
    return t.tv_sec * 1e6 + t.tv_nsec * 1e-3;
}

int main(int argc, char** argv) {
    if (argc != 13) {
        fprintf(stderr, "usage: %s M N K w_bit group_size x_dtype x Q S Z|- y calls\n", argv[0]);
        return 2;
    }
    int M = atoi(argv[1]), N = atoi(argv[2]), K = atoi(argv[3]), w_bit = atoi(argv[4]);
    int gs = atoi(argv[5]), xdt = atoi(argv[6]), calls = atoi(argv[12]);
    size_t nx, nq, ns, nz = 0;
    void* x = to_device(argv[7], &nx);
    void* Q = to_device(argv[8], &nq);
    void* S = to_device(argv[9], &ns);
    void* Z = argv[10][0] == '-' ? NULL : to_device(argv[10], &nz);
    float* y = NULL;
    size_t ny = (size_t)M * N * sizeof(float);
    if (!x || !Q || !S || (argv[10][0] != '-' && !Z) || hipMalloc((void**)&y, ny) != hipSuccess) {
        fprintf(stderr, "input or allocation failed\n");
        return 1;
    }
    hipStream_t st;
    hipStreamCreate(&st);
    qmm_status s = qmm_gemv(x, Q, S, Z, y, M, N, K, w_bit, gs, xdt, NULL, 0, st);
    if (s != QMM_OK) {
        fprintf(stderr, "qmm_gemv: %d %s\n", (int)s, qmm_last_error());
        return 1;
    }
    hipStreamSynchronize(st);
    float* yh = (float*)malloc(ny);
    hipMemcpy(yh, y, ny, hipMemcpyDeviceToHost);
    FILE* f = fopen(argv[11], "wb");
    if (!f || fwrite(yh, 1, ny, f) != ny) return 1;
    fclose(f);

    /* eager calls: host cost of each call, device time of the batch */
    hipEvent_t e0, e1;
    hipEventCreate(&e0);
    hipEventCreate(&e1);
    for (int i = 0; i < 20; ++i) qmm_gemv(x, Q, S, Z, y, M, N, K, w_bit, gs, xdt, NULL, 0, st);
    hipStreamSynchronize(st);
    double host = 0.0;
    hipEventRecord(e0, st);
    for (int i = 0; i < calls; ++i) {
        double t0 = now_us();
        s = qmm_gemv(x, Q, S, Z, y, M, N, K, w_bit, gs, xdt, NULL, 0, st);
        host += now_us() - t0;
        if (s != QMM_OK) return 1;
    }
    hipEventRecord(e1, st);
    hipEventSynchronize(e1);
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    printf("{\"calls\": %d, \"host_us_per_call\": %.3f, \"device_us_per_call\": %.3f}\n", calls,
           host / calls, 1e3 * ms / calls);
    return 0;
}
