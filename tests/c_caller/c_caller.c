/*
 * A plain C caller of liba2av.so (include/a2av.h): no Python, no torch.  It allocates
 * with the HIP runtime, builds a small routing step from integer formulas, runs
 * dispatch -> expert stand-in -> combine on the direct path and on the staged path,
 * and writes what came back (receive counts and offsets, receive rows, y) as raw bytes
 * to the file named by argv[1], for tests/test_c_caller_gpu.py to check against the
 * oracle.  Shape: 4 ranks x 64 tokens, hidden 128 float32, 8 experts (2 per rank), top-2.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "a2av.h"

enum { R = 4, T = 64, H = 128, EPR = 2, E = R * EPR, K = 2 };

#define HIP_OK(x) do { if ((x) != hipSuccess) { fprintf(stderr, "HIP call failed at line %d\n", __LINE__); return 1; } } while (0)
#define A2AV_OK_(x) do { int rc_ = (x); if (rc_ != A2AV_OK) { fprintf(stderr, "%s at line %d\n", a2av_error_string(rc_), __LINE__); return 1; } } while (0)

static int run(int path, FILE* out) {
    const int64_t cap = (int64_t)R * T * K;   /* worst case R*T*min(k, epr) */
    static float x[R][T][H], y[R][T][H], gates[R][T][K];
    static int32_t ids[R][T][K];
    for (int s = 0; s < R; ++s)
        for (int t = 0; t < T; ++t) {
            for (int h = 0; h < H; ++h) x[s][t][h] = (float)(s * 256 + t) + (float)h / 128.0f;
            for (int j = 0; j < K; ++j) {
                ids[s][t][j] = (s * 3 + t * 5 + j * 3) % E;   /* the two slots differ: 3 and 8 are coprime */
                gates[s][t][j] = j == 0 ? 0.75f : 0.25f;
            }
        }
    a2av_config_t cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.num_ranks = R; cfg.tokens_per_rank = T; cfg.hidden = H; cfg.dtype = A2AV_F32;
    cfg.experts_per_rank = EPR; cfg.top_k = K; cfg.recv_capacity_rows = cap;
    cfg.path = path; cfg.recv_layout = A2AV_LAYOUT_SOURCE_MAJOR;
    a2av_handle_t h;
    A2AV_OK_(a2av_create(&cfg, &h));
    void *dx, *dy, *dg, *dids, *drecv, *dcounts, *doffs, *dstatus;
    HIP_OK(hipMalloc(&dx, sizeof x));
    HIP_OK(hipMalloc(&dy, sizeof y));
    HIP_OK(hipMalloc(&dg, sizeof gates));
    HIP_OK(hipMalloc(&dids, sizeof ids));
    HIP_OK(hipMalloc(&drecv, sizeof(float) * R * cap * H));
    HIP_OK(hipMalloc(&dcounts, sizeof(int32_t) * R * R));
    HIP_OK(hipMalloc(&doffs, sizeof(int32_t) * R * (R + 1)));
    HIP_OK(hipMalloc(&dstatus, sizeof(uint32_t)));
    HIP_OK(hipMemset(dstatus, 0, sizeof(uint32_t)));
    HIP_OK(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dg, gates, sizeof gates, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dids, ids, sizeof ids, hipMemcpyHostToDevice));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    A2AV_OK_(a2av_dispatch(h, dx, (const int32_t*)dids, drecv, NULL, (int32_t*)dcounts, (int32_t*)doffs,
                           (uint32_t*)dstatus, st));
    A2AV_OK_(a2av_expert_apply(h, drecv, drecv, A2AV_EXPERT_IDENTITY, st));
    A2AV_OK_(a2av_combine(h, drecv, (const float*)dg, dy, (uint32_t*)dstatus, st));
    HIP_OK(hipStreamSynchronize(st));
    int32_t counts[R * R], offs[R * (R + 1)];
    uint32_t status;
    float* recv = (float*)malloc(sizeof(float) * R * cap * H);
    if (!recv) return 1;
    HIP_OK(hipMemcpy(counts, dcounts, sizeof counts, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(offs, doffs, sizeof offs, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&status, dstatus, sizeof status, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv, drecv, sizeof(float) * R * cap * H, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, dy, sizeof y, hipMemcpyDeviceToHost));
    fwrite(&status, sizeof status, 1, out);
    fwrite(counts, sizeof counts, 1, out);
    fwrite(offs, sizeof offs, 1, out);
    fwrite(recv, sizeof(float), (size_t)R * cap * H, out);
    fwrite(y, sizeof y, 1, out);
    free(recv);
    HIP_OK(hipStreamDestroy(st));
    HIP_OK(hipFree(dx)); HIP_OK(hipFree(dy)); HIP_OK(hipFree(dg)); HIP_OK(hipFree(dids));
    HIP_OK(hipFree(drecv)); HIP_OK(hipFree(dcounts)); HIP_OK(hipFree(doffs)); HIP_OK(hipFree(dstatus));
    A2AV_OK_(a2av_destroy(h));
    return 0;
}

int main(int argc, char** argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s OUT\n", argv[0]); return 2; }
    FILE* out = fopen(argv[1], "wb");
    if (!out) return 2;
    int rc = run(A2AV_PATH_DIRECT, out);
    if (rc == 0) rc = run(A2AV_PATH_STAGED, out);
    fclose(out);
    if (rc == 0) printf("c caller ok\n");
    return rc;
}
