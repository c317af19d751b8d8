/*
 * A C consumer of the library's C ABI (include/shortconv.h), for tests/test_gpu_c_abi.py: it
 * reads one prefill's inputs from raw files in a directory, copies them into device buffers it
 * allocates itself, calls shortconv_kv_prefill on the null stream, and writes the caches and the
 * state pools back to files. Nothing but the header and the HIP runtime: no torch, no Python
 * types, plain C99.
 *
 * Files (raw little-endian arrays): meta.txt ("T N H D W S num_slots dtype eps"), k.bin, v.bin
 * ([T][H][D], contiguous), kt.bin, vt.bin (fp32 [W][H][D]), kg.bin, vg.bin (fp32 [D]), cu.bin
 * (int32 [N+1]), sidx.bin (int32 [N]), hinit.bin (uint8 [N]), slot.bin (int64 [T]), ks.bin,
 * vs.bin ([S][W-1][H][D]), kc.bin, vc.bin ([num_slots][H][D], initial contents). Outputs:
 * kc_out.bin, vc_out.bin, ks_out.bin, vs_out.bin.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "shortconv.h"

#define MAXBUF 16

struct bufs {
    void* host[MAXBUF];
    void* dev[MAXBUF];
    int n;
};

static void* load(const char* dir, const char* name, size_t want, struct bufs* b) {
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* h = malloc(want > 0 ? want : 1);
    size_t got = want > 0 ? fread(h, 1, want, f) : 0;
    fclose(f);
    if (got != want) {
        free(h);
        return NULL;
    }
    void* d = NULL;
    if (want > 0 && (hipMalloc(&d, want) != hipSuccess ||
                     hipMemcpy(d, h, want, hipMemcpyHostToDevice) != hipSuccess)) {
        free(h);
        return NULL;
    }
    b->host[b->n] = h;
    b->dev[b->n] = d;
    b->n++;
    return d;
}

static int store(const char* dir, const char* name, const void* dev, size_t bytes) {
    char path[1024];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    void* h = malloc(bytes > 0 ? bytes : 1);
    if (bytes > 0 && hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
        free(h);
        return -1;
    }
    FILE* f = fopen(path, "wb");
    size_t put = f ? fwrite(h, 1, bytes, f) : 0;
    if (f) fclose(f);
    free(h);
    return put == bytes ? 0 : -1;
}

/* Returns the library's return code, or -100 for a file or runtime failure here. */
int sc_c_prefill(const char* dir) {
    char path[1024];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* m = fopen(path, "r");
    long long T, N, H, D, W, S, slots, dtype;
    float eps;
    if (!m) return -100;
    int ok = fscanf(m, "%lld %lld %lld %lld %lld %lld %lld %lld %f", &T, &N, &H, &D, &W, &S,
                    &slots, &dtype, &eps) == 9;
    fclose(m);
    if (!ok) return -100;
    const size_t e = dtype == SC_DTYPE_F32 ? 4 : 2;
    const size_t row = (size_t)(H * D) * e;
    const size_t srows = (size_t)(S * (W - 1));
    struct bufs b = {{0}, {0}, 0};
    void* k = load(dir, "k.bin", (size_t)T * row, &b);
    void* v = load(dir, "v.bin", (size_t)T * row, &b);
    void* kt = load(dir, "kt.bin", (size_t)(W * H * D) * 4, &b);
    void* vt = load(dir, "vt.bin", (size_t)(W * H * D) * 4, &b);
    void* kg = load(dir, "kg.bin", (size_t)D * 4, &b);
    void* vg = load(dir, "vg.bin", (size_t)D * 4, &b);
    void* cu = load(dir, "cu.bin", (size_t)(N + 1) * 4, &b);
    void* sidx = load(dir, "sidx.bin", (size_t)N * 4, &b);
    void* hinit = load(dir, "hinit.bin", (size_t)N, &b);
    void* slot = load(dir, "slot.bin", (size_t)T * 8, &b);
    void* ks = load(dir, "ks.bin", srows * row, &b);
    void* vs = load(dir, "vs.bin", srows * row, &b);
    void* kc = load(dir, "kc.bin", (size_t)slots * row, &b);
    void* vc = load(dir, "vc.bin", (size_t)slots * row, &b);
    int rc = -100;
    if (b.n == 14) {
        rc = shortconv_kv_prefill(k, v, H * D, H * D, (const int32_t*)cu, (int32_t)N, T,
                                  (const float*)kt, (const float*)vt, (const float*)kg,
                                  (const float*)vg, eps, ks, vs, S, (const int32_t*)sidx,
                                  (const uint8_t*)hinit, (const int64_t*)slot, kc, vc, slots,
                                  (int32_t)H, (int32_t)D, (int32_t)W, (int32_t)dtype, NULL);
        if (rc == SC_OK && hipDeviceSynchronize() != hipSuccess) rc = -100;
        if (rc == SC_OK &&
            (store(dir, "kc_out.bin", kc, (size_t)slots * row) ||
             store(dir, "vc_out.bin", vc, (size_t)slots * row) ||
             store(dir, "ks_out.bin", ks, srows * row) || store(dir, "vs_out.bin", vs, srows * row)))
            rc = -100;
    }
    for (int i = 0; i < b.n; ++i) {
        free(b.host[i]);
        if (b.dev[i]) hipFree(b.dev[i]);
    }
    return rc;
}
