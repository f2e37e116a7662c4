/* A plain C caller of the lookup library: device buffers from hipMalloc, a
 * stream of its own, no Python and no torch anywhere in the process.
 *
 * Usage: pkm_forward_main <inputs> <outputs>
 *
 * <inputs> (little-endian, written by the test that runs this program):
 *   char[8] "PKMIN1\0\0"; int32 D, H, n_keys, k, value_type, prepare;
 *   int64 B, max_batch;
 *   float wq[H*D*D], bn_mean[H*D], bn_var[H*D], bn_gamma[H*D], bn_beta[H*D],
 *         subkeys[H*2*n*(D/2)];
 *   uint8 values[N * row_bytes] (N = n*n; row_bytes per value_type);
 *   float value_scale[N]    (E4M3, int8 and int4 tables only);
 *   float x[B*D].
 * <outputs>: float out[B*D]; int32 idx[B*H*k]; float weights[B*H*k].
 *
 * prepare: 0 none; 1 or 2 call pkm_prepare with PKM_PREPARE_SPLIT or
 * PKM_PREPARE_FOLD before the lookup.
 *
 * Before the lookup it checks two calls that must not launch anything: a
 * negative B (PKM_E_ARG) and B = 0 (PKM_OK).  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pkm.h"

#define HIP_OK(call)                                                                     \
    do {                                                                                 \
        hipError_t e_ = (call);                                                          \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)

static void fail(const char *what)
{
    fprintf(stderr, "pkm_forward_main: %s\n", what);
    exit(1);
}

/* Reads n bytes from f into a fresh device buffer. */
static void *read_to_device(FILE *f, size_t n)
{
    void *host = malloc(n ? n : 1), *dev = NULL;
    if (!host) fail("out of host memory");
    if (n && fread(host, 1, n, f) != n) fail("short input file");
    HIP_OK(hipMalloc(&dev, n ? n : 1));
    if (n) HIP_OK(hipMemcpy(dev, host, n, hipMemcpyHostToDevice));
    free(host);
    return dev;
}

static size_t row_bytes(int32_t value_type, int32_t D)
{
    switch (value_type) {
    case PKM_VALUES_F32: return (size_t)D * 4;
    case PKM_VALUES_BF16: return (size_t)D * 2;
    case PKM_VALUES_FP8_E4M3:
    case PKM_VALUES_INT8: return (size_t)D;
    case PKM_VALUES_INT4: return (size_t)D / 2;
    default: fail("unknown value type");
    }
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 3) fail("usage: pkm_forward_main <inputs> <outputs>");
    FILE *f = fopen(argv[1], "rb");
    if (!f) fail("cannot open the inputs");
    char magic[8];
    int32_t hdr[6];
    int64_t sizes[2];
    if (fread(magic, 1, 8, f) != 8 || memcmp(magic, "PKMIN1\0\0", 8) != 0) fail("bad magic");
    if (fread(hdr, sizeof hdr, 1, f) != 1 || fread(sizes, sizeof sizes, 1, f) != 1) fail("short header");
    const int32_t D = hdr[0], H = hdr[1], n = hdr[2], k = hdr[3], vt = hdr[4], prepare = hdr[5];
    if (prepare < 0 || prepare > 2) fail("prepare must be 0, 1 or 2");
    const int64_t B = sizes[0];

    pkm_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.dim = D;
    cfg.heads = H;
    cfg.n_keys = n;
    cfg.k = k;
    cfg.value_type = vt;
    cfg.bn_eps = 1e-5f;
    cfg.max_batch = sizes[1];
    pkm_status st = pkm_config_check(&cfg);
    if (st != PKM_OK) {
        fprintf(stderr, "config: %s (%s)\n", pkm_status_str(st), pkm_last_error());
        return 1;
    }

    const size_t hd = (size_t)H * D, N = (size_t)n * n;
    const int scaled = vt == PKM_VALUES_FP8_E4M3 || vt == PKM_VALUES_INT8 || vt == PKM_VALUES_INT4;
    pkm_params p;
    p.wq = read_to_device(f, hd * D * 4);
    p.bn_mean = read_to_device(f, hd * 4);
    p.bn_var = read_to_device(f, hd * 4);
    p.bn_gamma = read_to_device(f, hd * 4);
    p.bn_beta = read_to_device(f, hd * 4);
    p.subkeys = read_to_device(f, (size_t)H * 2 * n * (D / 2) * 4);
    p.values = read_to_device(f, N * row_bytes(vt, D));
    p.value_scale = scaled ? read_to_device(f, N * 4) : NULL;
    float *x = read_to_device(f, (size_t)B * D * 4);
    fclose(f);

    float *out = NULL, *w = NULL;
    int32_t *idx = NULL;
    const size_t sel = (size_t)B * H * k;
    HIP_OK(hipMalloc((void **)&out, (size_t)B * D * 4 + 4));
    HIP_OK(hipMalloc((void **)&idx, sel * 4 + 4));
    HIP_OK(hipMalloc((void **)&w, sel * 4 + 4));

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    pkm_ctx *ctx = NULL;
    st = pkm_create(&cfg, &ctx);
    if (st != PKM_OK) {
        fprintf(stderr, "pkm_create: %s (%s)\n", pkm_status_str(st), pkm_last_error());
        return 1;
    }
    /* argument errors come back before anything is launched */
    if (pkm_forward(ctx, &p, -1, x, out, idx, w, stream) != PKM_E_ARG) fail("B = -1 was accepted");
    if (pkm_forward(ctx, &p, 0, x, out, idx, w, stream) != PKM_OK) fail("B = 0 was rejected");

    if (prepare) {
        st = pkm_prepare(ctx, &p, prepare == 2 ? PKM_PREPARE_FOLD : PKM_PREPARE_SPLIT, stream);
        if (st != PKM_OK) {
            fprintf(stderr, "pkm_prepare: %s (%s)\n", pkm_status_str(st), pkm_last_error());
            return 1;
        }
    }
    st = pkm_forward(ctx, &p, B, x, out, idx, w, stream);
    if (st != PKM_OK) {
        fprintf(stderr, "pkm_forward: %s (%s)\n", pkm_status_str(st), pkm_last_error());
        return 1;
    }
    HIP_OK(hipStreamSynchronize(stream));

    float *h_out = malloc((size_t)B * D * 4 + 4), *h_w = malloc(sel * 4 + 4);
    int32_t *h_idx = malloc(sel * 4 + 4);
    if (!h_out || !h_w || !h_idx) fail("out of host memory");
    HIP_OK(hipMemcpy(h_out, out, (size_t)B * D * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_idx, idx, sel * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_w, w, sel * 4, hipMemcpyDeviceToHost));
    FILE *o = fopen(argv[2], "wb");
    if (!o) fail("cannot open the outputs");
    if (fwrite(h_out, 4, (size_t)B * D, o) != (size_t)B * D || fwrite(h_idx, 4, sel, o) != sel ||
        fwrite(h_w, 4, sel, o) != sel)
        fail("short write");
    fclose(o);

    pkm_destroy(ctx);
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree((void *)p.wq));
    HIP_OK(hipFree((void *)p.bn_mean));
    HIP_OK(hipFree((void *)p.bn_var));
    HIP_OK(hipFree((void *)p.bn_gamma));
    HIP_OK(hipFree((void *)p.bn_beta));
    HIP_OK(hipFree((void *)p.subkeys));
    HIP_OK(hipFree((void *)p.values));
    if (p.value_scale) HIP_OK(hipFree((void *)p.value_scale));
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(idx));
    HIP_OK(hipFree(w));
    free(h_out);
    free(h_w);
    free(h_idx);
    printf("pkm_forward_main: %lld tokens, D %d, H %d, n_keys %d, k %d, value type %d: ok\n", (long long)B, D, H, n, k,
           vt);
    return 0;
}
