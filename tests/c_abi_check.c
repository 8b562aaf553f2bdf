/*
 * c_abi_check.c -- drives libar.so from plain C with raw device pointers:
 * no PyTorch, no Python in the call path.  Test helper, built by the
 * package's build step and run by tests/test_gpu_c_abi.py.
 *
 * usage: c_abi_check P n in.bin out.bin
 *   in.bin   P * n little-endian uint16 (bf16 bit patterns), rank-major
 *   out.bin  written: the n-element result of ar_oneshot_write_bcast
 * Exit status 0 when every call succeeds, the P write-mode outputs are
 * identical, and every other entry point agrees with them: ar_oneshot_sum,
 * ar_twoshot_share (every owner), ar_reduce_scatter_share (every block of
 * the first P * floor(n / P) elements), ar_ll_encode + ar_ll_decode of the
 * result, a fused packet call (all ranks, flag 1), the three-launch packet
 * decomposition (flag 2) and the epoch variant (flag 3), with no time-out in
 * any control block.
 */
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ar.h"

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
            return 2;                                                              \
        }                                                                          \
    } while (0)

#define AR_OK_(x)                                                                  \
    do {                                                                           \
        int rc_ = (x);                                                             \
        if (rc_ != AR_OK) {                                                        \
            fprintf(stderr, "%s failed: %s\n", #x, ar_strerror(rc_));              \
            return 3;                                                              \
        }                                                                          \
    } while (0)

int main(int argc, char **argv)
{
    if (argc != 5) {
        fprintf(stderr, "usage: %s P n in.bin out.bin\n", argv[0]);
        return 1;
    }
    const int P = atoi(argv[1]);
    const int64_t n = atoll(argv[2]);
    if (P < 2 || P > AR_MAX_P || n <= 0) return 1;
    const size_t bytes = (size_t)n * 2;

    uint16_t *host = malloc(bytes * P), *res = malloc(bytes), *chk = malloc(bytes);
    if (!host || !res || !chk) return 1;
    FILE *f = fopen(argv[3], "rb");
    if (!f || fread(host, 2, (size_t)n * P, f) != (size_t)n * P) return 1;
    fclose(f);

    ar_ptrs in = {{0}}, out = {{0}}, out2 = {{0}}, scratch = {{0}};
    const int64_t sbytes = ar_packet_scratch_bytes(P, n);
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMalloc(&in.p[p], bytes));
        HIP_OK(hipMalloc(&out.p[p], bytes));
        HIP_OK(hipMalloc(&out2.p[p], bytes));
        HIP_OK(hipMalloc(&scratch.p[p], (size_t)sbytes));
        HIP_OK(hipMemcpy(in.p[p], host + (size_t)p * n, bytes, hipMemcpyHostToDevice));
        HIP_OK(hipMemset(scratch.p[p], 0, (size_t)sbytes));
    }
    void *one = NULL, *ctrl = NULL;
    HIP_OK(hipMalloc(&one, bytes));
    HIP_OK(hipMalloc(&ctrl, AR_CTRL_BYTES));
    HIP_OK(hipMemset(ctrl, 0, AR_CTRL_BYTES));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    AR_OK_(ar_oneshot_write_bcast(in, out, P, n, s));
    AR_OK_(ar_oneshot_sum(in, one, P, n, s));
    AR_OK_(ar_packet_fused(in, scratch, out2, P, 0, P, n, 1u, ctrl, 0, s));
    HIP_OK(hipStreamSynchronize(s));

    ar_ctrl c;
    HIP_OK(hipMemcpy(&c, ctrl, sizeof c, hipMemcpyDeviceToHost));
    if (c.status != AR_OK) {
        fprintf(stderr, "packet call status %s\n", ar_strerror(c.status));
        return 4;
    }
    HIP_OK(hipMemcpy(res, out.p[0], bytes, hipMemcpyDeviceToHost));
    for (int p = 1; p < P; ++p) {
        HIP_OK(hipMemcpy(chk, out.p[p], bytes, hipMemcpyDeviceToHost));
        if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "write-mode output %d differs\n", p); return 5; }
    }
    HIP_OK(hipMemcpy(chk, one, bytes, hipMemcpyDeviceToHost));
    if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "one-shot differs\n"); return 5; }
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMemcpy(chk, out2.p[p], bytes, hipMemcpyDeviceToHost));
        if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "packet output %d differs\n", p); return 5; }
    }

    /* two-shot: every owner in turn fills its slice of every output */
    for (int p = 0; p < P; ++p) HIP_OK(hipMemset(out2.p[p], 0, bytes));
    for (int r = 0; r < P; ++r) AR_OK_(ar_twoshot_share(in, out2, P, r, n, s));
    HIP_OK(hipStreamSynchronize(s));
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMemcpy(chk, out2.p[p], bytes, hipMemcpyDeviceToHost));
        if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "two-shot output %d differs\n", p); return 5; }
    }

    /* reduce-scatter: block r of the first P * rc elements */
    const int64_t rc = n / P;
    for (int r = 0; r < P && rc > 0; ++r) {
        AR_OK_(ar_reduce_scatter_share(in, one, P, r, rc, s));
        HIP_OK(hipMemcpy(chk, one, (size_t)rc * 2, hipMemcpyDeviceToHost));
        if (memcmp(chk, res + (size_t)r * rc, (size_t)rc * 2) != 0) {
            fprintf(stderr, "reduce-scatter block %d differs\n", r);
            return 5;
        }
    }

    /* LL codec: encode the result, decode it without a control block */
    void *pk = NULL;
    HIP_OK(hipMalloc(&pk, (size_t)ar_ll_packets(n) * 16));
    AR_OK_(ar_ll_encode(out.p[0], pk, n, 7u, s));
    AR_OK_(ar_ll_decode(pk, one, n, 7u, NULL, 0, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(chk, one, bytes, hipMemcpyDeviceToHost));
    if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "codec round trip differs\n"); return 5; }
    HIP_OK(hipFree(pk));

    /* three-launch packet decomposition (flag 2), then the epoch kernel with
     * the control block's epoch set to 2, so that it takes flag 3 and leaves
     * the epoch at 3 */
    AR_OK_(ar_packet_send(in, scratch, P, 0, P, n, 2u, s));
    AR_OK_(ar_packet_recv_reduce_send(scratch, P, 0, P, n, 2u, ctrl, 0, s));
    AR_OK_(ar_packet_recv(scratch, out2, P, 0, P, n, 2u, ctrl, 0, s));
    HIP_OK(hipStreamSynchronize(s));
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMemcpy(chk, out2.p[p], bytes, hipMemcpyDeviceToHost));
        if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "three-op output %d differs\n", p); return 5; }
    }
    const uint32_t epoch = 2u;
    HIP_OK(hipMemcpy((char *)ctrl + offsetof(ar_ctrl, epoch), &epoch, sizeof epoch,
                     hipMemcpyHostToDevice));
    for (int p = 0; p < P; ++p) HIP_OK(hipMemset(out2.p[p], 0, bytes));
    AR_OK_(ar_packet_fused_epoch(in, scratch, out2, P, 0, P, n, ctrl, 0, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(&c, ctrl, sizeof c, hipMemcpyDeviceToHost));
    if (c.status != AR_OK || c.epoch != 3u) {
        fprintf(stderr, "epoch call: status %s, epoch %u\n", ar_strerror(c.status), c.epoch);
        return 4;
    }
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipMemcpy(chk, out2.p[p], bytes, hipMemcpyDeviceToHost));
        if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "epoch output %d differs\n", p); return 5; }
    }
    /* no-alloc packet share: the library's own scratch; beyond its size the
     * call must refuse with AR_ENOSPACE before touching the GPU */
    int32_t *st = NULL;
    HIP_OK(hipMalloc((void **)&st, sizeof *st));
    HIP_OK(hipMemset(st, 0x5A, sizeof *st));
    for (int p = 0; p < P; ++p) HIP_OK(hipMemset(out2.p[p], 0, bytes));
    const int64_t per_rank = (ar_packet_scratch_bytes(P, n) + 255) / 256 * 256;
    const int fits = 256 + (int64_t)P * per_rank <= (int64_t)AR_NOALLOC_SCRATCH_BYTES;
    const int nrc = ar_packet_fused_noalloc(in, out2, P, n, st, 0, s);
    if (!fits) {
        if (nrc != AR_ENOSPACE) { fprintf(stderr, "no-alloc: expected AR_ENOSPACE, got %d\n", nrc); return 6; }
    } else {
        AR_OK_(nrc);
        HIP_OK(hipStreamSynchronize(s));
        int32_t hs = -1;
        HIP_OK(hipMemcpy(&hs, st, sizeof hs, hipMemcpyDeviceToHost));
        if (hs != AR_OK) { fprintf(stderr, "no-alloc status %s\n", ar_strerror(hs)); return 4; }
        for (int p = 0; p < P; ++p) {
            HIP_OK(hipMemcpy(chk, out2.p[p], bytes, hipMemcpyDeviceToHost));
            if (memcmp(chk, res, bytes) != 0) { fprintf(stderr, "no-alloc output %d differs\n", p); return 5; }
        }
    }
    HIP_OK(hipFree(st));

    f = fopen(argv[4], "wb");
    if (!f || fwrite(res, 2, (size_t)n, f) != (size_t)n) return 1;
    fclose(f);

    for (int p = 0; p < P; ++p) {
        HIP_OK(hipFree(in.p[p]));
        HIP_OK(hipFree(out.p[p]));
        HIP_OK(hipFree(out2.p[p]));
        HIP_OK(hipFree(scratch.p[p]));
    }
    HIP_OK(hipFree(one));
    HIP_OK(hipFree(ctrl));
    HIP_OK(hipStreamDestroy(s));
    free(host); free(res); free(chk);
    printf("c_abi_check: ok\n");
    return 0;
}
