// probe.hip -- measurement kernels: the memory traffic of the reduce kernels
// without the reduction, to measure what the device delivers for the same
// bytes at the same size.
//
// Three kernels over 2P buffers of n bf16 (the P inputs and P outputs of a
// write-mode call): read every one of them (read-only), write every one of
// them (write-only), or copy input p to output p (the reduce kernel's bytes
// with no arithmetic).  They use the reduce kernels' accesses: 16-byte
// loads, 16-byte buffer stores (store_vec), U vectors in flight per lane,
// grid stride, with either cache policy the reduce kernels take (NT = false:
// plain loads, write-through streaming stores; NT = true: non-temporal loads
// and stores).  Results are meaningless by design (the read-only kernel keeps
// an xor of what it read only so that the loads cannot be dropped).
#include "device.h"
#include "host.h"

namespace ar {
namespace {

struct ProbeArgs {
    ar_ptrs in;
    ar_ptrs out;
    int64_t nvec;    // 16-byte vectors per buffer
    uint32_t *sink;  // read-only: one word written only if an impossible xor comes up
};

template <int P, int U, bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_read(ProbeArgs a) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (int64_t v0 = tid; v0 < a.nvec; v0 += nth * U) {
        u32x4 x[U][2 * P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nth;
            if (v < a.nvec) {
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    x[u][p] = load_vec<NT>(a.in.p[p], 8 * v);
                    x[u][P + p] = load_vec<NT>(a.out.p[p], 8 * v);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nth;
            if (v < a.nvec) {
#pragma unroll
                for (int b = 0; b < 2 * P; ++b) acc ^= x[u][b][0] ^ x[u][b][1] ^ x[u][b][2] ^ x[u][b][3];
            }
        }
    }
    if (acc == 0x9E3779B9u && a.sink) a.sink[0] = acc;
}

template <int P, int U, bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_write(ProbeArgs a) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t v0 = tid; v0 < a.nvec; v0 += nth * U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nth;
            if (v < a.nvec) {
                const u32x4 x = {(uint32_t)v, 0x3F803F80u, (uint32_t)v, 0x3F803F80u};
                const uint32_t off = (uint32_t)(16 * v);
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    store_vec<!NT>(a.in.p[p], off, x);
                    store_vec<!NT>(a.out.p[p], off, x);
                }
            }
        }
    }
}

template <int P, int U, bool NT>
__global__ __launch_bounds__(kThreads) void k_probe_copy(ProbeArgs a) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t v0 = tid; v0 < a.nvec; v0 += nth * U) {
        u32x4 x[U][P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nth;
            if (v < a.nvec) {
#pragma unroll
                for (int p = 0; p < P; ++p) x[u][p] = load_vec<NT>(a.in.p[p], 8 * v);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nth;
            if (v < a.nvec) {
#pragma unroll
                for (int p = 0; p < P; ++p) store_vec<!NT>(a.out.p[p], (uint32_t)(16 * v), x[u][p]);
            }
        }
    }
}

typedef void (*ProbeKernel)(ProbeArgs);

template <int P, bool NT>
ProbeKernel pick_probe(int kind, int U) {
    if (kind == 0) return U == 1 ? k_probe_read<P, 1, NT> : k_probe_read<P, 2, NT>;
    if (kind == 1)
        return U == 1 ? k_probe_write<P, 1, NT>
                      : (U == 2 ? k_probe_write<P, 2, NT> : k_probe_write<P, 4, NT>);
    return U == 1 ? k_probe_copy<P, 1, NT> : (U == 2 ? k_probe_copy<P, 2, NT> : k_probe_copy<P, 4, NT>);
}

// The bulk of one probe launch addresses at most this many elements per
// buffer, so every store offset stays inside store_vec's range.
constexpr int64_t kProbeMaxElems = 1ll << 29;
static_assert(2 * kProbeMaxElems <= (int64_t)kStoreRangeBytes, "probe offsets must fit the store range");

}  // namespace
}  // namespace ar

using namespace ar;

extern "C" {

int ar_probe_traffic(int kind, ar_ptrs in, ar_ptrs out, int P, int64_t n, int threads, int unroll,
                     int blocks, int policy, void *stream) {
    if (!(kind == 0 || kind == 1 || kind == 2) || !(P == 4 || P == 8) || n <= 0 || n % 8 != 0 ||
        !(policy == 0 || policy == 1) ||
        n > kProbeMaxElems || !(threads == 64 || threads == 128 || threads == 256) ||
        !(unroll == 1 || unroll == 2 || (unroll == 4 && kind != 0)) || blocks < 0)
        return AR_EINVAL;
    for (int p = 0; p < P; ++p) {
        if (!in.p[p] || !out.p[p] || !aligned_to(in.p[p], 16) || !aligned_to(out.p[p], 16))
            return AR_EINVAL;
        for (int q = 0; q < P; ++q) {
            if (overlap(span_of(in.p[p], 0, n, 2), span_of(out.p[q], 0, n, 2))) return AR_EALIAS;
            if (q > p && (overlap(span_of(in.p[p], 0, n, 2), span_of(in.p[q], 0, n, 2)) ||
                          overlap(span_of(out.p[p], 0, n, 2), span_of(out.p[q], 0, n, 2))))
                return AR_EALIAS;
        }
    }
    ProbeArgs a = {};
    a.in = in;
    a.out = out;
    a.nvec = n / 8;
    int64_t grid = (a.nvec + (int64_t)threads * unroll - 1) / ((int64_t)threads * unroll);
    if (blocks > 0 && grid > blocks) grid = blocks;
    ProbeKernel fn = policy ? (P == 4 ? pick_probe<4, true>(kind, unroll) : pick_probe<8, true>(kind, unroll))
                            : (P == 4 ? pick_probe<4, false>(kind, unroll) : pick_probe<8, false>(kind, unroll));
    return launch(reinterpret_cast<const void *>(fn), (unsigned)grid, (unsigned)threads, a, stream);
}

}  // extern "C"
