// reduce.hip -- one-shot sum, write-mode broadcast and two-shot slice share.
//
// One kernel family serves all three: read P peer inputs with 16-byte loads,
// widen bf16 -> binary32, add in rank order in VGPRs, round to bf16 (RNE),
// store the 16-byte result to one output (one-shot) or to all P outputs
// (write mode: aiter PR #1910 "optimize allreduce write mode by broadcast
// output ptr", Motivation -- the reduced data goes straight into every
// output, whose pointers reach the kernel by value).  The two-shot share is
// the same kernel on the owner's slice.
//
// The work is HBM-bound (about 0.4 flop per byte moved), so the design is
// about bytes in flight: each lane issues U x P independent 16-byte loads
// before it adds anything (16-byte units, as the one-shot kernel of
// torchcomms PR #3850 "Add HIP-graph capture coverage for the sharded-relay
// collectives", commit summary D117629704, found faster than element-wise
// moves), and a wavefront's 64 lanes touch 1 KiB of consecutive bytes per
// load instruction.  Alignment is checked, not assumed: when all pointers of
// a call share one 16-byte alignment the ragged head and tail take scalar
// accesses and the bulk takes vectors; otherwise the whole range is scalar.
// No LDS, no MFMA: there is no reuse to stage and no contraction.
#include "device.h"
#include "host.h"

namespace ar {
namespace {

struct ReduceArgs {
    ar_ptrs in;     // P inputs, already offset to the first element of the range
    ar_ptrs out;    // 1 or P outputs, offset likewise
    int64_t head;   // scalar elements before the 16-byte-aligned bulk
    int64_t nvec;   // 16-byte vectors (8 bf16) in the bulk
    int64_t ntail;  // scalar elements after the bulk
};

template <int P, bool BCAST, int U, bool NTL>
__global__ __launch_bounds__(kThreads) void k_reduce(ReduceArgs a) {
    constexpr int NOUT = BCAST ? P : 1;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;

    for (int64_t v0 = tid; v0 < a.nvec; v0 += nthreads * U) {
        u32x4 x[U][P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nthreads;
            if (v < a.nvec) {
#pragma unroll
                for (int p = 0; p < P; ++p) x[u][p] = load_vec<NTL>(a.in.p[p], a.head + 8 * v);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = v0 + u * nthreads;
            if (v < a.nvec) {
                const u32x4 r = reduce_vec<P>(x[u]);
                // byte offset from the output pointer: below 2**31 (launch_reduce
                // cuts longer ranges into pieces)
                const uint32_t off = (uint32_t)(2 * (a.head + 8 * v));
#pragma unroll
                for (int o = 0; o < NOUT; ++o) store_vec(a.out.p[o], off, r);
            }
        }
    }

    // Scalar elements: the head [0, head) and the tail after the bulk.
    const int64_t nscalar = a.head + a.ntail;
    for (int64_t s = tid; s < nscalar; s += nthreads) {
        const int64_t i = s < a.head ? s : a.head + 8 * a.nvec + (s - a.head);
        uint16_t e[P];
#pragma unroll
        for (int p = 0; p < P; ++p) e[p] = static_cast<const uint16_t *>(a.in.p[p])[i];
        const uint16_t r = reduce_elem<P>(e);
#pragma unroll
        for (int o = 0; o < NOUT; ++o) static_cast<uint16_t *>(a.out.p[o])[i] = r;
    }
}

// ---- kernel table ------------------------------------------------------------

typedef void (*ReduceKernel)(ReduceArgs);

template <int P, bool BCAST, bool NTL>
ReduceKernel pick_unroll(int U) {
    switch (U) {
        case 1: return k_reduce<P, BCAST, 1, NTL>;
        case 2: return k_reduce<P, BCAST, 2, NTL>;
        default: return k_reduce<P, BCAST, 4, NTL>;
    }
}

template <bool BCAST, bool NTL>
ReduceKernel pick_p(int P, int U) {
    switch (P) {
        case 2: return pick_unroll<2, BCAST, NTL>(U);
        case 3: return pick_unroll<3, BCAST, NTL>(U);
        case 4: return pick_unroll<4, BCAST, NTL>(U);
        case 5: return pick_unroll<5, BCAST, NTL>(U);
        case 6: return pick_unroll<6, BCAST, NTL>(U);
        case 7: return pick_unroll<7, BCAST, NTL>(U);
        default: return pick_unroll<8, BCAST, NTL>(U);
    }
}

ReduceKernel pick(bool bcast, bool ntl, int P, int U) {
    if (bcast) return ntl ? pick_p<true, true>(P, U) : pick_p<true, false>(P, U);
    return ntl ? pick_p<false, true>(P, U) : pick_p<false, false>(P, U);
}

// Bytes one launch touches beyond which its inputs take non-temporal loads:
// half the 256 MB MALL, so data that could stay cached keeps plain loads.
constexpr int64_t kStreamingBytes = 128ll << 20;

// Launch shape overrides for benchmark sweeps (0 = automatic).
int g_unroll_override = 0;
int g_threads_override = 0;
int g_max_blocks_override = 0;

// Splits the range into scalar head, 16-byte bulk and scalar tail.  The bulk
// exists only when every pointer has the same address mod 16.
void split_range(const ar_ptrs &in, const ar_ptrs &out, int P, int nout, int64_t len,
                 ReduceArgs *a) {
    const uintptr_t m = addr(in.p[0]) & 15u;
    bool same = true;
    for (int p = 0; p < P; ++p) same = same && (addr(in.p[p]) & 15u) == m;
    for (int o = 0; o < nout; ++o) same = same && (addr(out.p[o]) & 15u) == m;
    a->in = in;
    a->out = out;
    if (!same) {
        a->head = len;
        a->nvec = 0;
        a->ntail = 0;
        return;
    }
    const int64_t head = m == 0 ? 0 : (int64_t)((16u - m) / 2u);
    if (head >= len) {
        a->head = len;
        a->nvec = 0;
        a->ntail = 0;
        return;
    }
    a->head = head;
    a->nvec = (len - head) / 8;
    a->ntail = len - head - 8 * a->nvec;
}

ar_ptrs offset_ptrs(const ar_ptrs &p, int count, int64_t elem) {
    ar_ptrs r = {};
    for (int k = 0; k < count; ++k) r.p[k] = static_cast<uint16_t *>(p.p[k]) + elem;
    return r;
}

// One launch over a range of at most kPieceElems elements.
int launch_piece(const ar_ptrs &in_at, const ar_ptrs &out_at, int P, bool bcast, int64_t len,
                 bool ntl, const DeviceInfo &dev, void *stream) {
    ReduceArgs a;
    split_range(in_at, out_at, P, bcast ? P : 1, len, &a);

    // Launch shape (swept on MI355X over workgroup size, unroll and grid):
    //  - a small bulk (<= 256 lanes' worth per CU) is latency-bound: one vector
    //    per lane in 64-lane workgroups, so the work spreads over every CU;
    //  - a larger one takes 256-lane workgroups with two vectors in flight
    //    per lane and exactly two workgroups per CU, looping (grid stride)
    //    beyond that: a grid that is a multiple of the CU count keeps the
    //    CUs evenly loaded (550 workgroups on 256 CUs ran 19% slower than 512).
    int threads, U;
    int64_t blocks;
    if (a.nvec <= (int64_t)dev.cus * kThreads) {
        threads = 64;
        U = 1;
        blocks = (a.nvec + threads - 1) / threads;
    } else {
        threads = kThreads;
        U = 2;
        blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
        if (blocks > 2 * (int64_t)dev.cus) blocks = 2 * (int64_t)dev.cus;
    }
    if (g_unroll_override == 1 || g_unroll_override == 2 || g_unroll_override == 4) {
        U = g_unroll_override;
        blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
    }
    if (g_threads_override > 0) {
        threads = g_threads_override;
        blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
    }
    if (g_max_blocks_override > 0 && blocks > g_max_blocks_override) blocks = g_max_blocks_override;
    const int64_t scalar_blocks = (a.head + a.ntail + threads - 1) / threads;
    if (scalar_blocks > blocks) blocks = scalar_blocks;
    if (blocks > (int64_t)dev.cus * 16) blocks = (int64_t)dev.cus * 16;  // lanes loop beyond
    if (blocks < 1) blocks = 1;
    ReduceKernel fn = pick(bcast, ntl, P, U);
    return launch(reinterpret_cast<const void *>(fn), (unsigned)blocks, (unsigned)threads, a, stream);
}

// The kernel addresses its outputs with 32-bit byte offsets (see store_vec),
// so a range longer than kPieceElems elements (1 GiB per buffer) is cut into
// consecutive launches on the same stream.  The streaming decision is taken
// for the whole call.
constexpr int64_t kPieceElems = 1ll << 29;

int launch_reduce(const ar_ptrs &in_at, const ar_ptrs &out_at, int P, bool bcast, int64_t len,
                  void *stream) {
    if (len == 0) return AR_OK;
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    const int nout = bcast ? P : 1;
    const bool ntl = (int64_t)(P + nout) * len * 2 > kStreamingBytes;
    for (int64_t b = 0; b < len; b += kPieceElems) {
        const int64_t m = len - b < kPieceElems ? len - b : kPieceElems;
        const int rc = launch_piece(offset_ptrs(in_at, P, b), offset_ptrs(out_at, nout, b), P,
                                    bcast, m, ntl, dev, stream);
        if (rc != AR_OK) return rc;
    }
    return AR_OK;
}

// Common checks: P, n, non-null 2-byte-aligned pointers.
int check_buffers(const ar_ptrs &in, const void *const *outs, int nout, int P, int64_t n) {
    if (!valid_P(P) || n < 0) return AR_EINVAL;
    for (int p = 0; p < P; ++p)
        if (!in.p[p] || !aligned_to(in.p[p], 2)) return AR_EINVAL;
    for (int o = 0; o < nout; ++o)
        if (!outs[o] || !aligned_to(outs[o], 2)) return AR_EINVAL;
    return AR_OK;
}

// Outputs may coincide exactly with an input or with each other; any partial
// overlap involving an output over [begin, begin + len) is an alias.
int check_output_overlap(const ar_ptrs &in, const void *const *outs, int nout, int P,
                         int64_t begin, int64_t len) {
    for (int o = 0; o < nout; ++o) {
        const Span so = span_of(outs[o], begin, len, 2);
        for (int p = 0; p < P; ++p)
            if (partial_overlap(so, span_of(in.p[p], begin, len, 2))) return AR_EALIAS;
        for (int q = o + 1; q < nout; ++q)
            if (partial_overlap(so, span_of(outs[q], begin, len, 2))) return AR_EALIAS;
    }
    return AR_OK;
}

}  // namespace
}  // namespace ar

using namespace ar;

extern "C" {

int ar_oneshot_sum(ar_ptrs in, void *out, int P, int64_t n, void *stream) {
    const void *outs[1] = {out};
    int rc = check_buffers(in, outs, 1, P, n);
    if (rc == AR_OK) rc = check_output_overlap(in, outs, 1, P, 0, n);
    if (rc != AR_OK || n == 0) return rc;
    ar_ptrs o = {};
    o.p[0] = out;
    return launch_reduce(in, o, P, false, n, stream);
}

int ar_oneshot_write_bcast(ar_ptrs in, ar_ptrs out, int P, int64_t n, void *stream) {
    int rc = check_buffers(in, out.p, valid_P(P) ? P : 0, P, n);
    if (rc == AR_OK) rc = check_output_overlap(in, out.p, P, P, 0, n);
    if (rc != AR_OK || n == 0) return rc;
    return launch_reduce(in, out, P, true, n, stream);
}

int ar_twoshot_share(ar_ptrs in, ar_ptrs out, int P, int rank, int64_t n, void *stream) {
    int rc = check_buffers(in, out.p, valid_P(P) ? P : 0, P, n);
    if (rc != AR_OK) return rc;
    int64_t b = 0, e = 0;
    if (ar_slice_range(P, rank, n, &b, &e) != AR_OK) return AR_EINVAL;
    rc = check_output_overlap(in, out.p, P, P, b, e - b);
    if (rc != AR_OK || e == b) return rc;
    return launch_reduce(offset_ptrs(in, P, b), offset_ptrs(out, P, b), P, true, e - b, stream);
}

int ar_reduce_scatter_share(ar_ptrs in, void *out, int P, int rank, int64_t recvcount,
                            void *stream) {
    const void *outs[1] = {out};
    int rc = check_buffers(in, outs, 1, P, recvcount);
    if (rc != AR_OK) return rc;
    if (rank < 0 || rank >= P) return AR_EINVAL;
    const int64_t begin = (int64_t)rank * recvcount;
    // the output may be exactly this rank's own block of an input (in place)
    for (int p = 0; p < P; ++p)
        if (partial_overlap(span_of(out, 0, recvcount, 2), span_of(in.p[p], begin, recvcount, 2)))
            return AR_EALIAS;
    if (recvcount == 0) return AR_OK;
    ar_ptrs o = {};
    o.p[0] = out;
    return launch_reduce(offset_ptrs(in, P, begin), o, P, false, recvcount, stream);
}

// Benchmark-only launch-shape override for the reduce entry points above.
int ar_set_reduce_tuning(int unroll, int threads, int max_blocks) {
    if (!(unroll == 0 || unroll == 1 || unroll == 2 || unroll == 4) || max_blocks < 0 ||
        !(threads == 0 || threads == 64 || threads == 128 || threads == 256))
        return AR_EINVAL;
    g_unroll_override = unroll;
    g_threads_override = threads;
    g_max_blocks_override = max_blocks;
    return AR_OK;
}

}  // extern "C"
