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
//
// Three schedules of those loads and stores, chosen by size in launch_piece:
// grid-stride batches (k_reduce) for the latency-bound sizes; one pass in
// which every wave issues all its loads before any store (k_reduce_phased),
// at most one wave per SIMD in the middle range, which puts the device's
// reads first and its writes last, and several per SIMD for the largest
// one-output calls; and a two-stage software pipeline (k_reduce_pipe) just
// above the latency-bound sizes and for the largest calls with P outputs.
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

// Loads, for each u < U, the 16-byte vector v + u * nth of every input into
// x[u] (vectors past the bulk are skipped).
template <int P, int U, bool NTL>
__device__ __forceinline__ void load_stage(const ReduceArgs &a, int64_t v, int64_t nth,
                                           u32x4 (&x)[U][P]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = v + u * nth;
        if (w < a.nvec) {
#pragma unroll
            for (int p = 0; p < P; ++p) x[u][p] = load_vec<NTL>(a.in.p[p], a.head + 8 * w);
        }
    }
}

// Reduces x[u] in rank order and stores the result at vector v + u * nth of
// the output (one-shot) or of every output (write mode).
template <int P, bool BCAST, int U, bool WT = true>
__device__ __forceinline__ void store_stage(const ReduceArgs &a, int64_t v, int64_t nth,
                                            const u32x4 (&x)[U][P]) {
    constexpr int NOUT = BCAST ? P : 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = v + u * nth;
        if (w < a.nvec) {
            const u32x4 r = reduce_vec<P>(x[u]);
            // byte offset from the output pointer: inside the store range
            // (launch_reduce cuts longer ranges into pieces)
            const uint32_t off = (uint32_t)(2 * (a.head + 8 * w));
#pragma unroll
            for (int o = 0; o < NOUT; ++o) store_vec<WT>(a.out.p[o], off, r);
        }
    }
}

// Scalar elements: the head [0, head) and the tail after the bulk.
template <int P, bool BCAST>
__device__ __forceinline__ void scalar_part(const ReduceArgs &a, int64_t tid, int64_t nth) {
    constexpr int NOUT = BCAST ? P : 1;
    const int64_t nscalar = a.head + a.ntail;
    for (int64_t s = tid; s < nscalar; s += nth) {
        const int64_t i = s < a.head ? s : a.head + 8 * a.nvec + (s - a.head);
        uint16_t e[P];
#pragma unroll
        for (int p = 0; p < P; ++p) e[p] = static_cast<const uint16_t *>(a.in.p[p])[i];
        const uint16_t r = reduce_elem<P>(e);
#pragma unroll
        for (int o = 0; o < NOUT; ++o) static_cast<uint16_t *>(a.out.p[o])[i] = r;
    }
}

// Batches: each pass loads U vectors per input, then reduces and stores them.
// The next pass's loads are issued after this pass's stores, and CDNA's
// vector-memory counter retires loads and stores in issue order, so waiting
// for those loads also waits for the stores to be acknowledged.
//
// U = 4 takes non-temporal loads and non-temporal stores without the
// device-scope write-through at every size (NTL and WT are fixed by
// pick_unroll), as does k_reduce_phased below, which replaced it as the
// automatic one-pass shape: measured on MI355X in one process, interleaved,
// the write-mode share of 440x5120 x 8 ran 13.86 us per call from HBM against
// 14.33 us with plain loads and write-through stores (14.22 with NT loads
// alone, 14.24 with NT stores alone), and 10.79 against 10.96 us back to back
// on one buffer set; on a second box 14.18 against 14.55 us from HBM and
// 13.92 against 14.56 us cold (after a 512 MiB scrub).
template <int P, bool BCAST, int U, bool NTL, bool WT>
__global__ __launch_bounds__(kThreads) void k_reduce(ReduceArgs a) {
    const int64_t nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t v0 = tid; v0 < a.nvec; v0 += nth * U) {
        u32x4 x[U][P];
        load_stage<P, U, NTL>(a, v0, nth, x);
        store_stage<P, BCAST, U, WT>(a, v0, nth, x);
    }
    scalar_part<P, BCAST>(a, tid, nth);
}

// Software pipeline, straight-line: workgroup b owns the S x U x blockDim.x
// consecutive vectors from b x S x U x blockDim.x, taken in S stages of U per
// lane.  The loads of stage k+1 are issued before the stores of stage k, so
// the wait for stage k+1's data leaves stage k's stores in flight: reads of
// one stage overlap writes of the previous one.  No memory instruction sits
// behind a branch (a skipped instruction on one path would make the compiler
// count conservatively and wait for the stores as well): lanes past the bulk
// load the last vector again (in bounds) and store at an offset past the
// buffer resource's range, which the hardware drops.
template <int P, int U, bool NTL>
__device__ __forceinline__ void load_stage_clamped(const ReduceArgs &a, int64_t v, int64_t bd,
                                                   u32x4 (&x)[U][P]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t w = v + u * bd;
        w = w < a.nvec ? w : a.nvec - 1;
#pragma unroll
        for (int p = 0; p < P; ++p) x[u][p] = load_vec<NTL>(a.in.p[p], a.head + 8 * w);
    }
}

template <int P, bool BCAST, int U>
__device__ __forceinline__ void store_stage_masked(const ReduceArgs &a, int64_t v, int64_t bd,
                                                   const u32x4 (&x)[U][P]) {
    constexpr int NOUT = BCAST ? P : 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = v + u * bd;
        const u32x4 r = reduce_vec<P>(x[u]);
        const uint32_t off = w < a.nvec ? (uint32_t)(2 * (a.head + 8 * w)) : kDroppedStoreOffset;
#pragma unroll
        for (int o = 0; o < NOUT; ++o) store_vec(a.out.p[o], off, r);
    }
}

//
// The bulk is never empty here (launch_piece takes the batch kernel for a call
// with no 16-byte vectors), so the kernel needs no guard around it: a guard
// made the compiler wait for the vector count before it fetched the pointer
// table, two dependent rounds of kernel-argument loads before the first
// global load of every wave, where one is enough.
template <int P, bool BCAST, int U, int S, bool NTL>
__global__ __launch_bounds__(kThreads) void k_reduce_pipe(ReduceArgs a) {
    const int64_t bd = blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t v0 = (int64_t)blockIdx.x * S * U * bd + threadIdx.x;
    u32x4 x[2][U][P];
    load_stage_clamped<P, U, NTL>(a, v0, bd, x[0]);
#pragma unroll
    for (int k = 0; k < S; ++k) {
        if (k + 1 < S) load_stage_clamped<P, U, NTL>(a, v0 + (k + 1) * U * bd, bd, x[(k + 1) & 1]);
        store_stage_masked<P, BCAST, U>(a, v0 + k * U * bd, bd, x[k & 1]);
    }
    scalar_part<P, BCAST>(a, tid, (int64_t)gridDim.x * blockDim.x);
}

// One pass in three phases: global wave g (64 lanes) owns the U x 64
// consecutive vectors from g x U x 64 of every buffer -- at U = 5 that is
// 5 KiB of each input and each output -- and issues all U x P loads, then all
// U reductions, then all U x NOUT stores.  The scheduling barriers keep the
// compiler from starting a vector's stores while the wave still has loads to
// wait for.  Every wave therefore reads before it writes, and with every wave
// of the grid resident at once the device sees mostly reads first and
// mostly writes last, instead of the two mixed.  Measured on MI355X, write
// mode 440x5120 x 8 from HBM (buffer sets rotated through 576 MB), in one
// process, interleaved, at U = 4:
//  - 13.34 us per call against 13.64 us for the same loads and stores with a
//    stride of one grid between a lane's vectors;
//  - against 15.79 us when each vector's stores follow its own loads as soon
//    as they arrive (exact waits, so reads and writes overlap);
//  - 64-lane workgroups: the same layout in 256-lane workgroups ran 16.4 us.
// launch_piece picks U (see there); at U = 5 the same share runs 12.0 us.
// As in k_reduce_pipe, no memory instruction sits behind a branch: lanes past
// the bulk load the last vector again (in bounds) and store at an offset past
// the buffer resource's range, which the hardware drops; and the bulk is
// never empty.
template <int P, bool BCAST, int U>
__global__ __launch_bounds__(kThreads) void k_reduce_phased(ReduceArgs a) {
    constexpr int NOUT = BCAST ? P : 1;
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    {
        const int64_t base = (gtid >> 6) * (64 * U) + (gtid & 63);
        u32x4 x[U][P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t w = base + 64 * u;
            w = w < a.nvec ? w : a.nvec - 1;
#pragma unroll
            for (int p = 0; p < P; ++p) x[u][p] = load_vec<true>(a.in.p[p], a.head + 8 * w);
        }
        __builtin_amdgcn_sched_barrier(0);
        u32x4 r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = reduce_vec<P>(x[u]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t w = base + 64 * u;
            const uint32_t off = w < a.nvec ? (uint32_t)(2 * (a.head + 8 * w)) : kDroppedStoreOffset;
#pragma unroll
            for (int o = 0; o < NOUT; ++o) store_vec<false>(a.out.p[o], off, r[u]);
        }
    }
    scalar_part<P, BCAST>(a, gtid, (int64_t)gridDim.x * blockDim.x);
}

// ---- kernel table ------------------------------------------------------------

typedef void (*ReduceKernel)(ReduceArgs);

// Schedules: kBatch grid-stride batches; kPipe2/4/8 pipelined, that many
// stages; kPhased one pass, loads then reductions then stores.
enum Schedule { kBatch = 1, kPipe2 = 2, kPipe4 = 4, kPipe8 = 8, kPhased = 16 };

inline bool is_pipe(int sched) { return sched == kPipe2 || sched == kPipe4 || sched == kPipe8; }

template <int P, bool BCAST, bool NTL, int S>
ReduceKernel pick_pipe_unroll(int U) {
    return U == 1 ? k_reduce_pipe<P, BCAST, 1, S, NTL> : k_reduce_pipe<P, BCAST, 2, S, NTL>;
}

// Most vectors per lane k_reduce_phased takes for P inputs: a lane holds
// U x P loaded vectors (4 VGPRs each), and past 48 of them a wave outgrows
// 256 VGPRs.
constexpr int phased_max_unroll(int P) { return P >= 7 ? 6 : 8; }

template <int P, bool BCAST>
ReduceKernel pick_phased(int U) {
    constexpr int M = phased_max_unroll(P);
    switch (U < M ? U : M) {
        case 1: return k_reduce_phased<P, BCAST, 1>;
        case 2: return k_reduce_phased<P, BCAST, 2>;
        case 3: return k_reduce_phased<P, BCAST, 3>;
        case 4: return k_reduce_phased<P, BCAST, 4>;
        case 5: return k_reduce_phased<P, BCAST, 5>;
        case 6: return k_reduce_phased<P, BCAST, 6>;
        case 7: return k_reduce_phased<P, BCAST, (M >= 7 ? 7 : M)>;
        default: return k_reduce_phased<P, BCAST, M>;
    }
}

template <int P, bool BCAST, bool NTL>
ReduceKernel pick_unroll(int U, int sched) {
    if (sched == kPhased) return pick_phased<P, BCAST>(U);
    switch (sched) {
        case kPipe2: return pick_pipe_unroll<P, BCAST, NTL, 2>(U);
        case kPipe4: return pick_pipe_unroll<P, BCAST, NTL, 4>(U);
        case kPipe8: return pick_pipe_unroll<P, BCAST, NTL, 8>(U);
        default: break;
    }
    switch (U) {
        case 1: return k_reduce<P, BCAST, 1, NTL, true>;
        case 2: return k_reduce<P, BCAST, 2, NTL, true>;
        default: return k_reduce<P, BCAST, 4, true, false>;
    }
}

template <bool BCAST, bool NTL>
ReduceKernel pick_p(int P, int U, int sched) {
    switch (P) {
        case 2: return pick_unroll<2, BCAST, NTL>(U, sched);
        case 3: return pick_unroll<3, BCAST, NTL>(U, sched);
        case 4: return pick_unroll<4, BCAST, NTL>(U, sched);
        case 5: return pick_unroll<5, BCAST, NTL>(U, sched);
        case 6: return pick_unroll<6, BCAST, NTL>(U, sched);
        case 7: return pick_unroll<7, BCAST, NTL>(U, sched);
        default: return pick_unroll<8, BCAST, NTL>(U, sched);
    }
}

ReduceKernel pick(bool bcast, bool ntl, int P, int U, int sched) {
    if (bcast) return ntl ? pick_p<true, true>(P, U, sched) : pick_p<true, false>(P, U, sched);
    return ntl ? pick_p<false, true>(P, U, sched) : pick_p<false, false>(P, U, sched);
}

// Bytes one launch touches beyond which its inputs take non-temporal loads:
// half the 256 MB MALL, so data that could stay cached keeps plain loads.
constexpr int64_t kStreamingBytes = 128ll << 20;

// Launch shape overrides for benchmark sweeps (0 = automatic).
int g_unroll_override = 0;
int g_threads_override = 0;
int g_max_blocks_override = 0;
int g_schedule_override = 0;  // 0 automatic, or a Schedule

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

    // Launch shape, chosen from sweeps on MI355X with the data coming from HBM
    // (buffer sets rotated through 576 MB or more, interleaved in one process),
    // by the bulk's 16-byte vectors per input per CU (vpc; 256 CUs, 1024 SIMDs):
    //  - vpc <= 256: latency-bound; one vector per lane in 64-lane workgroups,
    //    so the work spreads over every CU;
    //  - vpc <= 768, P >= 4: the pipelined kernel in two stages, 64-lane
    //    workgroups (1M elements x 8 / x 4: 6.2 / 3.9 us instead of 6.7 / 4.1);
    //  - vpc <= 2560: one pass, every load before any store (k_reduce_phased),
    //    64-lane workgroups.  U, the vectors per lane per input, is the
    //    smallest that leaves at most one wave per SIMD (U = ceil(vpc / 256)),
    //    as far as the registers allow: the write-mode share of 440x5120 x 8
    //    (vpc 1100) runs 12.0-12.1 us with U = 5 (880 waves) against
    //    13.4-14.0 us with U = 4 (1100 waves, so 76 SIMDs run two) and 12.7
    //    with U = 6 (733 waves).  Past the register limit P = 8 takes U = 5
    //    (2048 vpc: 25.3 us against 28.0 with U = 6), P = 7 U = 6.  P <= 4
    //    keeps U = 4 up to vpc 1536 (x 4 at 1536: 8.7 us against 9.3 with
    //    U = 6), then one wave per SIMD up to U = 8 (x 4 at 2560: 14.1 us
    //    against 16.0 with U = 4);
    //  - beyond, with P outputs (write mode, two-shot): the two-stage
    //    pipelined kernel in 64-lane workgroups, one vector per lane per stage,
    //    a grid that covers the bulk: 16M elements x 4 (one owner of the 64 Mi
    //    two-shot) 47.9 against 51.0 us for 256-lane grid-stride batches, x 8
    //    103.4 against 110.2 us, x 6 72.1 against 78.2;
    //  - beyond, with one output (one-shot, reduce-scatter): one pass with
    //    U = 2 and a grid that covers the bulk, several waves per SIMD.  Median
    //    of 9 for 8M / 16M / 32M elements: x 8 26.9 / 49.7 / 97.1 us against
    //    27.5 / 51.9 / 100.1 for the pipelined kernel, x 4 15.7 / 28.8 / 54.5
    //    against 16.2 / 28.8 / 54.9, x 2 10.1 / 17.4 / 31.7 against 10.3 /
    //    18.4 / 32.7 (U = 3 or 4 won some of these by up to 6% and lost the
    //    32M ones by up to 3%).
    // With the data in the MALL instead (back-to-back calls on one buffer set
    // of up to 256 MB) the pipelined kernel is faster (9.0 against 10.1-11.1 us
    // for the 440x5120 x 8 share); the automatic choice is made for data from
    // HBM.
    int threads = 64, U = 1, sched = kBatch;
    int64_t blocks = 0;  // 0: the grid covers the bulk (set below)
    const int64_t vpc = (a.nvec + dev.cus - 1) / dev.cus;
    if (vpc <= 256) {
        blocks = (a.nvec + threads - 1) / threads;
    } else if (P >= 4 && vpc <= 768) {
        sched = kPipe2;
    } else if (vpc <= 2560) {
        sched = kPhased;
        const int one_wave_per_simd = (int)((vpc + 255) / 256);
        if (P >= 5)
            U = one_wave_per_simd <= phased_max_unroll(P) ? one_wave_per_simd
                                                          : (P == 8 ? 5 : phased_max_unroll(P));
        else
            U = vpc <= 1536 ? 4 : (one_wave_per_simd < 8 ? one_wave_per_simd : 8);
    } else if (!bcast) {
        sched = kPhased;
        U = 2;
    } else {
        sched = kPipe2;
    }
    if (g_unroll_override > 0) {
        U = g_unroll_override;
        blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
    }
    if (g_threads_override > 0) {
        threads = g_threads_override;
        blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
    }
    if (g_schedule_override != 0) sched = g_schedule_override;
    // the pipelined and phased kernels assume a non-empty bulk
    if (a.nvec == 0 && sched != kBatch) {
        sched = kBatch;
        U = 1;
        blocks = 0;
    }
    if (is_pipe(sched)) {
        // no grid stride: the grid covers the bulk, sched stages of U vectors per lane
        if (U > 2) U = 2;
        const int64_t per_block = (int64_t)threads * U * sched;
        blocks = (a.nvec + per_block - 1) / per_block;
    } else if (sched == kPhased) {
        // no grid stride: the grid covers the bulk, U vectors per lane
        if (U > phased_max_unroll(P)) U = phased_max_unroll(P);
        const int64_t per_block = (int64_t)threads * U;
        blocks = (a.nvec + per_block - 1) / per_block;
    } else {
        if (blocks == 0) blocks = (a.nvec + (int64_t)threads * U - 1) / ((int64_t)threads * U);
        if (g_max_blocks_override > 0 && blocks > g_max_blocks_override)
            blocks = g_max_blocks_override;
        if (blocks > (int64_t)dev.cus * 16) blocks = (int64_t)dev.cus * 16;  // lanes loop beyond
    }
    const int64_t scalar_blocks = (a.head + a.ntail + threads - 1) / threads;
    if (scalar_blocks > blocks) blocks = scalar_blocks;
    if (blocks < 1) blocks = 1;
    ReduceKernel fn = pick(bcast, ntl, P, U, sched);
    return launch(reinterpret_cast<const void *>(fn), (unsigned)blocks, (unsigned)threads, a, stream);
}

// The kernel addresses its outputs with 32-bit byte offsets (see store_vec),
// so a range longer than kPieceElems elements (1 GiB per buffer) is cut into
// consecutive launches on the same stream.  The streaming decision is taken
// for the whole call.
constexpr int64_t kPieceElems = 1ll << 29;
// the last 16-byte store of a piece ends at byte 2 * kPieceElems at most
static_assert(2 * kPieceElems + 16 <= (int64_t)kStoreRangeBytes,
              "a reduce piece must fit the output buffer resource's range");

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
int ar_set_reduce_tuning(int unroll, int threads, int max_blocks, int schedule) {
    const bool batch_unroll = unroll == 0 || unroll == 1 || unroll == 2 || unroll == 4;
    if (unroll < 0 || unroll > 8 || max_blocks < 0 ||
        !(threads == 0 || threads == 64 || threads == 128 || threads == 256) ||
        !(schedule == 0 || schedule == kBatch || is_pipe(schedule) || schedule == kPhased) ||
        (schedule != kPhased && !batch_unroll) || (is_pipe(schedule) && unroll == 4))
        return AR_EINVAL;
    g_unroll_override = unroll;
    g_threads_override = threads;
    g_max_blocks_override = max_blocks;
    g_schedule_override = schedule;
    return AR_OK;
}

}  // extern "C"
