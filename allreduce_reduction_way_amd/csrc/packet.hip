// packet.hip -- LL-packet codec and the fused packet allreduce share.
//
// Packets are 16 bytes {data0, flag, data1, flag}; each 8-byte half is one
// "word" {two bf16, flag} written and read as a single agent-scope atomic
// (see device.h), so a reader that sees the expected flag in a word also has
// that word's data.  Data and flag in one packet let the receiver detect
// arrival from the data itself (ARK PR #254 "Add monolithic fused packet
// allreduce kernel and Model::all_reduce_packet API", description).
//
// Work is laid out word-per-lane: lane t of a 256-lane workgroup handles word
// t (and t + 256 when a chunk is two words per lane) of each slot's chunk, so
// every 64-lane wavefront issues 512-byte contiguous atomic accesses and
// 256-byte contiguous element accesses.
//
// The fused kernel runs the P emulated ranks as groups of workgroups of one
// persistent grid: workgroup b serves rank lo + b % R and chunks m, m + B,
// m + 2B, ... with m = b / R (R ranks in the launch, B workgroups per rank).
// Rank r on chunk c does, for each of its words:
//   scatter    x_r[slice j] -> inbox_j[slot r]           for j = 0..P-1
//   reduce     inbox_r[slot 0..P-1] -> rank-order sum     (waits on flags)
//   broadcast  sum -> resbox_j[slot r]                    for j = 0..P-1
//   receive    resbox_r[slot 0..P-1] -> out_r             (waits on flags)
// and the three stages of consecutive chunks overlap in a software pipeline.
// The only synchronisation between workgroups is the flag inside each word:
// lane t of rank r waits only on lane t of the other ranks' workgroups of the
// same m, and everything a lane waits on was written before its producer
// could wait on anything later (torchcomms PR #3850 "Add HIP-graph capture
// coverage for the sharded-relay collectives", commit summary D117629704:
// pairwise handshakes, no global barrier, write and flag before waiting).
// The grid never exceeds the number of workgroups that fit on the device at
// once, so every workgroup a lane waits on is resident; all waits are bounded
// and report AR_ETIMEDOUT.
#include <mutex>

#include "device.h"
#include "host.h"

// Device memory of ar_packet_fused_noalloc, for callers that cannot allocate:
// its control block (first 256 bytes) and the P scratch buffers.  Every GPU
// the library runs on holds its own copy until the process ends; like any
// object of static storage it starts zeroed.  On the host this name is only
// a stand-in for the device object: host code never hands it to a kernel, it
// takes each device's address from hipGetSymbolAddress (noalloc_base).
static __device__ __align__(256) uint8_t scratch[AR_NOALLOC_SCRATCH_BYTES];

namespace ar {
namespace {

// Two bf16 starting at element e of a slice of `len` elements (e even, e < len
// or the word is padding), packed low element first; elements past the slice
// read as zero.  Every element is read once and written once per call, so
// the aligned case takes non-temporal (streaming) accesses: they leave L2 and
// the MALL to the packets, which are read back within the call.
__device__ __forceinline__ uint32_t load_pair(const uint16_t *p, int64_t e, int64_t len,
                                              bool aligned4) {
    if (e + 1 < len) {
        if (aligned4) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + e));
        return (uint32_t)p[e] | ((uint32_t)p[e + 1] << 16);
    }
    return e < len ? (uint32_t)p[e] : 0u;
}

__device__ __forceinline__ void store_pair(uint16_t *p, int64_t e, int64_t len, bool aligned4,
                                           uint32_t d) {
    if (e + 1 < len) {
        if (aligned4) {
            __builtin_nontemporal_store(d, reinterpret_cast<uint32_t *>(p + e));
        } else {
            p[e] = (uint16_t)d;
            p[e + 1] = (uint16_t)(d >> 16);
        }
    } else if (e < len) {
        p[e] = (uint16_t)d;
    }
}

// ---- standalone encode / decode ----------------------------------------------
//
// (Non-temporal element accesses: decode of 512x7168 on MI355X runs 3.85 us
// instead of 4.42 us per call.)

// 56 bytes, so that the grid size the runtime appends after them (read for
// the grid strides) shares their first 64-byte line: with a 64-byte struct it
// fell on a second line, whose fetch came as a second dependent round of
// kernel-argument loads at the start of every wave.  Measured on MI355X with
// an LL encode kernel on this struct, 512x7168 from HBM: 5.25 against 5.65 us
// per call.  The encode's own arguments (EncodeArgs) keep the same bound.
struct CodecArgs {
    uint16_t *elems;        // decode destination
    uint64_t *words;        // packet words (2 per packet)
    int64_t n;
    int64_t nwords;
    uint32_t flag;
    int aligned4;
    int32_t *status;
    uint64_t max_spins;
};
static_assert(sizeof(CodecArgs) <= 56, "the grid size must share the arguments' first 64-byte line");

// One encode launch: word w of `words` packs elements 2w and 2w+1 of
// `elems`.  Words [0, nbulk) are the bulk (both elements exist, `elems` is
// 4-byte aligned); words [nbulk, nwords) take one word per lane.
struct EncodeArgs {
    const uint16_t *elems;
    uint64_t *words;
    int64_t n;       // elements from `elems`
    int64_t nbulk;
    int64_t nwords;
    uint32_t flag;
};
static_assert(sizeof(EncodeArgs) <= 56, "the grid size must share the arguments' first 64-byte line");

// Encode.  The bulk goes kEncodeUnroll words per lane in one pass: global
// wave g takes the kEncodeUnroll x 64 consecutive words from
// g x kEncodeUnroll x 64 and issues all its loads before any store (the
// scheduling barrier keeps them apart), so the device sees mostly reads,
// then mostly writes.  Lanes past the bulk load its last word again (in
// bounds) and give their stores an offset past the resource's range, which
// the hardware drops: no branch around the stores.  The stores are the
// 8-byte device-scope (sc1) stores of an agent-scope atomic plus the
// streaming hint (nt), through one buffer resource per launch; a range
// longer than kEncodePieceWords runs as several launches so every offset
// fits the resource.  The rest -- the odd last element, the zero padding of
// the last packet, or the whole range for a 2-byte-aligned source -- takes
// one word per lane in a grid stride.  Measured on MI355X for 512x7168, in
// one process: from HBM (32 buffer pairs in turn) 4.8 us per call against
// 5.3 us for the same loads with per-lane agent-scope atomic stores behind
// bounds branches in a grid-stride loop; back to back on one buffer pair
// 3.37 against 3.63 us.
constexpr int kEncodeUnroll = 4;
constexpr int64_t kEncodePieceWords = 1ll << 27;
static_assert(8 * kEncodePieceWords + 8 <= (int64_t)kStoreRangeBytes,
              "every packet word of an encode piece must lie inside the store range");

// The 8-byte store of an agent-scope atomic (sc1: through to the device
// coherence point) with the streaming hint (nt), at byte offset `byte_off`
// from `base` (the same for every lane of the wavefront); dropped past
// kStoreRangeBytes.
__device__ __forceinline__ void store_word_stream(uint64_t *base, uint32_t byte_off, uint64_t w) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(base, (short)0, kStoreRangeBytes, 0x00020000);
    u32x2 v;
    v[0] = word_data(w);
    v[1] = word_flag(w);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 18);
}

// Words [from, nwords), one per lane, grid stride.
__device__ __forceinline__ void encode_words(const EncodeArgs &a, int64_t from) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t w = from + (int64_t)blockIdx.x * kThreads + threadIdx.x; w < a.nwords;
         w += stride)
        store_word(a.words + w, make_word(load_pair(a.elems, 2 * w, a.n, false), a.flag));
}

// The bulk (nbulk >= 1, one pass: the grid covers it), then the tail.
__global__ __launch_bounds__(kThreads) void k_ll_encode(EncodeArgs a) {
    constexpr int U = kEncodeUnroll;
    const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t base = (g >> 6) * (64 * U) + (g & 63);
    const uint32_t *src = reinterpret_cast<const uint32_t *>(a.elems);
    uint32_t d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t w = base + 64 * u;
        w = w < a.nbulk ? w : a.nbulk - 1;
        d[u] = __builtin_nontemporal_load(src + w);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = base + 64 * u;
        const uint32_t off = w < a.nbulk ? (uint32_t)(8 * w) : kDroppedStoreOffset;
        store_word_stream(a.words, off, make_word(d[u], a.flag));
    }
    encode_words(a, a.nbulk);
}

// No bulk: every word one per lane.
__global__ __launch_bounds__(kThreads) void k_ll_encode_words(EncodeArgs a) {
    encode_words(a, 0);
}

// Four words in flight per lane: 8-byte loads need many requests outstanding
// to keep HBM busy.  A word whose two elements both lie in a 4-byte-aligned
// destination is stored with one non-temporal 4-byte store; the rest go
// through store_pair.  (Measured on MI355X for 512x7168: 3.40-3.48 us per
// call back to back on one buffer pair against 3.75 us with store_pair for
// every word, 5.69-5.74 against 5.85 us from HBM.)
__global__ __launch_bounds__(kThreads) void k_ll_decode(CodecArgs a) {
    constexpr int K = 4;
    const int64_t nwhole = a.aligned4 ? a.n / 2 : 0;  // words with both elements
    uint32_t *dst32 = reinterpret_cast<uint32_t *>(a.elems);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t w0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; w0 < a.nwords;
         w0 += stride * K) {
        uint64_t v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t w = w0 + k * stride;
            v[k] = w < a.nwords ? load_word(a.words + w) : make_word(0, a.flag);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int64_t w = w0 + k * stride;
            if (w >= a.nwords) continue;
            if (word_flag(v[k]) != a.flag &&
                !wait_word(a.words + w, a.flag, v[k], a.status, a.max_spins))
                return;
            if (w < nwhole)
                __builtin_nontemporal_store(word_data(v[k]), dst32 + w);
            else
                store_pair(a.elems, 2 * w, a.n, a.aligned4, word_data(v[k]));
        }
    }
}

// ---- fused kernel ----------------------------------------------------------------

struct FusedArgs {
    ar_ptrs in;       // P inputs
    ar_ptrs scratch;  // P scratch buffers: [inbox: P slots][resbox: P slots]
    ar_ptrs out;      // P outputs
    int64_t n;
    int64_t L;        // length of slices 0..P-2; the last one is n - (P-1) L
    int64_t slot_words;  // 2 x packets per slot
    int64_t chunks;   // chunks of chunk_words words covering a slot
    int rank_lo;
    int nranks;       // R
    int per_rank;     // B
    uint32_t flag;
    int aligned4;
    int32_t *status;   // ar_ctrl.status (the control block's first word)
    uint32_t *epoch;   // ar_ctrl.epoch (second word)
    uint32_t *arrivals;  // ar_ctrl.arrivals (third word)
    uint64_t max_spins;
    // Library-owned control block (static scratch): at the end of an EPOCH
    // launch the last workgroup copies the status to status_out (if set) and
    // clears it, so the next call starts from AR_OK.
    int own_ctrl;
    int32_t *status_out;
};

// Elements in slice j (the last slice absorbs the remainder).
__device__ __forceinline__ int64_t slice_len(const FusedArgs &a, int j, int P) {
    return j == P - 1 ? a.n - (int64_t)(P - 1) * a.L : a.L;
}

// One pipeline step of rank r: scatter chunk cs (if do_s), reduce and
// broadcast chunk cr (if do_r), receive chunk cv (if do_v).  Every load of
// the step is issued before any store: on CDNA the vector-memory counter
// covers loads and stores alike, so a load issued after a write-through store
// would also wait for that store's acknowledgement.
//
// The element side takes non-temporal accesses (load_pair, store_pair), so it
// does not push the scratch packets, which are read back within the call, out
// of L2 and the MALL: 100.8 us instead of 111.3 us per call for 512x7168 x 8
// on MI355X (the loads give most of it).
//
// CARRY: the rank's own contributions come from registers instead of being
// read back from its own slots -- its scatter of chunk c into inbox_r[slot r]
// (one step before it reduces c) and its broadcast of chunk c into
// resbox_r[slot r] (one step before it receives c).  The packets are still
// written, so the scratch image is unchanged; only the read-back of the own
// slot, a local memory access, goes away.  `own_d` carries the scatter data
// and `own_res` the reduced words from one step to the next.
template <int P, int WPL, bool CARRY>
__device__ __forceinline__ bool pipeline_step(const FusedArgs &a, uint32_t flag, int r, bool do_s,
                                              int64_t cs, bool do_r, int64_t cr, bool do_v,
                                              int64_t cv, uint32_t (&own_d)[WPL],
                                              uint32_t (&own_res)[WPL]) {
    const uint16_t *x_r = static_cast<const uint16_t *>(a.in.p[r]);
    const uint64_t *mine = static_cast<const uint64_t *>(a.scratch.p[r]);
    constexpr int64_t CW = (int64_t)kThreads * WPL;
    const int64_t ws0 = cs * CW + threadIdx.x;
    const int64_t wr0 = cr * CW + threadIdx.x;
    const int64_t wv0 = cv * CW + threadIdx.x;
    const int64_t r_words = 2 * ((slice_len(a, r, P) + 3) / 4);

    // ---- loads
    uint32_t d[P][WPL];
    uint64_t vr[WPL][P];
    uint64_t vv[P][WPL];
    if (do_s) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int64_t len = slice_len(a, j, P);
#pragma unroll
            for (int k = 0; k < WPL; ++k)
                d[j][k] = load_pair(x_r + j * a.L, 2 * (ws0 + k * kThreads), len, a.aligned4);
        }
    }
    if (do_r) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int64_t w = wr0 + k * kThreads;
#pragma unroll
            for (int s = 0; s < P; ++s) {
                if (CARRY && s == r)
                    vr[k][s] = make_word(own_d[k], flag);
                else
                    vr[k][s] = w < r_words ? load_word(mine + (int64_t)s * a.slot_words + w) : 0;
            }
        }
    }
    if (do_v) {
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int64_t len = slice_len(a, s, P);
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                const int64_t w = wv0 + k * kThreads;
                if (CARRY && s == r)
                    vv[s][k] = make_word(own_res[k], flag);
                else
                    vv[s][k] = 2 * w < len ? load_word(mine + (int64_t)(P + s) * a.slot_words + w)
                                           : make_word(0, flag);
            }
        }
    }

    // ---- scatter: x_r[slice j] -> inbox_j[slot r]
    if (do_s) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int64_t words = 2 * ((slice_len(a, j, P) + 3) / 4);
            uint64_t *slot = static_cast<uint64_t *>(a.scratch.p[j]) + (int64_t)r * a.slot_words;
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                const int64_t w = ws0 + k * kThreads;
                if (w < words) store_word(slot + w, make_word(d[j][k], flag));
            }
        }
    }

    // ---- reduce inbox_r[slot 0..P-1] in rank order, broadcast to resbox_j[slot r]
    uint32_t res_d[WPL];
    if (do_r) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            const int64_t w = wr0 + k * kThreads;
            res_d[k] = 0;
            if (w >= r_words) continue;
            uint32_t dw[P];
#pragma unroll
            for (int s = 0; s < P; ++s) {
                if (word_flag(vr[k][s]) != flag &&
                    !wait_word(mine + (int64_t)s * a.slot_words + w, flag, vr[k][s], a.status,
                               a.max_spins))
                    return false;
                dw[s] = word_data(vr[k][s]);
            }
            res_d[k] = reduce_word<P>(dw);
            const uint64_t res = make_word(res_d[k], flag);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                uint64_t *resbox_j = static_cast<uint64_t *>(a.scratch.p[j]) + P * a.slot_words;
                store_word(resbox_j + r * a.slot_words + w, res);
            }
        }
    }

    // ---- receive resbox_r[slot s] (reduced slice s) -> out_r[slice s]
    if (do_v) {
        uint16_t *out_r = static_cast<uint16_t *>(a.out.p[r]);
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int64_t len = slice_len(a, s, P);
#pragma unroll
            for (int k = 0; k < WPL; ++k) {
                const int64_t w = wv0 + k * kThreads;
                if (2 * w >= len) continue;
                if (word_flag(vv[s][k]) != flag &&
                    !wait_word(mine + (int64_t)(P + s) * a.slot_words + w, flag, vv[s][k],
                               a.status, a.max_spins))
                    return false;
                store_pair(out_r + s * a.L, 2 * w, len, a.aligned4, word_data(vv[s][k]));
            }
        }
    }

    // hand this step's own-slot words to the next step
    if (CARRY) {
#pragma unroll
        for (int k = 0; k < WPL; ++k) {
            if (do_r) own_res[k] = res_d[k];
            if (do_s) own_d[k] = d[r][k];
        }
    }
    return true;
}

// Workgroup b serves rank lo + b % R and its chunks m, m + B, m + 2B, ...
// (m = b / R) as a three-stage software pipeline: step i scatters chunk i,
// reduces and broadcasts chunk i-1 and receives chunk i-2.  Everything a
// step waits on was produced by the other ranks' workgroups of the same m in
// their step i-1, before they could wait on anything in step i, so by
// induction over steps every wait is satisfied, and a wait normally finds its
// packets already there.
//
// EPOCH: the flag is not a kernel argument but ar_ctrl.epoch + 1, read by
// every lane at the start; the last workgroup to finish stores it back as the
// new epoch.  A launch captured in a graph then uses a new flag on every
// replay instead of the one baked in at capture (torchcomms PR #3850, PR
// summary, hazard G2: a by-value epoch replayed is already satisfied by every
// flag).  Every workgroup reads the epoch before it counts itself in, and the
// count completes only after the last one has, so all of them use one flag.
template <int P, int WPL, bool EPOCH>
__global__ __launch_bounds__(kThreads) void k_packet_fused(FusedArgs a) {
    // The arguments stay read-only (writing to them would move the whole
    // struct to scratch memory); the epoch is made wave-uniform.
    const uint32_t flag =
        EPOCH ? __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u)
              : a.flag;
    const int r = a.rank_lo + (int)(blockIdx.x % (unsigned)a.nranks);
    const int64_t m = blockIdx.x / (unsigned)a.nranks;
    const int64_t B = a.per_rank;
    const int64_t mine = m < a.chunks ? (a.chunks - 1 - m) / B + 1 : 0;
    uint32_t own_d[WPL] = {}, own_res[WPL] = {};
    for (int64_t i = 0; i < mine + 2; ++i) {
        if (!pipeline_step<P, WPL, true>(a, flag, r, i < mine, m + i * B, i >= 1 && i <= mine,
                                         m + (i - 1) * B, i >= 2, m + (i - 2) * B, own_d, own_res))
            break;
    }
    if (EPOCH) {
        __syncthreads();
        if (threadIdx.x == 0) {
            // With a library-owned block the arrival is a release and the last
            // one an acquire, so a status raised by any lane of any workgroup
            // is seen by the last workgroup before it reports and clears it.
            if (a.own_ctrl) __threadfence();
            const uint32_t before = __hip_atomic_fetch_add(a.arrivals, 1u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            if (before == gridDim.x - 1) {
                if (a.own_ctrl) {
                    // every workgroup has stopped waiting: nobody reads the status now
                    __threadfence();
                    const int32_t st = load_status(a.status);
                    if (a.status_out)
                        __hip_atomic_store(a.status_out, st, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(a.status, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __hip_atomic_store(a.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.epoch, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// The three-operation decomposition, one launch per phase (ARK PR #254,
// description: the send_packet -> recv_reduce_send_packet -> recv_packet
// pipeline that the fused kernel replaces): PHASE 0 scatters, 1 reduces and
// broadcasts, 2 receives.  Each (rank, chunk) item is independent within a
// launch; waits are on packets of the previous phase's launch (or of another
// stream's).
template <int P, int WPL, int PHASE>
__global__ __launch_bounds__(kThreads) void k_packet_phase(FusedArgs a) {
    const int64_t items = (int64_t)a.nranks * a.chunks;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int r = a.rank_lo + (int)(it % a.nranks);
        const int64_t c = it / a.nranks;
        uint32_t unused_d[WPL], unused_res[WPL];
        if (!pipeline_step<P, WPL, false>(a, a.flag, r, PHASE == 0, c, PHASE == 1, c, PHASE == 2,
                                          c, unused_d, unused_res))
            return;
    }
}

// Role-split schedule of the fused kernel: the grid is three consecutive
// ranges of R x B workgroups -- scatter, reduce-broadcast, receive -- and
// workgroup (role, r, m) runs its phase for rank r over chunks m, m + B, ...
// A role only waits on roles before it (reduce on scatter, receive on reduce),
// scatter never waits, and producers come first in workgroup order; with the
// whole grid resident every wait is satisfied.  The own slots are read back
// (no register carry across roles).
template <int P, int WPL>
__global__ __launch_bounds__(kThreads) void k_packet_roles(FusedArgs a) {
    const int64_t per_role = (int64_t)a.nranks * a.per_rank;
    const int role = (int)(blockIdx.x / per_role);
    const int64_t b = blockIdx.x % per_role;
    const int r = a.rank_lo + (int)(b % a.nranks);
    const int64_t m = b / a.nranks;
    uint32_t unused_d[WPL], unused_res[WPL];
    for (int64_t c = m; c < a.chunks; c += a.per_rank) {
        if (!pipeline_step<P, WPL, false>(a, a.flag, r, role == 0, c, role == 1, c, role == 2, c,
                                          unused_d, unused_res))
            return;
    }
}

typedef void (*FusedKernel)(FusedArgs);

template <int P, int WPL>
FusedKernel pick_kind(int kind) {
    switch (kind) {
        case 0: return k_packet_fused<P, WPL, false>;
        case 1: return k_packet_fused<P, WPL, true>;
        case 2: return k_packet_phase<P, WPL, 0>;
        case 3: return k_packet_phase<P, WPL, 1>;
        case 4: return k_packet_phase<P, WPL, 2>;
        default: return k_packet_roles<P, WPL>;
    }
}

template <int WPL>
FusedKernel pick_p(int P, int kind) {
    switch (P) {
        case 2: return pick_kind<2, WPL>(kind);
        case 3: return pick_kind<3, WPL>(kind);
        case 4: return pick_kind<4, WPL>(kind);
        case 5: return pick_kind<5, WPL>(kind);
        case 6: return pick_kind<6, WPL>(kind);
        case 7: return pick_kind<7, WPL>(kind);
        default: return pick_kind<8, WPL>(kind);
    }
}

enum Kind { kFused = 0, kFusedEpoch = 1, kSend = 2, kRecvReduceSend = 3, kRecv = 4, kRoles = 5 };

// Launch-shape overrides for benchmark sweeps: workgroups per rank and words
// per lane per chunk (0 = automatic).
int g_fused_per_rank_override = 0;
int g_fused_wpl_override = 0;
int g_fused_schedule = 0;  // 0 pipelined workgroups, 1 role-split workgroups

// Validates one packet-path call and fills the kernel arguments.  `use_in`,
// `use_out`, `use_ctrl` say which buffers the entry point touches; every
// table it uses needs P non-null pointers; no two distinct buffers it uses may
// share a byte (identical input pointers are fine: inputs are only read).
int prepare_packet(const ar_ptrs &in, const ar_ptrs &scratch, const ar_ptrs &out, bool use_in,
                   bool use_out, bool use_ctrl, int P, int rank_lo, int rank_hi, int64_t n,
                   uint32_t flag, bool need_flag, void *ctrl, uint64_t max_spins, int wpl,
                   FusedArgs *a) {
    if (!valid_P(P) || n < 0 || rank_lo < 0 || rank_hi > P || rank_lo >= rank_hi) return AR_EINVAL;
    if (need_flag && flag == 0) return AR_EINVAL;
    if (use_ctrl && (!ctrl || !aligned_to(ctrl, 4))) return AR_EINVAL;
    for (int p = 0; p < P; ++p) {
        if (!scratch.p[p] || !aligned_to(scratch.p[p], 16)) return AR_EINVAL;
        if (use_in && (!in.p[p] || !aligned_to(in.p[p], 2))) return AR_EINVAL;
        if (use_out && (!out.p[p] || !aligned_to(out.p[p], 2))) return AR_EINVAL;
    }
    if (n == 0) return AR_OK;
    const int64_t sbytes = ar_packet_scratch_bytes(P, n);
    Span spans[3 * AR_MAX_P + 1];
    int kind[3 * AR_MAX_P + 1];
    int ns = 0;
    for (int p = 0; p < P; ++p) {
        if (use_in) {
            spans[ns] = span_of(in.p[p], 0, n, 2);
            kind[ns++] = 0;
        }
        if (use_out) {
            spans[ns] = span_of(out.p[p], 0, n, 2);
            kind[ns++] = 1;
        }
        spans[ns] = span_of(scratch.p[p], 0, sbytes, 1);
        kind[ns++] = 2;
    }
    if (use_ctrl) {
        spans[ns] = span_of(ctrl, 0, AR_CTRL_BYTES, 1);
        kind[ns++] = 3;
    }
    for (int i = 0; i < ns; ++i)
        for (int k = i + 1; k < ns; ++k)
            if (overlap(spans[i], spans[k]) && !(kind[i] == 0 && kind[k] == 0)) return AR_EALIAS;

    *a = FusedArgs{};
    a->in = in;
    a->scratch = scratch;
    a->out = out;
    a->n = n;
    a->L = slice_len_unit(P, n);
    a->slot_words = 2 * ar_packet_slot_packets(P, n);
    const int64_t chunk_words = (int64_t)kThreads * wpl;
    a->chunks = (a->slot_words + chunk_words - 1) / chunk_words;
    a->rank_lo = rank_lo;
    a->nranks = rank_hi - rank_lo;
    a->flag = flag;
    bool al4 = true;
    for (int p = 0; p < P; ++p) {
        if (use_in) al4 = al4 && aligned_to(in.p[p], 4);
        if (use_out) al4 = al4 && aligned_to(out.p[p], 4);
    }
    a->aligned4 = al4;
    if (use_ctrl) {
        a->status = static_cast<int32_t *>(ctrl);
        a->epoch = static_cast<uint32_t *>(ctrl) + 1;
        a->arrivals = static_cast<uint32_t *>(ctrl) + 2;
    }
    a->max_spins = max_spins ? max_spins : AR_DEFAULT_MAX_SPINS;
    return AR_OK;
}

int packet_call(Kind kind_in, const ar_ptrs &in, const ar_ptrs &scratch, const ar_ptrs &out, int P,
                int rank_lo, int rank_hi, int64_t n, uint32_t flag, void *ctrl, uint64_t max_spins,
                void *stream, int32_t *status_out = nullptr, bool own_ctrl = false) {
    Kind kind = kind_in;
    if (kind == kFused && g_fused_schedule == 1) kind = kRoles;
    const bool use_in = kind == kFused || kind == kFusedEpoch || kind == kSend || kind == kRoles;
    const bool use_out = kind == kFused || kind == kFusedEpoch || kind == kRecv || kind == kRoles;
    const bool use_ctrl = kind != kSend;
    // Two words per lane per chunk: 98.3 us against 111.4 us with one word
    // for 512x7168 x 8 on MI355X (fewer, wider chunks; 155 VGPRs, 3
    // workgroups per CU; fewer workgroups per rank than fit ran slower).
    const int wpl = g_fused_wpl_override ? g_fused_wpl_override : 2;
    FusedArgs a;
    int rc = prepare_packet(in, scratch, out, use_in, use_out, use_ctrl, P, rank_lo, rank_hi, n,
                            flag, kind != kFusedEpoch, ctrl, max_spins, wpl, &a);
    if (rc != AR_OK || n == 0) return rc;
    a.own_ctrl = own_ctrl;
    a.status_out = status_out;
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    FusedKernel fn = wpl == 1 ? pick_p<1>(P, kind) : pick_p<2>(P, kind);

    if (kind == kSend || kind == kRecvReduceSend || kind == kRecv) {
        // Independent items, grid-stride.  The send phase never waits and
        // takes a full grid; a waiting phase takes at most half of what is
        // resident at once, leaving room for a producer that runs beside it.
        int64_t blocks = (int64_t)a.nranks * a.chunks;
        int64_t cap = (int64_t)dev.cus * 16;
        if (kind != kSend) {
            const int per_cu = blocks_per_cu(dev, reinterpret_cast<const void *>(fn));
            if (per_cu <= 0) return AR_ELAUNCH;
            cap = (int64_t)per_cu * dev.cus / 2;
            if (cap < 1) cap = 1;
        }
        if (blocks > cap) blocks = cap;
        a.per_rank = 0;
        return launch(reinterpret_cast<const void *>(fn), (unsigned)blocks, kThreads, a, stream);
    }

    // Persistent grid no larger than what is resident at once: B workgroups per
    // rank, every one that fits.  Only when that leaves at most two chunks per
    // workgroup is B lowered so that every workgroup runs the same number.
    // Measured on MI355X in one process (medians of 7, P x n): keeping every
    // resident workgroup ran 8 x 3.67M in 96.8-97.4 against 100.3-101.5 us
    // for the evened grid, 8 x 2M 55.9 against 58.7, 8 x 2.6M 71.5 against
    // 75.3, 8 x 6M 169.5 against 175.0, 8 x 12M 341.4 against 356.4, 4 x 3.67M
    // 48.1 against 51.8, 6 x 3.67M 73.5 against 82.4, 5 x 3.67M 62.2 against
    // 66.7, 3 x 3.67M 35.8 against 38.4; with two chunks per workgroup at most
    // the evened grid won (8 x 1M: 32.2 against 34.3 us) or tied (8 x 1.5M,
    // 6 x 1.5M, 8 x 0.8M).
    const int per_cu = blocks_per_cu(dev, reinterpret_cast<const void *>(fn));
    if (per_cu <= 0) return AR_ELAUNCH;
    const int64_t resident = (int64_t)per_cu * dev.cus;
    const int64_t roles = kind == kRoles ? 3 : 1;
    int64_t B = resident / (a.nranks * roles);
    if (g_fused_per_rank_override > 0 && g_fused_per_rank_override < B)
        B = g_fused_per_rank_override;
    if (B > a.chunks) B = a.chunks;
    if (B < 1) return AR_ELAUNCH;
    const int64_t rounds = (a.chunks + B - 1) / B;
    if (rounds <= 2) B = (a.chunks + rounds - 1) / rounds;
    a.per_rank = (int)B;
    return launch(reinterpret_cast<const void *>(fn), (unsigned)(roles * B * a.nranks), kThreads,
                  a, stream);
}

// ---- static scratch of ar_packet_fused_noalloc ----------------------------------

constexpr int64_t kNoallocCtrlRegion = 256;  // control block, padded to the array's alignment
constexpr int64_t kNoallocAlign = 256;       // each rank's scratch buffer starts 256-B aligned

std::mutex g_noalloc_mu;
uint8_t *g_noalloc_base[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of the static array on the current device, looked up once
// per device with that device current; AR_ELAUNCH if the lookup fails.
int noalloc_base(const DeviceInfo &dev, uint8_t **base) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_base[dev.device]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr ||
            !aligned_to(ptr, kNoallocAlign))
            return AR_ELAUNCH;
        g_noalloc_base[dev.device] = static_cast<uint8_t *>(ptr);
    }
    *base = g_noalloc_base[dev.device];
    return AR_OK;
}

// Bytes of one rank's scratch buffer inside the static array.
int64_t noalloc_rank_stride(int P, int64_t n) {
    return round_up(ar_packet_scratch_bytes(P, n), kNoallocAlign);
}

}  // namespace
}  // namespace ar

using namespace ar;

extern "C" {

int ar_ll_encode(const void *src, void *dst_pkts, int64_t n, uint32_t flag, void *stream) {
    if (n < 0 || flag == 0) return AR_EINVAL;
    if (n == 0) return AR_OK;
    if (!src || !dst_pkts || !aligned_to(src, 2) || !aligned_to(dst_pkts, 16)) return AR_EINVAL;
    if (overlap(span_of(src, 0, n, 2), span_of(dst_pkts, 0, ar_ll_packets(n), 16)))
        return AR_EALIAS;
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    const uint16_t *elems = static_cast<const uint16_t *>(src);
    uint64_t *words = static_cast<uint64_t *>(dst_pkts);
    const int64_t nwords = 2 * ar_ll_packets(n);
    const int64_t nbulk = aligned_to(src, 4) ? n / 2 : 0;
    if (nbulk == 0) {
        // a grid stride of at most 8 workgroups per CU over every word
        EncodeArgs a = {elems, words, n, 0, nwords, flag};
        int64_t blocks = (nwords + kThreads - 1) / kThreads;
        if (blocks > (int64_t)dev.cus * 8) blocks = (int64_t)dev.cus * 8;
        return launch(reinterpret_cast<const void *>(&k_ll_encode_words), (unsigned)blocks,
                      kThreads, a, stream);
    }
    // the bulk in pieces of at most kEncodePieceWords words, one pass each;
    // the last piece also takes the tail
    const int64_t per_block = (int64_t)kThreads * kEncodeUnroll;
    for (int64_t w0 = 0; w0 < nbulk; w0 += kEncodePieceWords) {
        const int64_t piece = nbulk - w0 < kEncodePieceWords ? nbulk - w0 : kEncodePieceWords;
        const bool last = w0 + piece == nbulk;
        EncodeArgs a = {elems + 2 * w0, words + w0, n - 2 * w0, piece,
                        last ? nwords - w0 : piece, flag};
        const int rc = launch(reinterpret_cast<const void *>(&k_ll_encode),
                              (unsigned)((piece + per_block - 1) / per_block), kThreads, a, stream);
        if (rc != AR_OK) return rc;
    }
    return AR_OK;
}

int ar_ll_decode(const void *src_pkts, void *dst, int64_t n, uint32_t flag, void *ctrl,
                 uint64_t max_spins, void *stream) {
    if (n < 0 || flag == 0) return AR_EINVAL;
    if (n == 0) return AR_OK;
    if (!src_pkts || !dst || !aligned_to(dst, 2) || !aligned_to(src_pkts, 16) ||
        (ctrl && !aligned_to(ctrl, 4)))
        return AR_EINVAL;
    const Span sd = span_of(dst, 0, n, 2), sp = span_of(src_pkts, 0, ar_ll_packets(n), 16);
    if (overlap(sd, sp)) return AR_EALIAS;
    if (ctrl) {
        const Span sc = span_of(ctrl, 0, AR_CTRL_BYTES, 1);
        if (overlap(sd, sc) || overlap(sp, sc)) return AR_EALIAS;
    }
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    CodecArgs a = {};
    a.elems = static_cast<uint16_t *>(dst);
    a.words = static_cast<uint64_t *>(const_cast<void *>(src_pkts));
    a.n = n;
    a.nwords = 2 * ar_ll_packets(n);
    a.flag = flag;
    a.aligned4 = aligned_to(dst, 4);
    a.status = static_cast<int32_t *>(ctrl);
    a.max_spins = max_spins ? max_spins : AR_DEFAULT_MAX_SPINS;
    // At most half of what is resident at once: decode may wait on a
    // producer that needs CUs of its own.
    const int per_cu = blocks_per_cu(dev, reinterpret_cast<const void *>(&k_ll_decode));
    if (per_cu <= 0) return AR_ELAUNCH;
    int64_t cap = (int64_t)per_cu * dev.cus / 2;
    if (cap < 1) cap = 1;
    int64_t blocks = (a.nwords + 4 * kThreads - 1) / (4 * kThreads);
    if (blocks > cap) blocks = cap;
    return launch(reinterpret_cast<const void *>(&k_ll_decode), (unsigned)blocks, kThreads, a,
                  stream);
}

int ar_packet_fused(ar_ptrs in, ar_ptrs scratch, ar_ptrs out, int P, int rank_lo, int rank_hi,
                    int64_t n, uint32_t flag, void *ctrl, uint64_t max_spins, void *stream) {
    return packet_call(kFused, in, scratch, out, P, rank_lo, rank_hi, n, flag, ctrl, max_spins,
                       stream);
}

int ar_packet_fused_epoch(ar_ptrs in, ar_ptrs scratch, ar_ptrs out, int P, int rank_lo,
                          int rank_hi, int64_t n, void *ctrl, uint64_t max_spins, void *stream) {
    return packet_call(kFusedEpoch, in, scratch, out, P, rank_lo, rank_hi, n, 0, ctrl, max_spins,
                       stream);
}

int ar_packet_fused_noalloc(ar_ptrs in, ar_ptrs out, int P, int64_t n, int32_t *d_status,
                            uint64_t max_spins, void *stream) {
    // host-only checks first: nothing touches the GPU for a call that cannot run
    if (!valid_P(P) || n < 0) return AR_EINVAL;
    if (d_status && !aligned_to(d_status, 4)) return AR_EINVAL;
    for (int p = 0; p < P; ++p) {
        if (!in.p[p] || !aligned_to(in.p[p], 2)) return AR_EINVAL;
        if (!out.p[p] || !aligned_to(out.p[p], 2)) return AR_EINVAL;
    }
    const int64_t stride = noalloc_rank_stride(P, n);
    if (kNoallocCtrlRegion + (int64_t)P * stride > (int64_t)AR_NOALLOC_SCRATCH_BYTES)
        return AR_ENOSPACE;
    if (d_status) {
        const Span ss = span_of(d_status, 0, 4, 1);
        for (int p = 0; p < P; ++p)
            if (overlap(ss, span_of(in.p[p], 0, n, 2)) || overlap(ss, span_of(out.p[p], 0, n, 2)))
                return AR_EALIAS;
    }
    if (n == 0) return AR_OK;
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    uint8_t *base = nullptr;
    if (noalloc_base(dev, &base) != AR_OK) return AR_ELAUNCH;
    ar_ptrs bufs = {};
    for (int p = 0; p < P; ++p) bufs.p[p] = base + kNoallocCtrlRegion + (int64_t)p * stride;
    return packet_call(kFusedEpoch, in, bufs, out, P, 0, P, n, 0, base, max_spins, stream,
                       d_status, true);
}

int ar_packet_send(ar_ptrs in, ar_ptrs scratch, int P, int rank_lo, int rank_hi, int64_t n,
                   uint32_t flag, void *stream) {
    return packet_call(kSend, in, scratch, ar_ptrs{}, P, rank_lo, rank_hi, n, flag, nullptr, 0,
                       stream);
}

int ar_packet_recv_reduce_send(ar_ptrs scratch, int P, int rank_lo, int rank_hi, int64_t n,
                               uint32_t flag, void *ctrl, uint64_t max_spins, void *stream) {
    return packet_call(kRecvReduceSend, ar_ptrs{}, scratch, ar_ptrs{}, P, rank_lo, rank_hi, n, flag,
                       ctrl, max_spins, stream);
}

int ar_packet_recv(ar_ptrs scratch, ar_ptrs out, int P, int rank_lo, int rank_hi, int64_t n,
                   uint32_t flag, void *ctrl, uint64_t max_spins, void *stream) {
    return packet_call(kRecv, ar_ptrs{}, scratch, out, P, rank_lo, rank_hi, n, flag, ctrl,
                       max_spins, stream);
}

// Benchmark-only override of the packet kernels' workgroups per rank (0 =
// auto; never above the resident limit) and words per lane per chunk.
int ar_set_packet_tuning(int per_rank, int words_per_lane, int schedule) {
    if (per_rank < 0 || !(words_per_lane == 0 || words_per_lane == 1 || words_per_lane == 2) ||
        !(schedule == 0 || schedule == 1))
        return AR_EINVAL;
    g_fused_per_rank_override = per_rank;
    g_fused_wpl_override = words_per_lane;
    g_fused_schedule = schedule;
    return AR_OK;
}

}  // extern "C"
