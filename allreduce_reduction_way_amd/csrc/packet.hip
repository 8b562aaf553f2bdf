// packet.hip -- LL-packet codec and the fused packet allreduce share.
//
// Packets are 16 bytes {data0, flag, data1, flag}; each 8-byte half is one
// "word" {two bf16, flag} written and read as a single agent-scope atomic
// (see device.h), so a reader that sees the expected flag in a word also has
// that word's data.  Data and flag in one packet let the receiver detect
// arrival from the data itself (ARK PR #254 "Add monolithic fused packet
// allreduce kernel and Model::all_reduce_packet API", description).
//
// Work is laid out word-per-lane: lane t of a 256-lane workgroup handles
// words t and t + 256 of a 512-word chunk, so every 64-lane wavefront issues
// one 512-byte contiguous atomic access per instruction and one 256-byte
// contiguous element access.
//
// The fused kernel runs the P emulated ranks as groups of workgroups of one
// persistent grid: workgroup b serves rank lo + b % R and chunks b / R,
// b / R + B, ... (R ranks in the launch, B workgroups per rank).  Rank r on
// chunk c does, for each of its words:
//   scatter    x_r[slice j] -> inbox_j[slot r]           for j = 0..P-1
//   reduce     inbox_r[slot 0..P-1] -> rank-order sum     (waits on flags)
//   broadcast  sum -> resbox_j[slot r]                    for j = 0..P-1
//   receive    resbox_r[slot 0..P-1] -> out_r             (waits on flags)
// The only synchronisation between workgroups is the flag inside each word:
// lane t of rank r waits only on lane t of the other ranks' workgroups of the
// same chunk, and every lane writes all it produces before it waits
// (torchcomms PR #3850 "Add HIP-graph capture coverage for the sharded-relay
// collectives", commit summary D117629704: pairwise handshakes, no global
// barrier, write and flag before waiting).  The grid never exceeds the number
// of workgroups that fit on the device at once, so every workgroup a lane
// waits on is resident; all waits are bounded and report AR_ETIMEDOUT.
#include "device.h"
#include "host.h"

namespace ar {
namespace {

constexpr int kWordsPerLane = 2;
constexpr int64_t kChunkWords = (int64_t)kThreads * kWordsPerLane;  // 512 words = 1024 bf16

// Two bf16 starting at element e of a slice of `len` elements (e even, e < len
// or the word is padding), packed low element first; elements past the slice
// read as zero.
__device__ __forceinline__ uint32_t load_pair(const uint16_t *p, int64_t e, int64_t len,
                                              bool aligned4) {
    if (e + 1 < len) {
        if (aligned4) return *reinterpret_cast<const uint32_t *>(p + e);
        return (uint32_t)p[e] | ((uint32_t)p[e + 1] << 16);
    }
    return e < len ? (uint32_t)p[e] : 0u;
}

__device__ __forceinline__ void store_pair(uint16_t *p, int64_t e, int64_t len, bool aligned4,
                                           uint32_t d) {
    if (e + 1 < len) {
        if (aligned4) {
            *reinterpret_cast<uint32_t *>(p + e) = d;
        } else {
            p[e] = (uint16_t)d;
            p[e + 1] = (uint16_t)(d >> 16);
        }
    } else if (e < len) {
        p[e] = (uint16_t)d;
    }
}

// ---- standalone encode / decode ----------------------------------------------

struct CodecArgs {
    const uint16_t *elems;  // encode: source; decode: unused
    uint16_t *dst;          // decode: destination
    uint64_t *words;        // packet words (2 per packet)
    int64_t n;
    int64_t nwords;
    uint32_t flag;
    int aligned4;
    int32_t *status;
    uint64_t max_spins;
};

__global__ __launch_bounds__(kThreads) void k_ll_encode(CodecArgs a) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < a.nwords; w += stride)
        store_word(a.words + w, make_word(load_pair(a.elems, 2 * w, a.n, a.aligned4), a.flag));
}

__global__ __launch_bounds__(kThreads) void k_ll_decode(CodecArgs a) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < a.nwords; w += stride) {
        uint64_t v;
        if (!wait_word(a.words + w, a.flag, v, a.status, a.max_spins)) return;
        store_pair(a.dst, 2 * w, a.n, a.aligned4, word_data(v));
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
    int64_t chunks;   // chunks of kChunkWords words covering a slot
    int rank_lo;
    int nranks;       // R
    int per_rank;     // B
    uint32_t flag;
    int aligned4;
    int32_t *status;
    uint64_t max_spins;
};

template <int P>
__global__ __launch_bounds__(kThreads) void k_packet_fused(FusedArgs a) {
    const int r = a.rank_lo + (int)(blockIdx.x % (unsigned)a.nranks);
    const int64_t first_chunk = blockIdx.x / (unsigned)a.nranks;
    const uint16_t *x_r = static_cast<const uint16_t *>(a.in.p[r]);
    uint16_t *out_r = static_cast<uint16_t *>(a.out.p[r]);
    uint64_t *mine = static_cast<uint64_t *>(a.scratch.p[r]);
    const int64_t last_len = a.n - (int64_t)(P - 1) * a.L;

    for (int64_t c = first_chunk; c < a.chunks; c += a.per_rank) {
        const int64_t w0 = c * kChunkWords + threadIdx.x;

        // scatter: every load first, then every store
        uint32_t d[P][kWordsPerLane];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int64_t len = j == P - 1 ? last_len : a.L;
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) {
                const int64_t w = w0 + k * kThreads;
                d[j][k] = load_pair(x_r + j * a.L, 2 * w, len, a.aligned4);
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const int64_t len = j == P - 1 ? last_len : a.L;
            const int64_t words = 2 * ((len + 3) / 4);
            uint64_t *slot = static_cast<uint64_t *>(a.scratch.p[j]) + (int64_t)r * a.slot_words;
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) {
                const int64_t w = w0 + k * kThreads;
                if (w < words) store_word(slot + w, make_word(d[j][k], a.flag));
            }
        }

        // reduce + broadcast of slice r
        {
            const int64_t len = r == P - 1 ? last_len : a.L;
            const int64_t words = 2 * ((len + 3) / 4);
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) {
                const int64_t w = w0 + k * kThreads;
                if (w >= words) continue;
                uint64_t v[P];
#pragma unroll
                for (int s = 0; s < P; ++s) v[s] = load_word(mine + (int64_t)s * a.slot_words + w);
                uint32_t dw[P];
#pragma unroll
                for (int s = 0; s < P; ++s) {
                    if (word_flag(v[s]) != a.flag &&
                        !wait_word(mine + (int64_t)s * a.slot_words + w, a.flag, v[s], a.status,
                                   a.max_spins))
                        return;
                    dw[s] = word_data(v[s]);
                }
                const uint64_t res = make_word(reduce_word<P>(dw), a.flag);
#pragma unroll
                for (int j = 0; j < P; ++j)
                    store_word(static_cast<uint64_t *>(a.scratch.p[j]) +
                                   (int64_t)(P + r) * a.slot_words + w,
                               res);
            }
        }

        // receive: resbox_r[slot s] holds the reduced slice s
        uint64_t v[P][kWordsPerLane];
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int64_t len = s == P - 1 ? last_len : a.L;
            const int64_t words = 2 * ((len + 3) / 4);
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) {
                const int64_t w = w0 + k * kThreads;
                v[s][k] = w < words ? load_word(mine + (int64_t)(P + s) * a.slot_words + w)
                                    : make_word(0, a.flag);
            }
        }
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int64_t len = s == P - 1 ? last_len : a.L;
#pragma unroll
            for (int k = 0; k < kWordsPerLane; ++k) {
                const int64_t w = w0 + k * kThreads;
                if (2 * w >= len) continue;
                if (word_flag(v[s][k]) != a.flag &&
                    !wait_word(mine + (int64_t)(P + s) * a.slot_words + w, a.flag, v[s][k],
                               a.status, a.max_spins))
                    return;
                store_pair(out_r + s * a.L, 2 * w, len, a.aligned4, word_data(v[s][k]));
            }
        }
    }
}

typedef void (*FusedKernel)(FusedArgs);

FusedKernel pick_fused(int P) {
    switch (P) {
        case 2: return k_packet_fused<2>;
        case 3: return k_packet_fused<3>;
        case 4: return k_packet_fused<4>;
        case 5: return k_packet_fused<5>;
        case 6: return k_packet_fused<6>;
        case 7: return k_packet_fused<7>;
        default: return k_packet_fused<8>;
    }
}

// Launch-shape override for benchmark sweeps: workgroups per rank (0 = auto).
int g_fused_per_rank_override = 0;

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
    CodecArgs a = {};
    a.elems = static_cast<const uint16_t *>(src);
    a.words = static_cast<uint64_t *>(dst_pkts);
    a.n = n;
    a.nwords = 2 * ar_ll_packets(n);
    a.flag = flag;
    a.aligned4 = aligned_to(src, 4);
    int64_t blocks = (a.nwords + kThreads - 1) / kThreads;
    if (blocks > (int64_t)dev.cus * 8) blocks = (int64_t)dev.cus * 8;
    return launch(reinterpret_cast<const void *>(&k_ll_encode), (unsigned)blocks, kThreads, a,
                  stream);
}

int ar_ll_decode(const void *src_pkts, void *dst, int64_t n, uint32_t flag, void *ctrl,
                 uint64_t max_spins, void *stream) {
    if (n < 0 || flag == 0) return AR_EINVAL;
    if (n == 0) return AR_OK;
    if (!src_pkts || !dst || !ctrl || !aligned_to(dst, 2) || !aligned_to(src_pkts, 16) ||
        !aligned_to(ctrl, 4))
        return AR_EINVAL;
    const Span sd = span_of(dst, 0, n, 2), sp = span_of(src_pkts, 0, ar_ll_packets(n), 16),
               sc = span_of(ctrl, 0, AR_CTRL_BYTES, 1);
    if (overlap(sd, sp) || overlap(sd, sc) || overlap(sp, sc)) return AR_EALIAS;
    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    CodecArgs a = {};
    a.dst = static_cast<uint16_t *>(dst);
    a.words = static_cast<uint64_t *>(const_cast<void *>(src_pkts));
    a.n = n;
    a.nwords = 2 * ar_ll_packets(n);
    a.flag = flag;
    a.aligned4 = aligned_to(dst, 4);
    a.status = static_cast<int32_t *>(ctrl);
    a.max_spins = max_spins ? max_spins : AR_DEFAULT_MAX_SPINS;
    // A modest grid: decode may wait on a producer that needs CUs of its own.
    int64_t blocks = (a.nwords + kThreads - 1) / kThreads;
    if (blocks > (int64_t)dev.cus * 2) blocks = (int64_t)dev.cus * 2;
    return launch(reinterpret_cast<const void *>(&k_ll_decode), (unsigned)blocks, kThreads, a,
                  stream);
}

int ar_packet_fused(ar_ptrs in, ar_ptrs scratch, ar_ptrs out, int P, int rank_lo, int rank_hi,
                    int64_t n, uint32_t flag, void *ctrl, uint64_t max_spins, void *stream) {
    if (!valid_P(P) || n < 0 || flag == 0 || rank_lo < 0 || rank_hi > P || rank_lo >= rank_hi)
        return AR_EINVAL;
    if (!ctrl || !aligned_to(ctrl, 4)) return AR_EINVAL;
    for (int p = 0; p < P; ++p) {
        if (!in.p[p] || !out.p[p] || !scratch.p[p]) return AR_EINVAL;
        if (!aligned_to(in.p[p], 2) || !aligned_to(out.p[p], 2) || !aligned_to(scratch.p[p], 16))
            return AR_EINVAL;
    }
    if (n == 0) return AR_OK;
    const int64_t sbytes = ar_packet_scratch_bytes(P, n);
    // No two distinct buffers may share a byte (identical input pointers are
    // fine: inputs are only read).
    Span spans[3 * AR_MAX_P];
    int kind[3 * AR_MAX_P];
    int ns = 0;
    for (int p = 0; p < P; ++p) {
        spans[ns] = span_of(in.p[p], 0, n, 2);
        kind[ns++] = 0;
        spans[ns] = span_of(out.p[p], 0, n, 2);
        kind[ns++] = 1;
        spans[ns] = span_of(scratch.p[p], 0, sbytes, 1);
        kind[ns++] = 2;
    }
    for (int i = 0; i < ns; ++i)
        for (int k = i + 1; k < ns; ++k)
            if (overlap(spans[i], spans[k]) && !(kind[i] == 0 && kind[k] == 0))
                return AR_EALIAS;
    const Span sc = span_of(ctrl, 0, AR_CTRL_BYTES, 1);
    for (int i = 0; i < ns; ++i)
        if (overlap(spans[i], sc)) return AR_EALIAS;

    DeviceInfo dev;
    if (current_device(&dev) != AR_OK) return AR_ELAUNCH;
    FusedKernel fn = pick_fused(P);
    const int per_cu = blocks_per_cu(dev, reinterpret_cast<const void *>(fn));
    if (per_cu <= 0) return AR_ELAUNCH;

    FusedArgs a = {};
    a.in = in;
    a.scratch = scratch;
    a.out = out;
    a.n = n;
    a.L = slice_len_unit(P, n);
    a.slot_words = 2 * ar_packet_slot_packets(P, n);
    a.chunks = (a.slot_words + kChunkWords - 1) / kChunkWords;
    a.rank_lo = rank_lo;
    a.nranks = rank_hi - rank_lo;
    a.flag = flag;
    bool al4 = true;
    for (int p = 0; p < P; ++p) al4 = al4 && aligned_to(in.p[p], 4) && aligned_to(out.p[p], 4);
    a.aligned4 = al4;
    a.status = static_cast<int32_t *>(ctrl);
    a.max_spins = max_spins ? max_spins : AR_DEFAULT_MAX_SPINS;

    // Persistent grid no larger than what is resident at once: B workgroups per
    // rank, then B rebalanced so that every workgroup runs the same number of
    // chunks.
    const int64_t resident = (int64_t)per_cu * dev.cus;
    int64_t B = resident / a.nranks;
    if (g_fused_per_rank_override > 0 && g_fused_per_rank_override < B)
        B = g_fused_per_rank_override;
    if (B > a.chunks) B = a.chunks;
    if (B < 1) return AR_ELAUNCH;
    const int64_t rounds = (a.chunks + B - 1) / B;
    B = (a.chunks + rounds - 1) / rounds;
    a.per_rank = (int)B;
    return launch(reinterpret_cast<const void *>(fn), (unsigned)(B * a.nranks), kThreads, a,
                  stream);
}

// Benchmark-only override of the fused kernel's workgroups per rank (0 = auto;
// never above the resident limit).
int ar_set_packet_tuning(int per_rank) {
    if (per_rank < 0) return AR_EINVAL;
    g_fused_per_rank_override = per_rank;
    return AR_OK;
}

}  // extern "C"
