/*
 * ar.h -- C ABI of libar.so: one rank's share of a small-message bf16
 * allreduce with fp32 accumulation, on AMD Instinct MI355X (gfx950).
 *
 * All P "peer" buffers live in the calling GPU's own HBM: the library runs the
 * share of one rank, or of several emulated ranks, on a single device.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Element type: bf16, passed as raw 16-bit patterns.  Element pointers must
 *    be 2-byte aligned; any further misalignment is allowed and takes a
 *    slower path (16-byte vectors are used where every pointer of a call
 *    shares one alignment, scalar accesses for the rest).
 *  - Arithmetic: element i of the result is the binary32 sum
 *    ((x_0[i] + x_1[i]) + x_2[i]) + ... + x_{P-1}[i], in rank order, each
 *    bf16 widened exactly, IEEE round-to-nearest-even adds with subnormals
 *    kept, then rounded to bf16 with round-to-nearest-even.  Any NaN result
 *    is stored as the quiet NaN 0x7FC0.  Results are bit-exact and identical
 *    for every output and every rank.
 *  - Pointers: device pointers (hipMalloc or torch CUDA tensors).  Arrays of
 *    P peer buffers are passed BY VALUE in an ar_ptrs struct, which the
 *    library copies into the kernel's arguments: no device-side pointer table
 *    and no extra launch to build one (Helion PR #245 "One shot all reduce
 *    Example", review thread on launching an extra kernel to turn a pointer
 *    array into a tensor versus passing pointers as kernel arguments).
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 *    stream).  Every call is asynchronous on that stream: the library never
 *    allocates, never synchronises and keeps no pointer after it returns.
 *    The caller owns and allocates every buffer.
 *  - Errors: argument errors are detected on the host before anything is
 *    launched and returned as a negative AR_E* code; a failed launch returns
 *    AR_ELAUNCH.  Errors found while the kernel runs (a bounded wait that ran
 *    out) are reported through the device control block (ar_ctrl).
 *  - n == 0 is a successful no-op.
 */
#ifndef AR_H
#define AR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_P 8

/* P device pointers (entries >= P are ignored), passed by value. */
typedef struct ar_ptrs {
    void *p[AR_MAX_P];
} ar_ptrs;

enum ar_status {
    AR_OK = 0,
    AR_EINVAL = -1,    /* bad argument: P, n, rank, flag, null or misaligned pointer */
    AR_EALIAS = -2,    /* buffers overlap where the call forbids it */
    AR_ELAUNCH = -3,   /* the HIP launch (or a device query it needs) failed */
    AR_ETIMEDOUT = -4, /* device side: a bounded wait for a packet ran out */
    AR_ENOSPACE = -5   /* the call needs more than the library's static scratch */
};

/*
 * Device control block of the packet kernels: 64 bytes of device memory the
 * caller allocates and zeroes once.
 *   status    AR_OK until a kernel's bounded wait runs out; the first waiter to
 *             time out stores AR_ETIMEDOUT and every waiter that polls the
 *             block afterwards stops waiting.  The library never clears it:
 *             the caller reads it back (after synchronising) and re-zeroes it.
 *   epoch     the flag of the last completed ar_packet_fused_epoch call on
 *             this block (the next call uses epoch + 1).
 *   arrivals  workgroups of the running ar_packet_fused_epoch launch that
 *             have finished; back to 0 when the launch completes.
 */
#define AR_CTRL_BYTES 64
typedef struct ar_ctrl {
    int32_t status;
    uint32_t epoch;
    uint32_t arrivals;
    uint32_t reserved[13];
} ar_ctrl;

/* Default bound on the polls of one packet word (0 passed as max_spins). */
#define AR_DEFAULT_MAX_SPINS (1ull << 22)

/* ---------------------------------------------------------------------------
 * ar_oneshot_sum -- one-shot allreduce share: out[i] = sum_r in.p[r][i].
 *
 * Every rank is owed the whole buffer and keeps the whole result: the
 * allreduce case of the one-shot push-reduce kernel (torchcomms PR #3850
 * "Add HIP-graph capture coverage for the sharded-relay collectives", commit
 * summary D117629707, srcStride = 0 and ownOffset = 0); the same one-shot sum
 * as Helion PR #245 "One shot all reduce Example".
 *   in   P input buffers of n bf16 each (read only).
 *   out  one output buffer of n bf16.  It may be identical to one of the
 *        inputs (in place); any other overlap with an input is AR_EALIAS.
 *   P    2..8.
 * ------------------------------------------------------------------------- */
int ar_oneshot_sum(ar_ptrs in, void *out, int P, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * ar_oneshot_write_bcast -- write mode: the reduced vector is stored straight
 * into all P output buffers, whose pointers reach the kernel by value
 * (aiter PR #1910 "optimize allreduce write mode by broadcast output ptr",
 * Motivation: stage 2 writes directly into the other ranks' outputs; Technical
 * Details: the output pointers are broadcast on the host).
 *   in   P input buffers of n bf16.
 *   out  P output buffers of n bf16; all P receive identical data.  out.p[k]
 *        may equal in.p[k'] exactly (in place); partial overlaps between any
 *        two buffers are AR_EALIAS.
 * ------------------------------------------------------------------------- */
int ar_oneshot_write_bcast(ar_ptrs in, ar_ptrs out, int P, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * ar_twoshot_share -- rank `rank`'s two-shot share: reduce its slice over the
 * P inputs and write that slice into all P outputs (reduce-scatter stage, then
 * the write-mode broadcast of aiter PR #1910, Motivation).  Slices: L =
 * floor(n / (128 P)) * 128; rank r owns [r L, (r+1) L), the last rank owns
 * [(P-1) L, n), so every slice boundary is 128-element aligned and the last
 * slice absorbs the remainder (torchcomms PR #3850, commit summary
 * D117629683).  Outputs outside the slice are not touched.
 *   in, out, P as for ar_oneshot_write_bcast; rank in [0, P).
 * ------------------------------------------------------------------------- */
int ar_twoshot_share(ar_ptrs in, ar_ptrs out, int P, int rank, int64_t n, void *stream);

/* ---------------------------------------------------------------------------
 * ar_reduce_scatter_share -- one-shot reduce-scatter share of `rank`: each
 * input holds P blocks of `recvcount` elements and the rank keeps the sum of
 * its own block, out[i] = sum_p in.p[p][rank * recvcount + i].  The same
 * push-reduce kernel serves reduce-scatter with a per-peer source stride of
 * recvcount and an owner offset of rank * recvcount, allreduce with both 0
 * (torchcomms PR #3850, commit summary D117629707).
 *   in    P inputs of P * recvcount bf16.
 *   out   recvcount bf16; may be exactly the rank's own block of an input
 *         (in place); any other overlap with an input block read is AR_EALIAS.
 *   rank  in [0, P).
 * ------------------------------------------------------------------------- */
int ar_reduce_scatter_share(ar_ptrs in, void *out, int P, int rank, int64_t recvcount,
                            void *stream);

/* ---------------------------------------------------------------------------
 * LL packets.  Data and flag travel in one packet so that arrival is read off
 * the data itself (ARK PR #254 "Add monolithic fused packet allreduce kernel
 * and Model::all_reduce_packet API", description).  Layout of packet k
 * (16 bytes, 16-byte aligned, four little-endian u32 words):
 *     word 0 = elem[4k]   | elem[4k+1] << 16      (data0)
 *     word 1 = flag                               (flag0)
 *     word 2 = elem[4k+2] | elem[4k+3] << 16      (data1)
 *     word 3 = flag                               (flag1)
 * Elements past n are encoded as 0.  Each 8-byte half {data, flag} is written
 * with one 8-byte device-scope store (the store of an agent-scope atomic; the
 * standalone encode adds the streaming hint) and read as one agent-scope
 * atomic, so a reader that sees the expected flag in a half also sees that
 * half's data.  A packet counts as arrived only when
 * both flags equal the expected value; flags are never cleared, so a packet
 * left by an earlier call (older flag) reads as not yet arrived (torchcomms
 * PR #3850, commit summary D117629704: flags never cleared, stale flags
 * compare as not arrived).
 * ------------------------------------------------------------------------- */

/* Number of packets for n elements: ceil(n / 4). */
int64_t ar_ll_packets(int64_t n);

/* Encode n bf16 from `src` into ceil(n/4) packets at `dst_pkts` (16-byte
 * aligned) with flag `flag` (!= 0).  src and dst must not overlap. */
int ar_ll_encode(const void *src, void *dst_pkts, int64_t n, uint32_t flag, void *stream);

/* Wait until every packet at `src_pkts` carries `flag` in both flag words,
 * then decode n bf16 into `dst`.  Each packet word is polled at most
 * `max_spins` times (0 = AR_DEFAULT_MAX_SPINS); on timeout AR_ETIMEDOUT is
 * stored in ctrl->status and dst is undefined.  `ctrl` may be NULL: the waits
 * stay bounded, but a timeout is then not reported (dst is undefined). */
int ar_ll_decode(const void *src_pkts, void *dst, int64_t n, uint32_t flag, void *ctrl,
                 uint64_t max_spins, void *stream);

/* ---------------------------------------------------------------------------
 * ar_packet_fused -- fused LL-packet allreduce for emulated ranks
 * [rank_lo, rank_hi) of P, in ONE launch: scatter, reduce and broadcast are
 * fused into one kernel and synchronised only by the flags inside the packets,
 * not by barriers between workgroups (ARK PR #254, description; a rotating
 * per-call flag, which that page lists as deferred under Known limitations).
 *
 * Each rank j owns the two-shot slice j (same rule as ar_twoshot_share) and a
 * scratch buffer scratch.p[j] of ar_packet_scratch_bytes(P, n) bytes laid out
 * as [inbox: P slots][resbox: P slots], each slot S = ar_packet_slot_packets
 * (P, n) packets (sized for the largest, i.e. last, slice).  Rank r:
 *   scatter    encodes in.p[r][slice j] into inbox_j[slot r], for every j;
 *   reduce     polls inbox_r[slot 0..P-1], decodes, sums in rank order;
 *   broadcast  encodes the reduced slice into resbox_j[slot r], for every j;
 *   receive    polls resbox_r[slot 0..P-1] and decodes into out.p[r].
 * Packets past a slice's length are never written.
 *   in       P inputs of n bf16 (all P are read by the ranks in the range).
 *   scratch  P scratch buffers, 16-byte aligned; zero them once before the
 *            first call; the library never clears them.
 *   out      P outputs of n bf16; out.p[r] is written for r in the range.
 *   flag     != 0, strictly increasing from call to call on one scratch set
 *            (call c uses flag c + 1).  Wrap-around is not supported.
 *   ctrl     control block (AR_CTRL_BYTES), required.
 * A range covering fewer than all P ranks completes once the packets of the
 * other ranks for this flag are in place: staged before (e.g. with
 * ar_ll_encode or an earlier launch on the same stream) or written by a launch
 * that runs at the same time.  HIP does not promise that launches on two
 * streams of one process run at the same time (streams share a few hardware
 * queues), so a launch that waits on one queued after it may end in
 * AR_ETIMEDOUT instead; it never hangs.  Inputs,
 * outputs and scratch buffers must not overlap each other (AR_EALIAS).  Two
 * calls in flight on one scratch set are not allowed.
 * ------------------------------------------------------------------------- */
int ar_packet_fused(ar_ptrs in, ar_ptrs scratch, ar_ptrs out, int P, int rank_lo, int rank_hi,
                    int64_t n, uint32_t flag, void *ctrl, uint64_t max_spins, void *stream);

/* ---------------------------------------------------------------------------
 * ar_packet_fused_epoch -- ar_packet_fused whose flag lives in the control
 * block instead of the argument list: the call uses flag = ctrl->epoch + 1,
 * read on the device, and its last workgroup stores that flag back as the new
 * epoch.  A launch captured into a HIP graph therefore rotates its flag on
 * every replay, where a by-value flag would be baked in at capture and every
 * stale packet would already match it (torchcomms PR #3850, PR summary,
 * hazard G2).  Same buffers and rules as ar_packet_fused; the first call on a
 * zeroed control block uses flag 1.  A rank range split over several launches
 * gives each launch its own control block: their epochs advance together as
 * long as every launch takes part in every call.
 * ------------------------------------------------------------------------- */
int ar_packet_fused_epoch(ar_ptrs in, ar_ptrs scratch, ar_ptrs out, int P, int rank_lo,
                          int rank_hi, int64_t n, void *ctrl, uint64_t max_spins, void *stream);

/* ---------------------------------------------------------------------------
 * ar_packet_fused_noalloc -- ar_packet_fused_epoch for all P ranks, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the control block
 * and the P scratch buffers live in one static device array of the library,
 * AR_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call
 * allocates nothing; the caller passes only inputs, outputs and an optional
 * status word.
 *   in, out   P inputs / P outputs of n bf16, as for ar_packet_fused (no
 *             overlaps: AR_EALIAS).  Every rank 0..P-1 runs in the launch.
 *   d_status  NULL, or a 4-byte aligned device int32 that receives AR_OK or
 *             AR_ETIMEDOUT when the call completes (written on the stream).
 *   max_spins as for ar_packet_fused.
 * Size limit: 256 + P * round_up(ar_packet_scratch_bytes(P, n), 256) must not
 * exceed AR_NOALLOC_SCRATCH_BYTES, otherwise AR_ENOSPACE is returned before
 * anything touches the GPU (at P = 8: n up to 1,047,676 elements).
 * The array starts zeroed; the flag of a call is the array's epoch + 1, so it
 * rises with every call on the GPU whatever P and n are, and a packet left by
 * an earlier call never matches.  Each call leaves the array's status word
 * cleared for the next one.  All calls on one GPU share its array: two calls
 * in flight at once on one GPU (two streams, two host threads) race and give
 * undefined results; calls ordered on one stream are safe.  The first call on
 * a device looks up the array's address there (hipGetSymbolAddress) and
 * returns AR_ELAUNCH if that fails.  Wrap-around after 2^32 - 1 calls is not
 * supported.
 * ------------------------------------------------------------------------- */
#define AR_NOALLOC_SCRATCH_BYTES (64ll << 20)
int ar_packet_fused_noalloc(ar_ptrs in, ar_ptrs out, int P, int64_t n, int32_t *d_status,
                            uint64_t max_spins, void *stream);

/* ---------------------------------------------------------------------------
 * The three-operation packet decomposition that the fused kernel replaces
 * (ARK PR #254, description: send_packet -> recv_reduce_send_packet ->
 * recv_packet, one launch per phase).  Same scratch layout, flags and results
 * as ar_packet_fused; for ranks [rank_lo, rank_hi):
 *   ar_packet_send              scatter: in.p[r][slice j] -> inbox_j[slot r]
 *   ar_packet_recv_reduce_send  wait for inbox_r[slot 0..P-1], sum in rank
 *                               order, broadcast into resbox_j[slot r]
 *   ar_packet_recv              wait for resbox_r[slot 0..P-1], decode into
 *                               out.p[r]
 * Launched in this order on one stream they reproduce ar_packet_fused bit for
 * bit.  Waits are bounded and report through ctrl like the fused kernel.
 * ------------------------------------------------------------------------- */
int ar_packet_send(ar_ptrs in, ar_ptrs scratch, int P, int rank_lo, int rank_hi, int64_t n,
                   uint32_t flag, void *stream);
int ar_packet_recv_reduce_send(ar_ptrs scratch, int P, int rank_lo, int rank_hi, int64_t n,
                               uint32_t flag, void *ctrl, uint64_t max_spins, void *stream);
int ar_packet_recv(ar_ptrs scratch, ar_ptrs out, int P, int rank_lo, int rank_hi, int64_t n,
                   uint32_t flag, void *ctrl, uint64_t max_spins, void *stream);

/* ---------------------------------------------------------------------------
 * Host-only helpers: no GPU needed, no HIP call made.
 * ------------------------------------------------------------------------- */

/* Slice [*begin, *end) of `rank` under the two-shot rule above. */
int ar_slice_range(int P, int rank, int64_t n, int64_t *begin, int64_t *end);

/* Packets per scratch slot (ceil of the last slice's length / 4), or < 0. */
int64_t ar_packet_slot_packets(int P, int64_t n);

/* Bytes of one rank's scratch buffer: 2 * P * slot_packets * 16, or < 0. */
int64_t ar_packet_scratch_bytes(int P, int64_t n);

/* Static, human-readable name of a status code. */
const char *ar_strerror(int code);

/* ---------------------------------------------------------------------------
 * Measurement helper: launch an empty kernel on `stream`.  Gives the dispatch
 * floor that latency-bound calls are compared against.
 * ------------------------------------------------------------------------- */
int ar_noop(void *stream);

/* Measurement helper: the traffic of a write-mode call without the reduction,
 * to measure what the device delivers for the same bytes at the same size.
 * kind 0 reads all 2P buffers (in.p[0..P-1] and out.p[0..P-1]), kind 1 writes
 * all 2P of them (contents become meaningless), kind 2 copies in.p[p] into
 * out.p[p].  The accesses are those of the reduce kernels: 16-byte loads,
 * 16-byte stores with the same cache policy, `unroll` vectors in flight per
 * lane (1 or 2 for kind 0; 1, 2 or 4 otherwise), `threads` in {64, 128, 256}
 * lanes per workgroup, `blocks` workgroups at most (0: one pass, one vector
 * per lane per unroll step), and either cache policy the reduce kernels use
 * (`policy` 0: plain loads, device-scope write-through streaming stores;
 * 1: non-temporal loads and stores).  P is 4 or 8; n elements per buffer, a
 * multiple of 8, at most 2^29; every buffer 16-byte aligned and none
 * overlapping. */
int ar_probe_traffic(int kind, ar_ptrs in, ar_ptrs out, int P, int64_t n, int threads, int unroll,
                     int blocks, int policy, void *stream);

/* Benchmark-only launch-shape overrides (process-global, not thread-safe).
 * ar_set_reduce_tuning: unroll (vectors in flight per lane) in {0 = automatic,
 * 1, 2, 4} (1 to 8 with schedule 16; above 6 taken as 6 for P >= 7), workgroup
 * size in {0 = automatic, 64, 128, 256}, a cap on
 * workgroups (0 = automatic; batches only) and the schedule (0 = automatic,
 * 1 = grid-stride batches: load U vectors, then store them; 2, 4 or 8 =
 * pipelined in that many stages of U vectors per lane, the next stage's loads
 * issued before the current stores, unroll 1 or 2; 16 = one pass in which
 * global wave g takes the U x 64 consecutive vectors from g x U x 64, all its
 * loads issued before any reduction and every reduction before any store) for
 * ar_oneshot_sum, ar_oneshot_write_bcast, ar_twoshot_share and
 * ar_reduce_scatter_share.  ar_set_packet_tuning: workgroups per emulated rank
 * of ar_packet_fused (0 = automatic; never more than fit on the device at once)
 * words per lane per chunk in {0 = automatic, 1, 2}, and the schedule of
 * ar_packet_fused: 0 = every workgroup runs all phases of its chunks as a
 * pipeline, 1 = separate scatter, reduce-broadcast and receive workgroups in
 * one grid.  Results do not depend on any of them. */
int ar_set_reduce_tuning(int unroll, int threads, int max_blocks, int schedule);
int ar_set_packet_tuning(int per_rank, int words_per_lane, int schedule);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
