// device.h -- gfx950 device helpers shared by the reduce and packet kernels.
//
// bf16 <-> binary32, the rank-order reduction of 16-byte vectors, and the
// agent-scope 8-byte packet words.  Written for CDNA4: 64-lane wavefronts,
// 16-byte global loads/stores (global_load_dwordx4), one L2 per XCD.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

// 16-byte vector of eight bf16 (four u32 words, element 2k in the low half
// of word k).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> binary32 ----------------------------------------------------

// Low / high bf16 of a 32-bit word widened to binary32.  Exact: the bf16 bits
// are the upper 16 bits of the binary32 encoding.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bits (in the low 16 bits), round to nearest even.
// Adding 0x7FFF plus the lowest kept bit carries into the kept part exactly
// when the dropped half is above the midpoint, or at it with an odd kept
// part; a carry out of the mantissa gives the next binade (or Inf).  NaN is
// the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// Rank-order sum of one 32-bit word (two bf16) over P sources.
template <int P>
__device__ __forceinline__ uint32_t reduce_word(const uint32_t (&w)[P]) {
    float lo = lo_f32(w[0]);
    float hi = hi_f32(w[0]);
#pragma unroll
    for (int p = 1; p < P; ++p) {
        lo = lo + lo_f32(w[p]);
        hi = hi + hi_f32(w[p]);
    }
    return pack_bf16x2(lo, hi);
}

// Rank-order sum of eight bf16 (one 16-byte vector) over P sources.
template <int P>
__device__ __forceinline__ u32x4 reduce_vec(const u32x4 (&x)[P]) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t w[P];
#pragma unroll
        for (int p = 0; p < P; ++p) w[p] = x[p][k];
        r[k] = reduce_word<P>(w);
    }
    return r;
}

// Rank-order sum of one bf16 over P sources (scalar path).
template <int P>
__device__ __forceinline__ uint16_t reduce_elem(const uint16_t (&e)[P]) {
    float acc = __uint_as_float((uint32_t)e[0] << 16);
#pragma unroll
    for (int p = 1; p < P; ++p) acc = acc + __uint_as_float((uint32_t)e[p] << 16);
    return (uint16_t)bf16_rne(acc);
}

// ---- plain 16-byte vector I/O ---------------------------------------------

// NT: non-temporal (streaming) load.  It keeps the data out of the 256 MB
// MALL, which costs when the data would have stayed there: measured on
// MI355X with grid-stride batches, the 4 x 64 Mi-element two-shot (268 MB per
// launch) runs 178 us per four owners with it against 190 us without, while
// the 72 MB write-mode share back to back on one buffer set slows from 9.9 to
// 13.7 us.  The batch and pipelined kernels therefore take it only past
// 128 MiB per launch; the one-pass phased kernel, tuned for data coming from
// HBM, always does.
template <bool NT>
__device__ __forceinline__ u32x4 load_vec(const void *base, int64_t elem) {
    const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + elem);
    if (NT) return __builtin_nontemporal_load(p);
    return *p;
}

// Results are written once and never read back by the kernel.  WT = true
// stores them with cache policy SC1 | NT (operand 18: SC1 = 16, NT = 2):
// device scope, so each store writes through this XCD's L2 instead of
// waiting there for the end-of-kernel write-back, plus the streaming hint.
// Measured on MI355X against NT alone, for the grid-stride shapes: write-mode
// 440x5120 x 8 9.58 instead of 10.18 us back to back (MALL-resident) and
// 15.57 instead of 15.72 us from HBM; two-shot rank 3 of 680x5120 x 8 3.20
// instead of 3.35 us.  (SC1 without NT: 9.30 us warm but 17.4 us from HBM;
// no policy bits: 17.7 against 14.4 us from HBM.)  WT = false stores with NT
// alone: the one-pass kernels that issue all their loads before storing any
// run better without the write-through (12.0 against 12.2 us for the phased
// write-mode share from HBM).
//
// The store goes through a buffer resource so the policy can be chosen:
// `base` must be the same for every lane of the wavefront (a kernel argument)
// and `byte_off + 16`, the end of the lane's store, at most kStoreRangeBytes.
// The hardware drops (does not fault on) a buffer store past the resource's
// range, so every caller must keep its offsets inside it.
constexpr uint32_t kStoreRangeBytes = 0x7FFFFFFFu;
// An offset whose 16-byte store lies wholly past the range: the hardware
// drops it.  Used on purpose for lanes with nothing to store, so that the
// store instruction need not sit behind a branch.
constexpr uint32_t kDroppedStoreOffset = 0x80000000u;
static_assert(kDroppedStoreOffset >= kStoreRangeBytes, "a dropped store must be out of range");

template <bool WT = true>
__device__ __forceinline__ void store_vec(void *base, uint32_t byte_off, u32x4 v) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(base, (short)0, kStoreRangeBytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, WT ? 18 : 2);
}

// ---- packet words -----------------------------------------------------------
//
// A packet word is the 8-byte half {data: two bf16, flag: u32} of an LL
// packet, flag in the upper 32 bits (little-endian: bytes 4..7).  Writers
// and readers run on different XCDs, each with its own L2, so both sides use
// agent-scope relaxed atomics: the compiler emits global_store_dwordx2 /
// global_load_dwordx2 with the sc1 (device coherence) bit, which writes
// through to and reads from the device coherence point instead of a possibly
// stale per-XCD L2 line.  No fence is needed: data and flag of a word are
// one single-copy-atomic access, so seeing the flag means seeing the data.

__device__ __forceinline__ uint64_t make_word(uint32_t data, uint32_t flag) {
    return (uint64_t)data | ((uint64_t)flag << 32);
}

__device__ __forceinline__ void store_word(uint64_t *p, uint64_t w) {
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t load_word(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t word_flag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ uint32_t word_data(uint64_t w) { return (uint32_t)w; }

// Status word of the control block: agent-scope so every XCD sees it.  A
// null status (a decode called without a control block) reads as 0 and is
// never raised.
__device__ __forceinline__ int32_t load_status(const int32_t *s) {
    if (!s) return 0;
    return __hip_atomic_load(const_cast<int32_t *>(s), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void raise_status(int32_t *s, int32_t code) {
    if (!s) return;
    int32_t expected = 0;
    __hip_atomic_compare_exchange_strong(s, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one packet word until its flag equals `flag`.  Bounded: after
// `max_spins` polls (or once another waiter has raised the status) it gives
// up, raises AR_ETIMEDOUT (-4) in the status word and returns false.
__device__ __forceinline__ bool wait_word(const uint64_t *p, uint32_t flag, uint64_t &w,
                                          int32_t *status, uint64_t max_spins) {
    w = load_word(p);
    uint64_t spins = 0;
    while (word_flag(w) != flag) {
        ++spins;
        if ((spins & 63u) == 0 && load_status(status) != 0) return false;
        if (spins >= max_spins) {
            raise_status(status, -4);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
        w = load_word(p);
    }
    return true;
}

}  // namespace ar
