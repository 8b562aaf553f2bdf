// host.h -- host-side helpers of libar.so: argument checks, buffer-overlap
// checks, per-device properties and a launch wrapper that reports errors as
// return codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ar.h"

namespace ar {

constexpr int kThreads = 256;  // four 64-lane wavefronts per workgroup
constexpr int kMaxDevices = 64;  // per-device host caches hold this many GPUs

inline bool valid_P(int P) { return P >= 2 && P <= AR_MAX_P; }

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

inline bool aligned_to(const void *p, uintptr_t a) { return (addr(p) & (a - 1)) == 0; }

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// A byte range [lo, lo + bytes) of one buffer argument.
struct Span {
    uintptr_t lo;
    uintptr_t bytes;
};

inline Span span_of(const void *p, int64_t elem_begin, int64_t elems, int64_t elem_bytes) {
    return Span{addr(p) + (uintptr_t)(elem_begin * elem_bytes), (uintptr_t)(elems * elem_bytes)};
}

// True when two non-empty spans share a byte.
inline bool overlap(Span a, Span b) {
    return a.bytes != 0 && b.bytes != 0 && a.lo < b.lo + b.bytes && b.lo < a.lo + a.bytes;
}

// True when two spans overlap without being the very same range.
inline bool partial_overlap(Span a, Span b) {
    return overlap(a, b) && !(a.lo == b.lo && a.bytes == b.bytes);
}

// Properties of the current device, queried once per device.
struct DeviceInfo {
    int device;
    int cus;  // compute units (256 on MI355X)
};

// Fills `out` for the current device; AR_OK or AR_ELAUNCH.
int current_device(DeviceInfo *out);

// Workgroups of `fn` (kThreads threads, no dynamic LDS) that fit on one CU at
// once, cached per device and kernel.  0 on error.
int blocks_per_cu(const DeviceInfo &dev, const void *fn);

// hipLaunchKernel of a kernel taking one by-value struct argument.
template <typename Args>
int launch(const void *fn, unsigned grid, unsigned block, const Args &a, void *stream) {
    void *args[] = {const_cast<Args *>(&a)};
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? AR_OK : AR_ELAUNCH;
}

// Two-shot slice rule (see ar_slice_range).
inline int64_t slice_len_unit(int P, int64_t n) { return (n / (128 * (int64_t)P)) * 128; }

}  // namespace ar
