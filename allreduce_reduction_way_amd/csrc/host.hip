// host.hip -- host-only entry points of libar.so (no GPU needed) plus the
// per-device property cache and the empty-kernel launch.
#include <map>
#include <mutex>
#include <utility>

#include "host.h"

namespace ar {

namespace {

std::mutex g_mu;
int g_cus[kMaxDevices];  // 0 = not queried yet
std::map<std::pair<const void *, int>, int> g_occupancy;  // (kernel, device) -> blocks per CU

__global__ void k_noop() {}

}  // namespace

int current_device(DeviceInfo *out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return AR_ELAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_cus[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return AR_ELAUNCH;
        g_cus[dev] = cus;
    }
    out->device = dev;
    out->cus = g_cus[dev];
    return AR_OK;
}

int blocks_per_cu(const DeviceInfo &dev, const void *fn) {
    const std::pair<const void *, int> key(fn, dev.device);
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_occupancy.find(key);
    if (it != g_occupancy.end()) return it->second;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, 0) != hipSuccess) nb = 0;
    if (nb > 0) g_occupancy.emplace(key, nb);
    return nb;
}

}  // namespace ar

using namespace ar;

extern "C" {

int ar_slice_range(int P, int rank, int64_t n, int64_t *begin, int64_t *end) {
    if (!valid_P(P) || rank < 0 || rank >= P || n < 0 || !begin || !end) return AR_EINVAL;
    const int64_t L = slice_len_unit(P, n);
    *begin = (int64_t)rank * L;
    *end = rank == P - 1 ? n : (int64_t)(rank + 1) * L;
    return AR_OK;
}

int64_t ar_ll_packets(int64_t n) { return n <= 0 ? 0 : (n + 3) / 4; }

int64_t ar_packet_slot_packets(int P, int64_t n) {
    if (!valid_P(P) || n < 0) return AR_EINVAL;
    return ar_ll_packets(n - (int64_t)(P - 1) * slice_len_unit(P, n));
}

int64_t ar_packet_scratch_bytes(int P, int64_t n) {
    const int64_t S = ar_packet_slot_packets(P, n);
    return S < 0 ? S : 2 * (int64_t)P * S * 16;
}

const char *ar_strerror(int code) {
    switch (code) {
        case AR_OK: return "AR_OK: success";
        case AR_EINVAL: return "AR_EINVAL: invalid argument";
        case AR_EALIAS: return "AR_EALIAS: buffers overlap";
        case AR_ELAUNCH: return "AR_ELAUNCH: kernel launch or device query failed";
        case AR_ETIMEDOUT: return "AR_ETIMEDOUT: a bounded packet wait ran out";
        case AR_ENOSPACE: return "AR_ENOSPACE: the call needs more than the static scratch";
        default: return "unknown ar status code";
    }
}

int ar_noop(void *stream) {
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&k_noop), dim3(1), dim3(64),
                                   nullptr, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? AR_OK : AR_ELAUNCH;
}

}  // extern "C"
