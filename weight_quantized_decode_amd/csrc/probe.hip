// Read-only stream probe (include/wqd_probe.h): the achievable HBM read rate for a plain stream of
// 16-byte nontemporal loads, as a ceiling for the decode kernels' rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/wqd_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRing = 8;  // wave loads in flight

__global__ __launch_bounds__(1024) void probe_read_kernel(const uint8_t *buf, int64_t chunks, uint32_t *sink) {
    // chunks: 1 KiB wave loads in the buffer; wave w of the grid reads [w*per, (w+1)*per)
    const int64_t waves = int64_t(gridDim.x) * 16;
    const int64_t w = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 6);
    const int64_t per = (chunks + waves - 1) / waves;
    const int64_t c0 = w * per, c1 = c0 + per < chunks ? c0 + per : chunks;
    const int lane = threadIdx.x & 63;
    uint32_t acc = 0;
    for (int64_t c = c0; c < c1; c += kRing) {
        u32x4 v[kRing];
#pragma unroll
        for (int i = 0; i < kRing; i++) {
            const int64_t cc = c + i < c1 ? c + i : c1 - 1;
            v[i] = __builtin_nontemporal_load((const u32x4 __attribute__((address_space(1))) *)(uintptr_t)(buf + cc * 1024 + lane * 16));
        }
#pragma unroll
        for (int i = 0; i < kRing; i++) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    sink[int64_t(blockIdx.x) * 1024 + threadIdx.x] = acc;
}

}  // namespace

extern "C" WQD_PROBE_API int wqd_probe_read(const void *buf, int64_t bytes, uint32_t *sink, int32_t workgroups,
                                            void *stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 16384 || (reinterpret_cast<uintptr_t>(buf) & 15) || workgroups < 0)
        return -1;
    int wg = workgroups;
    if (wg == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return -5;
        wg = cus;
    }
    hipLaunchKernelGGL(probe_read_kernel, dim3(unsigned(wg)), dim3(1024), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t *>(buf), bytes / 1024, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
