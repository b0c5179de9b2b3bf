// Test-only probe of the library's device random-number functions: the
// Philox4x32-10 block, the word layout of a draw, u24 and the Gumbel
// transform, exactly as the sampling kernels call them (same header). The GPU
// tests compare its outputs with the oracle's; nothing in the library uses it.
// Built by tests/device_probe_build.py into tests/_build/libss_device_probe.so.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../speculative_decoding_verification_pipeline_amd/csrc/ss_device.h"

namespace {

constexpr int kThreads = 256;

// in: [n][6] = counter words 0..3, key words 0..1; out: [n][4]
__global__ void k_philox(const uint32_t* in, uint32_t* out, int n) {
    const int i = (int)(blockIdx.x * kThreads + threadIdx.x);
    if (i >= n) return;
    const uint32_t* c = in + 6 * (size_t)i;
    const uint4 o = ss::philox4x32_10(make_uint4(c[0], c[1], c[2], c[3]), c[4], c[5]);
    uint32_t* r = out + 4 * (size_t)i;
    r[0] = o.x;
    r[1] = o.y;
    r[2] = o.z;
    r[3] = o.w;
}

// out[d] = the word of draw d at (seed, request, position, domain)
__global__ void k_words(uint64_t seed, uint32_t request, uint32_t position, uint32_t domain,
                        uint32_t* out, int n) {
    const int d = (int)(blockIdx.x * kThreads + threadIdx.x);
    if (d >= n) return;
    out[d] = ss::philox_word(seed, request, position, (uint32_t)d, domain);
}

__global__ void k_transforms(const uint32_t* w, float* u, float* g, int n) {
    const int i = (int)(blockIdx.x * kThreads + threadIdx.x);
    if (i >= n) return;
    u[i] = ss::u24(w[i]);
    g[i] = ss::gumbel32(w[i]);
}

int blocks(int n) { return (n + kThreads - 1) / kThreads; }

}  // namespace

extern "C" {

// All pointers are device pointers; n >= 0. Returns the hipError_t of the launch.
int ss_probe_philox(const uint32_t* in, uint32_t* out, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_philox, dim3(blocks(n)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), in, out, n);
    return (int)hipGetLastError();
}

int ss_probe_words(uint64_t seed, uint32_t request, uint32_t position, uint32_t domain,
                   uint32_t* out, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_words, dim3(blocks(n)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), seed, request, position, domain, out, n);
    return (int)hipGetLastError();
}

int ss_probe_transforms(const uint32_t* w, float* u, float* g, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_transforms, dim3(blocks(n)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), w, u, g, n);
    return (int)hipGetLastError();
}

}  // extern "C"
