// selfcheck.hip -- device self-checks for the test suite (libepcheck.so, not
// part of the library's ABI).
//
// ep_check_sigmoid_inrange: runs every fp32 bit pattern with |x| <= bound
// through the short sigmoid form (sigmoid_inrange) and the general one
// (sigmoid: cw_expf and the IEEE division) on the device and counts the
// inputs whose bits differ.  The general form is the one the oracle's
// definition is compared with elsewhere; this shows the short form equal to
// it on its whole domain, not only on sampled inputs.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "device.h"

namespace {

using namespace ep;

__global__ __launch_bounds__(256) void sigmoid_check_kernel(uint32_t lo, uint32_t count, float bound,
                                                            unsigned long long* __restrict__ out) {
    unsigned long long bad = 0, tested = 0;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < count; i += gridDim.x * blockDim.x) {
        const float x = __uint_as_float(lo + i);
        if (!(__builtin_fabsf(x) <= bound)) continue;
        ++tested;
        bad += __float_as_uint(sigmoid_inrange(x)) != __float_as_uint(sigmoid(x)) ? 1 : 0;
    }
    atomicAdd(&out[0], tested);
    atomicAdd(&out[1], bad);
}

}  // namespace

extern "C" {

// counts[0] = inputs tested, counts[1] = inputs whose bits differ (device
// memory, two zeroed words; the sweep is enqueued on `stream`).  bound must
// not exceed kSigmoidFastBound.
__attribute__((visibility("default"))) int ep_check_sigmoid_inrange(float bound, unsigned long long* counts,
                                                                      void* stream) {
    if (!counts || !(bound >= 0.0f) || bound > kSigmoidFastBound) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (uint64_t lo = 0; lo < (1ull << 32); lo += (1ull << 28))
        hipLaunchKernelGGL(sigmoid_check_kernel, dim3(65536), dim3(256), 0, st, (uint32_t)lo, (uint32_t)(1u << 28),
                           bound, counts);
    return (int)hipGetLastError();
}

}  // extern "C"
