// launch.h -- host-side launchers of the library's kernels (internal).
//
// Each launcher assumes its arguments were validated by the C ABI layer
// (api.hip): sizes within the documented limits, pointers non-null and
// aligned.  They enqueue on `stream` and return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

struct Shape {
    int T, H, E, G, TG, k, R, m;
};

hipError_t launch_route(const Shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                        hipStream_t stream);

size_t layout_workspace_bytes(const Shape& s);
hipError_t launch_layout(const Shape& s, const int32_t* topk_idx, int32_t* cnt, int32_t* ntok_rank,
                         int32_t* off, int32_t* slot, int32_t* recv_token, void* ws,
                         hipStream_t stream);

hipError_t launch_dispatch_fp8(const Shape& s, const uint16_t* x, const int32_t* slot, uint8_t* recv,
                               float* recv_scales, hipStream_t stream);
hipError_t launch_dispatch_bf16(const Shape& s, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                                hipStream_t stream);

hipError_t launch_combine(const Shape& s, const uint16_t* y, const int32_t* slot, const float* w,
                          uint16_t* out, hipStream_t stream);

// Workgroup geometry of the row kernels (dispatch, combine): a token's row is
// cut into `chunks` lane-sized pieces; a workgroup of `threads` lanes covers
// `threads` consecutive pieces of one token, and `segs` workgroups cover a
// row.  Large batches use one workgroup per row so that all stores of a row
// leave from one XCD's L2; small batches use one-wave workgroups so that the
// rows spread over every CU.
struct RowGeometry {
    int threads;
    int segs;
};

inline RowGeometry row_geometry(int T, int chunks) {
    const int waves_per_row = (chunks + 63) / 64;
    RowGeometry g;
    if ((long)T * 1 >= 2048 && waves_per_row <= 16) {
        g.threads = waves_per_row * 64;
    } else {
        g.threads = 64;
    }
    g.segs = (chunks + g.threads - 1) / g.threads;
    return g;
}

}  // namespace ep
