// device.h -- gfx950 device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Cache policy bits of buffer loads and stores (gfx950): 0 = default
// (cached), 2 = nt (streaming: the lines are not kept for reuse).
constexpr int kCached = 0;
constexpr int kStream = 2;

// Raw buffer resource over `bytes` bytes at `base`, a GLOBAL memory address
// (a buffer access addresses global memory, so a pointer into LDS must never
// be passed here).  Accesses at or past `bytes` read zero and drop stores,
// so each row gets its own resource and an access can never leave its row.
// Word 3 selects 32-bit raw data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2 (lo in bits 0..15), round to nearest even.
// gfx950 converts with v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Four fp32 -> four OCP E4M3 codes packed little-endian in one dword, round
// to nearest even.  gfx950's v_cvt_pk_fp8_f32 produces the OCP encoding.
// Callers keep |v| <= 448 * (1 + 2^-22), which rounds to at most 448.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// 2^n for n in the normal exponent range [-126, 127], from its bit pattern.
__device__ __forceinline__ float pow2_normal(int n) { return __uint_as_float((uint32_t)(n + 127) << 23); }

// exp(x), fp32, by Cody & Waite additive range reduction and a degree-7
// Taylor polynomial in Horner form with fused multiply-add.  Constants:
// L2E = fp32(log2 e); C1 = fp32(ln 2) with its low 12 significand bits
// cleared (n * C1 exact); C2 = fp32(ln 2 - C1); P_i = fp32(1 / i!).
// Range: +inf from 88.72283935546875 (the first fp32 value whose exponential
// exceeds FLT_MAX); 0 below -87.33654022216797 (the first fp32 value whose
// exponential is a normal number), so results are never subnormal.  In
// between n = rint(x * L2E) lies in [-126, 128], and 2^n is applied as two
// normal factors 2^n1 * 2^n2 (n1 = floor(n / 2)), so n = 128 needs no
// special case; every step is one correctly rounded operation.
__device__ __forceinline__ float cw_expf(float x) {
    constexpr float kLastFinite = 0x1.62e42ep+6f;  // largest fp32 with a finite exponential
    constexpr float kFirstNormal = -0x1.5d589ep+6f;  // smallest fp32 with a normal exponential
    // branch-free: the polynomial path runs on x clamped to the finite,
    // normal range (where it equals x) and the out-of-range results are
    // selected afterwards
    const float xc = __builtin_fminf(__builtin_fmaxf(x, kFirstNormal), kLastFinite);
    const float L2E = 0x1.715476p+0f;
    const float C1 = 0x1.62ep-1f;
    const float C2 = 0x1.0bfbe8p-15f;
    float n = __builtin_rintf(xc * L2E);
    float r = __builtin_fmaf(-n, C1, xc);
    r = __builtin_fmaf(-n, C2, r);
    float p = 0x1.a01a02p-13f;                 // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);  // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);   // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);   // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);   // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);             // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);             // 1/0!
    const int n1 = (int)__builtin_floorf(n * 0.5f);
    const int n2 = (int)n - n1;
    float y = (p * pow2_normal(n1)) * pow2_normal(n2);
    y = x > kLastFinite ? __builtin_huge_valf() : y;
    y = x < kFirstNormal ? 0.0f : y;
    return __builtin_isnan(x) ? x : y;
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + cw_expf(-x)); }

// sigmoid(x) for |x| <= kSigmoidFastBound, bit-identical there to sigmoid()
// in 17 instead of ~40 instructions.  Inside that range cw_expf's clamps and
// special cases never apply; 2^n is applied with one ldexp, which is exact
// because the result is a normal number (so it equals the two exact factor
// multiplications); and 1 / y, y = 1 + exp(-x) in [1, 2^116), is v_rcp_f32
// refined by one Newton step with fma.  That step gives the correctly rounded
// quotient for every such y: checked on gfx950 against the IEEE division for
// all 2,235,564,034 fp32 values with |x| <= 80.
constexpr float kSigmoidFastBound = 80.0f;

__device__ __forceinline__ float sigmoid_inrange(float x) {
    const float L2E = 0x1.715476p+0f;
    const float C1 = 0x1.62ep-1f;
    const float C2 = 0x1.0bfbe8p-15f;
    const float z = -x;
    const float n = __builtin_rintf(z * L2E);
    float r = __builtin_fmaf(-n, C1, z);
    r = __builtin_fmaf(-n, C2, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float y = 1.0f + __builtin_ldexpf(p, (int)n);
    const float q = __builtin_amdgcn_rcpf(y);
    return __builtin_fmaf(__builtin_fmaf(-y, q, 1.0f), q, q);
}

// In place: sigmoid of the N values one lane holds.  The short form runs
// when every value of every active lane lies within kSigmoidFastBound (a
// wave-uniform test, so only waves holding a value beyond it, or a NaN, take
// the general form).
template <int N>
__device__ __forceinline__ void sigmoid_lane(float (&v)[N]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < N; ++i) ok = ok && __builtin_fabsf(v[i]) <= kSigmoidFastBound;
    if (__all(ok)) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = sigmoid_inrange(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = sigmoid(v[i]);
    }
}

// DPP lane permutations (gfx9 encodings).  Each pairs every lane with one
// partner inside an aligned group of 2, 4, 8 or 16 lanes; used for
// symmetric merges, where any pairing across the two halves of the group
// works once each half holds identical values.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

// Every lane's source lane is valid for these permutations, so the `old`
// operand and bound_ctrl never take effect; old = 0 with bound_ctrl lets the
// compiler fold the move into the consuming v_max/v_min (one DPP
// instruction per butterfly step instead of three).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// Partner value across aligned lane groups of size 2D (D = 1 .. 32, a
// compile-time constant): lane i reads a lane of the other half of its
// group.  D = 16 swaps the halves of each 32-lane half-wave (ds_swizzle,
// xor mask 16); D = 32 the two half-waves.
template <int D>
__device__ __forceinline__ uint32_t partner_u32(uint32_t v) {
    if constexpr (D == 1) return dpp_u32<kDppXor1>(v);
    else if constexpr (D == 2) return dpp_u32<kDppXor2>(v);
    else if constexpr (D == 4) return dpp_u32<kDppHalfMirror>(v);
    else if constexpr (D == 8) return dpp_u32<kDppMirror>(v);
    else if constexpr (D == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
    else return (uint32_t)__shfl_xor((int)v, 32, kWave);
}

// Largest 32-bit unsigned value across a fully active wavefront, as a
// wave-uniform value: row-wise butterfly with DPP, then two row broadcasts
// (row_bcast:15 folds rows 0 -> 1 and 2 -> 3, row_bcast:31 row 1 -> rows 2
// and 3; rows outside the row mask keep v), so lane 63 holds the maximum.
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Largest 64-bit value across the wavefront (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, d, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// Sum of v over the lanes of a fully active wavefront that share lane % tpr
// (tpr a power of two <= 64), in each of those lanes: DPP rotations by tpr,
// 2 tpr, ... within each 16-lane row, then gfx950's row swaps.
// v_permlane16_swap(v, v) returns rows (0, 0, 2, 2) and (1, 1, 3, 3) of v,
// v_permlane32_swap(v, v) rows (0, 1, 0, 1) and (2, 3, 2, 3) (checked on the
// device), so the sum of the two halves is the sum over row pairs.
constexpr int kDppRowRor1 = 0x121;
constexpr int kDppRowRor2 = 0x122;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
template <int TPR>
__device__ __forceinline__ uint32_t lane_residue_sum(uint32_t v) {
    if constexpr (TPR <= 1) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor1, 0xF, 0xF, true);
    if constexpr (TPR <= 2) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor2, 0xF, 0xF, true);
    if constexpr (TPR <= 4) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor4, 0xF, 0xF, true);
    if constexpr (TPR <= 8) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor8, 0xF, 0xF, true);
    if constexpr (TPR <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = r[0] + r[1];
    }
    if constexpr (TPR <= 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = r[0] + r[1];
    }
    return v;
}

// lane_residue_sum over the N words of a lane, with tpr (a power of two <=
// 64) chosen at run time once for all of them
template <int N>
__device__ __forceinline__ void lane_residue_sums(uint32_t (&v)[N], int tpr) {
    switch (tpr) {
        case 1:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<1>(v[i]);
            break;
        case 2:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<2>(v[i]);
            break;
        case 4:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<4>(v[i]);
            break;
        case 8:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<8>(v[i]);
            break;
        case 16:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<16>(v[i]);
            break;
        case 32:
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = lane_residue_sum<32>(v[i]);
            break;
        default:
            break;  // 64: one lane per residue
    }
}

// Inclusive prefix sum across a fully active wavefront, with DPP: shifts by
// 1, 2, 4 and 8 lanes within each 16-lane row (lanes shifted in from before
// the row read 0), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then row 1's into rows 2 and 3 (row_bcast:31).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, true);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
    return v;
}

}  // namespace ep
