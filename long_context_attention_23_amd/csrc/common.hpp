// common.hpp -- device helpers shared by the CSA / HCA kernels (gfx950, wave64).
//
// Number formats are handled with bit operations (the CPU checker encodes the
// same byte layouts independently, by searching the value grids).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa_attn.h"

namespace csa {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even; NaN -> canonical quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- E4M3FN
// value = (-1)^s * (e ? (1 + m/8) 2^(e-7) : m 2^-9); 0x7F / 0xFF are NaN
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t s = (c & 0x80u) << 24, e = (c >> 3) & 15u, m = c & 7u;
    float v;
    if (e == 0) v = (float)m * 0.001953125f;                      // m * 2^-9
    else v = __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 15 && m == 7) v = __uint_as_float(0x7FC00000u);
    return __uint_as_float(__float_as_uint(v) | s);
}

// bf16 bit pattern of an E4M3 value (exact: bf16 holds every E4M3 value)
__device__ __forceinline__ uint16_t e4m3_to_bf16(uint32_t c) {
    return (uint16_t)(__float_as_uint(e4m3_to_f32(c)) >> 16);
}

// round to nearest even on the E4M3 grid, saturating to +-448; NaN -> 0x7F
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t s = (u >> 24) & 0x80u;
    float a = fabsf(x);
    if (a != a) return 0x7F;
    if (a >= 448.0f) return (uint8_t)(s | 0x7Eu);
    if (a < 0.015625f) {                                           // below 2^-6: quantum 2^-9
        uint32_t q = (uint32_t)rintf(a * 512.0f);                  // 0..8; 8 is the first normal
        return (uint8_t)(s | q);
    }
    uint32_t ua = __float_as_uint(a);
    ua += 0x7FFFFu + ((ua >> 20) & 1u);                            // RNE to 3 mantissa bits
    uint32_t e = (ua >> 23) - 120u, m = (ua >> 20) & 7u;
    return (uint8_t)(s | (e << 3) | m);
}

// ---------------------------------------------------------------- E2M1 / E8M0
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    uint32_t mag = c & 7u;
    float v = (mag < 2) ? 0.5f * (float)mag : __uint_as_float(((mag >> 1) + 126u) << 23 | (mag & 1u) << 22);
    return (c & 8u) ? -v : v;
}

// nearest E2M1 code, ties to even, saturating at +-6 (x already divided by the scale)
__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
    float a = fabsf(x);
    if (a != a) return 0;
    uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | ((__float_as_uint(x) >> 28) & 8u);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    // 2^(s-127); s = 0 is 2^-127 (subnormal float); 255 is NaN
    if (s == 255u) return __uint_as_float(0x7FC00000u);
    return s == 0 ? 5.877471754111438e-39f : __uint_as_float(s << 23);
}

// ---------------------------------------------------------------- RoPE
// Angle of pair i at position pos: pos * f_i with f_i = base^(-2i/dr) held in
// fp64 (positions reach 2^20 and more, where an fp32 product would be off by
// tens of milliradians).
// Copy the frequency table of the kernel's argument block to LDS, one entry
// per thread.  The block must be the kernel's first parameter (offset 0 of
// the kernel-argument segment); offset is offsetof(block, table).  Reading
// it through the segment pointer keeps a per-lane index off the by-value
// parameter (which would force a private copy of the whole block).  Needs
// blockDim >= npairs; the caller synchronises before use.
__device__ __forceinline__ void stage_rope_arg(size_t offset, double* lds, int npairs) {
    const double* t = (const double*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offset);
    if ((int)threadIdx.x < npairs) lds[threadIdx.x] = t[threadIdx.x];
}

// Load one dword of every 64-byte line of the first `bytes` of the kernel's
// argument block, all at once, and wait for them (the empty asm consumes the
// values).  The scalar loads of the argument fields spread through a kernel
// otherwise miss the scalar cache one line after another, each costing a
// memory round trip before the next can be issued; after this they hit.
__device__ __forceinline__ void warm_kernargs(size_t bytes) {
    const uint32_t* p = (const uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t acc = 0;
    for (size_t off = 0; off < bytes; off += 64) acc ^= p[off / 4];
    asm volatile("" ::"s"(acc));
}
// the same for BYTES bytes starting at a run-time offset: a fixed number of
// independent loads, one per 64-byte line
template <size_t BYTES>
__device__ __forceinline__ void warm_kernargs_at(size_t from) {
    constexpr int kLines = (int)((BYTES + 63) / 64) + 1;
    const uint32_t* p = (const uint32_t*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + (from & ~(size_t)63));
    uint32_t v[kLines];
#pragma unroll
    for (int i = 0; i < kLines; i++) v[i] = p[16 * i];
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kLines; i++) acc ^= v[i];
    asm volatile("" ::"s"(acc));
}

// A value every lane reads at the same address (a row's position), loaded
// through the scalar unit: waiting for it does not wait for the vector loads
// issued before it (they count on a different counter).  The memory is only
// read during the kernel.
__device__ __forceinline__ int32_t load_uniform_i32(const int32_t* p) {
    return *(const __attribute__((address_space(4))) int32_t*)p;
}

// the p-th frequency of a RopeTable passed by value at byte `offset` of the
// kernel arguments, read by one lane from the argument segment
__device__ __forceinline__ double rope_freq_arg(size_t offset, int p) {
    return ((const double*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offset))[p];
}


// sin and cos of pos * freq.  The angle is reduced in fp64 around the
// nearest multiple k of pi/2 (Cody-Waite: pi/2 as a double plus the double
// nearest its remainder, fused multiply-adds) to r in [-pi/4, pi/4]; sin r and
// cos r come from their Taylor series about 0 in fp32 (through r^9 and r^10:
// truncation error below 2e-9 on that interval) and k mod 4 picks the
// quadrant.  Branch-free and table-free.
__device__ __forceinline__ void rope_sincos(double pos, double freq, float& s, float& c) {
    const double x = pos * freq;
    const double k = rint(x * 0.6366197723675814);            // x / (pi / 2)
    double r = fma(-k, 1.5707963267948966, x);                 // pi / 2, leading double
    r = fma(-k, 6.123233995736766e-17, r);                     // pi / 2 - leading double
    const float f = (float)r, f2 = f * f;
    const float sp = f + f * f2 * (-1.0f / 6.0f + f2 * (1.0f / 120.0f + f2 * (-1.0f / 5040.0f + f2 * (1.0f / 362880.0f))));
    const float cp = 1.0f + f2 * (-0.5f + f2 * (1.0f / 24.0f + f2 * (-1.0f / 720.0f +
                                   f2 * (1.0f / 40320.0f + f2 * (-1.0f / 3628800.0f)))));
    const int q = (int)((long long)k & 3);
    // sin(q pi/2 + r), cos(q pi/2 + r) for q = 0..3: (s, c), (c, -s), (-s, -c), (-c, s)
    const float ss = (q & 1) ? cp : sp, cc = (q & 1) ? sp : cp;
    s = (q & 2) ? -ss : ss;
    c = ((q + 1) & 2) ? -cc : cc;
}

// ReLU on the bit pattern: a float with the sign bit set is a negative int32,
// so one integer max gives max(x, +0) for every non-NaN x, without the
// canonicalising pass a float max of an unknown value takes.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---------------------------------------------------------------- score keys
// order-preserving map float -> uint32 (larger float, larger key); NaN -> 0; -0 == +0
__device__ __forceinline__ uint32_t score_key(float s) {
    if (s != s) return 0u;
    s = s + 0.0f;
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// all-reduce over the 16 lanes of a DPP row (rotations, then quad swaps);
// commutative steps give every lane the same bits
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));     // row_ror:8
    v = fmaxf(v, dpp_f<0x124>(v));     // row_ror:4
    v = fmaxf(v, dpp_f<0x4E>(v));      // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0xB1>(v));      // quad_perm [1,0,3,2]
    return v;
}
__device__ __forceinline__ float row16_sum(float v) {
    v = v + dpp_f<0x128>(v);
    v = v + dpp_f<0x124>(v);
    v = v + dpp_f<0x4E>(v);
    v = v + dpp_f<0xB1>(v);
    return v;
}
// the same over all 64 lanes: the four row results are read as scalars and
// combined as (r0 + r1) + (r2 + r3); no LDS round trips
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = row16_sum(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = row16_max(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// wave ballot of a predicate, straight from its condition mask
__device__ __forceinline__ uint64_t ballot64(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// the value of v in lane `lane` (a wave-uniform index), as a scalar read
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// inclusive prefix sum over the 64 lanes: shifted adds inside each 16-lane
// DPP row (lanes shifted in from outside the row add 0), then the totals of
// the rows below, read as scalars
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
    v += dpp_u<0x111>(v);              // row_shr:1
    v += dpp_u<0x112>(v);              // row_shr:2
    v += dpp_u<0x114>(v);              // row_shr:4
    v += dpp_u<0x118>(v);              // row_shr:8
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const int rw = (threadIdx.x & 63) >> 4;
    return v + (rw >= 1 ? t0 : 0u) + (rw >= 2 ? t1 : 0u) + (rw >= 3 ? t2 : 0u);
}

// block-wide reductions; `red` is LDS scratch of >= blockDim/64 floats
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < nw; i++) t += red[i];
    return t;
}
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < nw; i++) t = fmaxf(t, red[i]);
    return t;
}

// load one scalar of an f32 / bf16 array as float
template <typename T> __device__ __forceinline__ float ld_scalar(const T* p, size_t i);
template <> __device__ __forceinline__ float ld_scalar<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld_scalar<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }

template <typename T> __device__ __forceinline__ void st_scalar(T* p, size_t i, float v);
template <> __device__ __forceinline__ void st_scalar<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void st_scalar<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }

}  // namespace csa
