// proj.hip -- attn_out_proj_grouped: block-diagonal output projection.
//
// Method: "DeepSeek-V4 ... open-source declaration" (peacm.com) section 3.2,
// CSA step 4 (the head-dim-512 attention outputs are projected in groups to
// cut the cost).  Reading: G independent [D/G x Hd/G] maps over consecutive
// head groups, no bias.
//
// Two kernels, both keeping every reduction inside one workgroup (no split
// across workgroups, fixed summation order):
//   decode (M <= 16): weight streaming.  The group's M activation rows sit in
//     LDS; each wave walks 16 / M weight rows with 16-byte coalesced loads
//     (every weight byte read once), accumulates M x rows dot products per
//     lane (bf16 pairs through v_dot2_f32_bf16), and reduces the 16 partial
//     sums across the wave by recursive halving (17 lane exchanges);
//   otherwise: a TM x TN tile of y per workgroup, walking the reduction
//     dimension in KC-wide slabs staged in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kProjThreads = 256;
constexpr int kProjTN = 16;
constexpr int kProjKC = 64;

template <typename T, typename YT, int TM>
__global__ __launch_bounds__(kProjThreads) void k_proj(ProjArgs a) {
    __shared__ float os[TM][kProjKC + 1];
    __shared__ float wsm[kProjTN][kProjKC + 1];
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int tpg = (dg + kProjTN - 1) / kProjTN;             // tiles per group
    const int g = (int)(blockIdx.x / tpg);
    const int i0 = (int)(blockIdx.x % tpg) * kProjTN;          // first row inside W[g]
    const int64_t m0 = (int64_t)blockIdx.y * TM;
    const T* o = reinterpret_cast<const T*>(a.o);
    const T* W = reinterpret_cast<const T*>(a.W);
    constexpr int kOwn = (TM * kProjTN + kProjThreads - 1) / kProjThreads;
    float acc[kOwn];
#pragma unroll
    for (int q = 0; q < kOwn; q++) acc[q] = 0.0f;

    for (int c0 = 0; c0 < cg; c0 += kProjKC) {
        for (int idx = threadIdx.x; idx < TM * kProjKC; idx += blockDim.x) {
            const int mi = idx / kProjKC, c = idx % kProjKC;
            const int64_t m = m0 + mi;
            float v = 0.0f;
            if (m < a.M && c0 + c < cg) v = ld_scalar<T>(o, (size_t)m * a.Hd + (size_t)g * cg + c0 + c);
            os[mi][c] = v;
        }
        for (int idx = threadIdx.x; idx < kProjTN * kProjKC; idx += blockDim.x) {
            const int ni = idx / kProjKC, c = idx % kProjKC;
            float v = 0.0f;
            if (i0 + ni < dg && c0 + c < cg) v = ld_scalar<T>(W, ((size_t)g * dg + i0 + ni) * cg + c0 + c);
            wsm[ni][c] = v;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kOwn; q++) {
            const int idx = threadIdx.x + q * kProjThreads;
            if (idx < TM * kProjTN) {
                const int mi = idx / kProjTN, ni = idx % kProjTN;
                float s = acc[q];
                for (int c = 0; c < kProjKC; c++) s = fmaf(os[mi][c], wsm[ni][c], s);
                acc[q] = s;
            }
        }
        __syncthreads();
    }
    YT* y = reinterpret_cast<YT*>(a.y);
#pragma unroll
    for (int q = 0; q < kOwn; q++) {
        const int idx = threadIdx.x + q * kProjThreads;
        if (idx < TM * kProjTN) {
            const int mi = idx / kProjTN, ni = idx % kProjTN;
            const int64_t m = m0 + mi;
            if (m < a.M && i0 + ni < dg) st_scalar<YT>(y, (size_t)m * a.D + (size_t)g * dg + i0 + ni, acc[q]);
        }
    }
}

typedef __bf16 bf16x2_p __attribute__((ext_vector_type(2)));

// 8 products of a 16-byte chunk pair, accumulated into acc
template <typename T>
__device__ __forceinline__ float chunk_dot(uint4 w, uint4 o, float acc);
template <>
__device__ __forceinline__ float chunk_dot<uint16_t>(uint4 w, uint4 o, float acc) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w}, ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
    for (int i = 0; i < 4; i++)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_p, wv[i]), __builtin_bit_cast(bf16x2_p, ov[i]),
                                              acc, false);
    return acc;
}
template <>
__device__ __forceinline__ float chunk_dot<float>(uint4 w, uint4 o, float acc) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(o.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(o.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(o.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(o.w), acc);
    return acc;
}

// sum v[0..16) over the 64 lanes; lane 4j..4j+3 end with the total of value j
__device__ __forceinline__ float wave_reduce16(float* v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 32, n = 16; b >= 4; b >>= 1, n >>= 1) {
        const bool hi = (lane & b) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; i++) {
            const float mine = hi ? v[i + n / 2] : v[i];
            const float other = hi ? v[i] : v[i + n / 2];
            v[i] = mine + __shfl_xor(other, b, 64);
        }
    }
    float r = v[0];
    r += __shfl_xor(r, 2, 64);
    r += __shfl_xor(r, 1, 64);
    return r;
}

constexpr int kGemvLdsBytes = 65536;

template <typename T, typename YT, int MR>
__global__ __launch_bounds__(256) void k_proj_gemv(ProjArgs a) {
    constexpr int R = 16 / MR;                 // weight rows per wave
    constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
    extern __shared__ uint4 osm[];             // [MR][chunks of the group's activation row]
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int nch = cg / EPC;
    const int rows_wg = 4 * R;
    const int tpg = dg / rows_wg;
    const int g = blockIdx.x / tpg;
    const int i0 = (blockIdx.x % tpg) * rows_wg;
    const T* o = reinterpret_cast<const T*>(a.o);
    const T* W = reinterpret_cast<const T*>(a.W);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r0 = i0 + w * R;
    const T* wr = W + ((size_t)g * dg + r0) * cg;
    // weight chunks are loaded in batches of kIt per lane; the first batch goes
    // out before the activations are staged, so both sets of loads are in
    // flight together
    constexpr int kIt = (32 / R) < 8 ? (32 / R) : 8;
    float acc[R * MR];
#pragma unroll
    for (int q = 0; q < R * MR; q++) acc[q] = 0.0f;
    for (int cb = 0; cb < nch; cb += 64 * kIt) {
        uint4 wv[kIt][R];
#pragma unroll
        for (int it = 0; it < kIt; it++) {
            const int c = cb + lane + 64 * it;
#pragma unroll
            for (int r = 0; r < R; r++)
                wv[it][r] = c < nch ? *reinterpret_cast<const uint4*>(wr + (size_t)r * cg + (size_t)c * EPC)
                                    : make_uint4(0u, 0u, 0u, 0u);
        }
        if (cb == 0) {
            for (int idx = threadIdx.x; idx < MR * nch; idx += blockDim.x) {
                const int m = idx / nch, c = idx % nch;
                osm[idx] = m < a.M ? *reinterpret_cast<const uint4*>(o + (size_t)m * a.Hd + (size_t)g * cg + (size_t)c * EPC)
                                   : make_uint4(0u, 0u, 0u, 0u);
            }
            __syncthreads();
        }
#pragma unroll
        for (int it = 0; it < kIt; it++) {
            const int c = cb + lane + 64 * it;
            if (c < nch) {
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    const uint4 ov = osm[m * nch + c];
#pragma unroll
                    for (int r = 0; r < R; r++) acc[r * MR + m] = chunk_dot<T>(wv[it][r], ov, acc[r * MR + m]);
                }
            }
        }
    }
    const float tot = wave_reduce16(acc);
    if ((lane & 3) == 0) {
        const int j = lane >> 2, r = j / MR, m = j % MR;
        if (m < a.M) st_scalar<YT>(reinterpret_cast<YT*>(a.y), (size_t)m * a.D + (size_t)g * dg + r0 + r, tot);
    }
}

template <typename T, typename YT>
static bool try_gemv(const ProjArgs& a, hipStream_t st) {
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int EPC = 16 / (int)sizeof(T);
    if (a.M > 16 || cg % EPC) return false;
    const int MR = a.M <= 1 ? 1 : a.M <= 2 ? 2 : a.M <= 4 ? 4 : a.M <= 8 ? 8 : 16;
    const int rows_wg = 4 * (16 / MR);
    const size_t lds = (size_t)MR * cg * sizeof(T);
    if (dg % rows_wg || lds > (size_t)kGemvLdsBytes) return false;
    if (((uintptr_t)a.o | (uintptr_t)a.W) & 15) return false;
    const unsigned grid = (unsigned)(a.G * (dg / rows_wg));
    switch (MR) {
        case 1: hipLaunchKernelGGL((k_proj_gemv<T, YT, 1>), dim3(grid), dim3(256), lds, st, a); break;
        case 2: hipLaunchKernelGGL((k_proj_gemv<T, YT, 2>), dim3(grid), dim3(256), lds, st, a); break;
        case 4: hipLaunchKernelGGL((k_proj_gemv<T, YT, 4>), dim3(grid), dim3(256), lds, st, a); break;
        case 8: hipLaunchKernelGGL((k_proj_gemv<T, YT, 8>), dim3(grid), dim3(256), lds, st, a); break;
        default: hipLaunchKernelGGL((k_proj_gemv<T, YT, 16>), dim3(grid), dim3(256), lds, st, a); break;
    }
    return true;
}

template <typename T, typename YT>
static void launch_t(const ProjArgs& a, hipStream_t st) {
    if (try_gemv<T, YT>(a, st)) return;
    const int dg = a.D / a.G;
    const unsigned gx = (unsigned)(a.G * ((dg + kProjTN - 1) / kProjTN));
    if (a.M <= 8) {
        hipLaunchKernelGGL((k_proj<T, YT, 8>), dim3(gx, 1), dim3(kProjThreads), 0, st, a);
    } else {
        const unsigned gy = (unsigned)((a.M + 31) / 32);
        hipLaunchKernelGGL((k_proj<T, YT, 32>), dim3(gx, gy), dim3(kProjThreads), 0, st, a);
    }
}

hipError_t launch_proj(const ProjArgs& a, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    const bool ib = a.fmt == CSA_BF16, yb = a.y_fmt == CSA_BF16;
    if (!ib && !yb) launch_t<float, float>(a, st);
    if (!ib && yb) launch_t<float, uint16_t>(a, st);
    if (ib && !yb) launch_t<uint16_t, float>(a, st);
    if (ib && yb) launch_t<uint16_t, uint16_t>(a, st);
    return hipGetLastError();
}

}  // namespace csa
