// proj.hip -- attn_out_proj_grouped: block-diagonal output projection.
//
// Method: "DeepSeek-V4 ... open-source declaration" (peacm.com) section 3.2,
// CSA step 4 (the head-dim-512 attention outputs are projected in groups to
// cut the cost).  Reading: G independent [D/G x Hd/G] maps over consecutive
// head groups, no bias.
//
// Tiled fp32 kernel: a workgroup computes a TM x TN tile of y for one group,
// walking the reduction dimension in KC-wide slabs staged in LDS.  Every
// reduction stays inside one workgroup (no split across workgroups), so the
// summation order is fixed.  In decode (M = batch) the tile covers all rows
// and each weight element is read exactly once.
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

template <typename T, typename YT>
static void launch_t(const ProjArgs& a, hipStream_t st) {
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
