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
//     LDS; the group's weight rows are dealt round-robin to its waves, which
//     read them with 16-byte coalesced loads (every weight byte read once),
//     accumulate M x rows dot products per lane (bf16 pairs through
//     v_dot2_f32_bf16), and reduce the partial sums across the wave by
//     recursive halving;
//   bf16, M > 16 (prefill chunks): a matrix-core GEMM per group, 256 x 128
//     tiles of y, the reduction walked in 32-wide slabs through LDS;
//   otherwise: a TM x TN tile of y per workgroup, walking the reduction
//     dimension in KC-wide slabs staged in LDS.
#include <type_traits>

#include <algorithm>

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

// Sum each of v[0..NV) over the 64 lanes (NV a power of two, at most 64):
// log2(NV) halving exchanges leave one value per lane group, then plain
// butterflies finish; value j ends in lanes [j * 64 / NV, (j + 1) * 64 / NV).
template <int NV>
__device__ __forceinline__ float wave_reduce_n(float* v) {
    static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
    const int lane = threadIdx.x & 63;
    int b = 32;
#pragma unroll
    for (int n = NV; n > 1; n >>= 1, b >>= 1) {
        const bool hi = (lane & b) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; i++) {
            const float mine = hi ? v[i + n / 2] : v[i];
            const float other = hi ? v[i] : v[i + n / 2];
            v[i] = mine + __shfl_xor(other, b, 64);
        }
    }
    float r = v[0];
#pragma unroll
    for (; b >= 1; b >>= 1) r += __shfl_xor(r, b, 64);
    return r;
}

constexpr int kGemvLdsBytes = 65536;

// Decode projection, M <= 16 activation rows.  Workgroup = NW waves of one
// group g; the group's M activation rows are staged in LDS once.  The group's
// dg weight rows are dealt to its waves round-robin: wave v of the group
// (V waves per group) takes rows v, v + V, v + 2V, ... (RT rows), so the grid
// streams one compact band of every group's weights at a time instead of
// scattering over all of them.  A wave walks its rows in batches of RB, the
// next batch's 16-byte loads in flight while the current one is reduced
// (lane l takes chunks l + 64 it of a row); weights are read once, with
// non-temporal loads since nothing reuses them.  kFull: the row length is a
// whole number of passes, so no load or product needs a bounds test (which
// would otherwise make every wait a full drain).
template <typename T, typename YT, int MR, int RT, int RB, int NW, bool kFull>
__global__ __launch_bounds__(64 * NW) void k_proj_gemv(ProjArgs a) {
    constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
    constexpr int NV = RT * MR;
    constexpr int NB = RT / RB;
    static_assert(RT % RB == 0, "row batches must tile the wave's rows");
    extern __shared__ uint4 osm[];             // [MR][chunks of the group's activation row]
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int nch = cg / EPC;
    const int V = dg / RT;                     // waves per group
    // consecutive workgroups take different groups: workgroups are dealt to
    // the 8 XCDs round-robin, so with G = 8 all of group g runs on one XCD
    const int g = blockIdx.x % a.G;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int v = (blockIdx.x / a.G) * NW + w;
    const T* o = reinterpret_cast<const T*>(a.o);
    const T* W = reinterpret_cast<const T*>(a.W) + ((size_t)g * dg + v) * cg;
    constexpr int kIt = RB <= 2 ? 8 : 16 / RB;  // chunks per lane per row and pass
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    float acc[NV];
#pragma unroll
    for (int q = 0; q < NV; q++) acc[q] = 0.0f;
    for (int cb = 0; cb < nch; cb += 64 * kIt) {
        v4u wv[2][RB][kIt];                    // ping-pong batch buffers
        auto issue = [&](v4u (&dst)[RB][kIt], int bt) {
#pragma unroll
            for (int r = 0; r < RB; r++) {
#pragma unroll
                for (int it = 0; it < kIt; it++) {
                    const int c = cb + lane + 64 * it;
                    const size_t row = (size_t)(bt * RB + r) * V;
                    dst[r][it] = kFull || c < nch ? __builtin_nontemporal_load(
                                               reinterpret_cast<const v4u*>(W + row * cg + (size_t)c * EPC))
                                         : v4u{0u, 0u, 0u, 0u};
                }
            }
        };
        issue(wv[0], 0);
        if (cb == 0) {
            for (int idx = threadIdx.x; idx < MR * nch; idx += blockDim.x) {
                const int m = idx / nch, c = idx % nch;
                osm[idx] = m < a.M ? *reinterpret_cast<const uint4*>(o + (size_t)m * a.Hd + (size_t)g * cg + (size_t)c * EPC)
                                   : make_uint4(0u, 0u, 0u, 0u);
            }
            __syncthreads();
        }
#pragma unroll
        for (int bt = 0; bt < NB; bt++) {
            if (bt + 1 < NB) issue(wv[(bt + 1) & 1], bt + 1);
#pragma unroll
            for (int it = 0; it < kIt; it++) {
                const int c = cb + lane + 64 * it;
                if (kFull || c < nch) {
#pragma unroll
                    for (int m = 0; m < MR; m++) {
                        const uint4 ov = osm[m * nch + c];
#pragma unroll
                        for (int r = 0; r < RB; r++) {
                            const v4u x = wv[bt & 1][r][it];
                            const int q = (bt * RB + r) * MR + m;
                            acc[q] = chunk_dot<T>(make_uint4(x[0], x[1], x[2], x[3]), ov, acc[q]);
                        }
                    }
                }
            }
        }
    }
    const float tot = wave_reduce_n<NV>(acc);
    if ((lane & (64 / NV - 1)) == 0) {
        const int j = lane / (64 / NV), r = j / MR, m = j % MR;
        if (m < a.M) st_scalar<YT>(reinterpret_cast<YT*>(a.y), (size_t)m * a.D + (size_t)g * dg + v + r * V, tot);
    }
}

// Launch shape, measured on the 8 x [896 x 4096] bf16 decode projection: two
// rows per wave, one row per batch, eight waves per workgroup (448
// workgroups) beat fewer, longer waves or all loads in flight at once.
constexpr int kGemvRows = 2, kGemvBatch = 1, kGemvWaves = 8;

template <typename T, typename YT, int MR>
static bool launch_gemv(const ProjArgs& a, hipStream_t st) {
    constexpr int RT = kGemvRows, RB = kGemvBatch, NW = kGemvWaves;
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const size_t lds = (size_t)MR * cg * sizeof(T);
    if (dg % (NW * RT) || lds > (size_t)kGemvLdsBytes) return false;
    const unsigned grid = (unsigned)(a.G * (dg / (NW * RT)));
    constexpr int kIt = RB <= 2 ? 8 : 16 / RB;
    if ((cg / (16 / (int)sizeof(T))) % (64 * kIt) == 0)
        hipLaunchKernelGGL((k_proj_gemv<T, YT, MR, RT, RB, NW, true>), dim3(grid), dim3(64 * NW), lds, st, a);
    else
        hipLaunchKernelGGL((k_proj_gemv<T, YT, MR, RT, RB, NW, false>), dim3(grid), dim3(64 * NW), lds, st, a);
    return true;
}

// ---- skinny bf16 projection on the matrix cores (4 < M <= 128 rows)
// A weight stream with a few activation rows: one workgroup per 16 output
// columns of one group, all M rows in blocks of 16 (v_mfma_f32_16x16x32_bf16:
// A = 16 activation rows x 32 k, B = 32 k x 16 weight rows).  The four waves
// split the group width into quarters; each streams its quarter of the 16
// weight rows straight into registers, KB K-steps per batch (every load of a
// batch in flight before its products), and re-reads the activation
// fragments per K-step (the M rows of o are a few hundred KB, resident in
// L2).  The parts' sums meet in LDS and are added in wave order, so the
// result depends neither on timing nor on M.
constexpr int kSkWaves = 4;                      // waves per workgroup at most
constexpr int64_t kSkMaxM = 128;                // rows handled by the skinny kernel
typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));
typedef float f32x4_s __attribute__((ext_vector_type(4)));

template <int MB, typename YT>
__global__ __launch_bounds__(64 * kSkWaves) void k_proj_skinny(ProjArgs a) {
    constexpr int KB = MB <= 2 ? 16 : (MB <= 4 ? 8 : 4);   // K-steps per load batch
    __shared__ f32x4_s part[kSkWaves][MB][64];
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (int)(blockDim.x >> 6);
    const int nbk = (dg + 15) / 16;              // 16-column blocks per group
    const int g = (int)(blockIdx.x / nbk), nb = (int)(blockIdx.x % nbk);
    const int l16 = lane & 15, kq = 8 * (lane >> 4);
    const int n = nb * 16 + l16;
    const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W) + ((size_t)g * dg + min(n, dg - 1)) * cg + kq;
    const uint16_t* o = reinterpret_cast<const uint16_t*>(a.o) + (size_t)g * cg + kq;
    const int nks = cg / 32;
    const int kper = (nks + nw - 1) / nw;
    const int kb0 = w * kper, kb1 = min(nks, kb0 + kper);     // this wave's K-steps
    typedef unsigned v4u_s __attribute__((ext_vector_type(4)));
    f32x4_s acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[mb] = f32x4_s{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = kb0; k0 < kb1; k0 += KB) {
        bf16x8_s bf[KB], af[MB][KB];
#pragma unroll
        for (int u = 0; u < KB; u++) {
            const bool kin = k0 + u < kb1;
            const v4u_s v = kin ? __builtin_nontemporal_load(reinterpret_cast<const v4u_s*>(W + (size_t)(k0 + u) * 32))
                                : v4u_s{0u, 0u, 0u, 0u};
            bf[u] = __builtin_bit_cast(bf16x8_s, v);
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
            const int m = mb * 16 + l16;
#pragma unroll
            for (int u = 0; u < KB; u++) {
                const bool in = m < a.M && k0 + u < kb1;
                const uint4 v = in ? *reinterpret_cast<const uint4*>(o + (size_t)m * a.Hd + (size_t)(k0 + u) * 32)
                                   : make_uint4(0u, 0u, 0u, 0u);
                af[mb][u] = __builtin_bit_cast(bf16x8_s, v);
            }
        }
#pragma unroll
        for (int u = 0; u < KB; u++)
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][u], bf[u], acc[mb], 0, 0, 0);
    }
#pragma unroll
    for (int mb = 0; mb < MB; mb++) part[w][mb][lane] = acc[mb];
    __syncthreads();
    if (w != 0) return;
    // lane l holds rows 4 (l / 16) + i of each block, column l % 16
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
        f32x4_s r = part[0][mb][lane];
        for (int q = 1; q < nw; q++) r += part[q][mb][lane];
        if (n < dg) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = mb * 16 + 4 * (lane >> 4) + i;
                if (m < a.M) st_scalar<YT>(reinterpret_cast<YT*>(a.y), (size_t)m * a.D + (size_t)g * dg + n, r[i]);
            }
        }
    }
}

template <typename YT>
static bool try_skinny(const ProjArgs& a, hipStream_t st) {
    const int cg = a.Hd / a.G, dg = a.D / a.G;
    if (a.fmt != CSA_BF16 || a.M <= 4 || a.M > kSkMaxM || cg % 32) return false;
    if (((uintptr_t)a.o | (uintptr_t)a.W) & 15) return false;
    const unsigned grid = (unsigned)((int64_t)a.G * ((dg + 15) / 16));
    // the group width split over up to kSkWaves waves, about 16 K-steps (one
    // load batch) each; fixed by the width alone, so a row's sum order does
    // not depend on M
    const int nw = (int)std::min<int64_t>(kSkWaves, std::max<int64_t>(1, (cg / 32 + 15) / 16));
    const dim3 blk(64 * nw);
    if (a.M <= 16) hipLaunchKernelGGL((k_proj_skinny<1, YT>), dim3(grid), blk, 0, st, a);
    else if (a.M <= 32) hipLaunchKernelGGL((k_proj_skinny<2, YT>), dim3(grid), blk, 0, st, a);
    else if (a.M <= 64) hipLaunchKernelGGL((k_proj_skinny<4, YT>), dim3(grid), blk, 0, st, a);
    else hipLaunchKernelGGL((k_proj_skinny<8, YT>), dim3(grid), blk, 0, st, a);
    return true;
}

// ---- bf16 GEMM on the matrix cores (M > 16)
// y_g[m][n] = sum_c o[m][g cg + c] W[g][n][c]: both operands are read along
// the reduction dimension, which is what the A (rows of o) and B (rows of W)
// operands of v_mfma_f32_32x32x16_bf16 want.  Workgroup tile 256 (m) x 128 (n)
// of one group, four waves each owning 64 rows x all 128 columns (2 x 4
// accumulators of 32 x 32).  The reduction goes in 32-wide slabs copied
// straight from global memory into LDS (global_load_lds_dwordx4, no register
// staging), three slabs in flight: slab s + 2 is sent while slab s is
// multiplied.  A slab row is 64 bytes (four 16-byte chunks), unpadded; chunk c
// of row r sits in slot c ^ ((r >> 1) & 3), so the fragment reads of 8
// consecutive rows hit 8 distinct bank groups.  72 KB of LDS: two workgroups
// per CU.  Rows past M and columns past D/G load clamped (valid) addresses and
// are never stored.  Tiles are dealt so that the dispatcher's round-robin over
// the 8 XCDs gives each XCD a contiguous run of tiles (neighbouring n-tiles
// share their rows of o in that XCD's L2).
constexpr int kPmBM = 256, kPmBN = 128, kPmBK = 32;
constexpr int kPmThreads = 256;
constexpr int kPmStages = 3;
constexpr int kPmAq = kPmBM * kPmBK / 8 / kPmThreads;   // 16-byte copies of o per thread and slab
constexpr int kPmBq = kPmBN * kPmBK / 8 / kPmThreads;   // 16-byte copies of W per thread and slab
constexpr int kPmSlabBytes = (kPmBM + kPmBN) * kPmBK * 2;
typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int pm_slot(int r, int c) { return 4 * r + (c ^ ((r >> 1) & 3)); }

template <typename YT>
__global__ __launch_bounds__(kPmThreads, 2) void k_proj_mfma(ProjArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[kPmStages][kPmSlabBytes];   // [A 256 rows | B 128 rows]
    const int dg = a.D / a.G, cg = a.Hd / a.G;
    const int tiles_n = (dg + kPmBN - 1) / kPmBN;
    const int64_t tiles_m = (a.M + kPmBM - 1) / kPmBM;
    // XCD-aware deal: workgroup id -> logical tile (n fastest, then m, then g)
    const int64_t id = blockIdx.x, nwg = gridDim.x, per = nwg / 8;
    const int64_t L = id < 8 * per ? (id % 8) * per + id / 8 : id;
    const int tn = (int)(L % tiles_n);
    const int64_t tm = (L / tiles_n) % tiles_m;
    const int g = (int)(L / tiles_n / tiles_m);
    const int64_t m0 = tm * kPmBM;
    const int n0 = tn * kPmBN;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const uint16_t* o = reinterpret_cast<const uint16_t*>(a.o) + (size_t)g * cg;
    const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W) + (size_t)g * dg * cg;
    // copy q of this wave fills slots [64 (4 q + w), +64) of the A (or B) part;
    // lane l's slot holds chunk (slot % 4) ^ ((row >> 1) & 3) of row slot / 4
    const uint16_t* ap[kPmAq];
    const uint16_t* bp[kPmBq];
#pragma unroll
    for (int q = 0; q < kPmAq; q++) {
        const int sl = 64 * (4 * q + w) + lane, r = sl >> 2;
        const int c = (sl & 3) ^ ((r >> 1) & 3);
        ap[q] = o + (size_t)min(m0 + r, a.M - 1) * a.Hd + 8 * c;
    }
#pragma unroll
    for (int q = 0; q < kPmBq; q++) {
        const int sl = 64 * (4 * q + w) + lane, r = sl >> 2;
        const int c = (sl & 3) ^ ((r >> 1) & 3);
        bp[q] = W + (size_t)min(n0 + r, dg - 1) * cg + 8 * c;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int s, int buf) __attribute__((always_inline)) {
        uint8_t* base = &sm[buf][0];
#pragma unroll
        for (int q = 0; q < kPmAq; q++)
            __builtin_amdgcn_global_load_lds(ap[q] + s * kPmBK, (lds_void*)(base + 1024 * (4 * q + w)), 16, 0, 0);
#pragma unroll
        for (int q = 0; q < kPmBq; q++)
            __builtin_amdgcn_global_load_lds(bp[q] + s * kPmBK,
                                             (lds_void*)(base + kPmBM * 64 + 1024 * (4 * q + w)), 16, 0, 0);
    };
    f32x16_p acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    auto compute = [&](int buf) __attribute__((always_inline)) {
        // every fragment of the slab is read before the first product
        const uint8_t* base = &sm[buf][0];
        constexpr int KK = kPmBK / 16;
        bf16x8_p fa[KK][2], fb[KK][4];
#pragma unroll
        for (int kk = 0; kk < KK; kk++) {
            const int c = 2 * kk + hl;
#pragma unroll
            for (int i = 0; i < 2; i++)
                fa[kk][i] = *reinterpret_cast<const bf16x8_p*>(base + 16 * pm_slot(64 * w + 32 * i + l32, c));
#pragma unroll
            for (int j = 0; j < 4; j++)
                fb[kk][j] = *reinterpret_cast<const bf16x8_p*>(base + kPmBM * 64 + 16 * pm_slot(32 * j + l32, c));
        }
        // the products take the fragments through an empty asm, so all twelve
        // reads go out before the first product
        static_assert(KK == 2, "fragment pinning is written for two K-steps");
        asm volatile("" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fb[0][0]), "+v"(fb[0][1]), "+v"(fb[0][2]),
                     "+v"(fb[0][3]), "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fb[1][0]), "+v"(fb[1][1]),
                     "+v"(fb[1][2]), "+v"(fb[1][3]));
#pragma unroll
        for (int kk = 0; kk < KK; kk++)
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][i], fb[kk][j], acc[i][j], 0, 0, 0);
    };
    // slab s lives in buffer s % 3.  Each thread waits for its own copies of
    // slab s (leaving those of slab s + 1 in flight); the barrier then makes
    // every thread's copies visible and frees the buffer of slab s - 1, which
    // receives slab s + 2.
    const int ns = cg / kPmBK;
    issue(0, 0);
    if (ns > 1) issue(1, 1);
    int buf = 0, buf2 = 2;
    for (int s = 0; s < ns; s++) {
        if (s + 1 < ns) __builtin_amdgcn_s_waitcnt(0x0F70 | (kPmAq + kPmBq));   // vmcnt(copies per slab)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                               // vmcnt(0)
        __syncthreads();
        if (s + 2 < ns) issue(s + 2, buf2);
        compute(buf);
        buf = buf == kPmStages - 1 ? 0 : buf + 1;
        buf2 = buf2 == kPmStages - 1 ? 0 : buf2 + 1;
    }
    // accumulator (i, j) element e: row 8 (e / 4) + 4 hl + e % 4, column l32
    YT* y = reinterpret_cast<YT*>(a.y) + (size_t)g * dg;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + 32 * j + l32;
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t m = m0 + 64 * w + 32 * i + 8 * (e / 4) + 4 * hl + (e % 4);
                if (m < a.M && n < dg) st_scalar<YT>(y, (size_t)m * a.D + n, acc[i][j][e]);
            }
        }
}

template <typename YT>
static bool try_mfma(const ProjArgs& a, hipStream_t st) {
    const int cg = a.Hd / a.G, dg = a.D / a.G;
    if (a.fmt != CSA_BF16 || a.M <= 16 || cg % kPmBK) return false;
    if (((uintptr_t)a.o | (uintptr_t)a.W) & 15) return false;
    const int64_t tiles = (int64_t)a.G * ((a.M + kPmBM - 1) / kPmBM) * ((dg + kPmBN - 1) / kPmBN);
    if (tiles > 0x7fffffff) return false;
    hipLaunchKernelGGL((k_proj_mfma<YT>), dim3((unsigned)tiles), dim3(kPmThreads), 0, st, a);
    return true;
}

template <typename T, typename YT>
static bool try_gemv(const ProjArgs& a, hipStream_t st) {
    const int cg = a.Hd / a.G;
    const int EPC = 16 / (int)sizeof(T);
    if (a.M > 16 || cg % EPC) return false;
    if (((uintptr_t)a.o | (uintptr_t)a.W) & 15) return false;
    if (a.M <= 1) return launch_gemv<T, YT, 1>(a, st);
    if (a.M <= 2) return launch_gemv<T, YT, 2>(a, st);
    if (a.M <= 4) return launch_gemv<T, YT, 4>(a, st);
    if (a.M <= 8) return launch_gemv<T, YT, 8>(a, st);
    return launch_gemv<T, YT, 16>(a, st);
}

template <typename T, typename YT>
static void launch_t(const ProjArgs& a, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        if (try_skinny<YT>(a, st)) return;
    }
    if (try_gemv<T, YT>(a, st)) return;
    if constexpr (sizeof(T) == 2) {
        if (try_mfma<YT>(a, st)) return;
    }
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
