// lin8.hip -- projections with FP8 weights: csa_linear_fp8 and the fused
// input projections of a layer (csa_layer_in_proj).
//
// Method: every parameter outside the MoE experts is stored in FP8
// ("DeepSeek-V4 preview review" (deepseek.csdn.net), section 6.2 on precision
// and deployment; "DeepSeek V4 (Flash & Pro)" (github wiki article),
// specification table).  Reading: E4M3 codes with one fp32 scale per output
// row, bf16 activations, fp32 accumulation, no bias:
//   y[r][g*(N/G) + i] = scale[g*(N/G) + i] * sum_c x[r][g*(K/G) + c] * e4m3(W[g*(N/G) + i][c])
//
// E4M3 values are all bf16 numbers, so a weight code is widened to bf16
// exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and the products run on
// the bf16 matrix cores; the row scale is applied to the fp32 sum.  Weights
// cross HBM as one byte each, which is what the decode shapes are bound by.
//
// Three kernels, each keeping every reduction inside one workgroup:
//   M <= 32 (decode): a weight stream.  A workgroup owns 16 output columns of
//     one group; its waves split the group width, each copies its share of
//     the 16 weight rows global -> LDS in 128-byte row runs and multiplies
//     with v_mfma_f32_16x16x32_bf16 (A = 16 activation rows, B = 16 weight
//     rows); the partial sums meet in LDS and are added in wave order;
//   32 < M <= 64: the same split with the weights loaded straight into
//     registers, 32 output columns per workgroup;
//   M > 64 (prefill): a GEMM with 256 x 128 tiles (v_mfma_f32_32x32x16_bf16),
//     the reduction walked in 32-wide slabs copied global -> LDS, the weight
//     bytes widened when each wave reads its fragments.
// A row's sum is ordered by the weight shape and M's size class alone, so a
// row's result does not depend on the other rows.
// The epilogue multiplies by the row scale and writes each output column to
// the segment that owns it (the fused input projection writes five outputs
// from one launch).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace csa {

typedef __bf16 bf16x8_l __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_l __attribute__((ext_vector_type(2)));
typedef float f32x4_l __attribute__((ext_vector_type(4)));
typedef float f32x16_l __attribute__((ext_vector_type(16)));
typedef unsigned v4u_l __attribute__((ext_vector_type(4)));

// 8 E4M3 codes (bytes 0..3 of lo, then of hi) -> 8 bf16, exactly
__device__ __forceinline__ bf16x8_l e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const bf16x2_l a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_l b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_l c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_l d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_l{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Output column n -> its segment (segments sorted by n0 and covering [0, N));
// the descriptors are uniform, the choice per lane.
struct SegSel {
    void* out;
    int64_t ld;
    int32_t n0, fmt;
};
__device__ __forceinline__ SegSel lin_seg(const LinArgs& a, int n) {
    SegSel s{a.seg[0].out, a.seg[0].ld, a.seg[0].n0, a.seg[0].fmt};
#pragma unroll
    for (int i = 1; i < kLinMaxSeg; i++) {
        if (i < a.nseg && n >= a.seg[i].n0) s = SegSel{a.seg[i].out, a.seg[i].ld, a.seg[i].n0, a.seg[i].fmt};
    }
    return s;
}
__device__ __forceinline__ void lin_store(const SegSel& s, int64_t m, int n, float v) {
    const size_t off = (size_t)m * s.ld + (size_t)(n - s.n0);
    if (s.fmt == CSA_BF16) reinterpret_cast<uint16_t*>(s.out)[off] = f32_to_bf16(v);
    else reinterpret_cast<float*>(s.out)[off] = v;
}

// ---- 32 < M <= 64: the weight stream into registers
// K-mapping of one 64-wide "double step": lane group q = lane / 16 owns
// reduction indices 16 q .. 16 q + 15 of the step; the first product takes
// the lower eight of them, the second the upper eight.  A lane's weight bytes
// for the step are one 16-byte load, its activation values two.
constexpr int kL8Waves = 4;

template <int MB, int NB, int KB>
__global__ __launch_bounds__(64 * kL8Waves) void k_lin8_skinny(LinArgs a) {
    __shared__ f32x4_l part[kL8Waves][MB * NB][64];
    const int ng = a.N / a.G, kg = a.K / a.G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    constexpr int kCols = 16 * NB;
    const int tiles = (ng + kCols - 1) / kCols;
    const int g = (int)(blockIdx.x / tiles), c0 = (int)(blockIdx.x % tiles) * kCols;
    const int l16 = lane & 15, q = lane >> 4;
    const int nds = kg / 64;
    const int per = (nds + kL8Waves - 1) / kL8Waves;
    const int d0 = w * per, d1 = min(nds, d0 + per);
    const uint8_t* wp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int n = min(c0 + 16 * nb + l16, ng - 1);
        wp[nb] = a.W + ((size_t)g * ng + n) * kg + 16 * q;
    }
    const uint16_t* xp = a.x + (size_t)g * kg + 16 * q;
    f32x4_l acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) acc[mb][nb] = f32x4_l{0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = d0; s0 < d1; s0 += KB) {
        v4u_l wv[NB][KB];
#pragma unroll
        for (int u = 0; u < KB; u++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
                wv[nb][u] = s0 + u < d1 ? *reinterpret_cast<const v4u_l*>(wp[nb] + (size_t)(s0 + u) * 64)
                                        : v4u_l{0u, 0u, 0u, 0u};
        bf16x8_l af[MB][KB][2];
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
            const int64_t m = 16 * mb + l16;
#pragma unroll
            for (int u = 0; u < KB; u++) {
                const bool in = m < a.M && s0 + u < d1;
                const uint4* p = reinterpret_cast<const uint4*>(xp + (size_t)m * a.K + (size_t)(s0 + u) * 64);
                af[mb][u][0] = __builtin_bit_cast(bf16x8_l, in ? p[0] : make_uint4(0u, 0u, 0u, 0u));
                af[mb][u][1] = __builtin_bit_cast(bf16x8_l, in ? p[1] : make_uint4(0u, 0u, 0u, 0u));
            }
        }
#pragma unroll
        for (int u = 0; u < KB; u++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const bf16x8_l b0 = e4m3x8_to_bf16x8(wv[nb][u][0], wv[nb][u][1]);
                const bf16x8_l b1 = e4m3x8_to_bf16x8(wv[nb][u][2], wv[nb][u][3]);
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][u][0], b0, acc[mb][nb], 0, 0, 0);
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb][u][1], b1, acc[mb][nb], 0, 0, 0);
                }
            }
    }
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
        for (int nb = 0; nb < NB; nb++) part[w][mb * NB + nb][lane] = acc[mb][nb];
    __syncthreads();
    // wave v finishes the (mb, nb) blocks with index = v mod 4; lane l holds
    // rows 4 (l / 16) + i of the block, column l % 16
    for (int b = w; b < MB * NB; b += kL8Waves) {
        const int mb = b / NB, nb = b % NB;
        f32x4_l r = part[0][b][lane];
#pragma unroll
        for (int v = 1; v < kL8Waves; v++) r += part[v][b][lane];
        const int c = c0 + 16 * nb + l16;
        if (c < ng) {
            const int n = g * ng + c;
            const float sc = a.scale[n];
            const SegSel sg = lin_seg(a, n);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t m = 16 * mb + 4 * q + i;
                if (m < a.M) lin_store(sg, m, n, r[i] * sc);
            }
        }
    }
}

// ---- decode, M <= 32: the weight stream through LDS
// The same products as above (16 output columns per workgroup, the group
// width split over four waves, partial sums added in wave order), with the
// weights copied global -> LDS (non-temporal: nothing re-reads them) in runs
// of 128 bytes per row: one 2 KB slab = 16 rows x 2 double steps per wave,
// two slabs in flight per wave, each wave on a ring of its own, so no barrier
// in the loop.  A plain 16-byte load per lane in the matrix-core layout would
// touch only 64 bytes of each row per instruction.  Slab row r keeps its
// chunks (16 bytes) in a permuted order (st_swz) so that the fragment reads
// of the 16 rows hit 16 different bank groups.  The activation fragments of
// slab s + 1 are loaded while slab s is multiplied, through a buffer
// resource: rows past M read as zero without touching memory.  Load order
// per iteration: activations of slab s + 1, then the weight copies of slab
// s + 2.  (Measured on the 4-row, 7168 x 33,604 input projection: 128-byte
// runs with six workgroups per CU beat 256-byte runs with three.)
constexpr int kStSD = 2;                        // double steps per slab
constexpr int kStStages = 3;
constexpr int kStMaxMB = 2;
constexpr int64_t kLinStreamMaxM = 16 * kStMaxMB;

// slot permutation of a slab row (CPR chunks): the fragment reads of rows
// 0..15 at one chunk land in 16 different 16-byte bank groups
template <int CPR>
__device__ __forceinline__ int st_swz(int r) { return (r * CPR / 16) % CPR; }

template <int MB, int NW>
__global__ __launch_bounds__(64 * NW) void k_lin8_stream(LinArgs a) {
    constexpr int SD = kStSD, ST = kStStages;
    constexpr int kCPR = 4 * SD;                 // 16-byte chunks per slab row
    constexpr int kNI = SD;                      // 1 KB copies per slab
    constexpr int kSlab = 1024 * kNI;
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][ST][kSlab];
    static_assert(sizeof(f32x4_l) * NW * MB * 64 <= sizeof(ring), "partial sums reuse the ring");
    const int ng = a.N / a.G, kg = a.K / a.G;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tiles = (ng + 15) / 16;
    const int g = (int)(blockIdx.x / tiles), c0 = (int)(blockIdx.x % tiles) * 16;
    const int l16 = lane & 15, q = lane >> 4;
    const int nds = kg / 64, per = (nds + NW - 1) / NW;
    const int d0 = min(nds, w * per), d1 = min(nds, d0 + per);
    const int nsl = (d1 - d0 + SD - 1) / SD;
    // copy i of a slab fills slots 64 i + lane: slab row r = slot / kCPR gets
    // its chunk c = (slot % kCPR) ^ swz(r) (double step c / 4, 16-byte part
    // c % 4); swz spreads the fragment reads of the 16 rows over 16 bank groups
    const uint8_t* wsrc[kNI];
    int wdu[kNI];
#pragma unroll
    for (int i = 0; i < kNI; i++) {
        const int slot = 64 * i + lane, r = slot / kCPR, c = (slot % kCPR) ^ st_swz<kCPR>(r);
        const int n = min(c0 + r, ng - 1);
        wsrc[i] = a.W + ((size_t)g * ng + n) * kg + 16 * (c & 3);
        wdu[i] = c >> 2;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int sl, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kNI; i++) {
            const int ds = min(d0 + sl * SD + wdu[i], d1 - 1);
            __builtin_amdgcn_global_load_lds(wsrc[i] + (size_t)ds * 64, (lds_void*)(&ring[w][buf][0] + 1024 * i), 16,
                                             0, 2);                // non-temporal
        }
    };
    // activations through a buffer resource over x (M K bf16, below 2 GiB:
    // checked by the launcher); a row past M gets an offset past the end and
    // reads zero, with no memory access and no branch
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, (int)(a.M * a.K * 2), 0x00020000);
    bf16x8_l af[2][MB][SD][2];
    auto load_act = [&](int sl, bf16x8_l (&dst)[MB][SD][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int mb = 0; mb < MB; mb++) {
            const int m = 16 * mb + l16;
#pragma unroll
            for (int u = 0; u < SD; u++) {
                // a double step past the range re-reads the last one (it meets
                // zero weights below)
                const int ds = min(d0 + sl * SD + u, d1 - 1);
                const int off = m < a.M ? 2 * (m * a.K + g * kg + ds * 64 + 16 * q) : 0x7FFFFFF0;
                dst[mb][u][0] = __builtin_bit_cast(bf16x8_l, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
                dst[mb][u][1] = __builtin_bit_cast(bf16x8_l, __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16, 0, 0));
            }
        }
    };
    f32x4_l acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; mb++) acc[mb] = f32x4_l{0.0f, 0.0f, 0.0f, 0.0f};
    // Every step issues its loads unconditionally (addresses clamped to the
    // wave's last valid slab, whose re-reads hit L2), so the loop is straight
    // code; a slab past the range meets zero weights.  Then the only loads
    // issued after slab s's activations are the copies of slab s + 1, and
    // vmcnt(copies per slab) is exact.
    int buf = 0;
    if (nsl > 0) {
        issue(0, 0);
        load_act(0, af[0]);
#pragma unroll
        for (int b = 1; b < ST - 1; b++) issue(b, b);
    }
    // one slab: af_cur holds its activations, af_nxt receives the next slab's
    auto step = [&](int sl, bf16x8_l (&af_cur)[MB][SD][2], bf16x8_l (&af_nxt)[MB][SD][2])
        __attribute__((always_inline)) {
        // nothing of the previous slab may move below this point: the
        // scheduler would otherwise hoist the wait above its products
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70 | kNI);                   // vmcnt: only the copies of slab s + 1 in flight
        load_act(sl + 1, af_nxt);
        // the copies of slab s + 2 overwrite the buffer of slab s - 1: its
        // fragment reads must have completed (the compiler may interleave
        // them with this step)
        __builtin_amdgcn_s_waitcnt(0xC07F);                         // lgkmcnt(0)
        issue(sl + ST - 1, buf == 0 ? ST - 1 : buf - 1);
        const uint8_t* base = &ring[w][buf][0];
#pragma unroll
        for (int u = 0; u < SD; u++) {
            // a double step past the wave's range (its copies re-read the last
            // valid step) multiplies zero weights
            const bool live = d0 + sl * SD + u < d1;
            v4u_l fw = *reinterpret_cast<const v4u_l*>(base + 16 * (kCPR * l16 + ((4 * u + q) ^ st_swz<kCPR>(l16))));
            fw = live ? fw : v4u_l{0u, 0u, 0u, 0u};
            const bf16x8_l b0 = e4m3x8_to_bf16x8(fw[0], fw[1]);
            const bf16x8_l b1 = e4m3x8_to_bf16x8(fw[2], fw[3]);
#pragma unroll
            for (int mb = 0; mb < MB; mb++) {
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af_cur[mb][u][0], b0, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af_cur[mb][u][1], b1, acc[mb], 0, 0, 0);
            }
        }
        buf = buf == ST - 1 ? 0 : buf + 1;
    };
    // two slabs per trip, so the activation buffers are named statically
    for (int sl = 0; sl < nsl; sl += 2) {
        step(sl, af[0], af[1]);
        step(sl + 1, af[1], af[0]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);                              // drain the trailing copies
    __syncthreads();                             // every wave is done with its ring
    f32x4_l (*part)[MB][64] = reinterpret_cast<f32x4_l (*)[MB][64]>(&ring[0][0][0]);
#pragma unroll
    for (int mb = 0; mb < MB; mb++) part[w][mb][lane] = acc[mb];
    __syncthreads();
    // wave v finishes row block v (lane l: rows 4 (l / 16) + i, column l % 16)
    for (int mb = w; mb < MB; mb += NW) {
        f32x4_l r = part[0][mb][lane];
#pragma unroll
        for (int v = 1; v < NW; v++) r += part[v][mb][lane];
        const int c = c0 + l16;
        if (c < ng) {
            const int n = g * ng + c;
            const float sc = a.scale[n];
            const SegSel sg = lin_seg(a, n);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t m = 16 * mb + 4 * q + i;
                if (m < a.M) lin_store(sg, m, n, r[i] * sc);
            }
        }
    }
}

// ---- prefill: 256 x 128 tiles on the matrix cores (M > 64)
// Slab = 32 reduction indices: the activation part is 256 rows x 64 bytes
// (bf16), the weight part 128 rows x 32 bytes (E4M3), both copied straight
// from global memory into LDS (global_load_lds_dwordx4), three slabs in
// flight.  K-mapping inside a slab: lane half h = lane / 32 owns indices
// 16 h .. 16 h + 15; the first product of the slab takes the lower eight, the
// second the upper eight.  So a lane's weight fragment of one 32-column block
// is one 16-byte LDS read (both products), widened to bf16 in registers.
// Activation rows: chunk c (16 bytes) of row r sits in slot c ^ ((r >> 1) & 3)
// of the row; weight rows: chunk c in slot c ^ (((r >> 2) ^ (r >> 3)) & 1),
// so the fragment reads of 16 consecutive rows spread over the banks.
constexpr int kL8BM = 256, kL8BN = 128, kL8BK = 32;
constexpr int kL8Threads = 256;
constexpr int kL8Stages = 3;
constexpr int kL8Aq = kL8BM * kL8BK * 2 / 16 / kL8Threads;   // 16-byte activation copies per thread and slab (4)
constexpr int kL8Bq = kL8BN * kL8BK / 16 / kL8Threads;       // 16-byte weight copies per thread and slab (1)
constexpr int kL8ABytes = kL8BM * kL8BK * 2;
constexpr int kL8SlabBytes = kL8ABytes + kL8BN * kL8BK;
static_assert(kL8Aq == 4 && kL8Bq == 1, "copy plan is written for 256 threads");

__device__ __forceinline__ int l8_aslot(int r, int c) { return 4 * r + (c ^ ((r >> 1) & 3)); }
__device__ __forceinline__ int l8_bslot(int r, int c) { return 2 * r + (c ^ (((r >> 2) ^ (r >> 3)) & 1)); }

__global__ __launch_bounds__(kL8Threads, 2) void k_lin8_mfma(LinArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t sm[kL8Stages][kL8SlabBytes];
    const int ng = a.N / a.G, kg = a.K / a.G;
    const int tiles_n = (ng + kL8BN - 1) / kL8BN;
    const int64_t tiles_m = (a.M + kL8BM - 1) / kL8BM;
    // XCD-aware deal (the dispatcher hands workgroups to the 8 XCDs
    // round-robin): each XCD gets a contiguous run of tiles, n fastest, so
    // neighbouring tiles share their activation rows in that XCD's L2
    const int64_t id = blockIdx.x, nwg = gridDim.x, per = nwg / 8;
    const int64_t L = id < 8 * per ? (id % 8) * per + id / 8 : id;
    const int tn = (int)(L % tiles_n);
    const int64_t tm = (L / tiles_n) % tiles_m;
    const int g = (int)(L / tiles_n / tiles_m);
    const int64_t m0 = tm * kL8BM;
    const int n0 = tn * kL8BN;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;
    const uint16_t* x = a.x + (size_t)g * kg;
    const uint8_t* W = a.W + (size_t)g * ng * kg;
    // copy q of wave w fills 16-byte slots [64 (4 q + w), +64) of the
    // activation part; the weight copy fills slots [64 w, +64) of its part
    const uint16_t* ap[kL8Aq];
#pragma unroll
    for (int q = 0; q < kL8Aq; q++) {
        const int sl = 64 * (4 * q + w) + lane, r = sl >> 2;
        const int c = (sl & 3) ^ ((r >> 1) & 3);
        ap[q] = x + (size_t)min(m0 + r, a.M - 1) * a.K + 8 * c;
    }
    const uint8_t* bp;
    {
        const int sl = 64 * w + lane, r = sl >> 1;
        const int c = (sl & 1) ^ (((r >> 2) ^ (r >> 3)) & 1);
        bp = W + (size_t)min(n0 + r, ng - 1) * kg + 16 * c;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto issue = [&](int s, int buf) __attribute__((always_inline)) {
        uint8_t* base = &sm[buf][0];
#pragma unroll
        for (int q = 0; q < kL8Aq; q++)
            __builtin_amdgcn_global_load_lds(ap[q] + s * kL8BK, (lds_void*)(base + 1024 * (4 * q + w)), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(bp + s * kL8BK, (lds_void*)(base + kL8ABytes + 1024 * w), 16, 0, 0);
    };
    f32x16_l acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    auto compute = [&](int buf) __attribute__((always_inline)) {
        const uint8_t* base = &sm[buf][0];
        bf16x8_l fa[2][2];
        v4u_l fw[4];
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
            for (int i = 0; i < 2; i++)
                fa[kk][i] = *reinterpret_cast<const bf16x8_l*>(base + 16 * l8_aslot(64 * w + 32 * i + l32, 2 * hl + kk));
#pragma unroll
        for (int j = 0; j < 4; j++)
            fw[j] = *reinterpret_cast<const v4u_l*>(base + kL8ABytes + 16 * l8_bslot(32 * j + l32, hl));
        asm volatile("" : "+v"(fa[0][0]), "+v"(fa[0][1]), "+v"(fa[1][0]), "+v"(fa[1][1]), "+v"(fw[0]), "+v"(fw[1]),
                     "+v"(fw[2]), "+v"(fw[3]));
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const bf16x8_l b0 = e4m3x8_to_bf16x8(fw[j][0], fw[j][1]);
            const bf16x8_l b1 = e4m3x8_to_bf16x8(fw[j][2], fw[j][3]);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][i], b0, acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][i], b1, acc[i][j], 0, 0, 0);
            }
        }
    };
    // slab s lives in buffer s % 3: each thread waits for its own copies of
    // slab s (those of slab s + 1 stay in flight), the barrier publishes every
    // thread's copies and frees the buffer of slab s - 1 for slab s + 2
    const int ns = kg / kL8BK;
    issue(0, 0);
    if (ns > 1) issue(1, 1);
    int buf = 0, buf2 = 2;
    for (int s = 0; s < ns; s++) {
        if (s + 1 < ns) __builtin_amdgcn_s_waitcnt(0x0F70 | (kL8Aq + kL8Bq));   // vmcnt(copies per slab)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                               // vmcnt(0)
        __syncthreads();
        if (s + 2 < ns) issue(s + 2, buf2);
        compute(buf);
        buf = buf == kL8Stages - 1 ? 0 : buf + 1;
        buf2 = buf2 == kL8Stages - 1 ? 0 : buf2 + 1;
    }
    // accumulator (i, j) element e: row 8 (e / 4) + 4 hl + e % 4, column l32
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int c = n0 + 32 * j + l32;
        if (c >= ng) continue;
        const int n = g * ng + c;
        const float sc = a.scale[n];
        const SegSel sg = lin_seg(a, n);
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int64_t m = m0 + 64 * w + 32 * i + 8 * (e / 4) + 4 * hl + (e % 4);
                if (m < a.M) lin_store(sg, m, n, acc[i][j][e] * sc);
            }
    }
}

// ---- FP4 quantisation of f32 rows (the indexer queries): one wave per row
// of n <= 256 values (a multiple of 32); blocks of 32 values get
// e = floor(log2 amax) - 2, raised to at least (row max e) - 14 and clamped to
// [-127, 127]; all-zero rows take e = 0; codes are the nearest E2M1 of
// x 2^-e, ties to even, saturating at +-6 (the indexer-key rule)
__global__ __launch_bounds__(256) void k_fp4_rows(const float* x, int64_t rows, int n, uint8_t* codes, uint8_t* scales) {
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int nb = n / 32;
    float v[4];
    int eb[4];
    int emax = INT32_MIN;
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int k = lane + 64 * t;
        v[t] = k < n ? x[row * n + k] : 0.0f;
        float bm = fabsf(v[t]);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 64));
        int e = INT32_MIN;
        if (k < n && bm > 0.0f) {
            int ex;
            frexpf(bm, &ex);                              // bm in [2^(ex-1), 2^ex)
            e = ex - 1 - 2;
        }
        eb[t] = e;
        emax = max(emax, e);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) emax = max(emax, __shfl_xor(emax, o, 64));
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const int k = lane + 64 * t;
        int e = emax == INT32_MIN ? 0 : max(eb[t], emax - 14);
        e = min(max(e, -127), 127);
        if (k < n && (k & 31) == 0) scales[row * nb + (k >> 5)] = (uint8_t)(e + 127);
        const uint32_t code = k < n ? f32_to_e2m1(ldexpf(v[t], -e)) : 0u;
        const uint32_t hi = __shfl_xor(code, 1, 64);
        if (k < n && (k & 1) == 0) codes[row * (n / 2) + (k >> 1)] = (uint8_t)(code | (hi << 4));
    }
}

hipError_t launch_fp4_rows(const float* x, int64_t rows, int n, uint8_t* codes, uint8_t* scales, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fp4_rows, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, x, rows, n, codes, scales);
    return hipGetLastError();
}

template <int MB, int NB, int KB>
static void launch_skinny(const LinArgs& a, hipStream_t st) {
    const int ng = a.N / a.G;
    const unsigned grid = (unsigned)((int64_t)a.G * ((ng + 16 * NB - 1) / (16 * NB)));
    hipLaunchKernelGGL((k_lin8_skinny<MB, NB, KB>), dim3(grid), dim3(64 * kL8Waves), 0, st, a);
}

hipError_t launch_lin8(const LinArgs& a, hipStream_t st) {
    if (a.M == 0) return hipSuccess;
    if (a.M <= kLinStreamMaxM && a.M * a.K * 2 < ((int64_t)1 << 31)) {
        const int ng = a.N / a.G;
        const unsigned grid = (unsigned)((int64_t)a.G * ((ng + 15) / 16));
        // (splitting the group width over eight waves for small grids was
        // measured slower on the 32768 -> 7168 grouped projection)
        if (a.M <= 16) hipLaunchKernelGGL((k_lin8_stream<1, kL8Waves>), dim3(grid), dim3(64 * kL8Waves), 0, st, a);
        else hipLaunchKernelGGL((k_lin8_stream<2, kL8Waves>), dim3(grid), dim3(64 * kL8Waves), 0, st, a);
    } else if (a.M <= kLinSkinnyMaxM) launch_skinny<4, 2, 2>(a, st);
    else {
        const int ng = a.N / a.G;
        const int64_t tiles = (int64_t)a.G * ((a.M + kL8BM - 1) / kL8BM) * ((ng + kL8BN - 1) / kL8BN);
        hipLaunchKernelGGL(k_lin8_mfma, dim3((unsigned)tiles), dim3(kL8Threads), 0, st, a);
    }
    return hipGetLastError();
}

int64_t lin8_max_tiles(int64_t M, int32_t N, int32_t G) {
    const int ng = N / G;
    return (int64_t)G * ((M + kL8BM - 1) / kL8BM) * ((ng + kL8BN - 1) / kL8BN);
}

}  // namespace csa
