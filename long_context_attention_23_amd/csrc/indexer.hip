// indexer.hip -- csa_indexer_topk: lightning-indexer scores and exact top-k.
//
// Method: "DeepSeek-V4 ... open-source declaration" (peacm.com) section 3.2,
// CSA step 2 (a lightweight indexer scores every query against the compressed
// blocks and the top-k blocks are kept); "technical report digest" section
// 3.2 (the indexer QK path in FP4 E2M1 with 1x32 scales).  Reading of the
// score: S_j = sum_h w_h * ReLU(<q_h, k_j>); of the selection: largest S,
// ties to the smaller block index, output in ascending block order.
//
// Exactness.  Scores are fp32; selection compares the 64-bit composite
// (order-preserving score key, inverted block index), which is unique per
// block, so "the k largest composites" is exactly the specified set.
//
// Small path (<= 4096 visible keys, e.g. prefill of a short context): one
//   workgroup per query row keeps every score in LDS, radix-selects in LDS and
//   emits the set by a j-ordered compaction.
// Large path (decode against 10^5..10^6 keys): after a kernel that clears
//   each row's histogram and counters, three kernels over key chunks and rows --
//   A  score + 4096-bin LDS histogram of the top 12 key bits, merged into a
//      per-row global histogram with integer atomics;
//   C  every chunk finds the threshold bin from that histogram and appends
//      keys above it to the row's "selected" list and keys in it to the
//      "candidate" list (wave-aggregated appends);
//   D  one workgroup per row finds the threshold score suffix among the
//      candidates (two 10-bit digit passes, skipped when all candidates share
//      one key), takes the tied ones at it by smallest block index, and emits
//      the k blocks in ascending order from LDS bitmaps (rows with more than
//      2^18 visible blocks: composite radix select and a bitonic sort).  The
//      append order of A/C does not matter: D's result depends only on the
//      sets.
// Prefill path (chunks of query rows): see the section further down.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kIdxThreads = 256;
constexpr int kIdxFinalThreads = 1024;
constexpr int kMaxHi = 16;
constexpr int kMaxDi = 256;

// ------------------------------------------------------------------ scoring
// decode 8 consecutive values [k0, k0+8) of an indexer row
template <int FMT>
__device__ __forceinline__ void load8(const uint8_t* row, const uint8_t* scales, int k0, float* v) {
    if constexpr (FMT == CSA_F32) {
        const float4* p = reinterpret_cast<const float4*>(row + 4 * k0);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else if constexpr (FMT == CSA_BF16) {
        uint4 a = *reinterpret_cast<const uint4*>(row + 2 * k0);
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {  // FP4: 8 codes in 4 bytes, one scale per 32 values
        uint32_t c = *reinterpret_cast<const uint32_t*>(row + k0 / 2);
        float s = e8m0_to_f32(scales[k0 / 32]);
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = e2m1_to_f32((c >> (4 * i)) & 15u) * s;
    }
}

__host__ __device__ constexpr int row_bytes(int fmt, int di) {
    return fmt == CSA_F32 ? 4 * di : fmt == CSA_BF16 ? 2 * di : di / 2;
}

// decode the query's Hi indexer rows into LDS as qs[k][h] (Hi contiguous per dim)
template <int QF>
__device__ void stage_query(const IndexerArgs& a, int64_t row, float* qs, float* ws) {
    const int di = a.di, Hi = a.Hi;
    const int rb = row_bytes(QF, di);
    for (int idx = threadIdx.x; idx < Hi * (di / 8); idx += blockDim.x) {
        int h = idx / (di / 8), k0 = (idx % (di / 8)) * 8;
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + (row * Hi + h) * rb;
        const uint8_t* qsc = a.q_scales ? a.q_scales + (row * Hi + h) * (di / 32) : nullptr;
        float v[8];
        load8<QF>(qrow, qsc, k0, v);
#pragma unroll
        for (int u = 0; u < 8; u++) qs[(k0 + u) * kMaxHi + h] = v[u];
    }
    for (int h = threadIdx.x; h < Hi; h += blockDim.x) ws[h] = a.w[row * Hi + h];
}

// S_j for one key row, fp32, dims in order then heads in order
template <int KF>
__device__ __forceinline__ float score_one(const IndexerArgs& a, const uint8_t* krow, const uint8_t* ksc,
                                           const float* qs, const float* ws) {
    float acc[kMaxHi];
#pragma unroll
    for (int h = 0; h < kMaxHi; h++) acc[h] = 0.0f;
    for (int k0 = 0; k0 < a.di; k0 += 8) {
        float v[8];
        load8<KF>(krow, ksc, k0, v);
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const float* qk = qs + (k0 + u) * kMaxHi;
#pragma unroll
            for (int h = 0; h < kMaxHi; h++)
                if (h < a.Hi) acc[h] = fmaf(qk[h], v[u], acc[h]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < kMaxHi; h++)
        if (h < a.Hi) s = fmaf(ws[h], fmaxf(acc[h], 0.0f), s);
    return s;
}

__device__ __forceinline__ int64_t visible_from(const IndexerArgs& a, int64_t t) {
    const int64_t n = t < 0 ? 0 : (t + 1) / a.m;
    return n < a.cap ? n : a.cap;
}
__device__ __forceinline__ int64_t visible_blocks(const IndexerArgs& a, int64_t row) {
    return visible_from(a, load_uniform_i32(a.q_pos + row));
}

// ------------------------------------------------------------------ radix helpers
// Find, in a 256-bin histogram (descending digit order), the digit whose
// cumulative count from the top first reaches `need`.  Executed by one full
// wave; returns (digit, count strictly above it) in every lane.
__device__ __forceinline__ void wave_pick_digit(const uint32_t* hist, uint32_t need, uint32_t& digit,
                                                uint32_t& above) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t h4[4], s = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) { h4[q] = hist[255 - 4 * lane - q]; s += h4[q]; }
    uint32_t incl = s;
    incl = wave_incl_scan_dpp(incl);
    uint64_t bal = __ballot(incl >= need);
    int L = bal ? __builtin_ctzll(bal) : kWave - 1;
    uint32_t cum = lane_u32(incl - s, L);
    uint32_t d = 0, ab = cum;
    if (lane == L) {
        uint32_t c = cum;
        d = 255 - 4 * L - 3;
        ab = c;
        for (int q = 0; q < 4; q++) {
            if (c + h4[q] >= need) { d = 255 - 4 * L - q; ab = c; break; }
            c += h4[q];
        }
    }
    digit = lane_u32(d, L);
    above = lane_u32(ab, L);
}

// Radix select over n composites get(i) (nbits significant bits): returns the
// composite of the need-th largest.  Block-wide; hist is LDS [256], sh LDS [4].
template <typename Get>
__device__ __forceinline__ uint64_t radix_select(Get get, int64_t n, int nbits, uint32_t need, uint32_t* hist, uint32_t* sh) {
    uint64_t prefix = 0, pmask = 0;
    for (int shift = ((nbits + 7) / 8) * 8 - 8; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        for (int64_t i0 = 0; i0 < n; i0 += blockDim.x) {
            // the whole block runs every round, so each wave's ballots are complete
            const int64_t i = i0 + threadIdx.x;
            const uint64_t c = i < n ? get(i) : 0;
            const bool in = i < n && (c & pmask) == prefix;
            const uint32_t dg = (uint32_t)(c >> shift) & 255u;
            // many equal digits (tied scores) would serialise on one LDS
            // address: a wave whose lanes mostly agree adds per distinct digit
            const uint64_t act = __ballot(in);
            const uint32_t d0 = lane_u32(dg, act ? __builtin_ctzll(act) : 0);
            if (__popcll(__ballot(in && dg == d0)) > 8) {
                uint64_t todo = act;
                while (todo) {
                    const int leader = __builtin_ctzll(todo);
                    const uint32_t dl = lane_u32(dg, leader);
                    const uint64_t same = __ballot(in && dg == dl) & todo;
                    if ((int)(threadIdx.x & (kWave - 1)) == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
                    todo &= ~same;
                }
            } else if (in) {
                atomicAdd(&hist[dg], 1u);
            }
        }
        __syncthreads();
        if (threadIdx.x < kWave) {
            uint32_t dg, ab;
            wave_pick_digit(hist, need, dg, ab);
            if (threadIdx.x == 0) { sh[0] = dg; sh[1] = ab; }
        }
        __syncthreads();
        prefix |= (uint64_t)sh[0] << shift;
        pmask |= (uint64_t)255u << shift;
        need -= sh[1];
        __syncthreads();
    }
    return prefix;
}

__device__ __forceinline__ int bits_for(int64_t n) {   // bits to hold values 0..n-1 (>= 1)
    int b = 1;
    while (b < 62 && ((int64_t)1 << b) < n) b++;
    return b;
}

// ------------------------------------------------------------------ small path
template <int QF, int KF>
__global__ __launch_bounds__(kIdxThreads) void k_idx_small(IndexerArgs a) {
    __shared__ float qs[kMaxDi * kMaxHi];
    __shared__ float ws[kMaxHi];
    __shared__ uint32_t keys[kIdxSmallMaxKeys];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t wcount[kIdxThreads / kWave];

    const int64_t row = blockIdx.x;
    const int64_t b = row / a.Tq;
    const int64_t n = visible_blocks(a, row);
    int32_t* out = a.out + row * a.topk;
    stage_query<QF>(a, row, qs, ws);
    __syncthreads();
    const int rb = row_bytes(KF, a.di);
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x) {
        const uint8_t* krow = a.keys + (b * a.cap + j) * rb;
        const uint8_t* ksc = a.key_scales ? a.key_scales + (b * a.cap + j) * (a.di / 32) : nullptr;
        keys[j] = score_key(score_one<KF>(a, krow, ksc, qs, ws));
    }
    __syncthreads();

    uint64_t thr = 0;                 // every composite >= thr is selected
    const int jb = bits_for(n);
    const uint64_t jmask = ((uint64_t)1 << jb) - 1;
    if (n > a.topk) {
        auto get = [&](int64_t i) -> uint64_t { return ((uint64_t)keys[i] << jb) | (jmask - (uint64_t)i); };
        thr = radix_select(get, n, 32 + jb, (uint32_t)a.topk, hist, sh);
    }
    // j-ordered compaction of the selected set
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    int base = 0;
    for (int64_t j0 = 0; j0 < n; j0 += blockDim.x) {
        int64_t j = j0 + threadIdx.x;
        bool sel = false;
        if (j < n) sel = ((((uint64_t)keys[j]) << jb) | (jmask - (uint64_t)j)) >= thr;
        uint64_t bal = __ballot(sel);
        if (lane == 0) wcount[wv] = __popcll(bal);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wv; w++) off += wcount[w];
        int tot = 0;
        for (int w = 0; w < (int)(blockDim.x / kWave); w++) tot += wcount[w];
        if (sel) out[off + __popcll(bal & ((1ull << lane) - 1))] = (int32_t)j;
        base += tot;
        __syncthreads();
    }
    for (int i = base + threadIdx.x; i < a.topk; i += blockDim.x) out[i] = -1;
}

// ------------------------------------------------------------------ large path
struct RowWs {
    uint32_t* hist;     // [4096]
    uint32_t* counts;   // [0] selected, [1] candidates
    uint32_t* scores;   // [cap]
    int32_t* sel;       // [topk]
    uint2* cand;        // [cap] (key, j)
};

__device__ __forceinline__ RowWs row_ws(const IndexerArgs& a, int64_t r) {
    uint8_t* base = a.ws + r * a.ws_row_bytes;
    RowWs w;
    w.hist = reinterpret_cast<uint32_t*>(base);
    w.counts = w.hist + kIdxHistBins;
    w.scores = w.counts + 4;
    w.sel = reinterpret_cast<int32_t*>(w.scores + a.cap);
    size_t off = (size_t)(kIdxHistBins + 4) * 4 + (size_t)a.cap * 4 + (size_t)a.topk * 4;
    off = (off + 15) & ~(size_t)15;
    w.cand = reinterpret_cast<uint2*>(base + off);
    return w;
}

int64_t idx_ws_row_bytes(int64_t cap, int32_t topk) {
    int64_t off = (int64_t)(kIdxHistBins + 4) * 4 + cap * 4 + (int64_t)topk * 4;
    off = (off + 15) & ~(int64_t)15;
    off += cap * 8;
    return (off + 255) & ~(int64_t)255;
}

__global__ void k_idx_zero(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    const int64_t r = blockIdx.x;
    uint32_t* p = reinterpret_cast<uint32_t*>(a.ws + r * a.ws_row_bytes);
    for (int i = threadIdx.x; i < kIdxHistBins + 4; i += blockDim.x) p[i] = 0;
}

template <int QF, int KF>
__global__ __launch_bounds__(kIdxThreads) void k_idx_score(IndexerArgs a) {
    __shared__ float qs[kMaxDi * kMaxHi];
    __shared__ float ws[kMaxHi];
    __shared__ uint32_t lh[kIdxHistBins];
    const int64_t r = blockIdx.y, row = a.row0 + r;
    const int64_t b = row / a.Tq;
    const int64_t n = visible_blocks(a, row);
    const int64_t c0 = (int64_t)blockIdx.x * kIdxChunk;
    if (n <= a.topk || c0 >= n) return;
    RowWs w = row_ws(a, r);
    stage_query<QF>(a, row, qs, ws);
    for (int i = threadIdx.x; i < kIdxHistBins; i += blockDim.x) lh[i] = 0;
    __syncthreads();
    const int rb = row_bytes(KF, a.di);
    const int64_t c1 = min(c0 + (int64_t)kIdxChunk, n);
    for (int64_t j = c0 + threadIdx.x; j < c1; j += blockDim.x) {
        const uint8_t* krow = a.keys + (b * a.cap + j) * rb;
        const uint8_t* ksc = a.key_scales ? a.key_scales + (b * a.cap + j) * (a.di / 32) : nullptr;
        uint32_t key = score_key(score_one<KF>(a, krow, ksc, qs, ws));
        w.scores[j] = key;
        atomicAdd(&lh[key >> 20], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kIdxHistBins; i += blockDim.x)
        if (lh[i]) atomicAdd(&w.hist[i], lh[i]);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_i __attribute__((ext_vector_type(8)));

constexpr int kIdxScoreThreads = 1024;  // 16 waves, four 32-key groups each (measured faster than 8 x 8)

// Score a chunk of 64-dim keys with the matrix cores.  C[head][key] = Q K^T:
// the query's Hi rows are the A operand (32 rows, rows >= Hi zero), 32 keys
// form the B operand, so accumulator lane l < 32 holds heads 0-3, 8-11, ...
// of key l and lane l + 32 heads 4-7, 12-15, ...; S = sum_h w_h ReLU(C[h][key])
// is completed with one lane exchange.
//   KF = FP4: v_mfma_scale_f32_32x32x64_f8f6f4 on E2M1 codes, the E8M0 block
//             scales applied by the instruction (one per 32 values);
//   KF = BF16: four v_mfma_f32_32x32x16_bf16 (queries FP4 or bf16, exact in bf16).
// Each wave loads kIdxMfmaBatch groups before computing them, to keep enough
// bytes in flight.
template <int QF, int KF>
__global__ __launch_bounds__(kIdxScoreThreads) void k_idx_score_mfma(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    constexpr int DI = 64;
    constexpr int NKS = KF == CSA_FP4_E2M1 ? 1 : 4;            // K steps per 32-key group
    // 32-key groups whose loads a wave issues before computing them
    constexpr int kIdxMfmaBatch = KF == CSA_FP4_E2M1 ? kIdxChunk / kIdxScoreThreads : 3;   // bf16: 4 would spill
    constexpr int KROW = KF == CSA_FP4_E2M1 ? DI / 2 : 2 * DI;  // key row bytes
    __shared__ uint32_t lh[kIdxHistBins];
    const int64_t r = blockIdx.y, row = a.row0 + r;
    const int64_t b = row / a.Tq;
    const int64_t c0 = (int64_t)blockIdx.x * kIdxChunk;
    RowWs ws = row_ws(a, r);
    for (int i = threadIdx.x; i < kIdxHistBins; i += blockDim.x) lh[i] = 0;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int l32 = lane & 31, half = lane >> 5;
    const int Hi = a.Hi;
    float wrow[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int h = 8 * (i / 4) + 4 * half + (i % 4);
        wrow[i] = h < Hi ? a.w[row * Hi + h] : 0.0f;
    }
    // A fragments: query row l32 (zero beyond Hi)
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(a.q) + row * Hi * row_bytes(QF, DI);
    i32x8_t qa4 = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    int qs4 = 127;
    bf16x8_i qab[NKS];
    if constexpr (KF == CSA_FP4_E2M1) {
        if (l32 < Hi) {
            const uint4 u = *reinterpret_cast<const uint4*>(qbase + (size_t)l32 * (DI / 2) + 16 * half);
            qa4[0] = (int)u.x; qa4[1] = (int)u.y; qa4[2] = (int)u.z; qa4[3] = (int)u.w;
            qs4 = a.q_scales[(row * Hi + l32) * (DI / 32) + half];
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) {
            float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if (l32 < Hi) {
                const uint8_t* qrow = qbase + (size_t)l32 * row_bytes(QF, DI);
                const uint8_t* qsc = a.q_scales ? a.q_scales + (row * Hi + l32) * (DI / 32) : nullptr;
                load8<QF>(qrow, qsc, 16 * ks + 8 * half, v);
            }
#pragma unroll
            for (int j = 0; j < 8; j++) qab[ks][j] = (__bf16)v[j];
        }
    }
    const uint8_t* kb = a.keys + (size_t)b * a.cap * KROW;
    const uint8_t* ksb = KF == CSA_FP4_E2M1 ? a.key_scales + (size_t)b * a.cap * (DI / 32) : nullptr;
    constexpr int kStride = 32 * (kIdxScoreThreads / 64);
    // key loads stay inside the cache's rows (cl); the first batch goes out
    // before the position arrives, and keys past the visible blocks (c1) are
    // scored but never stored or counted
    const int64_t cl = min(c0 + (int64_t)kIdxChunk, a.cap);
    uint4 kc[kIdxMfmaBatch][NKS];
    int ksc[kIdxMfmaBatch];
    auto load_batch = [&](int64_t gb) {
#pragma unroll
        for (int u = 0; u < kIdxMfmaBatch; u++) {
            const int64_t key = gb + (int64_t)u * kStride + l32;
            ksc[u] = 127;
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) kc[u][ks] = make_uint4(0u, 0u, 0u, 0u);
            if (key < cl) {
#pragma unroll
                for (int ks = 0; ks < NKS; ks++)
                    kc[u][ks] = *reinterpret_cast<const uint4*>(kb + key * KROW + 32 * ks + 16 * half);
                if constexpr (KF == CSA_FP4_E2M1) ksc[u] = ksb[key * (DI / 32) + half];
            }
        }
    };
    const int64_t gb0 = c0 + 32 * wv;
    load_batch(gb0);
    const int64_t n = visible_blocks(a, row);
    if (n <= a.topk || c0 >= n) return;
    __syncthreads();
    const int64_t c1 = min(c0 + (int64_t)kIdxChunk, n);
    for (int64_t gb = gb0; gb < c1; gb += (int64_t)kStride * kIdxMfmaBatch) {
        if (gb != gb0) load_batch(gb);
#pragma unroll
        for (int u = 0; u < kIdxMfmaBatch; u++) {
            const int64_t key = gb + (int64_t)u * kStride + l32;
            f32x16_t acc;
#pragma unroll
            for (int i = 0; i < 16; i++) acc[i] = 0.0f;
            if constexpr (KF == CSA_FP4_E2M1) {
                const i32x8_t kf = i32x8_t{(int)kc[u][0].x, (int)kc[u][0].y, (int)kc[u][0].z, (int)kc[u][0].w, 0, 0, 0, 0};
                acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa4, kf, acc, 4, 4, 0, qs4, 0, ksc[u]);
            } else {
#pragma unroll
                for (int ks = 0; ks < NKS; ks++)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qab[ks], __builtin_bit_cast(bf16x8_i, kc[u][ks]), acc, 0, 0, 0);
            }
            // rows 8 g + 4 half + (0..3) of group g hold heads; groups with no
            // head below Hi carry zero weights and are skipped (an fma with a
            // zero weight leaves the sum as it is), and with Hi <= 4 the upper
            // half of the wave holds no head at all
            float part = 0.0f;
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                if (8 * gq >= Hi) break;                          // wave-uniform
#pragma unroll
                for (int h = 0; h < 4; h++) part = fmaf(wrow[4 * gq + h], relu_bits(acc[4 * gq + h]), part);
            }
            const float sc = Hi > 4 ? part + __shfl_xor(part, 32, kWave) : part;
            if (half == 0 && key < c1) {
                const uint32_t k32 = score_key(sc);
                ws.scores[key] = k32;
                atomicAdd(&lh[k32 >> 20], 1u);
            }
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kIdxHistBins; i += blockDim.x)
        if (lh[i]) atomicAdd(&ws.hist[i], lh[i]);
}

// threshold bin of the 4096-bin histogram, computed by one wave
__device__ __forceinline__ void wave_pick_bin(const uint32_t* hist, uint32_t need, uint32_t& bin, uint32_t& above) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int per = kIdxHistBins / kWave;   // 64 bins per lane; lane 0 holds the top bins
    // this lane's bins [4096 - 64(lane+1), 4096 - 64 lane) with all loads in flight
    const uint4* hv = reinterpret_cast<const uint4*>(hist + kIdxHistBins - per * (lane + 1));
    uint4 v[per / 4];
#pragma unroll
    for (int i = 0; i < per / 4; i++) v[i] = hv[i];
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < per / 4; i++) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    uint32_t incl = s;
    incl = wave_incl_scan_dpp(incl);
    uint64_t bal = __ballot(incl >= need);
    int L = bal ? __builtin_ctzll(bal) : kWave - 1;
    const uint32_t cum = lane_u32(incl - s, L);
    // the bins of lane L, one per lane in descending bin order, prefix-summed
    const int bq = kIdxHistBins - 1 - per * L - lane;
    const uint32_t hb = hist[bq];
    uint32_t c = hb;
    c = wave_incl_scan_dpp(c);
    c += cum;
    const uint64_t hit = __ballot(c >= need);
    const int q = hit ? __builtin_ctzll(hit) : kWave - 1;
    bin = (uint32_t)lane_u32(bq, q);
    above = lane_u32(c - hb, q);
}

__global__ __launch_bounds__(kIdxThreads) void k_idx_collect(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    constexpr int kWaves = kIdxThreads / kWave;
    __shared__ uint32_t sh[2];
    __shared__ uint32_t wcnt[2][kWaves], base[2];
    const int64_t r = blockIdx.y, row = a.row0 + r;
    const int64_t c0 = (int64_t)blockIdx.x * kIdxChunk;
    RowWs w = row_ws(a, r);
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    constexpr int kPer = kIdxChunk / kIdxThreads;
    // every load goes out before the position is needed (they stay inside the
    // row's workspace; scores past the visible blocks are never used): the
    // chunk's scores, the position, and wave 0's bin search over the histogram
    const int64_t cl = min(c0 + (int64_t)kIdxChunk, a.cap);
    uint32_t keys[kPer];
#pragma unroll
    for (int u = 0; u < kPer; u++) {
        const int64_t j = c0 + (int64_t)u * kIdxThreads + threadIdx.x;
        keys[u] = j < cl ? w.scores[j] : 0u;
    }
    const int32_t tpos = load_uniform_i32(a.q_pos + row);
    if (threadIdx.x < kWave) {
        uint32_t bin, above;
        wave_pick_bin(w.hist, (uint32_t)a.topk, bin, above);
        if (threadIdx.x == 0) { sh[0] = bin; sh[1] = above; }
    }
    const int64_t n = visible_from(a, tpos);
    if (n <= a.topk || c0 >= n) return;
    const int64_t c1 = min(c0 + (int64_t)kIdxChunk, n);
    __syncthreads();
    const uint32_t tbin = sh[0];
    // per-wave counts of the two lists, one global reservation per list for
    // the workgroup, then slots in (wave, round, lane) order
    uint32_t kind = 0;                                   // bit u: 1 = sure, bit u+16: candidate
    uint32_t ns = 0, nc = 0;
#pragma unroll
    for (int u = 0; u < kPer; u++) {
        const int64_t j = c0 + (int64_t)u * kIdxThreads + threadIdx.x;
        const uint32_t bin = keys[u] >> 20;
        const bool sure = j < c1 && bin > tbin;
        const bool cand = j < c1 && bin == tbin;
        ns += (uint32_t)__popcll(__ballot(sure));
        nc += (uint32_t)__popcll(__ballot(cand));
        kind |= (sure ? 1u : 0u) << u;
        kind |= (cand ? 1u : 0u) << (u + 16);
    }
    if (lane == 0) { wcnt[0][wv] = ns; wcnt[1][wv] = nc; }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t ts = 0, tc = 0;
        for (int q = 0; q < kWaves; q++) { ts += wcnt[0][q]; tc += wcnt[1][q]; }
        base[0] = ts ? atomicAdd(&w.counts[0], ts) : 0u;
        base[1] = tc ? atomicAdd(&w.counts[1], tc) : 0u;
    }
    __syncthreads();
    uint32_t os = base[0], oc = base[1];
    for (int q = 0; q < wv; q++) { os += wcnt[0][q]; oc += wcnt[1][q]; }
    const uint64_t below = (1ull << lane) - 1;
#pragma unroll
    for (int u = 0; u < kPer; u++) {
        const int64_t j = c0 + (int64_t)u * kIdxThreads + threadIdx.x;
        const bool sure = (kind >> u) & 1u, cand = (kind >> (u + 16)) & 1u;
        const uint64_t bs = __ballot(sure), bc = __ballot(cand);
        if (sure) w.sel[os + __popcll(bs & below)] = (int32_t)j;
        if (cand) w.cand[oc + __popcll(bc & below)] = make_uint2(keys[u], (uint32_t)j);
        os += (uint32_t)__popcll(bs);
        oc += (uint32_t)__popcll(bc);
    }
}

constexpr int kIdxBitmapWords = 8192;    // words per LDS bitmap of blocks (caps up to 2^18)
constexpr int kIdxFinalLds = 4096;       // candidates held in registers across the digit passes
constexpr int kIdxDigitBins = 1024;      // 10-bit digits of the 20-bit score suffix
constexpr int kIdxCandPerThread = kIdxFinalLds / kIdxFinalThreads;
constexpr int kIdxWordsPerThread = kIdxBitmapWords / kIdxFinalThreads;
constexpr int kIdxSelPerThread = kIdxMaxTopk / kIdxFinalThreads;
// the large path runs only above kIdxSmallMaxKeys keys, so a row's candidate
// buffer (one entry per key) always holds kIdxFinalLds entries
static_assert(kIdxFinalLds <= kIdxSmallMaxKeys, "speculative candidate loads must stay in the buffer");

// wave_pick_digit over 1024 bins (16 per lane, lane 0 holding the top ones)
__device__ __forceinline__ void wave_pick_digit1024(const uint32_t* hist, uint32_t need, uint32_t& digit,
                                                    uint32_t& above) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int per = kIdxDigitBins / kWave;
    uint32_t h[per], s = 0;
#pragma unroll
    for (int q = 0; q < per; q++) { h[q] = hist[kIdxDigitBins - 1 - per * lane - q]; s += h[q]; }
    uint32_t incl = s;
    incl = wave_incl_scan_dpp(incl);
    const uint64_t bal = __ballot(incl >= need);
    const int L = bal ? __builtin_ctzll(bal) : kWave - 1;
    const uint32_t cum = lane_u32(incl - s, L);
    uint32_t d = 0, ab = cum;
    if (lane == L) {
        uint32_t c = cum;
        d = kIdxDigitBins - per * (L + 1);
        for (int q = 0; q < per; q++) {
            if (c + h[q] >= need) { d = kIdxDigitBins - 1 - per * L - q; ab = c; break; }
            c += h[q];
        }
    }
    digit = lane_u32(d, L);
    above = lane_u32(ab, L);
}

// one round of a 10-bit digit histogram: (key >> shift) & 1023 of the
// candidates `in`.  A wave whose lanes mostly share one digit (tied scores)
// adds once per distinct digit, and keeps its running count for the digit it
// meets most (run_dg, run_cnt: wave-uniform) in a register across rounds, so
// a long run of ties costs one LDS atomic per wave instead of one per round
// (many waves adding to one address serialise).  Every lane of the wave must
// take part; flush_digit_run adds the register count at the end.
__device__ __forceinline__ void digit_hist_round(uint32_t key, bool in, int shift, uint32_t* hist, uint32_t& run_dg,
                                                 uint32_t& run_cnt) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t dg = (key >> shift) & 1023u;
    const uint64_t act = __ballot(in);
    const uint32_t d0 = lane_u32(dg, act ? __builtin_ctzll(act) : 0);
    if (__popcll(__ballot(in && dg == d0)) > 8) {
        if (run_cnt == 0) run_dg = d0;
        uint64_t todo = act;
        while (todo) {
            const int leader = __builtin_ctzll(todo);
            const uint32_t dl = lane_u32(dg, leader);
            const uint64_t same = __ballot(in && dg == dl) & todo;
            if (dl == run_dg) run_cnt += (uint32_t)__popcll(same);
            else if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
            todo &= ~same;
        }
    } else if (in) {
        atomicAdd(&hist[dg], 1u);
    }
}
__device__ __forceinline__ void flush_digit_run(uint32_t* hist, uint32_t run_dg, uint32_t run_cnt) {
    if (run_cnt && (threadIdx.x & (kWave - 1)) == 0) atomicAdd(&hist[run_dg], run_cnt);
}

// the lowest k set bits of `bits` (k <= 0: none)
__device__ __forceinline__ uint32_t lowest_bits(uint32_t bits, int k) {
    uint32_t r = 0;
    while (k > 0 && bits) {
        const uint32_t low = bits & (0u - bits);
        r |= low;
        bits ^= low;
        k--;
    }
    return r;
}

// exclusive prefix sum of v over the block (wave scans, then wave totals in order)
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum) {
    const int lane = threadIdx.x & (kWave - 1), wvi = threadIdx.x / kWave;
    uint32_t incl = v;
    incl = wave_incl_scan_dpp(incl);
    if (lane == kWave - 1) wsum[wvi] = incl;
    __syncthreads();
    uint32_t off = 0;
    for (int q = 0; q < wvi; q++) off += wsum[q];
    return off + incl - v;
}

// D: one workgroup per row.  All candidates share the threshold bin (the top
// 12 key bits), so only the 20-bit score suffix s and the block index j
// separate them.  Two 10-bit digit passes find the suffix T of the need-th
// largest candidate; every candidate with s > T is in, and of those with
// s == T the (need - #{s > T}) smallest j are in (ties to the smaller index).
// The selected list and these sets are marked in two LDS bitmaps over j
// (members, ties at T); each thread then owns 8 consecutive words in
// registers, keeps the lowest tie bits up to the count and emits its members
// at its offset, so the output is in ascending j.  Up to 4096 candidates live
// in registers (4 per thread, loaded before the counts are known: the
// candidate and selected buffers always hold that many entries).
__global__ __launch_bounds__(kIdxFinalThreads) void k_idx_final(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    __shared__ uint4 bm4[2][kIdxBitmapWords / 4];        // members, ties at T
    __shared__ uint2 lc[kIdxFinalLds];                   // very large caps only
    __shared__ uint32_t hA[kIdxDigitBins], hB[kIdxDigitBins];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t wsum[2][kIdxFinalThreads / kWave];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x, row = a.row0 + r;
    int32_t* out = a.out + row * a.topk;
    // the workspace loads go out before the position arrives (a row with
    // fewer visible blocks than k ignores them)
    RowWs w = row_ws(a, r);
    uint2 cv[kIdxCandPerThread];
#pragma unroll
    for (int q = 0; q < kIdxCandPerThread; q++) cv[q] = w.cand[tid + q * kIdxFinalThreads];
    int32_t sv[kIdxSelPerThread];
#pragma unroll
    for (int q = 0; q < kIdxSelPerThread; q++) {
        const int idx = tid + q * kIdxFinalThreads;
        sv[q] = idx < a.topk ? w.sel[idx] : 0;
    }
    const uint32_t nsel = w.counts[0], ncand = w.counts[1];
    const int64_t n = visible_blocks(a, row);
    if (n <= a.topk) {
        for (int64_t i = tid; i < a.topk; i += blockDim.x) out[i] = i < n ? (int32_t)i : -1;
        return;
    }
    const uint32_t need = (uint32_t)a.topk - nsel;     // 1 <= need <= ncand by construction
    const bool in_reg = ncand <= (uint32_t)kIdxFinalLds;
    const int nwords = (int)((n + 31) / 32);
    // the bitmap selection, with R candidates per thread held in registers
    // across its three passes over them (R = 0: read from memory each pass)
    auto bitmap_select = [&](auto rc) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;
        uint2 cr[R > 0 ? R : 1];
        if constexpr (R == kIdxCandPerThread) {
#pragma unroll
            for (int q = 0; q < R; q++) cr[q] = cv[q];
        } else if constexpr (R > 0) {
#pragma unroll
            for (int q = 0; q < R; q++) {
                const uint32_t i = tid + q * kIdxFinalThreads;
                cr[q] = i < ncand ? w.cand[i] : make_uint2(0u, 0u);
            }
        }
        uint32_t* bmA = reinterpret_cast<uint32_t*>(bm4[0]);
        uint32_t* bmT = reinterpret_cast<uint32_t*>(bm4[1]);
        for (int i = tid; i < kIdxBitmapWords / 4; i += blockDim.x) {
            bm4[0][i] = make_uint4(0u, 0u, 0u, 0u);
            bm4[1][i] = make_uint4(0u, 0u, 0u, 0u);
        }
        for (int i = tid; i < kIdxDigitBins; i += blockDim.x) { hA[i] = 0u; hB[i] = 0u; }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kIdxSelPerThread; q++) {
            const uint32_t idx = tid + q * kIdxFinalThreads;
            if (idx < nsel) atomicOr(&bmA[(uint32_t)sv[q] >> 5], 1u << (sv[q] & 31));
        }
        // digit passes over the candidates (registers, or memory)
        auto pass = [&](int shift, bool filt, uint32_t upper, uint32_t* h) {
            uint32_t run_dg = 0, run_cnt = 0;
            if constexpr (R > 0) {
#pragma unroll
                for (int q = 0; q < R; q++) {
                    const uint32_t i = tid + q * kIdxFinalThreads;
                    const bool in = i < ncand && (!filt || ((cr[q].x >> 10) & 1023u) == upper);
                    digit_hist_round(cr[q].x, in, shift, h, run_dg, run_cnt);
                }
            } else {                                      // batches of 8 rounds, loads first
                for (uint32_t i0 = 0; i0 < ncand; i0 += 8 * blockDim.x) {
                    uint32_t kk[8];
#pragma unroll
                    for (int q = 0; q < 8; q++) {
                        const uint32_t i = i0 + q * blockDim.x + tid;
                        kk[q] = i < ncand ? w.cand[i].x : 0u;
                    }
#pragma unroll
                    for (int q = 0; q < 8; q++) {
                        const uint32_t i = i0 + q * blockDim.x + tid;
                        const bool in = i < ncand && (!filt || ((kk[q] >> 10) & 1023u) == upper);
                        digit_hist_round(kk[q], in, shift, h, run_dg, run_cnt);
                    }
                }
            }
            flush_digit_run(h, run_dg, run_cnt);
        };
        // beyond the first size class: the smallest and largest score suffix
        // among the candidates; when they are equal every candidate ties at T
        // (e.g. a row whose weights are all negative: the keys left to choose
        // from all score 0) and the digit passes are skipped
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        if constexpr (R == kIdxCandPerThread) {
            kmx = 1u;                                     // always the passes
        } else if constexpr (R > 0) {
#pragma unroll
            for (int q = 0; q < R; q++)
                if (tid + q * kIdxFinalThreads < ncand) {
                    kmn = min(kmn, cr[q].x & 0xFFFFFu);
                    kmx = max(kmx, cr[q].x & 0xFFFFFu);
                }
        } else {
            for (uint32_t i = tid; i < ncand; i += blockDim.x) {
                const uint32_t x = w.cand[i].x & 0xFFFFFu;
                kmn = min(kmn, x);
                kmx = max(kmx, x);
            }
        }
        if constexpr (R != kIdxCandPerThread) {
#pragma unroll
            for (int o = kWave / 2; o > 0; o >>= 1) {
                kmn = min(kmn, (uint32_t)__shfl_xor((int)kmn, o, kWave));
                kmx = max(kmx, (uint32_t)__shfl_xor((int)kmx, o, kWave));
            }
            if ((tid & (kWave - 1)) == 0) { wsum[0][tid / kWave] = kmn; wsum[1][tid / kWave] = kmx; }
            __syncthreads();
#pragma unroll
            for (int v = 0; v < kIdxFinalThreads / kWave; v++) {
                kmn = min(kmn, wsum[0][v]);
                kmx = max(kmx, wsum[1][v]);
            }
            __syncthreads();                              // wsum is reused by the scans below
        }
        uint32_t T;
        int needT;                                        // ties at T to take, >= 1
        if (kmn == kmx) {
            T = kmn;
            needT = (int)need;
        } else {
            pass(10, false, 0u, hA);
            __syncthreads();
            if (tid < kWave) {
                uint32_t dg, ab;
                wave_pick_digit1024(hA, need, dg, ab);
                if (tid == 0) { sh[0] = dg; sh[1] = ab; }
            }
            __syncthreads();
            const uint32_t dA = sh[0], needA = need - sh[1];
            pass(0, true, dA, hB);
            __syncthreads();
            if (tid < kWave) {
                uint32_t dg, ab;
                wave_pick_digit1024(hB, needA, dg, ab);
                if (tid == 0) { sh[2] = dg; sh[3] = ab; }
            }
            __syncthreads();
            T = (dA << 10) | sh[2];
            needT = (int)(needA - sh[3]);
        }
        auto mark = [&](uint2 c) {
            const uint32_t sfx = c.x & 0xFFFFFu;
            if (sfx >= T) atomicOr(&(sfx > T ? bmA : bmT)[c.y >> 5], 1u << (c.y & 31));
        };
        if constexpr (R > 0) {
#pragma unroll
            for (int q = 0; q < R; q++)
                if (tid + q * kIdxFinalThreads < ncand) mark(cr[q]);
        } else {
            for (uint32_t i0 = 0; i0 < ncand; i0 += 8 * blockDim.x) {
                uint2 cc[8];
#pragma unroll
                for (int q = 0; q < 8; q++) {
                    const uint32_t i = i0 + q * blockDim.x + tid;
                    cc[q] = i < ncand ? w.cand[i] : make_uint2(0u, 0u);
                }
#pragma unroll
                for (int q = 0; q < 8; q++)
                    if (i0 + q * blockDim.x + tid < ncand) mark(cc[q]);
            }
        }
        __syncthreads();
        // thread t owns words [8t, 8t + 8): bitmap words past nwords are zero
        uint32_t am[kIdxWordsPerThread], tm[kIdxWordsPerThread];
#pragma unroll
        for (int v = 0; v < kIdxWordsPerThread / 4; v++) {
            const uint4 x = bm4[0][tid * (kIdxWordsPerThread / 4) + v];
            const uint4 y = bm4[1][tid * (kIdxWordsPerThread / 4) + v];
            am[4 * v] = x.x; am[4 * v + 1] = x.y; am[4 * v + 2] = x.z; am[4 * v + 3] = x.w;
            tm[4 * v] = y.x; tm[4 * v + 1] = y.y; tm[4 * v + 2] = y.z; tm[4 * v + 3] = y.w;
        }
        uint32_t ct = 0;
#pragma unroll
        for (int q = 0; q < kIdxWordsPerThread; q++) ct += __popc(tm[q]);
        int rt = (int)block_exclusive_scan(ct, wsum[0]);  // ties in the words before mine
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < kIdxWordsPerThread; q++) {
            const uint32_t tb = tm[q];
            am[q] |= lowest_bits(tb, needT - rt);
            rt += __popc(tb);
            cnt += __popc(am[q]);
        }
        uint32_t off = block_exclusive_scan(cnt, wsum[1]);
        const int j0 = tid * kIdxWordsPerThread * 32;
#pragma unroll
        for (int q = 0; q < kIdxWordsPerThread; q++) {
            uint32_t bits = am[q];
            while (bits) {
                const int bpos = __builtin_ctz(bits);
                bits &= bits - 1;
                if (off < (uint32_t)a.topk) out[off] = j0 + 32 * q + bpos;
                off++;
            }
        }
    };
    if (nwords <= kIdxBitmapWords) {
        if (in_reg) bitmap_select(std::integral_constant<int, kIdxCandPerThread>{});
        else if (ncand <= 16u * kIdxFinalThreads) bitmap_select(std::integral_constant<int, 16>{});
        else if (ncand <= 20u * kIdxFinalThreads) bitmap_select(std::integral_constant<int, 20>{});
        else bitmap_select(std::integral_constant<int, 0>{});
        return;
    }
    // very large caps: radix-select the composite (score suffix, inverted
    // block index) among the candidates, gather the k indices, bitonic-sort
    int32_t* arr = reinterpret_cast<int32_t*>(bm4[0]);
    const int jb = bits_for(a.cap);
    const uint64_t jmask = ((uint64_t)1 << jb) - 1;
    if (in_reg) {
        for (uint32_t i = threadIdx.x; i < ncand; i += blockDim.x) lc[i] = w.cand[i];
        __syncthreads();
    }
    const uint2* cand = in_reg ? lc : w.cand;
    auto get = [&](int64_t i) -> uint64_t {
        uint2 c = cand[i];
        return ((uint64_t)(c.x & 0xFFFFFu) << jb) | (jmask - (uint64_t)c.y);
    };
    const uint64_t thr = radix_select(get, (int64_t)ncand, 20 + jb, need, hist, sh);
    for (uint32_t i = threadIdx.x; i < nsel && i < (uint32_t)a.topk; i += blockDim.x) arr[i] = w.sel[i];
    if (threadIdx.x == 0) sh[2] = nsel;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < ncand; i += blockDim.x)
        if (get(i) >= thr) {
            const uint32_t pos = atomicAdd(&sh[2], 1u);
            if (pos < (uint32_t)a.topk) arr[pos] = (int32_t)cand[i].y;
        }
    int P = 1;
    while (P < a.topk) P <<= 1;
    for (int i = a.topk + threadIdx.x; i < P; i += blockDim.x) arr[i] = INT32_MAX;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < P / 2; i += blockDim.x) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;
                int x = arr[lo], y = arr[hi];
                if ((x > y) == up) { arr[lo] = y; arr[hi] = x; }
            }
            __syncthreads();
        }
    }
    for (int i = threadIdx.x; i < a.topk; i += blockDim.x) out[i] = arr[i];
}

// ------------------------------------------------------------------ radix helpers
// In an nb-bin histogram (nb = BPT x the workgroup's threads), the digit whose
// cumulative count from the top first reaches need, and the count strictly
// above it, found by the whole workgroup: thread t sums the BPT bins
// [nb - BPT (t + 1), nb - BPT t) with one vector read (consecutive threads,
// consecutive bins: no bank conflicts), a workgroup scan orders the sums from
// the top, and the thread holding the need-th count writes (digit, above,
// count in the digit's bin) to sh[0..2].  Every thread calls it; read sh after
// a barrier.
template <int BPT>
__device__ __forceinline__ void block_pick(const uint32_t* hist, uint32_t need, uint32_t* wsum, uint32_t* sh) {
    static_assert(BPT == 1 || BPT == 2 || BPT == 4, "bins per thread");
    const int nb = BPT * (int)blockDim.x;
    const int lo = nb - BPT * ((int)threadIdx.x + 1);            // lowest bin of this thread's range
    uint32_t h[BPT];
    if constexpr (BPT == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(hist + lo);
        h[0] = v.w; h[1] = v.z; h[2] = v.y; h[3] = v.x;            // highest bin first
    } else if constexpr (BPT == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(hist + lo);
        h[0] = v.y; h[1] = v.x;
    } else {
        h[0] = hist[lo];
    }
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < BPT; q++) s += h[q];
    const uint32_t ex = block_exclusive_scan(s, wsum);            // counts in the bins above mine
    if (ex < need && ex + s >= need) {
        uint32_t c = ex;
#pragma unroll
        for (int q = 0; q < BPT; q++) {
            if (c + h[q] >= need) { sh[0] = (uint32_t)(lo + BPT - 1 - q); sh[1] = c; sh[2] = h[q]; break; }
            c += h[q];
        }
    }
}

// smallest and largest of v over the workgroup (all threads call; wv is the
// caller's scratch of one word pair per wave; a barrier inside)
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint2* wv) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
    }
    if ((threadIdx.x & (kWave - 1)) == 0) wv[threadIdx.x / kWave] = make_uint2(mn, mx);
    __syncthreads();
    const int nw = (int)(blockDim.x / kWave);
    for (int q = 0; q < nw; q++) {
        const uint2 x = wv[q];
        mn = min(mn, x.x);
        mx = max(mx, x.y);
    }
}

// One pass of a radix select over values known to lie in [base, base + 2^width)
// (width <= 32): the digit is (v - base) >> shift with shift = width - 11 (or
// 0), so the values spread over up to 2048 bins wherever the range starts --
// score keys crowd into a few top-bit bins, and LDS atomics on one address
// serialise.  add(f) calls f(v, in) for this thread's candidates; the bin
// holding the need-th largest becomes the new range.  With kTwo, passes
// alternate between two histograms of 2048 bins (hists + 2048 * (pass & 1)),
// both zero before the first pass: a pass clears its own after the last read
// of it, and the barriers of the next pass order that clear before the pass
// after it, so no pass needs a barrier of its own for the clearing.  Without
// kTwo (one histogram, where LDS is short) the clearing takes a barrier.
template <int NT, bool kTwo = true, typename Add>
__device__ __forceinline__ void span_pass(Add add, uint32_t& base, int& width, uint32_t& need, uint32_t& inbin,
                                          uint32_t* hists, int& pass, uint32_t* wsum, uint32_t* sh) {
    uint32_t* hist = kTwo ? hists + 2048 * (pass & 1) : hists;
    const int shift = width > 11 ? width - 11 : 0;
    const uint32_t lim = width >= 32 ? 0xFFFFFFFFu : (1u << width) - 1u;
    add([&](uint32_t v, bool in) {
        const uint32_t d = v - base;                   // wraps past lim for v below base
        if (in && d <= lim) atomicAdd(&hist[d >> shift], 1u);
    });
    __syncthreads();
    block_pick<2048 / NT>(hist, need, wsum, sh);
    __syncthreads();
    base += sh[0] << shift;
    need -= sh[1];
    inbin = sh[2];
    width = shift;
    pass++;
    for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0u;
    if constexpr (!kTwo) __syncthreads();
}

// A range [base, base + 2^width) left by span_pass that holds few values
// (inbin <= 64) is finished by one wave instead of further passes: the
// values in it go to fin[0..63] (fin[64] counts them, zero on entry), and
// lane i of wave 0 counts the listed values above and equal to its own; the
// lane whose value is the need-th largest gives base = that value and
// need -= the count above it, as the remaining passes would (width becomes
// 0).  Lanes holding equal values write equal results.  Two barriers.
template <typename Add>
__device__ __forceinline__ void span_finish(Add add, uint32_t& base, int& width, uint32_t& need, uint32_t* fin,
                                            uint32_t* sh) {
    const uint32_t lim = width >= 32 ? 0xFFFFFFFFu : (1u << width) - 1u;
    add([&](uint32_t v, bool in) {
        if (in && v - base <= lim) {
            const uint32_t i = atomicAdd(&fin[64], 1u);
            if (i < 64u) fin[i] = v;
        }
    });
    __syncthreads();
    if (threadIdx.x < kWave) {
        const uint32_t n = min(fin[64], 64u);
        const uint32_t lane = threadIdx.x;
        const uint32_t x = lane < n ? fin[lane] : 0u;
        uint32_t g = 0, e = 0;
        for (uint32_t j = 0; j < n; j++) {
            const uint32_t y = fin[j];
            g += y > x ? 1u : 0u;
            e += y == x ? 1u : 0u;
        }
        if (lane < n && g < need && need <= g + e) { sh[0] = x; sh[1] = g; }
    }
    __syncthreads();
    base = sh[0];
    need -= sh[1];
    width = 0;
}

__device__ __forceinline__ int bit_width(uint32_t x) { return x ? 32 - __builtin_clz(x) : 0; }

// ------------------------------------------------------------------ prefill path
// A chunk of many query rows with FP4 queries and keys (di = 64, Hi = 4):
// eight queries x four heads fill the 32 rows of one FP4 MFMA, so one
// 32x32x64 product scores 32 keys for 8 queries (the per-row path pads the
// four heads to 32 rows).  Kernels:
//   T  per query, the r-th largest score key of a systematic sample (every
//      stride-th 32-key tile); r * stride ~ 3k, so about 3k keys of the row
//      score at or above it (fewer than k only far in the sample's tail: the
//      row then goes to the exact kernel);
//   F  16 queries per workgroup stream every key tile once; keys scoring
//      above their query's threshold are appended (score bits, j) to per-(query,
//      wave) segments, keys tying with it (j) to per-(query, wave) tie
//      segments that keep each wave's first ties in ascending j (no atomics:
//      each wave counts its own);
//   S  per query: with at least k keys above the threshold, three 11-bit
//      digit passes over their score keys give the k-th largest value T1 and
//      ties at T1 go to the smaller block index (two 10-bit passes over the
//      inverted index find the cut); with fewer, all of them are in plus the
//      smallest j of the threshold ties.  Members are marked in an LDS bitmap
//      over j and emitted in ascending j.
//   X  a query whose above-threshold keys overflowed a segment, or whose
//      candidates are fewer than k (its sample ranked it too high), is flagged
//      by S and recomputed here exactly: the same digit passes over all its
//      recomputed scores.
// S is exact: the top k of a row lie among its keys at or above the
// threshold whenever those number at least k, and the smallest-j ties needed
// are among the stored ones (a wave's ties arrive in ascending j).
constexpr int kPfQ = 8;                  // queries per MFMA row block
constexpr int kPfRB = 2;                 // row blocks per filter workgroup
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kPfQB = kPfQ * kPfRB;      // queries per filter workgroup
constexpr int kPfThreads = 512;          // threshold, filter and exact workgroups
constexpr int kPfWaves = kPfThreads / kWave;
constexpr int kPfSelThreads = 512;       // select workgroups (16 candidates per thread: fewer unrolled masks than 32)
constexpr int kPfMaxSampTiles = 128;     // sample tiles per query (LDS: 8 x 4096 keys)
constexpr int kPfWords = 16384;          // bitmap words: caps up to 2^19 blocks
constexpr int kPfHdr = 128;              // per-row header: thr, flag, 8 above counts, 8 tie counts
constexpr int kPfSeg = kIdxPfCands / kPfWaves;     // above-threshold slots per (query, wave)
constexpr int kPfTieSeg = kIdxPfMaxTopk;           // tie slots per (query, wave)
static_assert(idx_prefill_row_bytes() == kPfHdr + (int64_t)kIdxPfCands * 8 + (int64_t)kPfWaves * kPfTieSeg * 4,
              "prefill row layout");

// row layout: header words [0] threshold key, [1] flag, [2..10) above counts
// per wave, [10..18) tie counts per wave; then the above-threshold (score
// bits, j) segments, then the tie j segments (each wave's first kPfTieSeg ties, in
// ascending j)
__device__ __forceinline__ uint32_t* pf_hdr(const IndexerArgs& a, int64_t row) {
    return reinterpret_cast<uint32_t*>(a.ws + row * a.ws_row_bytes);
}
__device__ __forceinline__ uint2* pf_cand(const IndexerArgs& a, int64_t row) {
    return reinterpret_cast<uint2*>(a.ws + row * a.ws_row_bytes + kPfHdr);
}
__device__ __forceinline__ uint32_t* pf_ties(const IndexerArgs& a, int64_t row) {
    return reinterpret_cast<uint32_t*>(a.ws + row * a.ws_row_bytes + kPfHdr + (int64_t)kIdxPfCands * 8);
}

// A operand of one row block: row l32 = query 4 * (l32 / 4) + head l32 % 4 of
// the 8 queries from tq (zero codes past Tq)
__device__ __forceinline__ void pf_load_a(const IndexerArgs& a, int b, int tq, int l32, int half, i32x8_t& qa,
                                          int& qs) {
    const int t = tq + l32 / 4, h = l32 & 3;
    qa = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    qs = 127;
    if (t < a.Tq) {
        const int64_t r = ((int64_t)b * a.Tq + t) * 4 + h;
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.q) + r * 32 + 16 * half);
        qa[0] = (int)u.x; qa[1] = (int)u.y; qa[2] = (int)u.z; qa[3] = (int)u.w;
        qs = a.q_scales[r * 2 + half];
    }
}

// key tile at j0: lane's 16 code bytes and scale of key j0 + l32 (clamped)
__device__ __forceinline__ void pf_load_keys(const IndexerArgs& a, int b, int64_t j0, int l32, int half, uint4& kc,
                                             int& ks) {
    const int64_t j = min(j0 + l32, a.cap - 1);
    const int64_t r = (int64_t)b * a.cap + j;
    kc = *reinterpret_cast<const uint4*>(a.keys + r * 32 + 16 * half);
    ks = a.key_scales[r * 2 + half];
}

__device__ __forceinline__ f32x16_t pf_mfma(const i32x8_t& qa, int qs, const uint4& kc, int ks) {
    const i32x8_t kf = i32x8_t{(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; i++) acc[i] = 0.0f;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, kf, acc, 4, 4, 0, qs, 0, ks);
}

// score of slot s (query 2s + half of the row block): heads in order, from +0
__device__ __forceinline__ float pf_score(const f32x16_t& acc, int s, const float* w4) {
    float v = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; h++) v = fmaf(w4[h], relu_bits(acc[4 * s + h]), v);
    return v;
}

__global__ __launch_bounds__(kPfThreads) void k_idxp_thresh(IndexerArgs a, int32_t stride, int32_t rank) {
    warm_kernargs(sizeof(IndexerArgs));
    __shared__ uint32_t ss[kPfQ][kPfMaxSampTiles * 32];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int b = blockIdx.y, tq = blockIdx.x * kPfQ;
    i32x8_t qa;
    int qs;
    pf_load_a(a, b, tq, l32, half, qa, qs);
    float w[4][4];
    int32_t nq[4];
    int32_t nmax = 0;
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const int t = tq + 2 * s + half;
        const int64_t row = (int64_t)b * a.Tq + t;
        nq[s] = t < a.Tq ? (int32_t)visible_blocks(a, row) : 0;
        nmax = max(nmax, nq[s]);
#pragma unroll
        for (int h = 0; h < 4; h++) w[s][h] = t < a.Tq ? a.w[row * 4 + h] : 0.0f;
    }
    nmax = (int32_t)wave_max_dpp((float)nmax);          // exact: counts < 2^24
    const int ntile = (nmax + 31) / 32;
    const int nst = min((ntile + stride - 1) / stride, kPfMaxSampTiles);
    for (int i = wv; i < nst; i += kPfWaves) {
        const int64_t j0 = (int64_t)i * stride * 32;
        uint4 kc;
        int ks;
        pf_load_keys(a, b, j0, l32, half, kc, ks);
        const f32x16_t acc = pf_mfma(qa, qs, kc, ks);
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const float v = pf_score(acc, s, w[s]);
            ss[2 * s + half][i * 32 + l32] = j0 + l32 < nq[s] ? score_key(v) : 0u;
        }
    }
    __syncthreads();
    // wave q: the rank-th largest of query q's samples (largest T with at least
    // rank samples >= T, built bit by bit); padding counts only at T = 0
    const int q = wv;
    const int t = tq + q;
    uint32_t v[kPfMaxSampTiles * 32 / kWave];
#pragma unroll
    for (int i = 0; i < kPfMaxSampTiles * 32 / kWave; i++) {
        const int idx = lane + kWave * i;
        v[i] = idx < nst * 32 ? ss[q][idx] : 0u;
    }
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; bit--) {
        const uint32_t c = T | (1u << bit);
        float cnt = 0.0f;
#pragma unroll
        for (int i = 0; i < kPfMaxSampTiles * 32 / kWave; i++) cnt += v[i] >= c ? 1.0f : 0.0f;
        if (wave_sum_dpp(cnt) >= (float)rank) T = c;
    }
    if (t < a.Tq && lane < kPfHdr / 4) {
        uint32_t* hd = pf_hdr(a, (int64_t)b * a.Tq + t);
        hd[lane] = lane == 0 ? T : 0u;                     // thr, flag, counts
    }
}

// compare predicates of the lane-mask compare builtin (LLVM's numbering)
constexpr int kFcmpOeq = 1, kFcmpOgt = 2, kFcmpOge = 3;

__global__ __launch_bounds__(kPfThreads, 4) void k_idxp_filter(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int b = blockIdx.y, t0 = blockIdx.x * kPfQB;
    // the head weights of the 16 queries sit in LDS (read per tile as one
    // 16-byte broadcast per query slot), which keeps four waves per SIMD
    __shared__ float4 wl[kPfRB][4][2];
    i32x8_t qa[kPfRB];
    int qs[kPfRB];
    float thr[kPfRB][4];                                  // threshold key as a float (NaN for key 0)
    int32_t nq[kPfRB][4];
    int32_t nmax = 0;
#pragma unroll
    for (int rb = 0; rb < kPfRB; rb++) {
        pf_load_a(a, b, t0 + kPfQ * rb, l32, half, qa[rb], qs[rb]);
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int t = t0 + kPfQ * rb + 2 * s + half;
            const int64_t row = (int64_t)b * a.Tq + min(t, a.Tq - 1);
            nq[rb][s] = t < a.Tq ? (int32_t)visible_blocks(a, row) : 0;
            nmax = max(nmax, nq[rb][s]);
            {
                // inverse of score_key: key > T <=> score > thr and key == T <=>
                // score == thr for every score (NaN and T = 0: neither)
                const uint32_t T = pf_hdr(a, row)[0];
                thr[rb][s] = __uint_as_float((T & 0x80000000u) ? (T & 0x7FFFFFFFu) : ~T);
            }
            if (lane == 0 && wv == 0) {
#pragma unroll
                for (int hf = 0; hf < 2; hf++) {
                    const int tt = t0 + kPfQ * rb + 2 * s + hf;
                    const int64_t rw = (int64_t)b * a.Tq + min(tt, a.Tq - 1);
                    wl[rb][s][hf] = tt < a.Tq ? make_float4(a.w[rw * 4], a.w[rw * 4 + 1], a.w[rw * 4 + 2], a.w[rw * 4 + 3])
                                              : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
            }
        }
    }
    __syncthreads();
    int32_t nmin = nq[0][0];
#pragma unroll
    for (int rb = 0; rb < kPfRB; rb++)
#pragma unroll
        for (int s = 0; s < 4; s++) nmin = min(nmin, nq[rb][s]);
    nmax = (int32_t)wave_max_dpp((float)nmax);
    nmin = -(int32_t)wave_max_dpp(-(float)nmin);
    const int ntile = (nmax + 31) / 32;
    const int nfull = nmin / 32;                          // tiles every query of the workgroup sees whole
    // this wave's running counts per query (above the threshold, at it):
    // slot (rb, s, half) -> query 8 rb + 2 s + half
    uint32_t cnt[kPfRB][4][2], tcnt[kPfRB][4][2];
#pragma unroll
    for (int rb = 0; rb < kPfRB; rb++)
#pragma unroll
        for (int s = 0; s < 4; s++) { cnt[rb][s][0] = cnt[rb][s][1] = tcnt[rb][s][0] = tcnt[rb][s][1] = 0u; }
    const int64_t rowb = a.ws_row_bytes;
    uint8_t* wbase = a.ws + ((int64_t)b * a.Tq + t0) * rowb;   // this workgroup's first query row
    // appends go through a buffer resource over the workgroup's query rows:
    // 32-bit offsets (the uniform part on the scalar unit), no 64-bit
    // address arithmetic per append
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        wbase, (short)0, (int)(min(kPfQB, a.Tq - t0) * rowb), 0x00020000);
    const int wvs = __builtin_amdgcn_readfirstlane(wv);
    uint4 kc;
    int ks;
    if (wv < ntile) pf_load_keys(a, b, (int64_t)wv * 32, l32, half, kc, ks);
    for (int tile = wv; tile < ntile; tile += kPfWaves) {
        // odd queries of a slot pair: one row further (re-derived every tile,
        // so that no per-slot offsets are kept in registers across the loop)
        uint32_t hoff = half ? (uint32_t)rowb : 0u;
        asm volatile("" : "+v"(hoff));
        const uint4 kcur = kc;
        const int kscur = ks;
        if (tile + kPfWaves < ntile) pf_load_keys(a, b, (int64_t)(tile + kPfWaves) * 32, l32, half, kc, ks);
        const int32_t j = tile * 32 + l32;
        // tiles below every query's visible count skip the visibility test
        auto body = [&](auto visc) __attribute__((always_inline)) {
        constexpr bool kVis = decltype(visc)::value;
        // both row blocks' products first, so the second runs on the matrix
        // core while the first one's scores are formed
        f32x16_t accs[kPfRB];
#pragma unroll
        for (int rb = 0; rb < kPfRB; rb++) accs[rb] = pf_mfma(qa[rb], qs[rb], kcur, kscur);
#pragma unroll
        for (int rb = 0; rb < kPfRB; rb++) {
            const f32x16_t& acc = accs[rb];
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const float4 w4 = wl[rb][s][half];
                const float wv4[4] = {w4.x, w4.y, w4.z, w4.w};
                const float sc = pf_score(acc, s, wv4);
                // one compare decides whether any lane appends (ordered: a NaN
                // score is neither above nor at the threshold); above and at
                // are told apart only on that rarer path
                uint64_t bge = __builtin_amdgcn_fcmpf(sc, thr[rb][s], kFcmpOge);
                if constexpr (kVis) bge &= ballot64(j < nq[rb][s]);
                if (bge) {
                    // this lane's own tests as vector compares (exec masks
                    // straight from them, no bit extraction from the ballots)
                    bool above = sc > thr[rb][s], tie = sc == thr[rb][s];
                    if constexpr (kVis) {
                        const bool vis = j < nq[rb][s];
                        above = above && vis;
                        tie = tie && vis;
                    }
                    const uint64_t bal = ballot64(above), bt = ballot64(tie);
                    // rank among this half's hits: mbcnt over the whole wave,
                    // less the lower half's count for the upper half
                    const uint32_t alo = (uint32_t)bal, ahi = (uint32_t)(bal >> 32);
                    const uint32_t tlo = (uint32_t)bt, thi = (uint32_t)(bt >> 32);
                    const int slot = (kPfQ * rb + 2 * s) * (int)rowb;   // the pair's even query row
                    if (above) {
                        const uint32_t r = __builtin_amdgcn_mbcnt_hi(ahi, __builtin_amdgcn_mbcnt_lo(alo, 0u));
                        const uint32_t pos = r + (half ? cnt[rb][s][1] - __popc(alo) : cnt[rb][s][0]);
                        if (pos < (uint32_t)kPfSeg) {                    // the select forms the key
                            const u32x2_t v = {__float_as_uint(sc), (uint32_t)j};
                            __builtin_amdgcn_raw_buffer_store_b64(v, wres, (int)(hoff + 8 * pos),
                                                                  slot + kPfHdr + 8 * kPfSeg * wvs, 0);
                        }
                    }
                    if (tie) {
                        const uint32_t r = __builtin_amdgcn_mbcnt_hi(thi, __builtin_amdgcn_mbcnt_lo(tlo, 0u));
                        const uint32_t pos = r + (half ? tcnt[rb][s][1] - __popc(tlo) : tcnt[rb][s][0]);
                        if (pos < (uint32_t)kPfTieSeg)
                            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)j, wres, (int)(hoff + 4 * pos),
                                                                  slot + kPfHdr + kIdxPfCands * 8 + 4 * kPfTieSeg * wvs, 0);
                    }
                    cnt[rb][s][0] += __popc(alo);
                    cnt[rb][s][1] += __popc(ahi);
                    tcnt[rb][s][0] += __popc(tlo);
                    tcnt[rb][s][1] += __popc(thi);
                }
            }
        }
        };
        if (tile < nfull) body(std::false_type{});
        else body(std::true_type{});
    }
    if (lane == 0) {
#pragma unroll
        for (int rb = 0; rb < kPfRB; rb++)
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int hf = 0; hf < 2; hf++) {
                    const int t = t0 + kPfQ * rb + 2 * s + hf;
                    if (t < a.Tq) {
                        uint32_t* hd = pf_hdr(a, (int64_t)b * a.Tq + t);
                        hd[2 + wv] = cnt[rb][s][hf];
                        hd[2 + kPfWaves + wv] = tcnt[rb][s][hf];
                    }
                }
    }
}

// histogram of the 11-bit (or narrower) digit (v >> shift) & mask of the values
// `in`, a wave whose lanes mostly agree adding once per distinct digit (as
// digit_hist_round, without the run register)
__device__ __forceinline__ void pf_hist_round(uint32_t v, bool in, int shift, uint32_t mask, uint32_t* hist) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t dg = (v >> shift) & mask;
    const uint64_t act = __ballot(in);
    const uint32_t d0 = lane_u32(dg, act ? __builtin_ctzll(act) : 0);
    if (__popcll(__ballot(in && dg == d0)) > 8) {
        uint64_t todo = act;
        while (todo) {
            const int leader = __builtin_ctzll(todo);
            const uint32_t dl = lane_u32(dg, leader);
            const uint64_t same = __ballot(in && dg == dl) & todo;
            if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
            todo &= ~same;
        }
    } else if (in) {
        atomicAdd(&hist[dg], 1u);
    }
}

// in an nb-bin histogram (nb a multiple of 64), the digit whose cumulative
// count from the top first reaches need, and the count strictly above it;
// one wave, result in every lane
template <int NB>
__device__ __forceinline__ void pf_pick(const uint32_t* hist, uint32_t need, uint32_t& digit, uint32_t& above) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int per = NB / kWave;
    uint32_t h[per], s = 0;
#pragma unroll
    for (int q = 0; q < per; q++) { h[q] = hist[NB - 1 - per * lane - q]; s += h[q]; }
    const uint32_t incl = wave_incl_scan_dpp(s);
    const uint64_t bal = __ballot(incl >= need);
    const int L = bal ? __builtin_ctzll(bal) : kWave - 1;
    const uint32_t cum = lane_u32(incl - s, L);
    uint32_t d = 0, ab = cum;
    if (lane == L) {
        uint32_t c = cum;
        d = NB - per * (L + 1);
        for (int q = 0; q < per; q++) {
            if (c + h[q] >= need) { d = NB - 1 - per * L - q; ab = c; break; }
            c += h[q];
        }
    }
    digit = lane_u32(d, L);
    above = lane_u32(ab, L);
}

// emit the members marked in the first nw4 16-byte groups of bitmap bm (the
// words that can hold a visible block) in ascending j: thread t owns groups
// [t g, (t + 1) g), g = ceil(nw4 / threads), counted in one pass and emitted
// in a second (the callers mark exactly topk members, so every output slot
// is written)
__device__ __forceinline__ void pf_emit(const uint4* bm4, int nw4, int32_t* out, int topk, uint32_t* wsum) {
    const int g = (nw4 + (int)blockDim.x - 1) / (int)blockDim.x;
    const int v0 = (int)threadIdx.x * g, v1 = min(v0 + g, nw4);
    uint32_t cnt = 0;
    for (int v = v0; v < v1; v++) {
        const uint4 x = bm4[v];
        cnt += __popc(x.x) + __popc(x.y) + __popc(x.z) + __popc(x.w);
    }
    uint32_t off = block_exclusive_scan(cnt, wsum);
    for (int v = v0; v < v1; v++) {
        const uint4 x = bm4[v];
        const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            uint32_t bits = wd[e];
            while (bits) {
                const int bpos = __builtin_ctz(bits);
                bits &= bits - 1;
                if (off < (uint32_t)topk) out[off] = 128 * v + 32 * e + bpos;
                off++;
            }
        }
    }
}

// the need-th smallest j among the slots flagged in ok (CPT per thread): two
// 10-bit digit passes over 2^20 - 1 - j; ties with j <= the result are in
template <int CPT>
__device__ __forceinline__ uint32_t pf_jcut(const uint32_t (&jv)[CPT], const bool (&ok)[CPT], uint32_t nslots,
                                            uint32_t need, uint32_t* hist, uint32_t* sh) {
    const uint32_t jm = (1u << 20) - 1u;
    uint32_t jp = 0, jmsk = 0;
    const int js[2] = {10, 0};
    for (int p = 0; p < 2; p++) {
        for (int i = threadIdx.x; i < 1024; i += blockDim.x) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < CPT; q++) {
            if (q * (int)blockDim.x >= (int)nslots) break;   // block-uniform
            const uint32_t iv = jm - jv[q];
            pf_hist_round(iv, ok[q] && (iv & jmsk) == jp, js[p], 1023u, hist);
        }
        __syncthreads();
        if (threadIdx.x < kWave) {
            uint32_t dg, ab;
            pf_pick<1024>(hist, need, dg, ab);
            if (threadIdx.x == 0) { sh[0] = dg; sh[1] = ab; }
        }
        __syncthreads();
        jp |= sh[0] << js[p];
        jmsk |= 1023u << js[p];
        need -= sh[1];
        __syncthreads();
    }
    return jm - jp;
}

// entry i of the concatenation of NW segments (counts c[], stride seg) -> slot
template <int NW>
__device__ __forceinline__ uint32_t pf_slot(uint32_t i, const uint32_t (&c)[NW], int seg) {
    uint32_t w = 0;
#pragma unroll
    for (int s = 0; s < NW - 1; s++)
        if (w == (uint32_t)s && i >= c[s]) { i -= c[s]; w++; }
    return w * seg + i;
}

__global__ __launch_bounds__(kPfSelThreads) void k_idxp_select(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    constexpr int kCPT = kIdxPfCands / kPfSelThreads;          // candidates per thread
    __shared__ uint4 bm4[kPfWords / 4];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t fin[65];
    __shared__ uint2 mm[kPfSelThreads / kWave];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t wsum[kPfSelThreads / kWave];
    uint32_t* bm = reinterpret_cast<uint32_t*>(bm4);
    const int tid = threadIdx.x;
    const int b = blockIdx.y, t = blockIdx.x;
    const int64_t row = (int64_t)b * a.Tq + t;
    const int64_t n = visible_blocks(a, row);
    const int nw4 = (int)min<int64_t>((n + 127) / 128, kPfWords / 4);   // bitmap groups holding visible blocks
    int32_t* out = a.out + row * a.topk;
    if (n <= a.topk) {
        for (int64_t i = tid; i < a.topk; i += blockDim.x) out[i] = i < n ? (int32_t)i : -1;
        return;
    }
    uint32_t* hd = pf_hdr(a, row);
    uint32_t segc[kPfWaves], tiec[kPfWaves], tot = 0, ttot = 0, tstored = 0;
    bool over = false;
#pragma unroll
    for (int w = 0; w < kPfWaves; w++) {
        segc[w] = hd[2 + w];
        tiec[w] = hd[2 + kPfWaves + w];
        over |= segc[w] > (uint32_t)kPfSeg;
        tot += segc[w];
        ttot += tiec[w];
        tiec[w] = min(tiec[w], (uint32_t)kPfTieSeg);           // entries stored
        tstored += tiec[w];
    }
    const uint32_t k = (uint32_t)a.topk;
    if (over || tot + ttot < k) {
        if (tid == 0) hd[1] = 1u;                              // left to the exact kernel
        return;
    }
    const uint2* cand = pf_cand(a, row);
    uint2 cv[kCPT];
#pragma unroll
    for (int q = 0; q < kCPT; q++) {
        const uint32_t i = tid + q * kPfSelThreads;
        cv[q] = make_uint2(0u, 0u);
        if (i < tot) cv[q] = cand[pf_slot(i, segc, kPfSeg)];
    }
#pragma unroll
    for (int q = 0; q < kCPT; q++) cv[q].x = score_key(__uint_as_float(cv[q].x));   // the filter stores score bits
    for (int i = tid; i < nw4; i += blockDim.x) bm4[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tot >= k) {
        // the top k lie among the keys above the threshold: range-adaptive
        // radix passes over their score keys, finished in one wave once the
        // range holds at most 64 of them, give the k-th largest key; then the
        // smallest j of the ties at it
        for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;
        if (tid == 0) fin[64] = 0u;
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
        for (int q = 0; q < kCPT; q++)
            if (tid + q * kPfSelThreads < (int)tot) { mn = min(mn, cv[q].x); mx = max(mx, cv[q].x); }
        block_minmax(mn, mx, mm);                                // barrier inside: hist and fin cleared
        uint32_t need = k, prefix = mn, inbin = 0;
        int width = bit_width(mx - mn), pass = 0;
        auto cands = [&](auto f) {
#pragma unroll
            for (int q = 0; q < kCPT; q++) f(cv[q].x, tid + q * kPfSelThreads < (int)tot);
        };
        while (width > 0) {                                      // workgroup-uniform
            span_pass<kPfSelThreads, false>(cands, prefix, width, need, inbin, hist, pass, wsum, sh);
            if (width > 0 && inbin <= 64u) span_finish(cands, prefix, width, need, fin, sh);
        }
        const uint32_t T1 = prefix;
        uint32_t jv[kCPT];
        bool ok[kCPT];
        uint32_t ntie = 0;
#pragma unroll
        for (int q = 0; q < kCPT; q++) {
            jv[q] = cv[q].y;
            ok[q] = tid + q * kPfSelThreads < tot && cv[q].x == T1;
            ntie += ok[q] ? 1u : 0u;
        }
        if (tid == 0) sh[2] = 0u;
        __syncthreads();
        if (ntie) atomicAdd(&sh[2], ntie);
        __syncthreads();
        const uint32_t jcut = sh[2] > need ? pf_jcut<kCPT>(jv, ok, tot, need, hist, sh) : 0xFFFFFFFFu;
#pragma unroll
        for (int q = 0; q < kCPT; q++) {
            const uint2 c = cv[q];
            if (tid + q * kPfSelThreads < tot && (c.x > T1 || (c.x == T1 && c.y <= jcut)))
                atomicOr(&bm[c.y >> 5], 1u << (c.y & 31));
        }
    } else {
        // every key above the threshold is in, and the (k - tot) smallest j of
        // those at it: each wave stored its own first ties, so they are here
        const uint32_t* ties = pf_ties(a, row);
        uint32_t jv[kCPT];
        bool ok[kCPT];
#pragma unroll
        for (int q = 0; q < kCPT; q++) {
            const uint32_t i = tid + q * kPfSelThreads;
            ok[q] = i < tstored;
            jv[q] = ok[q] ? ties[pf_slot(i, tiec, kPfTieSeg)] : 0u;
        }
        const uint32_t jcut = pf_jcut<kCPT>(jv, ok, tstored, k - tot, hist, sh);
#pragma unroll
        for (int q = 0; q < kCPT; q++) {
            if (tid + q * kPfSelThreads < tot) atomicOr(&bm[cv[q].y >> 5], 1u << (cv[q].y & 31));
            if (ok[q] && jv[q] <= jcut) atomicOr(&bm[jv[q] >> 5], 1u << (jv[q] & 31));
        }
    }
    __syncthreads();
    pf_emit(bm4, nw4, out, a.topk, wsum);
}

// exact selection of one query row from its recomputed scores: digit passes
// over the score key, then over the inverted block index of the ties, then the
// members marked in bm4 (LDS, >= (n + 127) / 128 groups) and emitted.  Every
// thread of the workgroup calls it; the waves take the key tiles in turn.
__device__ void exact_row(const IndexerArgs& a, int b, int64_t row, int64_t n, int32_t* out, uint4* bm4,
                          uint32_t* hist, uint32_t* sh, uint32_t* wsum) {
    uint32_t* bm = reinterpret_cast<uint32_t*>(bm4);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l32 = lane & 31, half = lane >> 5;
    const int nwv = (int)(blockDim.x >> 6);
    const int nw4 = (int)((n + 127) / 128);
    // A operand: rows 0..3 = the four heads of this query, the rest zero
    i32x8_t qa = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    int qs = 127;
    if (l32 < 4) {
        const int64_t r = row * 4 + l32;
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.q) + r * 32 + 16 * half);
        qa[0] = (int)u.x; qa[1] = (int)u.y; qa[2] = (int)u.z; qa[3] = (int)u.w;
        qs = a.q_scales[r * 2 + half];
    }
    float w4[4];
#pragma unroll
    for (int h = 0; h < 4; h++) w4[h] = a.w[row * 4 + h];
    const int ntile = (int)((n + 31) / 32);
    // every key of the row, lanes < 32 holding the score key of key j (the
    // other half of the wave holds zero rows); fn(key, j, valid) per lane
    auto sweep = [&](auto fn) {
        for (int tile = wv; tile < ntile; tile += nwv) {
            uint4 kc;
            int ks;
            pf_load_keys(a, b, (int64_t)tile * 32, l32, half, kc, ks);
            const f32x16_t acc = pf_mfma(qa, qs, kc, ks);
            const float v = pf_score(acc, 0, w4);
            const int32_t j = tile * 32 + l32;
            fn(score_key(v), (uint32_t)j, half == 0 && j < n);
        }
    };
    uint32_t need = (uint32_t)a.topk, prefix = 0, pmask = 0;
    const int shifts[3] = {21, 10, 0};
    const uint32_t masks[3] = {2047u, 2047u, 1023u};
    for (int p = 0; p < 3; p++) {
        for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;
        __syncthreads();
        sweep([&](uint32_t key, uint32_t, bool ok) {
            pf_hist_round(key, ok && (key & pmask) == prefix, shifts[p], masks[p], hist);
        });
        __syncthreads();
        if (tid < kWave) {
            uint32_t dg, ab;
            if (p < 2) pf_pick<2048>(hist, need, dg, ab);
            else pf_pick<1024>(hist, need, dg, ab);
            if (tid == 0) { sh[0] = dg; sh[1] = ab; }
        }
        __syncthreads();
        prefix |= sh[0] << shifts[p];
        pmask |= masks[p] << shifts[p];
        need -= sh[1];
        __syncthreads();
    }
    const uint32_t T1 = prefix;
    const uint32_t jm = (1u << 20) - 1u;
    uint32_t jp = 0, jmsk = 0, jneed = need;
    const int js[2] = {10, 0};
    for (int p = 0; p < 2; p++) {
        for (int i = tid; i < 1024; i += blockDim.x) hist[i] = 0u;
        __syncthreads();
        sweep([&](uint32_t key, uint32_t j, bool ok) {
            const uint32_t iv = jm - j;
            pf_hist_round(iv, ok && key == T1 && (iv & jmsk) == jp, js[p], 1023u, hist);
        });
        __syncthreads();
        if (tid < kWave) {
            uint32_t dg, ab;
            pf_pick<1024>(hist, jneed, dg, ab);
            if (tid == 0) { sh[0] = dg; sh[1] = ab; }
        }
        __syncthreads();
        jp |= sh[0] << js[p];
        jmsk |= 1023u << js[p];
        jneed -= sh[1];
        __syncthreads();
    }
    const uint32_t jcut = jm - jp;
    for (int i = tid; i < nw4; i += blockDim.x) bm4[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    sweep([&](uint32_t key, uint32_t j, bool ok) {
        if (ok && (key > T1 || (key == T1 && j <= jcut))) atomicOr(&bm[j >> 5], 1u << (j & 31));
    });
    __syncthreads();
    pf_emit(bm4, nw4, out, a.topk, wsum);
}

// a query row the select kernel flagged, recomputed exactly
__global__ __launch_bounds__(kPfThreads) void k_idxp_exact(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    __shared__ uint4 bm4[kPfWords / 4];
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t wsum[kPfWaves];
    const int b = blockIdx.y, t = blockIdx.x;
    const int64_t row = (int64_t)b * a.Tq + t;
    if (pf_hdr(a, row)[1] == 0u) return;
    exact_row(a, b, row, visible_blocks(a, row), a.out + row * a.topk, bm4, hist, sh, wsum);
}

// ------------------------------------------------------------------ decode path
// Query rows of short chunks (decode: one or a few queries per sequence) with
// FP4 queries and keys (di = 64, Hi = 4) against a large key set (up to 2^18
// blocks).  Two kernels:
//   F  the row's keys are split over workgroups of kDfChunk consecutive
//      blocks.  Every workgroup of a row first scores the same sample of the
//      row's keys (kDsSampTiles 32-key tiles, one in each window of stride
//      tiles, stride and rank from the row's visible count: mostly cache
//      hits), then issues its own keys and, while they are in flight, takes
//      T, the rank-th largest sample score key itself (at least rank samples
//      score at or above T; about 4k keys of the row do) by radix passes;
//      every workgroup gets the same T.  Keys scoring above T go (key, j) to the workgroup's own
//      segment of the row's candidate area, keys equal to T (j) to its tie
//      segment, both in ascending j; the counts go to the row header.  No
//      atomics and nothing to clear: each workgroup writes its own counts.
//   S  one workgroup per row: the above-threshold segments are compacted
//      into LDS; with at least k of them, three digit passes (11, 11, 10
//      bits) over their score keys give the k-th largest key T1 and members
//      are the keys above T1 plus the smallest-j keys at T1; with fewer,
//      every key above T plus the smallest-j keys at T.  Members and the
//      ties to choose from are marked in two LDS bitmaps over j; the lowest
//      tie bits up to the count join the members, emitted in ascending j.
//      A row with more candidates than LDS holds, or fewer than k at or
//      above T (a sample ranked too high), is recomputed exactly in place.
// Every kernel forms a key's score from the same MFMA result and the same
// fp32 operations, so the score is the same number in all of them.

constexpr int kDfThreads = 512;
constexpr int kDfWaves = kDfThreads / kWave;
constexpr int kDfTiles = 16;                                         // 32-key tiles per wave
constexpr int kDfChunk = kDfWaves * kDfTiles * 32;                   // keys per filter workgroup
constexpr int kDfSegCands = 1024;                                    // above-threshold slots per workgroup
constexpr int kDsSampTiles = 32;                                     // sample tiles per row
constexpr int kDsSampPerWave = kDsSampTiles / kDfWaves;
constexpr int kDecMaxSeg = (int)(kIdxDecMaxCap / kDfChunk);          // workgroups per row at most
constexpr int kDecHdr = 1024;                                        // T, counts per segment
constexpr int kDsThreads = 1024;
constexpr int kDsWords = (int)(kIdxDecMaxCap / 32);                  // bitmap words
constexpr int kDsWPT = kDsWords / kDsThreads;                        // bitmap words per thread
constexpr int kDsCPT = kIdxPfCands / kDsThreads;                     // compacted candidates per thread
static_assert(kDecHdr >= 4 * (2 + 2 * kDecMaxSeg), "decode header");
static_assert(idx_decode_row_bytes(kIdxDecMaxCap) ==
                  kDecHdr + (int64_t)kDecMaxSeg * (kDfSegCands * 8 + kDfChunk * 4) &&
              idx_decode_row_bytes(kDfChunk + 1) == kDecHdr + 2 * (kDfSegCands * 8 + kDfChunk * 4), "decode row layout");
static_assert(kDsWords * 32 >= kIdxDecMaxCap && kDsWords % (4 * kDsThreads) == 0, "decode bitmaps");
static_assert(kDecMaxSeg <= kWave && kDsThreads % kDecMaxSeg == 0, "decode segments");
static_assert(2048 % kDfThreads == 0 && 2048 % kDsThreads == 0 && 1024 % kDsThreads == 0, "histogram picks");

// decode row layout (idx_decode_row_bytes): header words [0] T, [2 + s]
// above count of segment s, [2 + kDecMaxSeg + s] tie count of segment s;
// then, for the cache's S = ceil(cap / kDfChunk) segments, each segment's
// above slots (key, j), then each segment's tie slots (j)
__device__ __forceinline__ uint32_t* dec_hdr(const IndexerArgs& a, int64_t row) {
    return reinterpret_cast<uint32_t*>(a.ws + row * a.ws_row_bytes);
}
__device__ __forceinline__ uint2* dec_cand(const IndexerArgs& a, int64_t row, int seg) {
    return reinterpret_cast<uint2*>(a.ws + row * a.ws_row_bytes + kDecHdr) + (int64_t)seg * kDfSegCands;
}
__device__ __forceinline__ uint32_t* dec_ties(const IndexerArgs& a, int64_t row, int seg) {
    const int64_t nseg_cap = (a.cap + kDfChunk - 1) / kDfChunk;
    return reinterpret_cast<uint32_t*>(a.ws + row * a.ws_row_bytes + kDecHdr + nseg_cap * kDfSegCands * 8) +
           (int64_t)seg * kDfChunk;
}

// A operand of one query row: rows 0..3 its four heads, the rest zero
// The row's FP4 query as the product's A operand: lanes l32 < 4 hold head
// l32's row, the others zero rows.  Split in two so that the loads (every
// lane reads, head l32 & 3) go out before the key loads and the selects come
// after them: a wait for a load issued after the keys would wait for the keys.
struct PdQuery {
    uint4 u;
    int s;
};
__device__ __forceinline__ PdQuery pd_issue_q(const IndexerArgs& a, int64_t row, int l32, int half) {
    const int64_t r = row * 4 + (l32 & 3);
    return PdQuery{*reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(a.q) + r * 32 + 16 * half),
                   (int)a.q_scales[r * 2 + half]};
}
__device__ __forceinline__ void pd_form_a(const PdQuery& p, int l32, i32x8_t& qa, int& qs) {
    const bool on = l32 < 4;
    qa = i32x8_t{on ? (int)p.u.x : 0, on ? (int)p.u.y : 0, on ? (int)p.u.z : 0, on ? (int)p.u.w : 0, 0, 0, 0, 0};
    qs = on ? p.s : 127;
}

// score of key l32 of a tile for the row's four heads (lanes of the upper
// half hold zero rows).  The product reads operands from every lane, so it
// is kept out of any lane-divergent select that consumes it (the compiler
// would otherwise issue it under a partial exec mask).
__device__ __forceinline__ float pd_score(const i32x8_t& qa, int qs, const uint4& kc, int ks, const float* w4) {
    const f32x16_t acc = pf_mfma(qa, qs, kc, ks);
    float v = pf_score(acc, 0, w4);
    asm volatile("" : "+v"(v));
    return v;
}

// Sample tile i of a decode row: one tile in each window of `stride` tiles,
// at an offset that varies with i (((37 i + 11) mod 64) / 64 of the window,
// no division).  Tiles at a power-of-two stride would all fall into a few
// cache sets (and every workgroup of the row reads them).
__device__ __forceinline__ int64_t dec_sample_tile(int i, int stride) {
    return (int64_t)i * stride + (int64_t)((((uint32_t)i * 37u + 11u) & 63u) * (uint32_t)stride >> 6);
}

__global__ __launch_bounds__(kDfThreads) void k_idxd_filter(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    __shared__ __attribute__((aligned(16))) uint32_t hist[2 * 2048];
    __shared__ uint32_t fin[65];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t wcnt[2][kDfWaves];
    __shared__ uint32_t wsum[kDfWaves];
    __shared__ uint2 mm[kDfWaves];
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);           // uniform: tile math on the scalar unit
    const int64_t row = blockIdx.y;
    const int b = (int)(row / a.Tq);
    const int seg = (int)blockIdx.x;
    const int64_t t0 = (int64_t)seg * kDfChunk + (int64_t)wv * kDfTiles * 32;    // this wave's first key
    // loads return in order: the query and head weights (independent of the
    // position) go first, then the row's sample.  The chunk's keys are issued
    // once the sample has been scored: issued together, every CU's chunk
    // competes with the sample for HBM and the sample arrives late; issued
    // after it, the chunk is in flight while the threshold is formed.
    const PdQuery pq = pd_issue_q(a, row, l32, half);
    float w4[4];
#pragma unroll
    for (int h = 0; h < 4; h++) w4[h] = a.w[row * 4 + h];
    const int64_t n = visible_blocks(a, row);
    if (n <= a.topk || (int64_t)seg * kDfChunk >= n) return;                     // workgroup-uniform
    // the sample's stride comes from the row's visible count
    const int ntile = (int)((n + 31) / 32);
    const int stride = (ntile + kDsSampTiles - 1) / kDsSampTiles;
    const int nst = (ntile + stride - 1) / stride;                               // sample tiles, <= kDsSampTiles
    uint4 sc[kDsSampPerWave];
    int ss[kDsSampPerWave];
#pragma unroll
    for (int i = 0; i < kDsSampPerWave; i++)
        pf_load_keys(a, b, dec_sample_tile(wv + kDfWaves * i, stride) * 32, l32, half, sc[i], ss[i]);
    for (int i = tid; i < 2 * 2048; i += kDfThreads) hist[i] = 0u;
    if (tid == 0) fin[64] = 0u;
    i32x8_t qa;
    int qs;
    pd_form_a(pq, l32, qa, qs);
    uint32_t skey[kDsSampPerWave];
#pragma unroll
    for (int i = 0; i < kDsSampPerWave; i++) {
        const int tile = wv + kDfWaves * i;
        const int64_t j = dec_sample_tile(tile, stride) * 32 + l32;
        const float v = pd_score(qa, qs, sc[i], ss[i], w4);
        skey[i] = (half == 0 && tile < nst && j < n) ? score_key(v) : 0u;
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 kc[kDfTiles];
    int ks[kDfTiles];
#pragma unroll
    for (int i = 0; i < kDfTiles; i++) pf_load_keys(a, b, t0 + 32 * i, l32, half, kc[i], ks[i]);
    __builtin_amdgcn_sched_barrier(0);
    // T: the rank-th largest sample key itself, by range-adaptive radix
    // passes over the samples (key 0 marks no sample).  At least rank samples
    // score at or above T; an exact sample value (not a bin edge) keeps a
    // mass of equal scores (e.g. the zeros of a row whose weights are all
    // negative) on the tie list instead of the above-threshold one.
    uint32_t mn = 0xFFFFFFFFu, mx = 0u, nv = 0u;
#pragma unroll
    for (int i = 0; i < kDsSampPerWave; i++) {
        nv += (uint32_t)__popcll(ballot64(half == 0 && skey[i] != 0u));
        if (half == 0 && skey[i] != 0u) { mn = min(mn, skey[i]); mx = max(mx, skey[i]); }
    }
    if (lane == 0) wcnt[0][wv] = nv;
    block_minmax(mn, mx, mm);                          // barrier inside: wcnt complete
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < kDfWaves; q++) valid += wcnt[0][q];
    uint32_t T = score_key(-__builtin_huge_valf());    // no sample: every non-NaN score is above it
    if (valid > 0) {
        uint32_t need = (uint32_t)min<int64_t>(max<int64_t>(((int64_t)4 * a.topk * valid + n - 1) / n, 1), valid);
        uint32_t base = mn, inbin = 0;
        int width = bit_width(mx - mn), pass = 0;
        auto samples = [&](auto f) {
#pragma unroll
            for (int i = 0; i < kDsSampPerWave; i++) f(skey[i], half == 0 && skey[i] != 0u);
        };
        while (width > 0) {                                                      // workgroup-uniform
            span_pass<kDfThreads>(samples, base, width, need, inbin, hist, pass, wsum, sh);
            if (width > 0 && inbin <= 64u) span_finish(samples, base, width, need, fin, sh);
        }
        T = base;
    }
    __syncthreads();                                   // wcnt is reused below
    // key > T <=> score > thr, key == T <=> score == thr
    const float thr = __uint_as_float((T & 0x80000000u) ? (T & 0x7FFFFFFFu) : ~T);
    uint64_t ab[kDfTiles], tb[kDfTiles];
    uint32_t kk[kDfTiles];
    uint32_t na = 0, nt = 0;
#pragma unroll
    for (int i = 0; i < kDfTiles; i++) {
        const float v = pd_score(qa, qs, kc[i], ks[i], w4);
        const uint64_t vm = ballot64(half == 0 && t0 + 32 * i + l32 < n);
        ab[i] = __builtin_amdgcn_fcmpf(v, thr, kFcmpOgt) & vm;
        tb[i] = __builtin_amdgcn_fcmpf(v, thr, kFcmpOeq) & vm;
        kk[i] = score_key(v);
        na += (uint32_t)__popcll(ab[i]);
        nt += (uint32_t)__popcll(tb[i]);
    }
    if (lane == 0) { wcnt[0][wv] = na; wcnt[1][wv] = nt; }
    __syncthreads();
    uint32_t oa = 0, ot = 0, ta = 0, tt = 0;
#pragma unroll
    for (int q = 0; q < kDfWaves; q++) {
        const uint32_t ca = wcnt[0][q], ct = wcnt[1][q];
        if (q < wv) { oa += ca; ot += ct; }
        ta += ca;
        tt += ct;
    }
    uint32_t* hd = dec_hdr(a, row);
    if (tid == 0) {
        hd[2 + seg] = ta;                        // true counts (above may exceed the slots)
        hd[2 + kDecMaxSeg + seg] = tt;
        if (seg == 0) hd[0] = T;
    }
    uint2* cand = dec_cand(a, row, seg);
    uint32_t* ties = dec_ties(a, row, seg);
    const uint64_t below = (1ull << lane) - 1;
#pragma unroll
    for (int i = 0; i < kDfTiles; i++) {
        const uint32_t j = (uint32_t)(t0 + 32 * i + l32);
        if ((ab[i] >> lane) & 1u) {
            const uint32_t pos = oa + (uint32_t)__popcll(ab[i] & below);
            if (pos < (uint32_t)kDfSegCands) cand[pos] = make_uint2(kk[i], j);
        }
        if ((tb[i] >> lane) & 1u) ties[ot + (uint32_t)__popcll(tb[i] & below)] = j;   // < kDfChunk
        oa += (uint32_t)__popcll(ab[i]);
        ot += (uint32_t)__popcll(tb[i]);
    }
}

__global__ __launch_bounds__(kDsThreads) void k_idxd_select(IndexerArgs a) {
    warm_kernargs(sizeof(IndexerArgs));
    __shared__ uint4 bmA4[kDsWords / 4];                             // members (also the exact path's bitmap)
    __shared__ uint4 bmT4[kDsWords / 4];                             // ties to choose from
    __shared__ uint2 cl[kIdxPfCands];                                // compacted above-threshold candidates
    __shared__ __attribute__((aligned(16))) uint32_t hist[2 * 2048];
    __shared__ uint32_t fin[65];
    __shared__ uint32_t sh[4];
    __shared__ uint32_t segoff[2][kDecMaxSeg];
    __shared__ uint32_t segcnt[kDecMaxSeg];                          // stored above-threshold entries
    __shared__ uint2 mm[kDsThreads / kWave];
    __shared__ uint32_t wsum[2][kDsThreads / kWave];
    uint32_t* bmA = reinterpret_cast<uint32_t*>(bmA4);
    uint32_t* bmT = reinterpret_cast<uint32_t*>(bmT4);
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t row = blockIdx.x;
    const int b = (int)(row / a.Tq);
    uint32_t* hd = dec_hdr(a, row);
    // the segment counts go out before the position arrives (always inside the header)
    uint32_t ca = 0, ct = 0;
    if (tid < kDecMaxSeg) { ca = hd[2 + tid]; ct = hd[2 + kDecMaxSeg + tid]; }
    const int64_t n = visible_blocks(a, row);
    int32_t* out = a.out + row * a.topk;
    const uint32_t k = (uint32_t)a.topk;
    if (n <= a.topk) {
        for (int64_t i = tid; i < a.topk; i += kDsThreads) out[i] = i < n ? (int32_t)i : -1;
        return;
    }
    const int nseg = (int)((n + kDfChunk - 1) / kDfChunk);
    if (wv == 0) {                                                   // kDecMaxSeg <= 64: one wave
        if (lane >= nseg) { ca = 0; ct = 0; }
        const bool over = __ballot(ca > (uint32_t)kDfSegCands) != 0;
        const uint32_t ia = wave_incl_scan_dpp(ca), it = wave_incl_scan_dpp(ct);
        if (lane < kDecMaxSeg) {
            segoff[0][lane] = ia - ca;
            segoff[1][lane] = it - ct;
            segcnt[lane] = min(ca, (uint32_t)kDfSegCands);
        }
        if (lane == kWave - 1) { sh[0] = ia; sh[1] = it; sh[2] = over ? 1u : 0u; }
    }
    __syncthreads();
    const uint32_t tot = sh[0], ttot = sh[1];
    if (sh[2] || tot > (uint32_t)kIdxPfCands || tot + ttot < k) {
        exact_row(a, b, row, n, out, bmA4, hist, sh, wsum[0]);
        return;
    }
    // compaction: kDsThreads / kDecMaxSeg threads per segment, each copying
    // every (that many)-th entry, four loads in flight (clamped to the
    // segment's last entry, so none is conditional) before the first store
    {
        constexpr int kTps = kDsThreads / kDecMaxSeg;
        const int sg = tid / kTps, sub = tid % kTps;
        const uint32_t c = segcnt[sg], o = segoff[0][sg];           // zero past the row's segments
        const uint2* src = dec_cand(a, row, sg);
        for (uint32_t e0 = sub; e0 < c; e0 += 4 * kTps) {
            uint2 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) v[u] = src[min(e0 + u * kTps, c - 1)];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (e0 + u * kTps < c) cl[o + e0 + u * kTps] = v[u];
        }
    }
    const int nwords = (int)((n + 31) / 32);
    const int nw4 = (nwords + 3) / 4;
    for (int i = tid; i < nw4; i += kDsThreads) {
        bmA4[i] = make_uint4(0u, 0u, 0u, 0u);
        bmT4[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    for (int i = tid; i < 2 * 2048; i += kDsThreads) hist[i] = 0u;
    if (tid == 0) fin[64] = 0u;
    __syncthreads();
    uint2 cv[kDsCPT];
#pragma unroll
    for (int q = 0; q < kDsCPT; q++) {
        const uint32_t i = tid + q * kDsThreads;
        cv[q] = i < tot ? cl[i] : make_uint2(0u, 0u);
    }
    uint32_t needT;                                                  // ties to take
    if (tot >= k) {
        // the k-th largest key among those above T: range-adaptive radix
        // passes until the range is one key
        uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
        for (int q = 0; q < kDsCPT; q++)
            if (tid + q * kDsThreads < (int)tot) { mn = min(mn, cv[q].x); mx = max(mx, cv[q].x); }
        block_minmax(mn, mx, mm);
        uint32_t need = k, prefix = mn, inbin = 0;
        int width = bit_width(mx - mn), pass = 0;
        auto cands = [&](auto f) {
#pragma unroll
            for (int q = 0; q < kDsCPT; q++) f(cv[q].x, tid + q * kDsThreads < (int)tot);
        };
        while (width > 0) {                                          // workgroup-uniform
            span_pass<kDsThreads>(cands, prefix, width, need, inbin, hist, pass, wsum[0], sh);
            if (width > 0 && inbin <= 64u) span_finish(cands, prefix, width, need, fin, sh);
        }
        const uint32_t T1 = prefix;
        needT = need;
#pragma unroll
        for (int q = 0; q < kDsCPT; q++) {
            const uint2 c = cv[q];
            if (tid + q * kDsThreads < (int)tot && c.x >= T1)
                atomicOr(&(c.x > T1 ? bmA : bmT)[c.y >> 5], 1u << (c.y & 31));
        }
    } else {
        // every key above T is in, and the (k - tot) smallest j of those at T
        needT = k - tot;
#pragma unroll
        for (int q = 0; q < kDsCPT; q++)
            if (tid + q * kDsThreads < (int)tot) atomicOr(&bmA[cv[q].y >> 5], 1u << (cv[q].y & 31));
        for (int s = wv; s < nseg; s += kDsThreads / kWave) {
            const uint32_t c = hd[2 + kDecMaxSeg + s];
            const uint32_t* src = dec_ties(a, row, s);
            for (uint32_t e0 = 0; e0 < c; e0 += 4 * kWave) {
                uint32_t v[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const uint32_t e = e0 + u * kWave + lane;
                    v[u] = e < c ? src[e] : 0u;
                }
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (e0 + u * kWave + lane < c) atomicOr(&bmT[v[u] >> 5], 1u << (v[u] & 31));
            }
        }
    }
    __syncthreads();
    // thread t owns words [kDsWPT t, kDsWPT (t + 1)); words past nwords are not read
    uint32_t am[kDsWPT], tm[kDsWPT];
    const int w0 = tid * kDsWPT;
#pragma unroll
    for (int v = 0; v < kDsWPT / 4; v++) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u), y = x;
        if (w0 + 4 * v < nwords) { x = bmA4[tid * (kDsWPT / 4) + v]; y = bmT4[tid * (kDsWPT / 4) + v]; }
        am[4 * v] = x.x; am[4 * v + 1] = x.y; am[4 * v + 2] = x.z; am[4 * v + 3] = x.w;
        tm[4 * v] = y.x; tm[4 * v + 1] = y.y; tm[4 * v + 2] = y.z; tm[4 * v + 3] = y.w;
    }
    uint32_t cnt_t = 0;
#pragma unroll
    for (int q = 0; q < kDsWPT; q++) cnt_t += __popc(tm[q]);
    int rt = (int)block_exclusive_scan(cnt_t, wsum[0]);              // ties in the words before mine
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < kDsWPT; q++) {
        am[q] |= lowest_bits(tm[q], (int)needT - rt);
        rt += __popc(tm[q]);
        cnt += __popc(am[q]);
    }
    uint32_t off = block_exclusive_scan(cnt, wsum[1]);
#pragma unroll
    for (int q = 0; q < kDsWPT; q++) {
        uint32_t bits = am[q];
        while (bits) {
            const int bpos = __builtin_ctz(bits);
            bits &= bits - 1;
            if (off < k) out[off] = (w0 + q) * 32 + bpos;
            off++;
        }
    }
}

// ------------------------------------------------------------------ launcher
template <int QF, int KF>
static hipError_t launch_tpl(IndexerArgs a, int64_t total_rows, int64_t ws_bytes, hipStream_t st) {
    if (total_rows == 0) return hipSuccess;
    if (a.cap <= kIdxSmallMaxKeys) {
        a.row0 = 0;
        a.rows = (int32_t)total_rows;
        hipLaunchKernelGGL((k_idx_small<QF, KF>), dim3((unsigned)total_rows), dim3(kIdxThreads), 0, st, a);
        return hipGetLastError();
    }
    if constexpr (QF == CSA_FP4_E2M1 && KF == CSA_FP4_E2M1) {
        if (idx_prefill_eligible(a.di, a.Hi, a.Tq, a.cap, a.topk) &&
            ws_bytes >= total_rows * idx_prefill_row_bytes()) {
            const unsigned B = (unsigned)(total_rows / a.Tq);
            const int64_t ntile = (a.cap + 31) / 32;
            const int64_t stride = std::max<int64_t>(64, (ntile + kPfMaxSampTiles - 1) / kPfMaxSampTiles);
            const int32_t rank = (int32_t)((3 * (int64_t)a.topk + stride - 1) / stride);
            a.row0 = 0;
            a.rows = (int32_t)total_rows;
            a.ws_row_bytes = idx_prefill_row_bytes();
            hipLaunchKernelGGL(k_idxp_thresh, dim3((unsigned)((a.Tq + kPfQ - 1) / kPfQ), B), dim3(kPfThreads), 0, st,
                               a, (int32_t)stride, rank);
            hipLaunchKernelGGL(k_idxp_filter, dim3((unsigned)((a.Tq + kPfQB - 1) / kPfQB), B), dim3(kPfThreads), 0, st, a);
            hipLaunchKernelGGL(k_idxp_select, dim3((unsigned)a.Tq, B), dim3(kPfSelThreads), 0, st, a);
            hipLaunchKernelGGL(k_idxp_exact, dim3((unsigned)a.Tq, B), dim3(kPfThreads), 0, st, a);
            return hipGetLastError();
        }
    }
    if constexpr (QF == CSA_FP4_E2M1 && KF == CSA_FP4_E2M1) {
        if (idx_decode_eligible(a.di, a.Hi, a.Tq, a.cap, a.topk) && ws_bytes >= total_rows * idx_decode_row_bytes(a.cap)) {
            a.row0 = 0;
            a.rows = (int32_t)total_rows;
            a.ws_row_bytes = idx_decode_row_bytes(a.cap);
            hipLaunchKernelGGL(k_idxd_filter, dim3((unsigned)((a.cap + kDfChunk - 1) / kDfChunk), (unsigned)total_rows),
                               dim3(kDfThreads), 0, st, a);
            hipLaunchKernelGGL(k_idxd_select, dim3((unsigned)total_rows), dim3(kDsThreads), 0, st, a);
            return hipGetLastError();
        }
    }
    const int64_t per_batch = ws_bytes / a.ws_row_bytes;
    const unsigned nchunk = (unsigned)((a.cap + kIdxChunk - 1) / kIdxChunk);
    for (int64_t r0 = 0; r0 < total_rows; r0 += per_batch) {
        const int64_t nr = min(per_batch, total_rows - r0);
        a.row0 = (int32_t)r0;
        a.rows = (int32_t)nr;
        hipLaunchKernelGGL(k_idx_zero, dim3((unsigned)nr), dim3(256), 0, st, a);
        const bool mfma_ok = a.di == 64 && a.Hi <= 32 && ((KF == CSA_FP4_E2M1 && QF == CSA_FP4_E2M1) ||
                                                          (KF == CSA_BF16 && QF != CSA_F32));
        if constexpr ((KF == CSA_FP4_E2M1 && QF == CSA_FP4_E2M1) || (KF == CSA_BF16 && QF != CSA_F32)) {
            if (mfma_ok) hipLaunchKernelGGL((k_idx_score_mfma<QF, KF>), dim3(nchunk, (unsigned)nr), dim3(kIdxScoreThreads), 0, st, a);
            else hipLaunchKernelGGL((k_idx_score<QF, KF>), dim3(nchunk, (unsigned)nr), dim3(kIdxThreads), 0, st, a);
        } else {
            hipLaunchKernelGGL((k_idx_score<QF, KF>), dim3(nchunk, (unsigned)nr), dim3(kIdxThreads), 0, st, a);
        }
        hipLaunchKernelGGL(k_idx_collect, dim3(nchunk, (unsigned)nr), dim3(kIdxThreads), 0, st, a);
        hipLaunchKernelGGL(k_idx_final, dim3((unsigned)nr), dim3(kIdxFinalThreads), 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_indexer_topk(IndexerArgs a, int64_t total_rows, int64_t ws_bytes, hipStream_t st) {
    const int qf = a.q_fmt, kf = a.key_fmt;
#define CSA_IDX_CASE(Q, K) if (qf == Q && kf == K) return launch_tpl<Q, K>(a, total_rows, ws_bytes, st);
    CSA_IDX_CASE(CSA_F32, CSA_F32)
    CSA_IDX_CASE(CSA_F32, CSA_BF16)
    CSA_IDX_CASE(CSA_F32, CSA_FP4_E2M1)
    CSA_IDX_CASE(CSA_BF16, CSA_F32)
    CSA_IDX_CASE(CSA_BF16, CSA_BF16)
    CSA_IDX_CASE(CSA_BF16, CSA_FP4_E2M1)
    CSA_IDX_CASE(CSA_FP4_E2M1, CSA_F32)
    CSA_IDX_CASE(CSA_FP4_E2M1, CSA_BF16)
    CSA_IDX_CASE(CSA_FP4_E2M1, CSA_FP4_E2M1)
#undef CSA_IDX_CASE
    return hipErrorInvalidValue;
}

}  // namespace csa
