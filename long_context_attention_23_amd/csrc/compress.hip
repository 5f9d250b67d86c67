// compress.hip -- csa_compress_kv: block pooling, RMSNorm, partial RoPE and the
// cache quantisers.
//
// Method: "DeepSeek-V4 ... open-source declaration" (peacm.com) section 3.2,
// CSA step 1 (every m tokens become one compressed KV entry through an
// attention-like mechanism; HCA uses 128:1) and the four tricks (KV RMSNorm,
// RoPE on the last 64 dims); "technical report digest" section 2.1.4 (FP8
// non-RoPE dims + BF16 RoPE dims) and section 3.2 (FP4 indexer keys with 1x32
// scales).  Reading of "attention-like": softmax weights over a learned
// m-position score vector (plus an optional content score), summed over the
// block's tokens.
//
// One workgroup of 512 threads per output block.  The work is streaming and
// memory-bound (m tokens of d values in, one record out); the block's pooled
// vector lives in LDS between the pooling, normalisation, rotation and
// quantisation phases.  A decode step compresses one block per sequence, so
// a workgroup's own latency is the cost: the token rows are read with many
// independent 16-byte loads in flight per thread.
#include <stddef.h>

#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace csa {

constexpr int kCompThreads = 512;
constexpr int kMaxD = 1024;
constexpr int kMaxM = 1024;


template <typename XT>
__global__ __launch_bounds__(kCompThreads) void k_compress(CompressArgs a) {
    __shared__ float sv[kMaxD];
    __shared__ float sz[kMaxM];
    __shared__ float red[kCompThreads / kWave];
    __shared__ int se[kMaxD / 32];
    __shared__ float part[kCompThreads * 8];      // token-group partial sums of the pooling (TG * d <= 8 * threads)
    __shared__ double rf[64];

    const int tid = threadIdx.x;
    const int b = blockIdx.y;
    const int64_t i = blockIdx.x;
    const int d = a.d, m = a.m;
    const int64_t j = (int64_t)a.tok_start[b] / m + i;
    if (!a.ring && j >= a.cap) return;
    const int64_t slot = a.ring ? j % a.cap : j;
    const XT* xb = reinterpret_cast<const XT*>(a.x) + ((int64_t)b * a.T + i * m) * d;
    stage_rope_arg(offsetof(CompressArgs, rope), rf, a.dr / 2);

    // ---- pooling weights: z_r = bias_r + <u, x_r>, softmax over r
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    for (int r = 0; r < m; r += kCompThreads / kWave) {
        int rr = r + wv;
        float z = 0.0f;
        if (a.sproj && rr < m) {
            for (int k = lane; k < d; k += kWave) z += a.sproj[k] * ld_scalar<XT>(xb, (size_t)rr * d + k);
            z = wave_sum(z);
        }
        if (rr < m && lane == 0) sz[rr] = a.sbias[rr] + z;
    }
    __syncthreads();
    float zmax = -INFINITY;
    for (int r = tid; r < m; r += kCompThreads) zmax = fmaxf(zmax, sz[r]);
    zmax = block_max(zmax, red);
    float zsum = 0.0f;
    for (int r = tid; r < m; r += kCompThreads) zsum += expf(sz[r] - zmax);
    zsum = block_sum(zsum, red);
    for (int r = tid; r < m; r += kCompThreads) sz[r] = expf(sz[r] - zmax) / zsum;
    __syncthreads();

    // ---- pooled vector c = sum_r pi_r x_r.  16-byte chunks of the token rows;
    // the threads of one chunk column split the block's tokens into TG groups
    // (token order inside a group), and the group sums are added in group order.
    constexpr int EPC = 16 / (int)sizeof(XT);
    const int nch = d / EPC;
    if (d % EPC == 0 && nch <= kCompThreads) {
        const int TG = kCompThreads / nch;
        const int c = tid % nch, tg = tid / nch;
        if (tg < TG) {
            float acc[EPC];
#pragma unroll
            for (int e = 0; e < EPC; e++) acc[e] = 0.0f;
            // batches of kBatch rows: all loads of a batch are issued before any
            // is consumed (token order is kept inside the group)
            constexpr int kBatch = 8;
            for (int r0 = tg; r0 < m; r0 += kBatch * TG) {
                uint4 u[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; q++) {
                    const int r = r0 + q * TG;
                    u[q] = r < m ? *reinterpret_cast<const uint4*>(xb + (size_t)r * d + (size_t)c * EPC)
                                 : make_uint4(0u, 0u, 0u, 0u);
                }
#pragma unroll
                for (int q = 0; q < kBatch; q++) {
                    const int r = r0 + q * TG;
                    if (r >= m) break;
                    const float p = sz[r];
                    if constexpr (sizeof(XT) == 2) {
                        const uint32_t wd[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            acc[2 * e] = fmaf(p, __uint_as_float(wd[e] << 16), acc[2 * e]);
                            acc[2 * e + 1] = fmaf(p, __uint_as_float(wd[e] & 0xFFFF0000u), acc[2 * e + 1]);
                        }
                    } else {
                        acc[0] = fmaf(p, __uint_as_float(u[q].x), acc[0]);
                        acc[1] = fmaf(p, __uint_as_float(u[q].y), acc[1]);
                        acc[2] = fmaf(p, __uint_as_float(u[q].z), acc[2]);
                        acc[3] = fmaf(p, __uint_as_float(u[q].w), acc[3]);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < EPC; e++) part[tg * d + c * EPC + e] = acc[e];
        }
        __syncthreads();
        for (int k = tid; k < d; k += kCompThreads) {
            float v = 0.0f;
            for (int q = 0; q < TG; q++) v += part[q * d + k];
            sv[k] = v;
        }
    } else {
        for (int k = tid; k < d; k += kCompThreads) {
            float acc = 0.0f;
            for (int r = 0; r < m; r++) acc += sz[r] * ld_scalar<XT>(xb, (size_t)r * d + k);
            sv[k] = acc;
        }
    }
    __syncthreads();
    float ss = 0.0f;
    for (int k = tid; k < d; k += kCompThreads) ss += sv[k] * sv[k];
    if (a.gamma) {
        ss = block_sum(ss, red);
        const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
        for (int k = tid; k < d; k += kCompThreads) sv[k] = sv[k] * inv * a.gamma[k];
    }
    __syncthreads();

    // ---- RoPE at the block's start position j*m on the last dr dims
    const int off = d - a.dr;
    for (int p = tid; p < a.dr / 2; p += kCompThreads) {
        float sn, cs;
        rope_sincos((double)(j * m), rf[p], sn, cs);
        float x0 = sv[off + 2 * p], x1 = sv[off + 2 * p + 1];
        sv[off + 2 * p] = x0 * cs - x1 * sn;
        sv[off + 2 * p + 1] = x0 * sn + x1 * cs;
    }
    __syncthreads();

    // ---- quantise into the output record
    const size_t r = (size_t)b * a.cap + slot;
    uint8_t* rec = a.out + r * a.rec_bytes;
    if (a.fmt == CSA_F32) {
        for (int k = tid; k < d; k += kCompThreads) reinterpret_cast<float*>(rec)[k] = sv[k];
    } else if (a.fmt == CSA_BF16) {
        for (int k = tid; k < d; k += kCompThreads) reinterpret_cast<uint16_t*>(rec)[k] = f32_to_bf16(sv[k]);
    } else if (a.fmt == CSA_FP8_E4M3) {
        const int dn = d - a.dr;
        float amax = 0.0f;
        for (int k = tid; k < dn; k += kCompThreads) amax = fmaxf(amax, fabsf(sv[k]));
        amax = block_max(amax, red);
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
        for (int k = tid; k < dn; k += kCompThreads) rec[k] = f32_to_e4m3(sv[k] / scale);
        for (int k = tid; k < a.dr; k += kCompThreads)
            reinterpret_cast<uint16_t*>(rec + dn)[k] = f32_to_bf16(sv[dn + k]);
        const int tail = dn + 2 * a.dr;
        for (int k = tail + 4 + tid; k < a.rec_bytes; k += kCompThreads) rec[k] = 0;
        if (tid == 0) *reinterpret_cast<float*>(rec + tail) = scale;
    } else {  // FP4 E2M1 indexer row with one E8M0 scale per 32 values
        const int nb = d / 32;
        if (tid < nb) {
            float amax = 0.0f;
            for (int k = 0; k < 32; k++) amax = fmaxf(amax, fabsf(sv[tid * 32 + k]));
            int e = INT32_MIN;
            if (amax > 0.0f) {
                int ex;
                frexpf(amax, &ex);          // amax in [2^(ex-1), 2^ex)
                e = ex - 1 - 2;
            }
            se[tid] = e;
        }
        __syncthreads();
        int emax = INT32_MIN;
        for (int q = 0; q < nb; q++) emax = max(emax, se[q]);
        __syncthreads();
        if (tid < nb) {
            int e = se[tid];
            if (emax == INT32_MIN) e = 0;             // all-zero row
            else e = max(e, emax - 14);               // keep FP4 -> FP8 lossless
            e = min(max(e, -127), 127);
            se[tid] = e;
            a.out_scales[r * nb + tid] = (uint8_t)(e + 127);
        }
        __syncthreads();
        for (int k = tid; k < d / 2; k += kCompThreads) {
            int e = se[(2 * k) / 32];
            uint32_t c0 = f32_to_e2m1(ldexpf(sv[2 * k], -e));
            uint32_t c1 = f32_to_e2m1(ldexpf(sv[2 * k + 1], -e));
            rec[k] = (uint8_t)(c0 | (c1 << 4));
        }
    }
}

// Decode-latency form of the same computation, for position-only pooling
// scores (no content projection), d % (16-byte chunk) == 0, d <= 1024 and at
// most QR token rows per thread.  Every global load is issued up front (token
// rows, pooling biases, gamma); each wave finds the softmax maximum and sum
// itself; element k of the block belongs to thread k (and k + 512), so RoPE
// pairs are lane pairs and the whole tail needs three barriers.  The RoPE
// frequencies come straight from the argument segment, and the destination
// slot (which depends on the sequence's token start) is found after the loads
// are out, so the block costs one memory round trip before its arithmetic.  The
// arithmetic is that of k_compress (token order inside each token group,
// group sums in group order); the softmax sum and the square sums are reduced
// in DPP row order instead of a butterfly, so the last bits may differ.
struct CompFastSmem {
    float part[kCompThreads * 8];
    float pw[kMaxM];                      // pooling weight of each token row of the block
    float red_z[kCompThreads / kWave];    // per-wave partials of a token's content score
    float red_ss[kCompThreads / kWave];
    float red_mx[kCompThreads / kWave];
    int se[kMaxD / 32];
};

// block i of sequence b; `a` lives in the argument segment with its RoPE table
// at byte rope_off of the segment
// The tail of a block's compression, shared by the block and the per-token
// kernels: RMSNorm, RoPE at j*m on the last dr dims, the quantiser into slot
// j of the output (a block beyond a linear cache's capacity is not stored).
// v: the pooled vector, element tid + t * threads in v[t]; gk, fk: gamma and
// the RoPE frequency of those elements.  Every thread of the workgroup calls it.
template <int KT>
__device__ __forceinline__ void finish_block(const CompressArgs& a, size_t rope_off, CompFastSmem& sm, float (&v)[KT],
                                             const float (&gk)[KT], const double (&fk)[KT], int64_t j, int b) {
    float* red_ss = sm.red_ss;
    float* red_mx = sm.red_mx;
    int* se = sm.se;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int d = a.d, m = a.m;
    const int off = d - a.dr;
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < KT; t++) {
        const int k = tid + t * kCompThreads;
        if (k < d) ss += v[t] * v[t];
    }
    if (a.gamma) {                                        // RMSNorm
        ss = wave_sum_dpp(ss);
        if (lane == 0) red_ss[wv] = ss;
        __syncthreads();                                  // barrier 2
        float tot = 0.0f;
        for (int w = 0; w < kCompThreads / kWave; w++) tot += red_ss[w];
        const float inv = 1.0f / sqrtf(tot / (float)d + a.eps);
#pragma unroll
        for (int t = 0; t < KT; t++) v[t] = v[t] * inv * gk[t];
    }
    // ---- RoPE at j*m on the last dr dims: the pair (off + 2p, off + 2p + 1) is a lane pair
#pragma unroll
    for (int t = 0; t < KT; t++) {
        const int k = tid + t * kCompThreads;
        const float other = __shfl_xor(v[t], 1, kWave);
        if (k < d && k >= off) {
            float sn, cs;
            rope_sincos((double)(j * m), fk[t], sn, cs);
            const bool odd = (k - off) & 1;
            const float x0 = odd ? other : v[t], x1 = odd ? v[t] : other;
            v[t] = odd ? x0 * sn + x1 * cs : x0 * cs - x1 * sn;
        }
    }

    // ---- quantise into the output record (a block beyond a linear cache's
    // capacity is not stored; the test sits here, after every load, so that
    // no load waits for the block index)
    if (!a.ring && j >= a.cap) return;                   // the whole workgroup
    const int64_t slot = a.ring ? j % a.cap : j;
    const size_t rrow = (size_t)b * a.cap + slot;
    uint8_t* rec = a.out + rrow * a.rec_bytes;
    if (a.fmt == CSA_F32) {
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            if (k < d) reinterpret_cast<float*>(rec)[k] = v[t];
        }
    } else if (a.fmt == CSA_BF16) {
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            if (k < d) reinterpret_cast<uint16_t*>(rec)[k] = f32_to_bf16(v[t]);
        }
    } else if (a.fmt == CSA_FP8_E4M3) {
        const int dn = d - a.dr;
        float amax = 0.0f;
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            if (k < dn) amax = fmaxf(amax, fabsf(v[t]));
        }
        amax = wave_max_dpp(amax);
        if (lane == 0) red_mx[wv] = amax;
        __syncthreads();                                  // barrier 3
        amax = red_mx[0];
        for (int w = 1; w < kCompThreads / kWave; w++) amax = fmaxf(amax, red_mx[w]);
        const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            if (k < dn) rec[k] = f32_to_e4m3(v[t] / scale);
            else if (k < d) reinterpret_cast<uint16_t*>(rec + dn)[k - dn] = f32_to_bf16(v[t]);
        }
        const int tail = dn + 2 * a.dr;
        for (int k = tail + 4 + tid; k < a.rec_bytes; k += kCompThreads) rec[k] = 0;
        if (tid == 0) *reinterpret_cast<float*>(rec + tail) = scale;
    } else {  // FP4 E2M1 indexer row with one E8M0 scale per 32 values (32 consecutive lanes)
        const int nb = d / 32;
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            float bm = k < d ? fabsf(v[t]) : 0.0f;
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, kWave));
            if (k < d && (k & 31) == 0) {
                int e = INT32_MIN;
                if (bm > 0.0f) {
                    int ex;
                    frexpf(bm, &ex);                      // bm in [2^(ex-1), 2^ex)
                    e = ex - 1 - 2;
                }
                se[k >> 5] = e;
            }
        }
        __syncthreads();                                  // barrier 3
        int emax = INT32_MIN;
        for (int q = 0; q < nb; q++) emax = max(emax, se[q]);
#pragma unroll
        for (int t = 0; t < KT; t++) {
            const int k = tid + t * kCompThreads;
            int e = 0;
            if (k < d) {
                e = se[k >> 5];
                if (emax == INT32_MIN) e = 0;             // all-zero row
                else e = max(e, emax - 14);               // keep FP4 -> FP8 lossless
                e = min(max(e, -127), 127);
                if ((k & 31) == 0) a.out_scales[rrow * nb + (k >> 5)] = (uint8_t)(e + 127);
            }
            const uint32_t code = k < d ? f32_to_e2m1(ldexpf(v[t], -e)) : 0u;
            const uint32_t hi = __shfl_xor(code, 1, kWave);
            if (k < d && (k & 1) == 0) rec[k >> 1] = (uint8_t)(code | (hi << 4));
        }
    }
}

template <typename XT, int QR>
__device__ __forceinline__ void compress_fast_body(const CompressArgs& a, size_t rope_off, CompFastSmem& sm, int b,
                                                   int i) {
    float* part = sm.part;
    constexpr int EPC = 16 / (int)sizeof(XT);
    constexpr int KT = kMaxD / kCompThreads;              // elements per thread
    constexpr int SB = 2 * QR < 16 ? 2 * QR : 16;        // pooling biases per lane (m <= 64 SB)
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int d = a.d, m = a.m;
    const XT* xb = reinterpret_cast<const XT*>(a.x) + ((int64_t)b * a.T + (int64_t)i * m) * d;
    const int nch = d / EPC, TG = kCompThreads / nch;
    const int c = tid % nch, tg = tid / nch;
    const int off = d - a.dr;

    // ---- every load first: the biases (the lane's share of all of them, and
    // those of the rows whose pooling weight this thread forms), gamma, the
    // RoPE frequencies of this thread's elements, then the token rows (one
    // load per row slot, clamped to a valid row: the softmax below waits for
    // the biases only, with the rows still in flight)
    float sb[SB];
#pragma unroll
    for (int s = 0; s < SB; s++) sb[s] = lane + s * kWave < m ? a.sbias[lane + s * kWave] : -INFINITY;
    constexpr int PR = kMaxM / kCompThreads;             // pooling weights formed per thread
    float bo[PR];
#pragma unroll
    for (int t = 0; t < PR; t++) bo[t] = tid + t * kCompThreads < m ? a.sbias[tid + t * kCompThreads] : 0.0f;
    float gk[KT];
    double fk[KT];
#pragma unroll
    for (int t = 0; t < KT; t++) {
        const int k = tid + t * kCompThreads;
        gk[t] = (a.gamma && k < d) ? a.gamma[k] : 1.0f;
        fk[t] = (k < d && k >= off) ? rope_freq_arg(rope_off, (k - off) >> 1) : 0.0;
    }
    const int64_t tok0 = a.tok_start[b];
    uint4 u[QR];
#pragma unroll
    for (int q = 0; q < QR; q++) {
        const int r = min(tg + q * TG, m - 1);
        u[q] = *reinterpret_cast<const uint4*>(xb + (size_t)r * d + (size_t)c * EPC);
    }
    __builtin_amdgcn_sched_barrier(0);                   // the rows go out before the softmax waits for the biases
    const int64_t j = (int64_t)(tok0 / m) + i;

    // ---- softmax of the biases: every wave reduces the same values itself
    float zmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < SB; s++) zmax = fmaxf(zmax, sb[s]);
    zmax = wave_max_dpp(zmax);
    float zsum = 0.0f;
#pragma unroll
    for (int s = 0; s < SB; s++)
        if (lane + s * kWave < m) zsum += expf(sb[s] - zmax);
    zsum = wave_sum_dpp(zsum);
    // the pooling weight of each row, formed once (row r by thread r % threads)
#pragma unroll
    for (int t = 0; t < PR; t++)
        if (tid + t * kCompThreads < m) sm.pw[tid + t * kCompThreads] = expf(bo[t] - zmax) / zsum;
    __syncthreads();                                      // barrier 0: pooling weights

    // ---- pooled partial sums of this thread's token group
    if (tg < TG) {
        float acc[EPC];
#pragma unroll
        for (int e = 0; e < EPC; e++) acc[e] = 0.0f;
#pragma unroll
        for (int q = 0; q < QR; q++) {
            if (tg + q * TG >= m) break;
            const float p = sm.pw[tg + q * TG];
            if constexpr (sizeof(XT) == 2) {
                const uint32_t wd[4] = {u[q].x, u[q].y, u[q].z, u[q].w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    acc[2 * e] = fmaf(p, __uint_as_float(wd[e] << 16), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(p, __uint_as_float(wd[e] & 0xFFFF0000u), acc[2 * e + 1]);
                }
            } else {
                acc[0] = fmaf(p, __uint_as_float(u[q].x), acc[0]);
                acc[1] = fmaf(p, __uint_as_float(u[q].y), acc[1]);
                acc[2] = fmaf(p, __uint_as_float(u[q].z), acc[2]);
                acc[3] = fmaf(p, __uint_as_float(u[q].w), acc[3]);
            }
        }
#pragma unroll
        for (int e = 0; e < EPC; e++) part[tg * d + c * EPC + e] = acc[e];
    }
    __syncthreads();                                      // barrier 1: partials
    const int tgu = m < TG ? m : TG;                      // token groups that hold rows
    float v[KT];
#pragma unroll
    for (int t = 0; t < KT; t++) {
        const int k = tid + t * kCompThreads;
        v[t] = 0.0f;
        if (k < d)
            for (int q = 0; q < tgu; q++) v[t] += part[q * d + k];
    }
    finish_block<KT>(a, rope_off, sm, v, gk, fk, j, b);
}

template <typename XT, int QR>
__global__ __launch_bounds__(kCompThreads) void k_compress_fast(CompressArgs a) {
    warm_kernargs(offsetof(CompressArgs, rope));
    __shared__ CompFastSmem sm;
    compress_fast_body<XT, QR>(a, offsetof(CompressArgs, rope), sm, blockIdx.y, blockIdx.x);
}

// Several independent compressions in one launch (blockIdx.z = job): the
// blocks of one decode step (window entry, compressed block, indexer key)
// otherwise cost a dispatch each.  Jobs with at most one token row per
// thread run the QR = 1 body, the others the QRB body.
template <typename XT, int QRB>
__global__ __launch_bounds__(kCompThreads) void k_compress_batch(CompressBatch bt) {
    __shared__ CompFastSmem sm;
    const int z = blockIdx.z;
    const CompressArgs& a = bt.job[z];
    const size_t off = (size_t)z * sizeof(CompressArgs);
    warm_kernargs_at<offsetof(CompressArgs, rope)>(off);
    if ((int64_t)(blockIdx.x + 1) * a.m > a.T || (int)blockIdx.y >= a.B) return;   // block x of this job is complete iff (x+1) m <= T
    constexpr int EPC = 16 / (int)sizeof(XT);
    const int TG = kCompThreads / (a.d / EPC);
    if (a.m <= TG) compress_fast_body<XT, 1>(a, off + offsetof(CompressArgs, rope), sm, blockIdx.y, blockIdx.x);
    else compress_fast_body<XT, QRB>(a, off + offsetof(CompressArgs, rope), sm, blockIdx.y, blockIdx.x);
}

// One token of each sequence per call (decode): the block compression in
// its incremental form.  The pooling softmax over a block's m scores is an
// online softmax over its tokens (peacm.com section 3.2, CSA step 1: every
// m tokens become one entry), kept per sequence in a state of d + 2 floats:
// the running weighted sum of the tokens, the running maximum score and the
// running sum of exp(score - maximum).  Token r = t % m of block j = t / m:
//   r == 0     the state starts from the token (weight 1);
//   r > 0      max' = max(max, z); sum and the weighted sum are rescaled by
//              exp(max - max') and the token added with exp(z - max');
//   r == m - 1 the block is finished like a whole block (RMSNorm, RoPE at
//              j * m, quantiser into slot j) from weighted sum / sum; the
//              state is not written back (the next block starts afresh).
// m == 1 (window entries) needs no state: the token is the entry.  The
// result equals the block kernel's up to rounding in the pooling (the two
// forms add the same terms with other roundings); m == 1 entries are the
// same bits.  One workgroup per (sequence, job); a.tok_start holds each
// sequence's token position t.
template <typename XT>
__device__ __forceinline__ void compress_step_body(const CompressArgs& a, size_t rope_off, CompFastSmem& sm, int b) {
    constexpr int KT = kMaxD / kCompThreads;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int d = a.d, m = a.m;
    const int off = d - a.dr;
    // ---- every load first: the position, the token, gamma, the RoPE
    // frequencies, the content-score weights and the state
    const int64_t t = a.tok_start[b];
    if (t < 0) return;                                    // no position, no entry (the whole workgroup)
    const XT* xr = reinterpret_cast<const XT*>(a.x) + (size_t)b * d;
    float xv[KT], gk[KT], uk[KT], acc[KT];
    double fk[KT];
#pragma unroll
    for (int q = 0; q < KT; q++) {
        const int k = tid + q * kCompThreads;
        if constexpr (sizeof(XT) == 2) xv[q] = k < d ? __uint_as_float((uint32_t)xr[k] << 16) : 0.0f;
        else xv[q] = k < d ? xr[k] : 0.0f;
        gk[q] = (a.gamma && k < d) ? a.gamma[k] : 1.0f;
        fk[q] = (k < d && k >= off) ? rope_freq_arg(rope_off, (k - off) >> 1) : 0.0;
        uk[q] = (a.sproj && k < d) ? a.sproj[k] : 0.0f;
        acc[q] = (a.state && k < d) ? a.state[(size_t)b * (d + 2) + k] : 0.0f;
    }
    const float smax = a.state ? a.state[(size_t)b * (d + 2) + d] : 0.0f;
    const float ssum = a.state ? a.state[(size_t)b * (d + 2) + d + 1] : 0.0f;
    const int64_t j = t / m;
    const int r = (int)(t - j * m);
    float z = a.sbias[r];
    if (a.sproj) {                                        // z += <u, x>: fixed-order block sum
        float pz = 0.0f;
#pragma unroll
        for (int q = 0; q < KT; q++) pz = fmaf(uk[q], xv[q], pz);
        pz = wave_sum_dpp(pz);
        if (lane == 0) sm.red_z[wv] = pz;
        __syncthreads();
        float tot = 0.0f;
        for (int w = 0; w < kCompThreads / kWave; w++) tot += sm.red_z[w];
        z += tot;
    }
    float v[KT];
    if (m == 1) {
#pragma unroll
        for (int q = 0; q < KT; q++) v[q] = xv[q];
    } else {
        float mx, sw;
        if (r == 0) {
            mx = z;
            sw = 1.0f;
#pragma unroll
            for (int q = 0; q < KT; q++) acc[q] = xv[q];
        } else {
            mx = fmaxf(smax, z);
            const float a1 = expf(smax - mx), a2 = expf(z - mx);
            sw = fmaf(ssum, a1, a2);
#pragma unroll
            for (int q = 0; q < KT; q++) acc[q] = fmaf(a2, xv[q], acc[q] * a1);
        }
        if (r < m - 1) {                                  // the block goes on: keep the state
            float* st = a.state + (size_t)b * (d + 2);
#pragma unroll
            for (int q = 0; q < KT; q++) {
                const int k = tid + q * kCompThreads;
                if (k < d) st[k] = acc[q];
            }
            if (tid == 0) {
                st[d] = mx;
                st[d + 1] = sw;
            }
            return;                                       // the whole workgroup
        }
#pragma unroll
        for (int q = 0; q < KT; q++) v[q] = acc[q] / sw;
    }
    finish_block<KT>(a, rope_off, sm, v, gk, fk, j, b);
}

// a decode step's per-token compressions (blockIdx.y = job), one workgroup
// per sequence
template <typename XT>
__global__ __launch_bounds__(kCompThreads) void k_compress_step(CompressBatch bt) {
    __shared__ CompFastSmem sm;
    const int z = blockIdx.y;
    const CompressArgs& a = bt.job[z];
    const size_t off = (size_t)z * sizeof(CompressArgs);
    warm_kernargs_at<offsetof(CompressArgs, rope)>(off);
    if ((int)blockIdx.x >= a.B) return;
    compress_step_body<XT>(a, off + offsetof(CompressArgs, rope), sm, blockIdx.x);
}

// token rows per thread of the fast kernel for this job, or 0 when the job
// needs the general kernel (content scores, d not a whole number of 16-byte
// chunks, or more pooling biases than the kernel's lanes hold)
template <typename XT>
static int fast_rows(const CompressArgs& a) {
    constexpr int EPC = 16 / (int)sizeof(XT);
    const int nch = a.d / EPC;
    const bool fast0 = !a.sproj && a.d % EPC == 0 && a.d <= kMaxD && nch <= kCompThreads && a.dr % 2 == 0 &&
                       (a.d - a.dr) % 2 == 0 && a.d % 32 == 0;
    if (!fast0) return 0;
    const int TG = kCompThreads / nch;
    const int qr = (a.m + TG - 1) / TG;
    const int sb = qr <= 1 ? 2 : qr <= 2 ? 4 : qr <= 4 ? 8 : 16;        // SB of the kernel for qr
    return (qr <= 16 && a.m <= kWave * sb) ? qr : 0;
}

template <typename XT>
static void launch_compress_t(const CompressArgs& a, dim3 grid, hipStream_t st) {
    const int qr = fast_rows<XT>(a);
    const bool fast = qr > 0;
    if (fast && qr <= 1) hipLaunchKernelGGL((k_compress_fast<XT, 1>), grid, dim3(kCompThreads), 0, st, a);
    else if (fast && qr <= 2) hipLaunchKernelGGL((k_compress_fast<XT, 2>), grid, dim3(kCompThreads), 0, st, a);
    else if (fast && qr <= 4) hipLaunchKernelGGL((k_compress_fast<XT, 4>), grid, dim3(kCompThreads), 0, st, a);
    else if (fast && qr <= 8) hipLaunchKernelGGL((k_compress_fast<XT, 8>), grid, dim3(kCompThreads), 0, st, a);
    else if (fast && qr <= 16) hipLaunchKernelGGL((k_compress_fast<XT, 16>), grid, dim3(kCompThreads), 0, st, a);
    else hipLaunchKernelGGL(k_compress<XT>, grid, dim3(kCompThreads), 0, st, a);
}

hipError_t launch_compress(const CompressArgs& a, int x_dtype, hipStream_t st) {
    int64_t nblk = a.T / a.m;
    if (nblk == 0 || a.B == 0) return hipSuccess;
    dim3 grid((unsigned)nblk, (unsigned)a.B);
    if (x_dtype == CSA_F32) launch_compress_t<float>(a, grid, st);
    else launch_compress_t<uint16_t>(a, grid, st);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_compress_batch_t(const CompressArgs* jobs, int n, hipStream_t st) {
    int qmax = 0;
    int64_t gx = 0, gy = 0;
    bool one = n <= kCompBatchMax;
    for (int k = 0; k < n; k++) {
        const int q = fast_rows<XT>(jobs[k]);
        one = one && q > 0;
        qmax = q > qmax ? q : qmax;
        gx = std::max(gx, jobs[k].T / jobs[k].m);
        gy = std::max(gy, (int64_t)jobs[k].B);
    }
    if (!one) {                                         // one launch per job
        for (int k = 0; k < n; k++) {
            const hipError_t e = launch_compress(jobs[k], sizeof(XT) == 4 ? CSA_F32 : CSA_BF16, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (gx == 0 || gy == 0) return hipSuccess;
    CompressBatch bt{};
    for (int k = 0; k < n; k++) bt.job[k] = jobs[k];
    const dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)n);
    if (qmax <= 1) hipLaunchKernelGGL((k_compress_batch<XT, 1>), grid, dim3(kCompThreads), 0, st, bt);
    else if (qmax <= 2) hipLaunchKernelGGL((k_compress_batch<XT, 2>), grid, dim3(kCompThreads), 0, st, bt);
    else if (qmax <= 4) hipLaunchKernelGGL((k_compress_batch<XT, 4>), grid, dim3(kCompThreads), 0, st, bt);
    else if (qmax <= 8) hipLaunchKernelGGL((k_compress_batch<XT, 8>), grid, dim3(kCompThreads), 0, st, bt);
    else hipLaunchKernelGGL((k_compress_batch<XT, 16>), grid, dim3(kCompThreads), 0, st, bt);
    return hipGetLastError();
}

hipError_t launch_compress_batch(const CompressArgs* jobs, int n, int x_dtype, hipStream_t st) {
    if (x_dtype == CSA_F32) return launch_compress_batch_t<float>(jobs, n, st);
    return launch_compress_batch_t<uint16_t>(jobs, n, st);
}

template <typename XT>
static hipError_t launch_compress_step_t(const CompressArgs* jobs, int n, hipStream_t st) {
    for (int k0 = 0; k0 < n; k0 += kCompBatchMax) {
        const int nk = n - k0 < kCompBatchMax ? n - k0 : kCompBatchMax;
        CompressBatch bt{};
        int64_t gx = 0;
        for (int k = 0; k < nk; k++) {
            bt.job[k] = jobs[k0 + k];
            gx = std::max(gx, (int64_t)jobs[k0 + k].B);
        }
        if (gx == 0) continue;
        hipLaunchKernelGGL(k_compress_step<XT>, dim3((unsigned)gx, (unsigned)nk), dim3(kCompThreads), 0, st, bt);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_compress_step(const CompressArgs* jobs, int n, int x_dtype, hipStream_t st) {
    if (x_dtype == CSA_F32) return launch_compress_step_t<float>(jobs, n, st);
    return launch_compress_step_t<uint16_t>(jobs, n, st);
}

}  // namespace csa
