// launch.hpp -- argument blocks and launchers of the CSA / HCA kernels.
// Host validation lives in api.cpp; each .hip file defines its launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa_attn.h"

namespace csa {

// fp64 inverse frequencies base^(-2i/dr), i < dr/2 (dr <= 128), filled on the host
struct RopeTable {
    double f[64];
};
void fill_rope_table(RopeTable& t, int dr, float base);

struct CompressArgs {
    const void* x;
    int32_t B, d, m;
    int64_t T;
    const int32_t* tok_start;
    const float* sbias;
    const float* sproj;
    const float* gamma;
    float eps;
    int32_t dr;
    float base;
    int32_t out_kind;   // 0: KV record, 1: indexer row
    int32_t fmt;
    uint8_t* out;
    uint8_t* out_scales;
    int64_t cap;
    int32_t ring;
    int32_t rec_bytes;
    float* state;       // per-token compression: [B][d + 2] running pooled state (null: m == 1 or block kernels)
    RopeTable rope;
};
hipError_t launch_compress(const CompressArgs& a, int x_dtype, hipStream_t st);
// independent compressions of one x dtype; up to kCompBatchMax share a launch
constexpr int kCompBatchMax = 4;
struct CompressBatch {
    CompressArgs job[kCompBatchMax];
};
hipError_t launch_compress_batch(const CompressArgs* jobs, int n, int x_dtype, hipStream_t st);
// one token per sequence of each job (tok_start: the token's position), the
// per-token form of the block compression with a running state per sequence
hipError_t launch_compress_step(const CompressArgs* jobs, int n, int x_dtype, hipStream_t st);

// ---- indexer + top-k
constexpr int kIdxSmallMaxKeys = 4096;   // one workgroup per query row up to this key count
constexpr int kIdxHistBins = 4096;       // first-level radix histogram (top 12 key bits)
constexpr int kIdxChunk = 4096;          // keys per workgroup in the large path
constexpr int kIdxMaxTopk = 2048;

struct IndexerArgs {
    const void* q;              // [rows][Hi][row bytes]
    const uint8_t* q_scales;    // [rows][Hi][di/32] (FP4)
    int32_t q_fmt;
    const float* w;             // [rows][Hi]
    const uint8_t* keys;        // [B][cap][row bytes]
    const uint8_t* key_scales;  // [B][cap][di/32] (FP4)
    int32_t key_fmt;
    int64_t cap;
    int32_t di, Hi, m, topk, Tq;
    const int32_t* q_pos;       // [rows]
    int32_t* out;               // [rows][topk]
    int32_t row0;               // first row of this launch batch
    int32_t rows;               // rows in this batch
    uint8_t* ws;                // per-row workspace slabs (large path)
    int64_t ws_row_bytes;
};
int64_t idx_ws_row_bytes(int64_t cap, int32_t topk);
// query-batched prefill path of the indexer (FP4 queries and keys): chunks of
// at least 32 query rows, di 64, four heads, caps up to 2^19 blocks, topk up
// to 1024; per query row a header, 8192 above-threshold candidate slots and
// 8 x 1024 tie slots
constexpr int kIdxPfMinTq = 32;
constexpr int64_t kIdxPfMaxCap = (int64_t)1 << 19;
constexpr int kIdxPfMaxTopk = 1024;
constexpr int kIdxPfCands = 8192;
inline bool idx_prefill_eligible(int32_t di, int32_t Hi, int32_t Tq, int64_t cap, int32_t topk) {
    return di == 64 && Hi == 4 && Tq >= kIdxPfMinTq && cap > kIdxSmallMaxKeys && cap <= kIdxPfMaxCap &&
           topk <= kIdxPfMaxTopk;
}
// the decode path (short chunks, FP4 queries and keys, caps up to 2^18):
// sampled thresholds, per-workgroup candidate segments, exact select
constexpr int64_t kIdxDecMaxCap = (int64_t)1 << 18;
inline bool idx_decode_eligible(int32_t di, int32_t Hi, int32_t Tq, int64_t cap, int32_t topk) {
    return di == 64 && Hi == 4 && Tq < kIdxPfMinTq && cap > kIdxSmallMaxKeys && cap <= kIdxDecMaxCap &&
           topk <= kIdxPfMaxTopk;
}
constexpr int64_t idx_prefill_row_bytes() { return 128 + (int64_t)kIdxPfCands * 8 + 8 * kIdxPfMaxTopk * 4; }
// decode rows: a 1024-byte header, then per 4096-key segment 1024 (key, j)
// slots, then per segment 4096 tie slots
constexpr int64_t idx_decode_row_bytes(int64_t cap) {
    return 1024 + (cap + 4095) / 4096 * (1024 * 8 + 4096 * 4);
}
hipError_t launch_indexer_topk(IndexerArgs a, int64_t total_rows, int64_t ws_bytes, hipStream_t st);

// ---- attention
struct AttnArgs {
    const void* q;              // [rows][H][d]
    int32_t q_fmt;
    const int32_t* q_pos;       // [rows]
    const int32_t* topk;        // [rows][k] or null (dense)
    int32_t k;
    const uint8_t* comp;        // [B][ccap] records
    int32_t comp_fmt;
    int64_t ccap;
    int32_t comp_rec;
    const uint8_t* win;         // [B][wcap] records (ring)
    int32_t win_fmt;
    int64_t wcap;
    int32_t win_rec;
    const float* gamma_q;       // [d] or null
    const float* sink;          // [H]
    int32_t d, dr, W, m;
    float base, scale, eps;
    int32_t Tq, H, rows;
    int32_t split_tq;           // chunk length the split policy sees (1: the decode splits always)
    void* out;                  // [rows][H][d]
    int32_t out_fmt;
    void* ws;
    int64_t ws_bytes;
    int32_t nsplit_max;         // splits per row in the partial buffers (set by the launcher)
    int32_t part_bf16;          // split partials of O stored in bf16 (set by the launcher)
    RopeTable rope;
};
int64_t attn_ws_bytes(int64_t rows, int32_t split_tq, int32_t H, int32_t d, int64_t max_entries);

// Split policy of the attention kernels: entries per split for a query row
// with n entries.  It depends only on the row's own entry count and on the
// chunk length Tq, never on the batch size, so a sequence's result does not
// depend on the batch it is in (the fixed policy passes Tq = 1 for every
// chunk, so neither does it depend on the chunk length).  Chunks of >= 64 queries give one split per
// row (enough rows to fill the chip); shorter chunks (decode) cut a row into
// at most 64 splits of at least 32 entries, a multiple of 32.
// (templated on the integer type: device code uses 32-bit arithmetic)
template <typename I>
__host__ __device__ inline I attn_split_len(I n, int32_t Tq) {
    if (n <= 0) return 32;
    if (Tq >= 64) return (n + 31) / 32 * 32;
    I s = (n + 63) / 64;
    s = (s + 31) / 32 * 32;
    return s < 32 ? 32 : s;
}
template <typename I>
__host__ __device__ inline I attn_nsplit(I n, int32_t Tq) {
    return n <= 0 ? 1 : (n + attn_split_len(n, Tq) - 1) / attn_split_len(n, Tq);
}
// an upper bound of attn_nsplit over rows with at most max_n entries
inline int64_t attn_nsplit_bound(int64_t max_n, int32_t Tq) {
    if (Tq >= 64 || max_n <= 0) return 1;
    int64_t b = (max_n + 31) / 32;
    return b > 64 ? 64 : b;
}
hipError_t launch_attention(const AttnArgs& a, int64_t max_entries, hipStream_t st);
bool attn_mfma_supported(const AttnArgs& a);
hipError_t launch_attention_mfma(const AttnArgs& a, int64_t max_entries, hipStream_t st);

// ---- grouped projection
struct ProjArgs {
    const void* o;
    const void* W;
    void* y;
    int64_t M;
    int32_t Hd, D, G;
    int32_t fmt;                // o / W dtype
    int32_t y_fmt;
};
hipError_t launch_proj(const ProjArgs& a, hipStream_t st);

// ---- projections with FP8 weights (csa_linear_fp8, csa_layer_in_proj)
// Output columns [n0, next segment's n0) go to out[m * ld + (n - n0)] in fmt
// (CSA_F32 or CSA_BF16); segments sorted by n0, the first at 0.
constexpr int kLinMaxSeg = 5;
constexpr int64_t kLinSkinnyMaxM = 64;   // rows handled by the weight-stream kernel
struct LinSeg {
    int32_t n0;
    int32_t fmt;
    int64_t ld;
    void* out;
};
struct LinArgs {
    const uint16_t* x;          // [M][K] bf16
    int64_t M;
    int32_t K, N, G;
    const uint8_t* W;           // [N][K/G] E4M3 codes
    const float* scale;         // [N]
    int32_t nseg;
    LinSeg seg[kLinMaxSeg];
};
hipError_t launch_lin8(const LinArgs& a, hipStream_t st);
int64_t lin8_max_tiles(int64_t M, int32_t N, int32_t G);
// FP4 quantisation of rows of n f32 values (the indexer-key rule)
hipError_t launch_fp4_rows(const float* x, int64_t rows, int n, uint8_t* codes, uint8_t* scales, hipStream_t st);

}  // namespace csa
