// attn_mfma.hip -- MFMA kernel of csa_sparse_mqa_attn / hca_dense_mqa_attn for
// bf16 queries over bf16 / FP8 caches (gfx950, v_mfma_f32_16x16x32_bf16).
//
// Same method and decomposition as attn.hip (peacm.com section 3.2: MQA over
// the selected compressed entries plus the raw window, Q/KV RMSNorm, partial
// RoPE with the -i output RoPE, sink logit in the denominator), arranged for
// the matrix cores of one CU:
//   - one query row (up to 64 heads) per workgroup and split, eight waves
//     (two per SIMD): wave w takes the 32 heads of half w/4 (with at most 32
//     heads, the 16 heads of group w/4) and the quarter w%4 of the head
//     dimension D.  It holds those queries as MFMA A-fragments and that
//     block of the output as accumulators (64 fp32 per lane at D = 512, so
//     everything stays in plain VGPRs);
//   - a tile of 32 entries is shared by all heads (MQA: one KV vector per
//     entry serves every head).  FP8 records are expanded exactly to bf16
//     codes with the hardware OCP-E4M3 conversion; the row scale multiplies
//     the non-RoPE part of the logits and the probabilities used for the
//     non-RoPE output dims (scale * <q, code> = <q, scale * code>);
//   - the partial logits of the four quarters meet in LDS; wave g (< 4) owns
//     16-head group g, adds them in quarter order and runs the online softmax of
//     those heads (base-2 exponentials; the running maximum is raised only
//     when a tile exceeds it by more than a factor 2^8, so the accumulators
//     are rescaled rarely); P goes to LDS entry-major;
//   - P and V reach the MFMA through the gfx950 transposing LDS read
//     (ds_read_b64_tr_b16).  The P V k index runs over the tile's entries in
//     a permuted order chosen so that the rows read together fall in disjoint
//     LDS banks;
//   - records are fetched straight into LDS with the gfx950 global-to-LDS
//     load (global_load_lds_dwordx4) by waves 4..7; record addresses are
//     computed one lane per entry and the top-k indices are read ahead.
//     When every record is FP8 (the layout the method stores), the records
//     stay as fetched in a ring of three tile buffers and the MFMA operands
//     are converted on the way out of LDS: K rows with 64-bit reads, V
//     columns with the byte-transposing read (ds_read_b64_tr_b8).  Other
//     formats go through a staging area and are expanded to bf16 rows;
//   - software pipeline, two LDS-only barriers per tile: phase 1 (all waves)
//     runs P V of tile t-1 and Q K^T of tile t back to back on the matrix
//     cores; phase 2 runs the softmax of tile t (waves 0..3) beside the fetch
//     work (waves 4..7), whose copies stay in flight through the next phase 1.
//     The dispatch on the dim quarter (which K-steps and N-tiles are FP8
//     codes, which RoPE dims) sits outside the tile loop.
#include <map>
#include <mutex>
#include <stddef.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kMTE = 32;                  // entries per LDS tile
constexpr int kNW = 8;                    // waves per workgroup
constexpr int kFetchers = 4;              // waves 4..7 fetch and expand the tiles
constexpr int kEntPerWave = kMTE / kFetchers;   // entries of a tile per fetching wave (slots f + 4u)
constexpr int kPRow = 80;                 // bf16 per P row (64 heads + pad: 160-byte rows)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;          // base-2 headroom before the running max is raised

// FP8 record bytes: D - DR codes, DR bf16, the f32 scale, padded to 16 bytes
template <int D, int DR>
constexpr int fp8_rec_bytes() { return ((D - DR) + 2 * DR + 4 + 15) / 16 * 16; }

template <int D, int DR, bool F8>
struct MfmaTiles;
// any record formats: a staging area and double-buffered bf16 rows
template <int D, int DR>
struct MfmaTiles<D, DR, false> {
    static constexpr int kBufs = 2;
    uint8_t tile[2][kMTE][D * 2 + 16];    // bf16 entries (FP8 codes expanded), 16-byte row pad
    uint8_t raw[kMTE][D * 2];             // records of the next tile as fetched (bf16 records are the largest)
    float scale[2][kMTE];                 // FP8 row scale (1 for bf16 records)
    int valid[2][kMTE];
};
// all FP8: the records as fetched, a ring of three tiles
template <int D, int DR>
struct MfmaTiles<D, DR, true> {
    static constexpr int kBufs = 3;
    uint8_t ring[3][kMTE][fp8_rec_bytes<D, DR>()];
    int valid[3][kMTE];
};

template <int D, int DR, bool F8>
struct MfmaSmem : MfmaTiles<D, DR, F8> {
    float zx[kNW][2][2][64][4];           // partial logits [wave][local head group][n][lane][i]
    uint16_t pt[2][kMTE][kPRow];          // P [scaled, plain] by (k index, head)
    float alpha[64];                      // per-head rescale factor of the current tile
    float fin[64];                        // per-head final factor (single-split rows)
    float ssq[4][64];                     // per-quarter sums of squares of the queries
    alignas(8) int moved[4];              // per head group: accumulators need rescaling
    float2 qsc[DR / 2];                   // (sin, cos) of t * freq, per RoPE pair (query)
    float2 osc[DR / 2];                   // (sin, cos) of -t * freq (output)
};

// ---- per-row entry enumeration (wave-uniform)
struct RowCtx {
    const uint8_t* comp;      // this sequence's compressed records
    const int32_t* top;       // this row's top-k list (null: dense)
    const uint8_t* win;       // this sequence's window ring
    int32_t nc, vis;          // compressed slots, visible blocks
    int32_t slot0;            // ring slot of entry nc (< 0: before the sequence start)
};

__device__ __forceinline__ uint32_t pack_bf16x2(bf16x2_t v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}

// Per-wave fetch state of one tile: lane u < 8 holds the record address of
// the fetching wave's entry u (tile slot f + 4u); the masks say which entries exist
// and which are FP8 records.
struct Fetch {
    uint64_t ptr;         // per lane
    uint32_t vmask, fmask;
};

// index of this lane's entry in the top-k list (lanes 0..7), read ahead of use
__device__ __forceinline__ int32_t fetch_index(const AttnArgs& a, const RowCtx& c, int32_t et, int32_t e1, int w,
                                               int lane) {
    // unconditional load at a clamped entry (no branch around it, so the
    // compiler's wait counts stay exact); the value is used only where valid
    const int32_t e = et + w + kFetchers * lane;
    return c.top ? c.top[min(e, c.nc - 1)] : 0;
}

// record addresses of the wave's entries of the tile at et (j: fetch_index).
// Branch-free over lanes: both the compressed and the window address are
// formed and one is selected (a per-lane choice between two argument fields
// would otherwise become a vector load from the argument segment).
__device__ __forceinline__ Fetch fetch_plan(const AttnArgs& a, const RowCtx& c, int32_t et, int32_t e1, int w,
                                            int lane, int32_t j) {
    const int32_t e = et + w + kFetchers * lane;
    const bool comp8 = a.comp_fmt == CSA_FP8_E4M3, win8 = a.win_fmt == CSA_FP8_E4M3;
    const bool inr = lane < kEntPerWave && e < e1;
    const bool isc = e < c.nc;
    const int32_t jj = c.top ? j : e;
    int32_t sl = c.slot0 + (e - c.nc);
    if (sl >= a.wcap) sl -= (int32_t)a.wcap;
    const bool ok = inr && (isc ? (jj >= 0 && jj < c.vis) : sl >= 0);
    const uint8_t* p = isc ? c.comp + (int64_t)jj * a.comp_rec : c.win + (int64_t)sl * a.win_rec;
    const bool fp8 = isc ? comp8 : win8;
    Fetch f;
    f.ptr = (uint64_t)(uintptr_t)p;
    f.vmask = (uint32_t)__ballot(ok);
    f.fmask = (uint32_t)__ballot(ok && fp8);
    return f;
}

// issue the global-to-LDS copies of the wave's records: entry u to row
// dst + (w + 4u) * stride
template <int D, int DR>
__device__ __forceinline__ void fetch_issue(uint8_t* dst, int stride, int w, int lane, const Fetch& f) {
    constexpr int fp8_pieces = (D - DR) / 16 + DR / 8 + 1;
    constexpr uint32_t kAll = (1u << kEntPerWave) - 1;
    if (f.vmask == kAll && f.fmask == kAll) {
        // every entry present and an FP8 record: one exec mask for all copies
        if (lane < fp8_pieces) {
#pragma unroll
            for (int u = 0; u < kEntPerWave; u++) {
                const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)f.ptr, u);
                const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(f.ptr >> 32), u);
                const uint8_t* rec = (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
                __builtin_amdgcn_global_load_lds(rec + 16 * lane,
                                                 (__attribute__((address_space(3))) void*)(dst + (w + kFetchers * u) * stride), 16, 0, 0);
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        if (f.vmask & (1u << u)) {
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)f.ptr, u);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(f.ptr >> 32), u);
            const uint8_t* rec = (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
            const int npieces = (f.fmask & (1u << u)) ? fp8_pieces : D / 8;
            if (lane < npieces)
                __builtin_amdgcn_global_load_lds(rec + 16 * lane,
                                                 (__attribute__((address_space(3))) void*)(dst + (w + kFetchers * u) * stride), 16, 0, 0);
        }
    }
}

// expand the wave's fetched records into bf16 tile rows: FP8 codes exactly,
// RoPE dims copied, row scale and validity aside.  Branch-free over lanes:
// lane l writes bytes 16l..16l+15 of the row (FP8: codes 8l..8l+7 expanded,
// or a RoPE piece; bf16: the same bytes of the record); all reads first.
template <int D, int DR, typename Smem>
__device__ __forceinline__ void fetch_expand(Smem& sm, int buf, int w, int lane, const Fetch& f) {
    constexpr int dn = D - DR;
    constexpr uint32_t kAll = (1u << kEntPerWave) - 1;
    if (f.vmask == kAll && f.fmask == kAll) {
        // every entry present and an FP8 record: straight-line, selects only
        const bool code = lane < dn / 8;
        const int off = code ? 8 * lane : (lane < D / 8 ? dn + 16 * (lane - dn / 8) : 0);
        uint2 x[kEntPerWave], y[kEntPerWave];
        float sc[kEntPerWave];
#pragma unroll
        for (int u = 0; u < kEntPerWave; u++) {
            const uint8_t* src = sm.raw[w + kFetchers * u];
            x[u] = *reinterpret_cast<const uint2*>(src + off);
            y[u] = *reinterpret_cast<const uint2*>(src + off + 8);
            sc[u] = *reinterpret_cast<const float*>(src + dn + 2 * DR);
        }
        float mysc = sc[0];
#pragma unroll
        for (int u = 0; u < kEntPerWave; u++) {
            const uint32_t c0 = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].x, 1.0f, false));
            const uint32_t c1 = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].x, 1.0f, true));
            const uint32_t c2 = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].y, 1.0f, false));
            const uint32_t c3 = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].y, 1.0f, true));
            const uint4 o = code ? make_uint4(c0, c1, c2, c3) : make_uint4(x[u].x, x[u].y, y[u].x, y[u].y);
            if (lane < D / 8) *reinterpret_cast<uint4*>(&sm.tile[buf][w + kFetchers * u][16 * lane]) = o;
            mysc = lane == u ? sc[u] : mysc;
        }
        if (lane < kEntPerWave) {
            sm.scale[buf][w + kFetchers * lane] = mysc;
            sm.valid[buf][w + kFetchers * lane] = 1;
        }
        return;
    }
    uint2 x[kEntPerWave], y[kEntPerWave];
    float sc[kEntPerWave];
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        const bool fp8 = (f.fmask >> u) & 1u;
        const uint8_t* src = sm.raw[w + kFetchers * u];
        int off = fp8 ? (lane < dn / 8 ? 8 * lane : dn + 16 * (lane - dn / 8)) : 16 * lane;
        if (lane >= D / 8) off = 0;
        x[u] = *reinterpret_cast<const uint2*>(src + off);
        y[u] = *reinterpret_cast<const uint2*>(src + off + 8);
        sc[u] = fp8 ? *reinterpret_cast<const float*>(src + dn + 2 * DR) : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < kEntPerWave; u++) {
        const int ee = w + kFetchers * u;
        const bool ok = (f.vmask >> u) & 1u, fp8 = (f.fmask >> u) & 1u;
        uint4 o;
        if (fp8 && lane < dn / 8) {
            o.x = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].x, 1.0f, false));
            o.y = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].x, 1.0f, true));
            o.z = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].y, 1.0f, false));
            o.w = pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[u].y, 1.0f, true));
        } else {
            o = make_uint4(x[u].x, x[u].y, y[u].x, y[u].y);
        }
        // a masked entry becomes a zero row, which keeps 0 * garbage out of P V
        if (!ok) o = make_uint4(0u, 0u, 0u, 0u);
        if (lane < D / 8) *reinterpret_cast<uint4*>(&sm.tile[buf][ee][16 * lane]) = o;
        if (lane == 0) {
            sm.scale[buf][ee] = ok ? sc[u] : 1.0f;
            sm.valid[buf][ee] = ok ? 1 : 0;
        }
    }
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations
// complete, then s_barrier.  __syncthreads() would also wait for every
// global-to-LDS copy in flight (they count as LDS writes); the copies of a
// ring buffer are waited for explicitly (wait_vm) by the waves that issued
// them, before the barrier that publishes the buffer.  The memory clobber
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait for this wave's global-to-LDS copies (vmcnt 0), and for its LDS reads
// before the staging area is refilled (lgkmcnt 0)
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// gfx950 transposing LDS read of four bf16 (ds_read_b64_tr_b16).  Within each
// 16-lane group, lane s points at 4 consecutive bf16; lane i then receives,
// for j = 0..3, element i%4 of the 4 values addressed by lane i/4 + 4j.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* p) {
    typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// eight bf16 from two transposing reads (one vector reinterpretation: element
// by element casts of the 16-bit lanes have been lowered incorrectly)
__device__ __forceinline__ bf16x8_t tr_pair(const void* p0, const void* p1) {
    const s16x4_t v0 = lds_read_tr16(p0), v1 = lds_read_tr16(p1);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// eight E4M3 codes to eight bf16 (exact)
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint2 c) {
    const uint4 o = make_uint4(pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false)),
                               pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true)),
                               pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false)),
                               pack_bf16x2(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true)));
    return __builtin_bit_cast(bf16x8_t, o);
}

// gfx950 byte-transposing LDS read (ds_read_b64_tr_b8).  Within each 16-lane
// group, lane s points at 8 consecutive bytes; lane i then receives, for
// j = 0..7, byte i%8 of the 8 bytes addressed by lane i/8 + 2j.
__device__ __forceinline__ uint2 lds_read_tr8(const void* p) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p));
}

// position of tile entry e in the P V k order: k = 8g + 4h + j holds entry
// 8g + h + 2j, so the four V rows one transposing read covers are two apart
// (row pitch = 4 banks mod 32: offsets 0, 8, 16, 24 banks)
__device__ __forceinline__ int pv_k_of_entry(int e) { return (e & ~7) + 4 * (e & 1) + ((e & 7) >> 1); }

// MTW: 16-head groups per wave.  2: wave w takes the 32 heads of half w / 4
// (64 heads per workgroup); 1: wave w takes the 16 heads of group w / 4 (a
// workgroup of at most 32 heads keeps all eight waves busy in the products).
// LOOP: the workgroup runs splits blockIdx.x, blockIdx.x + gridDim.x, ...
// of its row (instantiated for d = 512 and launched only when a row's splits
// outnumber its workgroups: the loop keeps the query fragments live through
// the epilogue, more registers than a single split needs).
template <int D, int DR, bool F8, typename OT, int MTW, bool LOOP>
__global__ __launch_bounds__(kNW * 64) void k_attn_mfma(AttnArgs a) {
    warm_kernargs(offsetof(AttnArgs, rope));
    constexpr int DQ = D / 4;              // dims per quarter
    constexpr int KS = DQ / 32;            // Q K^T K-steps per wave
    constexpr int NT = DQ / 16;            // P V N-tiles per wave
    constexpr int dn = D - DR;             // non-RoPE dims (multiple of 32)
    static_assert(DR / 2 <= 32, "one RoPE pair per lane of half a wave");
    constexpr int RS = D * 2 + 16;         // bf16 tile row stride in bytes
    constexpr int REC = fp8_rec_bytes<D, DR>();   // FP8 ring row stride in bytes
    constexpr uint32_t kAll = (1u << kEntPerWave) - 1;
    __shared__ MfmaSmem<D, DR, F8> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qd = w & 3, hp = w >> 2;                 // dim quarter, head half
    const int g0 = MTW * hp;                           // this wave's first 16-head group
    const int l16 = lane & 15, g4 = lane >> 4;
    const int row = blockIdx.y;
    const int h0 = blockIdx.z * 64;
    const int MT = min(4, (a.H - h0) / 16);           // 16-head groups in this workgroup
    const int dbase = qd * DQ;                         // first dim of this wave's quarter

    // ---- sparse rows: the entry layout (k top-k entries, then the window)
    // does not depend on the position, so the fetching waves read the first
    // tiles' top-k indices first of all.  Loads return in order: issued after
    // the query, the wait for an index would wait for the whole query, and
    // the first records would go out only once the query had arrived.
    const int fw = w - (kNW - kFetchers);              // fetching wave index (>= 0 for waves 4..7)
    const bool fetcher = fw >= 0;
    const bool sparse = a.topk != nullptr;
    int32_t jf0 = 0, jf1 = 0, jf2 = 0;
    if (sparse && fetcher && a.k > 0) {
        const int32_t split_s = attn_split_len<int32_t>(a.k + a.W, a.split_tq);
        const int32_t eb = (int32_t)blockIdx.x * split_s + fw + kFetchers * lane;
        const int32_t* top = a.topk + (int64_t)row * a.k;
        jf0 = top[min(eb, a.k - 1)];
        jf1 = top[min(eb + kMTE, a.k - 1)];
        jf2 = top[min(eb + 2 * kMTE, a.k - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- then the query loads (they do not depend on the position either).
    // No load sits under a branch: a head group beyond MT reads group 0 (its
    // results are never stored), and without gamma the loads read the query
    // and are replaced by ones.
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)row * a.H + h0) * D;
    uint4 qraw[MTW][KS];
#pragma unroll
    for (int mt = 0; mt < MTW; mt++) {
        const int hg = (g0 + mt < MT) ? 16 * (g0 + mt) : 0;
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            qraw[mt][ks] = *reinterpret_cast<const uint4*>(qb + (hg + l16) * D + dbase + 32 * ks + 8 * g4);
    }
    float4 gam[KS][2];
    const bool hasg = a.gamma_q != nullptr;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const float* gsrc = hasg ? a.gamma_q + dbase + 32 * ks + 8 * g4 : reinterpret_cast<const float*>(a.q);
        const float4 g0 = reinterpret_cast<const float4*>(gsrc)[0], g1 = reinterpret_cast<const float4*>(gsrc)[1];
        // component selects (a select of whole vectors became a private-array lookup)
        gam[ks][0] = make_float4(hasg ? g0.x : 1.0f, hasg ? g0.y : 1.0f, hasg ? g0.z : 1.0f, hasg ? g0.w : 1.0f);
        gam[ks][1] = make_float4(hasg ? g1.x : 1.0f, hasg ? g1.y : 1.0f, hasg ? g1.z : 1.0f, hasg ? g1.w : 1.0f);
    }

    const int b = row / a.Tq;
    const int t = load_uniform_i32(a.q_pos + row);
    // the RoPE factors of the position, for the query (t) and the output
    // (-t), one pair per lane of wave 0, computed while the query loads are
    // in flight (read after the prologue's barrier)
    if (w == 0 && (lane & 31) < DR / 2) {
        const double* rfa = (const double*)((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(AttnArgs, rope));
        const int p = lane & 31;
        float sn, cs;
        rope_sincos(lane < 32 ? (double)t : -(double)t, rfa[p], sn, cs);
        (lane < 32 ? sm.qsc : sm.osc)[p] = make_float2(sn, cs);
    }
    RowCtx c;
    c.vis = t < 0 ? 0 : (t + 1) / a.m;
    if (c.vis > a.ccap) c.vis = (int32_t)a.ccap;
    c.nc = a.topk ? a.k : c.vis;
    c.comp = a.comp + (int64_t)b * a.ccap * a.comp_rec;
    c.top = a.topk ? a.topk + (int64_t)row * a.k : nullptr;
    c.win = a.win + (int64_t)b * a.wcap * a.win_rec;
    {
        const int32_t s0 = t - a.W + 1;
        c.slot0 = (a.W > 0 && s0 >= 0) ? s0 % (int32_t)a.wcap : s0;
    }
    const int32_t ne = c.nc + a.W;
    const int32_t split = attn_split_len<int32_t>(ne, a.split_tq);
    const int32_t nsplit = attn_nsplit<int32_t>(ne, a.split_tq);
    // with LOOP the workgroup runs splits blockIdx.x, blockIdx.x + gridDim.x,
    // ... of its row one after another (the query prologue once); each split
    // is computed and stored exactly as by a workgroup of its own
    int32_t sp = blockIdx.x;
    if (sp >= nsplit) return;
    int32_t e0 = sp * split, e1 = min(e0 + split, ne);
    const bool active = g0 < MT;                       // this wave's first head group exists
    const bool owner = w < MT;                         // wave w runs the softmax of head group w
    // non-RoPE K-steps / N-tiles of this quarter
    const int nks = max(0, min(KS, (dn - dbase) / 32));
    const int nnt = max(0, min(NT, (dn - dbase) / 16));
    const float zscale = a.scale * kLog2e;             // logits in base-2 units

    int ntiles = (e1 - e0 + kMTE - 1) / kMTE;
    // the first tile's records go out before the query prologue; the top-k
    // indices are read two tiles ahead of their records
    Fetch fr;
    int32_t jn = 0;
    // FP8 ring: plan and send tile tt into ring buffer rb; record validity, and
    // zero the rows of missing entries (no stale codes reach P V)
    auto ring_issue = [&](int tt, int rb, int32_t j) __attribute__((always_inline)) {
        if constexpr (F8) {
            const Fetch f = fetch_plan(a, c, e0 + tt * kMTE, e1, fw, lane, j);
            fetch_issue<D, DR>(&sm.ring[rb][0][0], REC, fw, lane, f);
            if (lane < kEntPerWave) sm.valid[rb][fw + kFetchers * lane] = (f.vmask >> lane) & 1u;
            if (f.vmask != kAll) {
#pragma unroll
                for (int u = 0; u < kEntPerWave; u++)
                    if (!(f.vmask & (1u << u)) && lane < REC / 16)
                        *reinterpret_cast<uint4*>(&sm.ring[rb][fw + kFetchers * u][16 * lane]) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    // the first tiles' records go out as soon as their addresses are known:
    // the barrier after the query's square sums does not wait for them
    auto first_tiles = [&]() __attribute__((always_inline)) {
        if (fetcher) {
            if constexpr (F8) {
                jn = jf2;
                ring_issue(0, 0, jf0);
                if (ntiles > 1) ring_issue(1, 1, jf1);
            } else {
                jn = jf1;
                fr = fetch_plan(a, c, e0, e1, fw, lane, jf0);
                fetch_issue<D, DR>(&sm.raw[0][0], D * 2, fw, lane, fr);
            }
        }
    };
    first_tiles();
    // (LOOP) the next split's first top-k indices, read while this split runs
    int32_t nj0 = 0, nj1 = 0, nj2 = 0;
    auto next_indices = [&]() __attribute__((always_inline)) {
        if constexpr (LOOP) {
            const int32_t sn = sp + (int32_t)gridDim.x;
            if (sparse && fetcher && a.k > 0 && sn < nsplit) {
                const int32_t eb = sn * split + fw + kFetchers * lane;
                const int32_t* top = a.topk + (int64_t)row * a.k;
                nj0 = top[min(eb, a.k - 1)];
                nj1 = top[min(eb + kMTE, a.k - 1)];
                nj2 = top[min(eb + 2 * kMTE, a.k - 1)];
            }
        }
    };
    next_indices();

    // ---- query prologue: q^ = RoPE_t(RMSNorm(q)), this wave's 32 heads and quarter
#pragma unroll
    for (int mt = 0; mt < MTW; mt++) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const uint32_t wd[4] = {qraw[mt][ks].x, qraw[mt][ks].y, qraw[mt][ks].z, qraw[mt][ks].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(wd[j] << 16), x1 = __uint_as_float(wd[j] & 0xFFFF0000u);
                ss += x0 * x0 + x1 * x1;
            }
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        if (g4 == 0) sm.ssq[qd][16 * (g0 + mt) + l16] = ss;
    }
    lds_barrier();
    float inv[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; mt++) {
        const int hl = 16 * (g0 + mt) + l16;
        const float ss = ((sm.ssq[0][hl] + sm.ssq[1][hl]) + sm.ssq[2][hl]) + sm.ssq[3][hl];
        inv[mt] = 1.0f / sqrtf(ss / (float)D + a.eps);
    }
    bf16x8_t qf[MTW][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const float gv[8] = {gam[ks][0].x, gam[ks][0].y, gam[ks][0].z, gam[ks][0].w,
                             gam[ks][1].x, gam[ks][1].y, gam[ks][1].z, gam[ks][1].w};
        float sn[4], cs[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            sn[j] = 0.0f;
            cs[j] = 1.0f;
        }
        if (ks >= nks) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float2 v = sm.qsc[(dbase + 32 * ks + 8 * g4 + 2 * j - dn) / 2];
                sn[j] = v.x;
                cs[j] = v.y;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MTW; mt++) {
            const uint32_t wd[4] = {qraw[mt][ks].x, qraw[mt][ks].y, qraw[mt][ks].z, qraw[mt][ks].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x0 = __uint_as_float(wd[j] << 16) * inv[mt] * gv[2 * j];
                const float x1 = __uint_as_float(wd[j] & 0xFFFF0000u) * inv[mt] * gv[2 * j + 1];
                qf[mt][ks][2 * j] = (__bf16)(x0 * cs[j] - x1 * sn[j]);
                qf[mt][ks][2 * j + 1] = (__bf16)(x0 * sn[j] + x1 * cs[j]);
            }
        }
    }

    // P rows of a head group beyond MT are never written: its accumulators
    // collect garbage and are never stored
    f32x4_t o[MTW][NT];
#pragma unroll
    for (int mt = 0; mt < MTW; mt++)
#pragma unroll
        for (int nd = 0; nd < NT; nd++) o[mt][nd] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // running max (base 2) of the owned heads 16w + 4*g4 + i, and this lane's
    // part of their running sums (the 16 lanes of a row are added at the end)
    float mrun[4], lrun[4];
#pragma unroll
    for (int i = 0; i < 4; i++) { mrun[i] = -INFINITY; lrun[i] = 0.0f; }

    // (any formats) expand tile tt into buffer tt % 2, send the fetch of tile tt + 1;
    // (FP8 ring) wait for tile tt, send the fetch of tile tt + 1 into ring (tt + 1) % 3
    auto fetch_step = [&](int tt, int rb_next) __attribute__((always_inline)) {
        if (!fetcher || tt >= ntiles) return;
        const int32_t et = e0 + tt * kMTE;
        wait_vm();
        if constexpr (F8) {
            if (tt + 1 < ntiles) {
                ring_issue(tt + 1, rb_next, jn);
                jn = fetch_index(a, c, et + 2 * kMTE, e1, fw, lane);
            }
        } else {
            fetch_expand<D, DR>(sm, tt & 1, fw, lane, fr);
            wait_lgkm();
            if (tt + 1 < ntiles) {
                fr = fetch_plan(a, c, et + kMTE, e1, fw, lane, jn);
                fetch_issue<D, DR>(&sm.raw[0][0], D * 2, fw, lane, fr);
                jn = fetch_index(a, c, et + 2 * kMTE, e1, fw, lane);
            }
        }
    };
    // partial logits of tile tt (buffer tt % 2), this quarter, the wave's head
    // groups: scale * <q, code>_non-RoPE + <q, k>_RoPE, to LDS.  The quarter is
    // a template constant (QD), so the FP8/RoPE split of its K-steps is known at
    // compile time and every K fragment is read before the first product.
    auto qk_step = [&](auto qdc, int bq) __attribute__((always_inline)) {
        constexpr int DC = decltype(qdc)::value * DQ;
        constexpr int NKS = (dn - DC) / 32 < 0 ? 0 : ((dn - DC) / 32 > KS ? KS : (dn - DC) / 32);
        float esc[2];
        bf16x8_t kb[2][KS];
        if constexpr (F8) {
            uint2 kc[2][KS];
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const uint8_t* kr = &sm.ring[bq][16 * n + l16][0];
                esc[n] = *reinterpret_cast<const float*>(kr + dn + 2 * DR);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int dim = dbase + 32 * ks + 8 * g4;
                    if (ks < NKS) kc[n][ks] = *reinterpret_cast<const uint2*>(kr + dim);
                    else kb[n][ks] = *reinterpret_cast<const bf16x8_t*>(kr + dn + 2 * (dim - dn));
                }
            }
#pragma unroll
            for (int n = 0; n < 2; n++)
#pragma unroll
                for (int ks = 0; ks < NKS; ks++) kb[n][ks] = fp8x8_to_bf16(kc[n][ks]);
        } else {
#pragma unroll
            for (int n = 0; n < 2; n++) {
                const uint8_t* kr = &sm.tile[bq][16 * n + l16][2 * dbase + 16 * g4];
                esc[n] = sm.scale[bq][16 * n + l16];
#pragma unroll
                for (int ks = 0; ks < KS; ks++) kb[n][ks] = *reinterpret_cast<const bf16x8_t*>(kr + 64 * ks);
            }
        }
#pragma unroll
        for (int n = 0; n < 2; n++) {
            f32x4_t acc[MTW];
#pragma unroll
            for (int mt = 0; mt < MTW; mt++) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                if (ks == NKS && ks > 0) {
#pragma unroll
                    for (int mt = 0; mt < MTW; mt++) acc[mt] *= esc[n];
                }
#pragma unroll
                for (int mt = 0; mt < MTW; mt++)
                    acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mt][ks], kb[n][ks], acc[mt], 0, 0, 0);
            }
            if (NKS == KS) {
#pragma unroll
                for (int mt = 0; mt < MTW; mt++) acc[mt] *= esc[n];
            }
#pragma unroll
            for (int mt = 0; mt < MTW; mt++)
                *reinterpret_cast<f32x4_t*>(&sm.zx[w][mt][n][lane][0]) = acc[mt];
        }
    };
    // owner waves: add the quarters of tile tt in order, online softmax, publish P
    auto softmax_step = [&](int bq) __attribute__((always_inline)) {
        float esc[2];
        bool eok[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
            if constexpr (F8) esc[n] = *reinterpret_cast<const float*>(&sm.ring[bq][16 * n + l16][dn + 2 * DR]);
            else esc[n] = sm.scale[bq][16 * n + l16];
            eok[n] = sm.valid[bq][16 * n + l16] != 0;
        }
        const int src = 4 * (w / MTW), lg = w % MTW;    // waves holding this group's quarters
        f32x4_t z[2];
#pragma unroll
        for (int n = 0; n < 2; n++) {
            z[n] = *reinterpret_cast<const f32x4_t*>(&sm.zx[src][lg][n][lane][0]);
#pragma unroll
            for (int q = 1; q < 4; q++) z[n] += *reinterpret_cast<const f32x4_t*>(&sm.zx[src + q][lg][n][lane][0]);
        }
        float zz[2][4];
        bool over = false;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int n = 0; n < 2; n++) {
                zz[n][i] = eok[n] ? z[n][i] * zscale : -INFINITY;
                over |= zz[n][i] > mrun[i] + kLazyMax;
            }
        // the running max is raised only past the headroom (also for the first
        // finite logits); then the exact row max is taken and O, l rescaled
        if (__any(over)) {
            bool moved = false;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float mx = row16_max(fmaxf(zz[0][i], zz[1][i]));
                const bool up = mx > mrun[i] + kLazyMax;
                const float al = up ? __builtin_amdgcn_exp2f(mrun[i] - mx) : 1.0f;   // 0 from -inf
                moved |= up && mrun[i] != -INFINITY;
                mrun[i] = up ? mx : mrun[i];
                lrun[i] *= al;
                if (l16 == 0) sm.alpha[16 * w + 4 * g4 + i] = al;
            }
            const bool any_moved = __any(moved);
            if (lane == 0) sm.moved[w] = any_moved ? 1 : 0;
        } else if (lane == 0) {
            sm.moved[w] = 0;
        }
        float pz[2][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int n = 0; n < 2; n++)
                pz[n][i] = mrun[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(zz[n][i] - mrun[i]);
            lrun[i] += pz[0][i] + pz[1][i];           // per-lane partial row sums
        }
#pragma unroll
        for (int n = 0; n < 2; n++) {
            const int kk = pv_k_of_entry(16 * n + l16);
            uint2 ps, pp;
            ps.x = pack_bf16x2(bf16x2_t{(__bf16)(pz[n][0] * esc[n]), (__bf16)(pz[n][1] * esc[n])});
            ps.y = pack_bf16x2(bf16x2_t{(__bf16)(pz[n][2] * esc[n]), (__bf16)(pz[n][3] * esc[n])});
            pp.x = pack_bf16x2(bf16x2_t{(__bf16)pz[n][0], (__bf16)pz[n][1]});
            pp.y = pack_bf16x2(bf16x2_t{(__bf16)pz[n][2], (__bf16)pz[n][3]});
            *reinterpret_cast<uint2*>(&sm.pt[0][kk][16 * w + 4 * g4]) = ps;
            *reinterpret_cast<uint2*>(&sm.pt[1][kk][16 * w + 4 * g4]) = pp;
        }
    };
    // per-lane LDS coordinates of the transposing reads
    const int v_row = 8 * g4 + 2 * (l16 >> 2);
    const int p_row = 8 * g4 + (l16 >> 2);
    const int p_col = 16 * g0 + 4 * (l16 & 3);
    // rescale O of the head groups whose max moved at tile tt (rare), then
    // O += P V.  The quarter is a template constant: the FP8/RoPE split of its
    // N-tiles is static, and the flags, P fragments and V fragments are all
    // read before the first product.
    auto pv_step = [&](auto qdc, int bq) __attribute__((always_inline)) {
        constexpr int DC = decltype(qdc)::value * DQ;
        constexpr int NNT = (dn - DC) / 16 < 0 ? 0 : ((dn - DC) / 16 > NT ? NT : (dn - DC) / 16);
        int mv[MTW];
#pragma unroll
        for (int mt = 0; mt < MTW; mt++) mv[mt] = sm.moved[g0 + mt];      // g0 + mt <= 3
        // P A-fragments: scaled P for the non-RoPE dims, plain P for the RoPE dims
        bf16x8_t pfs[MTW], pfp[MTW];
#pragma unroll
        for (int mt = 0; mt < MTW; mt++) {
            if (NNT > 0) pfs[mt] = tr_pair(&sm.pt[0][p_row][16 * mt + p_col], &sm.pt[0][p_row + 4][16 * mt + p_col]);
            if (NNT < NT) pfp[mt] = tr_pair(&sm.pt[1][p_row][16 * mt + p_col], &sm.pt[1][p_row + 4][16 * mt + p_col]);
        }
        bf16x8_t vb[NT];
        if constexpr (F8) {
            // lane (g4, s) addresses entry pi(8*g4 + s/2): bytes of 8 FP8 dims,
            // or 4 bf16 RoPE dims of rows pi(8*g4 + 4h + s/4)
            const uint8_t* rb = &sm.ring[bq][0][0];
            uint2 vc[NT];
#pragma unroll
            for (int nd = 0; nd < NT; nd++) {
                if (nd < NNT) {
                    const int r = 8 * g4 + (l16 >> 3) + 2 * ((l16 >> 1) & 3);
                    vc[nd] = lds_read_tr8(rb + r * REC + dbase + 16 * nd + 8 * (l16 & 1));
                } else {
                    const int cb = dn + 2 * (dbase + 16 * nd - dn + 4 * (l16 & 3));
                    vb[nd] = tr_pair(rb + v_row * REC + cb, rb + (v_row + 1) * REC + cb);
                }
            }
#pragma unroll
            for (int nd = 0; nd < NNT; nd++) vb[nd] = fp8x8_to_bf16(vc[nd]);
        } else {
            const uint8_t* vp = &sm.tile[bq][v_row][2 * (dbase + 4 * (l16 & 3))];
#pragma unroll
            for (int nd = 0; nd < NT; nd++) vb[nd] = tr_pair(vp + 32 * nd, vp + RS + 32 * nd);
        }
#pragma unroll
        for (int mt = 0; mt < MTW; mt++) {
            const int g = g0 + mt;
            if (g < MT && mv[mt]) {
                const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[16 * g + 4 * g4]);
#pragma unroll
                for (int nd = 0; nd < NT; nd++) {
                    o[mt][nd][0] *= al.x;
                    o[mt][nd][1] *= al.y;
                    o[mt][nd][2] *= al.z;
                    o[mt][nd][3] *= al.w;
                }
            }
        }
#pragma unroll
        for (int nd = 0; nd < NT; nd++)
#pragma unroll
            for (int mt = 0; mt < MTW; mt++)
                o[mt][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(nd < NNT ? pfs[mt] : pfp[mt], vb[nd], o[mt][nd], 0, 0, 0);
    };
    // the tile loop for this wave's quarter (wave-uniform dispatch, outside
    // the loop).  Quarters with the same split into non-RoPE and RoPE dims
    // share one instantiation (the quarter's base dim is a runtime value):
    // quarters 0 .. QF-1 hold only non-RoPE dims, quarter QF holds the
    // boundary (or only RoPE dims, as do the ones after it).  Dispatching per
    // tile instead made the register allocator move the output accumulators
    // between the instantiations' registers on every tile.
    constexpr int QF = dn / DQ;
    static_assert(QF < 4, "the RoPE dims take part of the last quarter");
    constexpr bool kMixed = dn % DQ != 0;
    auto with_quarter = [&](auto&& f) {
        if (qd < QF) f(std::integral_constant<int, 0>{});
        else if (!kMixed || qd == QF) f(std::integral_constant<int, QF>{});
        else f(std::integral_constant<int, 3>{});
    };

    // ---- software pipeline over the tiles; per tile two barriers:
    //   phase 1 (all waves):   O += P V of tile t-1, partial logits of tile t
    //   phase 2: waves < MT run the softmax of tile t while the fetching waves
    //            expand tile t+1 and send the fetch of tile t+2
    // buffers: any formats, tile t in bf16 buffer t % 2; FP8 ring, tile t in ring t % 3
    constexpr int NB = MfmaTiles<D, DR, F8>::kBufs;
    // the quarter dispatch sits outside the split loop too, so that the
    // output accumulators keep one register set (the epilogue's returns end
    // the kernel)
    with_quarter([&](auto qdc) {
    for (;;) {                                          // this workgroup's splits
    if constexpr (F8) {
        if (fetcher) wait_vm();
    } else {
        fetch_step(0, 0);
    }
    __syncthreads();
    {
        int bcur = 0, bprev = NB - 1;
        for (int tt = 0; tt < ntiles; tt++) {
            if (active) {
                if (tt > 0) pv_step(qdc, bprev);
                qk_step(qdc, bcur);
            }
            lds_barrier();
            if (owner) softmax_step(bcur);
            if constexpr (F8) {
                int bn2 = bcur + 2;
                if (bn2 >= NB) bn2 -= NB;
                fetch_step(tt + 1, bn2);      // waits for tile tt+1, sends tile tt+2
            } else {
                fetch_step(tt + 1, 0);
            }
            // LDS-only barriers: the copies of the tile just sent stay in
            // flight through the next step (fetch_step waits for them)
            lds_barrier();
            bprev = bcur;
            bcur = bcur + 1 == NB ? 0 : bcur + 1;
        }
        if (active && ntiles > 0) pv_step(qdc, bprev);
    }

    // ---- epilogue
#pragma unroll
    for (int i = 0; i < 4; i++) lrun[i] = row16_sum(lrun[i]);
    if (nsplit <= 1) {
        if (owner) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int hr = 16 * w + 4 * g4 + i;
                const float sk = a.sink[h0 + hr] * kLog2e, mr = mrun[i];
                const float M = fmaxf(mr, sk);
                float f = 0.0f;
                if (mr != -INFINITY && M != -INFINITY) {
                    const float em = exp2f(mr - M);
                    f = em / (lrun[i] * em + exp2f(sk - M));
                }
                if (l16 == 0) sm.fin[hr] = f;
            }
        }
        __syncthreads();
        if (!active) return;
        OT* out = reinterpret_cast<OT*>(a.out) + ((int64_t)row * a.H + h0) * D;
#pragma unroll
        for (int nd = 0; nd < NT; nd++) {
            const int dim = dbase + 16 * nd + l16;
            const bool rope = nd >= nnt;
            float sn = 0.0f, cs = 1.0f;
            if (rope) {
                const float2 v = sm.osc[(dim - dn) / 2];
                sn = v.x;
                cs = v.y;
            }
#pragma unroll
            for (int mt = 0; mt < MTW; mt++) {
                const int g = g0 + mt;
                if (g < MT) {
                    const float4 f = *reinterpret_cast<const float4*>(&sm.fin[16 * g + 4 * g4]);
                    const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        float v = o[mt][nd][i] * fv[i];
                        if (rope) {
                            const float pv = __shfl_xor(v, 1, kWave);
                            v = (dim & 1) ? pv * sn + v * cs : v * cs - pv * sn;
                        }
                        st_scalar<OT>(out, (size_t)(16 * g + 4 * g4 + i) * D + dim, v);
                    }
                }
            }
        }
        return;
    }
    // partial results of this split: unnormalised O, and (max, sum) in natural-log units.
    // O goes through LDS (the tile and logit areas are free now) so that the
    // global stores are whole 16-byte vectors: in bf16 (bf16 outputs: the
    // partial is rounded once more, half the bytes of the split round trip)
    // all heads at once, in fp32 32 heads at a time.
    float* wo = reinterpret_cast<float*>(a.ws);
    float* wml = wo + (size_t)a.rows * a.nsplit_max * a.H * D;
    const size_t base = ((size_t)row * a.nsplit_max + sp) * a.H + h0;
    static_assert(sizeof(MfmaTiles<D, DR, F8>) + sizeof(sm.zx) >= 32 * (D + 4) * sizeof(float),
                  "partial staging does not fit");
    static_assert(sizeof(MfmaTiles<D, DR, F8>) + sizeof(sm.zx) >= 64 * (D + 8) * sizeof(uint16_t),
                  "bf16 partial staging does not fit");
    if constexpr (sizeof(OT) == 2) {
        uint16_t* ost = reinterpret_cast<uint16_t*>(&sm);     // [64 heads][D + 8]
        __syncthreads();
        if (active) {
#pragma unroll
            for (int mt = 0; mt < MTW; mt++)
#pragma unroll
                for (int nd = 0; nd < NT; nd++)
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        ost[(16 * (g0 + mt) + 4 * g4 + i) * (D + 8) + dbase + 16 * nd + l16] =
                            f32_to_bf16(o[mt][nd][i]);
        }
        __syncthreads();
        const int nv = 16 * MT * (D / 8);                  // 16-byte vectors of the valid heads
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.ws) + base * D);
        for (int v = tid; v < nv; v += kNW * 64) {
            const int h = v / (D / 8), c8 = v % (D / 8);
            dst[v] = *reinterpret_cast<const uint4*>(&ost[h * (D + 8) + 8 * c8]);
        }
    } else {
        float* ost = reinterpret_cast<float*>(&sm);     // [32 heads][D + 4]
#pragma unroll
        for (int half = 0; half < 2; half++) {
            if (2 * half >= MT) break;
            __syncthreads();
#pragma unroll
            for (int mt = 0; mt < MTW; mt++) {
                const int g = g0 + mt;                       // head group; half g / 2
                if ((g >> 1) == half) {
#pragma unroll
                    for (int nd = 0; nd < NT; nd++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            ost[(16 * (g & 1) + 4 * g4 + i) * (D + 4) + dbase + 16 * nd + l16] = o[mt][nd][i];
                }
            }
            __syncthreads();
            const int nv = min(32, 16 * MT - 32 * half) * (D / 4);      // float4s of the valid heads
            float4* dst = reinterpret_cast<float4*>(wo + (base + 32 * half) * D);
            for (int v = tid; v < nv; v += kNW * 64) {
                const int h = v / (D / 4), c4 = v % (D / 4);
                dst[v] = *reinterpret_cast<const float4*>(&ost[h * (D + 4) + 4 * c4]);
            }
        }
    }
    if (owner && l16 == 0) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const size_t hr = base + 16 * w + 4 * g4 + i;
            wml[hr * 2] = mrun[i] * kLn2;
            wml[hr * 2 + 1] = lrun[i];
        }
    }
    // ---- the next split of this workgroup: its entries, top-k indices and
    // first records (once every wave has read the staged partial out of
    // LDS), then fresh accumulators
    sp += (int32_t)gridDim.x;
    if (!LOOP || sp >= nsplit) return;                  // workgroup-uniform
    e0 = sp * split;
    e1 = min(e0 + split, ne);
    ntiles = (e1 - e0 + kMTE - 1) / kMTE;
    __syncthreads();
    jf0 = nj0;
    jf1 = nj1;
    jf2 = nj2;
    first_tiles();
    next_indices();
#pragma unroll
    for (int mt = 0; mt < MTW; mt++)
#pragma unroll
        for (int nd = 0; nd < NT; nd++) o[mt][nd] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    mrun[0] = mrun[1] = mrun[2] = mrun[3] = -INFINITY;
    lrun[0] = lrun[1] = lrun[2] = lrun[3] = 0.0f;
    }
    });
}

bool attn_mfma_supported(const AttnArgs& a) {
    if (a.q_fmt != CSA_BF16) return false;
    if (a.comp_fmt == CSA_F32 || (a.W > 0 && a.win_fmt == CSA_F32)) return false;
    if (a.d != 128 && a.d != 256 && a.d != 512) return false;
    if (a.H % 16 != 0) return false;
    if (a.dr != 64) return false;
    return true;
}

// Workgroups of kernel k resident on the whole current device at once (CUs
// times the workgroups one CU holds), cached per (device, kernel); 0 when
// the runtime cannot say.
static int resident_wgs(const void* k) {
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    const auto key = std::make_pair(dev, k);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, kNW * 64, 0) != hipSuccess)
        return 0;
    const int v = cus * (per > 0 ? per : 1);
    cache[key] = v;
    return v;
}

template <bool F8, typename OT>
static void launch_d(const AttnArgs& a0, int nsplit, hipStream_t st) {
    AttnArgs a = a0;
    a.nsplit_max = nsplit;                              // part_bf16: set by launch_attention
    const int groups = (a.H + 63) / 64;
    // eight waves per workgroup always (head groups x dim quarters); a
    // workgroup covers up to 64 heads, or with at most 32 heads (d 512) one
    // 16-head group per wave, so that all eight waves multiply
    void (*k)(AttnArgs) = a.d == 128 ? k_attn_mfma<128, 64, F8, OT, 2, false>
                        : a.d == 256 ? k_attn_mfma<256, 64, F8, OT, 2, false>
                        : a.H <= 32  ? k_attn_mfma<512, 64, F8, OT, 1, false>
                                     : k_attn_mfma<512, 64, F8, OT, 2, false>;
    // split slots per row: every split its own workgroup while they all fit
    // on the chip at once; beyond that (d = 512) as many slots as fit, each
    // workgroup running several splits of its row in turn (the query
    // prologue is paid once per workgroup, not once per split).  A split's
    // result does not depend on the workgroup that runs it, so neither does
    // any output bit.
    int gx = nsplit;
    const int64_t per_slot = (int64_t)a.rows * groups;
    const int slots = a.d == 512 ? resident_wgs(reinterpret_cast<const void*>(k)) : 0;
    if (slots > 0 && nsplit > 1 && per_slot * nsplit > slots) {
        gx = (int)std::max<int64_t>(1, slots / per_slot);
        k = a.H <= 32 ? k_attn_mfma<512, 64, F8, OT, 1, true> : k_attn_mfma<512, 64, F8, OT, 2, true>;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)gx, (unsigned)a.rows, (unsigned)groups), dim3(kNW * 64), 0, st, a);
}

hipError_t launch_attention_mfma(const AttnArgs& a, int64_t nsplit_bound, hipStream_t st) {
    // all records FP8: the ring kernel; otherwise the expanding one
    const bool f8 = a.comp_fmt == CSA_FP8_E4M3 && (a.W == 0 || a.win_fmt == CSA_FP8_E4M3);
    if (f8) {
        if (a.out_fmt == CSA_BF16) launch_d<true, uint16_t>(a, (int)nsplit_bound, st);
        else launch_d<true, float>(a, (int)nsplit_bound, st);
    } else {
        if (a.out_fmt == CSA_BF16) launch_d<false, uint16_t>(a, (int)nsplit_bound, st);
        else launch_d<false, float>(a, (int)nsplit_bound, st);
    }
    return hipGetLastError();
}

}  // namespace csa
