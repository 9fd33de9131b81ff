// Pieces shared by the INT4 and the fp16 paged decode kernels: their common
// work schedule (per-sequence splits, or balanced ranges over the whole
// batch), the partial-state layout the merge kernel reads, and row-of-16
// lane reductions.  Internal; the public interface is include/kvq.h.
#pragma once

#include "kvq_internal.h"

namespace kvq {
namespace dec {

constexpr int kWaves = 4;                 // waves per block: 4 head slots
constexpr int kThreads = 64 * kWaves;
constexpr int kH = kHeadsPerChunk;        // query heads per head slot

__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// All-reduce inside each row of 16 lanes; every lane of the row gets the
// result.  (DPP: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror.)
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x141>(v));
    v = fmaxf(v, dpp_f<0x140>(v));
    return v;
}

// Row max as an integer max (one DPP-fused instruction per step): float
// order equals signed-integer order of the key b ^ ((b >> 31) & 0x7fffffff)
// for all non-NaN floats, -inf included.
__device__ __forceinline__ int row_max16_key(int k) {
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0xB1, 0xF, 0xF, true));
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0x4E, 0xF, 0xF, true));
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0x141, 0xF, 0xF, true));
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0x140, 0xF, 0xF, true));
    return k;
}
__device__ __forceinline__ float row_max16_fast(float v) {
    const int b = __builtin_bit_cast(int, v);
    const int k = row_max16_key(b ^ ((b >> 31) & 0x7fffffff));
    return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7fffffff));
}
// For v >= 0 (no -0, no NaN) the bits themselves order like the values.
__device__ __forceinline__ float row_max16_nonneg(float v) {
    return __builtin_bit_cast(float, row_max16_key(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}

__device__ __forceinline__ int row_sum16_i(int v) {
    v += dpp_i<0xB1>(v);
    v += dpp_i<0x4E>(v);
    v += dpp_i<0x141>(v);
    v += dpp_i<0x140>(v);
    return v;
}

// 2^x with the hardware exponential alone (v_exp_f32, about 1 ulp): the
// softmax arguments are <= 0, and where the exact result would be an fp32
// denormal (x < -126) this may give 0 instead, a weight below 2^-126 of the
// largest one.  -inf gives 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp16 query words holding dims 8j .. 8j + 7 with the channels set in byte
// j of the 128-bit sign mask negated (exact: sign-bit flips).
__device__ __forceinline__ uint4 sign_flip_query(uint4 w, const uint32_t (&mask)[4], int j) {
    const uint32_t b = (mask[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    w.x ^= ((b & 1u) << 15) | ((b & 2u) << 30);
    w.y ^= ((b & 4u) << 13) | ((b & 8u) << 28);
    w.z ^= ((b & 16u) << 11) | ((b & 32u) << 26);
    w.w ^= ((b & 64u) << 9) | ((b & 128u) << 24);
    return w;
}

// Orders LDS traffic between the lanes of one wave (no cross-wave sharing).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Partial softmax state of one work range, as lane (g, j) holds it: head g,
// dims 16 m + j of the unnormalised output, running max and sum (log2 units).
struct PartialState {
    float o[8];
    float m, l;
};

// Writes the state of query head qh0 + g to unit u0 + g * head_stride of the
// workspace (o: kHeadDim floats, then (max, sum) in ws_ml).  DEVICE_SCOPE:
// as device-scope stores, which go through to the level the whole device
// shares instead of waiting in this XCD's L2 for the write-back at the end of
// the kernel (measured: the batch-1 decode's partial kernel, whose last
// action is this write, 12.15 -> 11.66 us; the batch-wide schedule, which
// writes states while it streams the cache, got 1.5% slower with them).
template <bool DEVICE_SCOPE = false>
__device__ __forceinline__ void write_partial(const DecodeArgs &a, const PartialState &st, const int lane,
                                              const int nheads, const int64_t u0, const int64_t head_stride) {
    const int g = lane >> 4;
    const int j = lane & 15;
    auto put = [](float *p, const float v) {
        if constexpr (DEVICE_SCOPE)
            __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            *p = v;
    };
    if (g < nheads) {
        const int64_t unit = u0 + g * head_stride;
        float *dst = a.ws_o + unit * kHeadDim + j;
#pragma unroll
        for (int m = 0; m < 8; ++m) put(&dst[16 * m], st.o[m]);
        if (j == 0) {
            put(&a.ws_ml[unit * 2 + 0], st.m);
            put(&a.ws_ml[unit * 2 + 1], st.l);
        }
    }
}

// ---- split mode: one page range of one sequence per wave ----
//
// blockIdx.x = (sequence, quad of head slots), blockIdx.y = page range; a
// head slot is (KV head, chunk of 4 of its query heads).  A sequence's
// chunks are shared out evenly over nsplit_b = ceil(npages /
// pages_per_split) ranges (no short remainder range), each a whole number of
// chunks and at most pages_per_split pages; the sequence's last range is at
// the highest blockIdx.y.
struct SplitItem {
    int b, hk, chunk_id, L, s, p0, p1;
    bool live;
};

template <int P>
__device__ __forceinline__ SplitItem split_item(const DecodeArgs &a, const int wave) {
    SplitItem it{};
    it.live = false;
    const int head_slots = a.num_kv_heads * a.head_chunks;
    const int quads = (head_slots + kWaves - 1) / kWaves;
    it.b = blockIdx.x / quads;
    const int slot = (blockIdx.x - it.b * quads) * kWaves + wave;
    if (slot >= head_slots) return it;
    it.hk = slot / a.head_chunks;
    it.chunk_id = slot - it.hk * a.head_chunks;
    it.L = decode_len(a, it.b);
    if (it.L <= 0) return it;
    const int npages = (it.L + P - 1) / P;
    constexpr int kChunkPages = kChunkTokens / P;
    const int nch_b = (npages + kChunkPages - 1) / kChunkPages;
    const int nsplit_b = (npages + a.pages_per_split - 1) / a.pages_per_split;
    it.s = (int)blockIdx.y - (a.num_splits - nsplit_b);
    if (it.s < 0) return it;
    it.p0 = (it.s * nch_b / nsplit_b) * kChunkPages;
    it.p1 = min(((it.s + 1) * nch_b / nsplit_b) * kChunkPages, npages);
    it.live = true;
    return it;
}

// ---- balanced mode: equal ranges of the batch's concatenated chunks ----
//
// The chunks (kChunkTokens each) of all sequences, in sequence order, form
// one list of tot chunks cut into G equal ranges; block (range gi, head quad
// qd) processes range gi for the 4 head slots of quad qd, one partial state
// per (sequence b it meets, head), stored at position gi + b of that head's
// (sk_groups + batch) states (so a head's states for one sequence are
// contiguous).  Every block streams the same amount of cache whatever the
// mix of context lengths.

// LDS of the schedule's set-up (reused by the kernels once it is done).
struct ScanSpace {
    int32_t prefix[kMaxScanBatch + 1];
    int32_t part[kThreads];
};

struct BlockRange {
    int tot, G, gi, qd, start, end, b0, pb0;
};

// Exclusive prefix sums of the per-sequence chunk counts (batch <=
// kMaxScanBatch) into sp.prefix, block 0 also into the workspace (for the
// merge), then the block's range.  Ends with a block barrier, after which
// sp may be reused.
__device__ __forceinline__ BlockRange balanced_range(const DecodeArgs &a, ScanSpace &sp, const int wave,
                                                     const int lane) {
    const int B = a.batch;
    if (B <= 64) {
        // one wave: lane i holds sequence i; shuffle scan, no block barriers
        if (wave == 0) {
            const int L = lane < B ? decode_len(a, lane) : 0;
            const int nch = L > 0 ? (L + kChunkTokens - 1) / kChunkTokens : 0;
            int inc = nch;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_up(inc, off);
                if (lane >= off) inc += v;
            }
            if (lane < B) sp.prefix[lane] = inc - nch;
            if (lane == B - 1) sp.prefix[B] = inc;
        }
    } else {
        const int per = (B + kThreads - 1) / kThreads;
        const int i0 = threadIdx.x * per;
        const int i1 = min(i0 + per, B);
        int local = 0;
        for (int i = i0; i < i1; ++i) {
            const int L = decode_len(a, i);
            local += L > 0 ? (L + kChunkTokens - 1) / kChunkTokens : 0;
        }
        sp.part[threadIdx.x] = local;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            const int v = threadIdx.x >= off ? sp.part[threadIdx.x - off] : 0;
            __syncthreads();
            sp.part[threadIdx.x] += v;
            __syncthreads();
        }
        int run = sp.part[threadIdx.x] - local;
        for (int i = i0; i < i1; ++i) {
            sp.prefix[i] = run;
            const int L = decode_len(a, i);
            run += L > 0 ? (L + kChunkTokens - 1) / kChunkTokens : 0;
        }
        if (threadIdx.x == kThreads - 1) sp.prefix[B] = sp.part[kThreads - 1];
    }
    __syncthreads();
    BlockRange r;
    r.tot = __builtin_amdgcn_readfirstlane(sp.prefix[B]);
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i <= B; i += kThreads) a.sk_prefix[i] = sp.prefix[i];

    r.G = balanced_groups(a.sk_min, a.sk_target, r.tot);
    // Blocks go to the 8 XCDs in turn (block i to XCD i % 8); with the grid
    // a multiple of 8, logical block (i % 8) * (grid / 8) + i / 8 keeps the
    // head quads of one range and consecutive ranges on one XCD, whose L2
    // then serves their shared page-table lines (measured: 0.6% faster).
    int lb = blockIdx.x;
    if ((gridDim.x & 7) == 0) lb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    r.gi = lb / a.quads;
    r.qd = lb - r.gi * a.quads;
    r.start = (int)(((int64_t)r.gi * r.tot) / r.G);
    r.end = (int)(((int64_t)(r.gi + 1) * r.tot) / r.G);
    // First sequence of the range: the last b with prefix[b] <= start.
    int b0 = 0;
    if (r.tot > 0 && r.gi < r.G) {
        int hi = B;
        while (hi - b0 > 1) {
            const int mid = (b0 + hi) >> 1;
            if (sp.prefix[mid] <= r.start) b0 = mid;
            else hi = mid;
        }
    }
    r.b0 = __builtin_amdgcn_readfirstlane(b0);   // uniform: keep sequence state scalar
    r.pb0 = __builtin_amdgcn_readfirstlane(sp.prefix[r.b0]);
    __syncthreads();   // the scan space may now be reused
    return r;
}

}  // namespace dec
}  // namespace kvq
