// Split-K merge of partial softmax states and inverse rotation of the output.
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "回転のトリック — ブロック対角アダマール": the rotation R = H/sqrt(Bh)
// is orthogonal and its own inverse, so the attention output computed in the
// rotated basis is brought back by applying R once more.  That is done after
// the merge, since merging (a weighted sum) commutes with R.
//
// Partial state of split s: running max M_s (log2 units), running sum l_s,
// unnormalised output o_s.  Merge: M = max M_s, l = sum l_s 2^(M_s - M),
// o = sum o_s 2^(M_s - M) / l.
//
// One wave merges one (sequence, query head): lane t owns dims 2t and 2t+1,
// so the butterflies of the inverse FWHT are one in-register step (span 1)
// and lane exchanges (spans 2..64); no LDS and no block barrier on that path.
// With many splits per sequence (batch 1, long context) 4 or 16 waves share
// one (sequence, head): each merges every 4th (16th) split, and their partial
// states are merged once more through LDS.  The merge is latency-bound there
// (few units), so more waves means fewer dependent load rounds per wave.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
static_assert(kWaves == 4, "the balanced decode's partial layout assumes 4 waves per block");
constexpr int kWideWaves = 16;     // waves per unit for very many splits

__device__ __forceinline__ float wave_max(float v) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Merge the partial states s0, s0 + step, ... < nsplit of one unit, state s
// stored at position s * stride: returns (M, l) and o for dims 2t, 2t + 1
// (relative to M).
__device__ __forceinline__ void merge_splits(const float *ml, const float *po, int nsplit, int64_t stride, int s0,
                                             int step, int t, float &M, float &lsum, float &o0, float &o1) {
    float mloc = -INFINITY;
    for (int s = s0 + t * step; s < nsplit; s += 64 * step) mloc = fmaxf(mloc, ml[2 * s * stride]);
    M = wave_max(mloc);
    float lloc = 0.0f;
    for (int s = s0 + t * step; s < nsplit; s += 64 * step)
        lloc = fmaf(ml[2 * s * stride + 1], exp2f(ml[2 * s * stride] - M), lloc);
    lsum = wave_sum(lloc);
    o0 = 0.0f;
    o1 = 0.0f;
#pragma unroll 8
    for (int s = s0; s < nsplit; s += step) {
        const float w = exp2f(ml[2 * s * stride] - M);
        const float2 v = *reinterpret_cast<const float2 *>(po + (int64_t)s * stride * kHeadDim + 2 * t);
        o0 = fmaf(v.x, w, o0);
        o1 = fmaf(v.y, w, o1);
    }
}

// Inverse rotation of 128 values held as (2t, 2t+1) by lane t, then store.
__device__ __forceinline__ void rotate_back_and_store(float o0, float o1, int bh, int t, float *out) {
    if (bh > 0) {
        float u = o0 + o1, v = o0 - o1;          // span 1: inside the lane
        o0 = u;
        o1 = v;
        for (int span = 2; span < bh; span <<= 1) {
            const int m = span >> 1;              // partner lane for dims 2t ^ span
            const bool upper = (t & m) != 0;
            const float p0 = __shfl_xor(o0, m);
            const float p1 = __shfl_xor(o1, m);
            o0 = upper ? (p0 - o0) : (o0 + p0);
            o1 = upper ? (p1 - o1) : (o1 + p1);
        }
        const float c = rsqrtf(static_cast<float>(bh));
        o0 *= c;
        o1 *= c;
    }
    *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(o0, o1);
}

// Merge of a unit with at most kFewSplits partial states (the common case
// with many sequences): lane t loads the (M, l) pair of split t while every
// lane loads its two dims of every split's o, all in one round of loads (an
// index past the last split is clamped and its weight is zero); the maxima
// and sums then come from lane reads, with no cross-lane reduction.
constexpr int kFewSplits = 8;
__device__ __forceinline__ void merge_few(const float *ml, const float *po, int nsplit, int t, float &lsum,
                                          float &o0, float &o1) {
    const int mine = min(t, nsplit - 1);
    const float2 mlt = *reinterpret_cast<const float2 *>(ml + 2 * mine);
    float2 v[kFewSplits];
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k)
        v[k] = *reinterpret_cast<const float2 *>(po + (int64_t)min(k, nsplit - 1) * kHeadDim + 2 * t);
    float mk[kFewSplits];
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
        mk[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlt.x), k));
        if (k < nsplit) M = fmaxf(M, mk[k]);
    }
    lsum = 0.0f;
    o0 = 0.0f;
    o1 = 0.0f;
#pragma unroll
    for (int k = 0; k < kFewSplits; ++k) {
        const float w = k < nsplit ? exp2f(mk[k] - M) : 0.0f;
        lsum = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlt.y), k)), w, lsum);
        o0 = fmaf(v[k].x, w, o0);
        o1 = fmaf(v[k].y, w, o1);
    }
}

// NW = 1: 4 units per block, one wave each.  NW = 4 or 16: one unit per block,
// NW waves each merging every NW-th split.
template <int NW>
__global__ __launch_bounds__(NW == 1 ? kThreads : 64 * NW) void combine_kernel(DecodeArgs a, int rotate_back) {
    constexpr bool WIDE = NW > 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads below
    const int t = threadIdx.x & 63;
    const int unit = WIDE ? blockIdx.x : blockIdx.x * kWaves + wave;   // b * num_q_heads + qh
    if (unit >= a.batch * a.num_q_heads) return;
    const int b = unit / a.num_q_heads;
    float *out = a.out + (int64_t)unit * kHeadDim;
    const int qh = unit - b * a.num_q_heads;
    int nsplit;
    int64_t first;
    if (a.sk_groups > 0) {
        // Balanced decode: the partial states of (b, qh) come from the ranges
        // g_first .. g_last that meet sequence b, at positions
        // ((quad * 4 + wave) * 4 + head) * (sk_groups + batch) + g + b.  A
        // sequence with no chunks (context length <= 0) has none.
        const int tot = a.sk_prefix[a.batch];
        const int pb = a.sk_prefix[b], pb1 = a.sk_prefix[b + 1];
        if (pb1 == pb || tot <= 0) {   // (tot > 0 whenever pb1 > pb: the test only orders the loads)
            if (!WIDE || wave == 0) *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(0.0f, 0.0f);
            return;
        }
        const int G = balanced_groups(a.sk_min, a.sk_target, tot);
        const int g_first = (int)((((int64_t)pb + 1) * G - 1) / tot);
        const int g_last = (int)(((int64_t)pb1 * G - 1) / tot);
        const int hk = qh / a.group;
        const int chunk_id = (qh - hk * a.group) / kHeadsPerChunk;
        const int slot = hk * a.head_chunks + chunk_id;
        const int local = (slot % kWaves) * kHeadsPerChunk + (qh - hk * a.group) % kHeadsPerChunk;
        nsplit = g_last - g_first + 1;
        first = ((int64_t)(slot / kWaves) * kWaves * kHeadsPerChunk + local) * (a.sk_groups + a.batch) + g_first + b;
    } else {
        const int L = a.context_lens[b];
        if (L <= 0) {
            if (!WIDE || wave == 0) *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(0.0f, 0.0f);
            return;
        }
        const int npages = (L + a.page_size - 1) >> a.page_shift;
        nsplit = (npages + a.pages_per_split - 1) / a.pages_per_split;
        first = (int64_t)unit * a.num_splits;
    }
    const float *ml = a.ws_ml + first * 2;
    const float *po = a.ws_o + first * kHeadDim;
    const int bh = rotate_back ? a.had_block : 0;

    float M, lsum, o0, o1;
    if constexpr (!WIDE) {
        if (nsplit <= kFewSplits) merge_few(ml, po, nsplit, t, lsum, o0, o1);
        else merge_splits(ml, po, nsplit, 1, 0, 1, t, M, lsum, o0, o1);
    } else {
        merge_splits(ml, po, nsplit, 1, wave, NW, t, M, lsum, o0, o1);
        __shared__ float sm[NW], sl[NW];
        __shared__ float so[NW][kHeadDim];
        if (t == 0) {
            sm[wave] = M;
            sl[wave] = lsum;
        }
        so[wave][2 * t] = o0;
        so[wave][2 * t + 1] = o1;
        __syncthreads();
        if (wave != 0) return;
        M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w]);
        lsum = 0.0f;
        o0 = 0.0f;
        o1 = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = (sm[w] == -INFINITY) ? 0.0f : exp2f(sm[w] - M);
            lsum = fmaf(sl[w], f, lsum);
            o0 = fmaf(so[w][2 * t], f, o0);
            o1 = fmaf(so[w][2 * t + 1], f, o1);
        }
    }
    const float inv = 1.0f / lsum;
    rotate_back_and_store(o0 * inv, o1 * inv, bh, t, out);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, bool rotate_back, hipStream_t stream) {
    const int units = a.batch * a.num_q_heads;
    const int rb = rotate_back ? 1 : 0;
    // Many splits per sequence (long context, small batch): spread each unit's
    // splits over 4 or 16 waves; otherwise one wave per unit.
    const int per_unit = a.sk_groups > 0 ? a.sk_groups / a.batch + 2 : a.num_splits;
    if (per_unit >= 128) {
        hipLaunchKernelGGL(combine_kernel<kWideWaves>, dim3((unsigned)units), dim3(64 * kWideWaves), 0, stream, a, rb);
    } else if (per_unit >= 32) {
        hipLaunchKernelGGL(combine_kernel<kWaves>, dim3((unsigned)units), dim3(kThreads), 0, stream, a, rb);
    } else {
        hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                           stream, a, rb);
    }
    return hipGetLastError();
}

}  // namespace kvq
