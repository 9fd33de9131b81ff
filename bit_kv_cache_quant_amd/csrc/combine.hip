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
// A wave takes its partial states 8 at a time, every load of a round issued
// before any is used (the merge is latency-bound: few dependent rounds of
// loads matter more than instruction counts).  With many splits per
// sequence (batch 1, long context) 4 or 16 waves share one (sequence, head):
// each merges every 4th (16th) split, and their states are merged once more
// through LDS.
#include "decode_common.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
static_assert(kWaves == 4, "the balanced decode's partial layout assumes 4 waves per block");
constexpr int kWideWaves = 16;     // waves per unit for very many splits

// A unit's partial states are merged kRound at a time: lane k < kRound of a
// round loads the (max, sum) pair of its state and every lane loads its two
// output dims of all kRound states, all before any is used; maxima and sums
// then come from lane reads.  Positions past the unit's states are read
// clamped to limit - 1 (every position below limit is readable) and never
// enter the result, so a round can be issued before nsplit is known.
constexpr int kRound = 8;
struct Round {
    float2 mlt;           // (max, sum) of state base + t * step, t < kRound
    float2 v[kRound];     // output dims 2t, 2t + 1 of states base + k * step
};

__device__ __forceinline__ Round load_round(const float *ml, const float *po, const int base, const int step,
                                            const int limit, const int t) {
    Round r;
    const int sl = min(base + min(t, kRound - 1) * step, limit - 1);
    r.mlt = *reinterpret_cast<const float2 *>(ml + 2 * (int64_t)sl);
#pragma unroll
    for (int k = 0; k < kRound; ++k)
        r.v[k] = *reinterpret_cast<const float2 *>(po + (int64_t)min(base + k * step, limit - 1) * kHeadDim + 2 * t);
    return r;
}

// Folds the states base + k * step < nsplit of round r into (M, l, o0, o1)
// (M = -inf and everything 0 while no state has been seen; branch-free).
__device__ __forceinline__ void add_round(const Round &r, const int base, const int step, const int nsplit, float &M,
                                          float &lsum, float &o0, float &o1) {
    float mk[kRound], lk[kRound];
    float Mr = M;
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
        mk[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.mlt.x), k));
        lk[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.mlt.y), k));
        if (base + k * step < nsplit) Mr = fmaxf(Mr, mk[k]);
    }
    const float corr = Mr == -INFINITY ? 1.0f : dec::fast_exp2(M - Mr);
    lsum *= corr;
    o0 *= corr;
    o1 *= corr;
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
        const bool live = base + k * step < nsplit;   // unwritten positions may hold anything
        const float w = dec::fast_exp2(mk[k] - Mr);
        lsum = live ? fmaf(lk[k], w, lsum) : lsum;
        o0 = live ? fmaf(r.v[k].x, w, o0) : o0;
        o1 = live ? fmaf(r.v[k].y, w, o1) : o1;
    }
    M = Mr;
}

// Inverse rotation of 128 values held as (2t, 2t+1) by lane t (S R: the
// block rotation, then the sign mask), then store.
__device__ __forceinline__ void rotate_back_and_store(float o0, float o1, int bh, int t, const uint32_t (&mask)[4],
                                                      float *out) {
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
    const uint32_t bits = (mask[t >> 4] >> (2 * (t & 15))) & 3u;   // channels 2t, 2t + 1
    o0 = (bits & 1u) ? -o0 : o0;
    o1 = (bits & 2u) ? -o1 : o1;
    *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(o0, o1);
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
    const int s0 = WIDE ? wave : 0, step = WIDE ? NW : 1;
    int nsplit, limit;
    Round r0;   // the first round of this wave's states
    const float *ml, *po;
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
        limit = nsplit;
        const int64_t first =
            ((int64_t)(slot / kWaves) * kWaves * kHeadsPerChunk + local) * (a.sk_groups + a.batch) + g_first + b;
        ml = a.ws_ml + first * 2;
        po = a.ws_o + first * kHeadDim;
        r0 = load_round(ml, po, s0, step, limit, t);
    } else {
        // Split mode: the unit owns num_splits positions, the first nsplit of
        // them written (none if the context is empty); the first round of
        // loads is issued before the context length is known.
        const int64_t first = (int64_t)unit * a.num_splits;
        ml = a.ws_ml + first * 2;
        po = a.ws_o + first * kHeadDim;
        limit = a.num_splits;
        r0 = load_round(ml, po, s0, step, limit, t);
        const int L = decode_len(a, b);
        const int npages = (L + a.page_size - 1) >> a.page_shift;
        nsplit = L > 0 ? (npages + a.pages_per_split - 1) / a.pages_per_split : 0;
    }
    const int bh = rotate_back ? a.had_block : 0;

    float M = -INFINITY, lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    add_round(r0, s0, step, nsplit, M, lsum, o0, o1);
    for (int base = s0 + kRound * step; base < nsplit; base += kRound * step)
        add_round(load_round(ml, po, base, step, limit, t), base, step, nsplit, M, lsum, o0, o1);
    if constexpr (WIDE) {
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
            const float f = (sm[w] == -INFINITY) ? 0.0f : dec::fast_exp2(sm[w] - M);
            lsum = fmaf(sl[w], f, lsum);
            o0 = fmaf(so[w][2 * t], f, o0);
            o1 = fmaf(so[w][2 * t + 1], f, o1);
        }
    }
    if (nsplit == 0) {   // empty context: a zero row
        *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(0.0f, 0.0f);
        return;
    }
    const float inv = 1.0f / lsum;
    rotate_back_and_store(o0 * inv, o1 * inv, bh, t, a.sign_mask, out);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, bool rotate_back, hipStream_t stream) {
    const int units = a.batch * a.num_q_heads;
    const int rb = rotate_back ? 1 : 0;
    // Many splits per sequence (long context, small batch): spread each unit's
    // splits over 4 or 16 waves, so that a wave merges about one round
    // (kRound states); otherwise one wave per unit.
    const int per_unit = a.sk_groups > 0 ? a.sk_groups / a.batch + 2 : a.num_splits;
    if (per_unit > 4 * kRound) {
        hipLaunchKernelGGL(combine_kernel<kWideWaves>, dim3((unsigned)units), dim3(64 * kWideWaves), 0, stream, a, rb);
    } else if (per_unit > kRound) {
        hipLaunchKernelGGL(combine_kernel<kWaves>, dim3((unsigned)units), dim3(kThreads), 0, stream, a, rb);
    } else {
        hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)((units + kWaves - 1) / kWaves)), dim3(kThreads), 0,
                           stream, a, rb);
    }
    return hipGetLastError();
}

}  // namespace kvq
