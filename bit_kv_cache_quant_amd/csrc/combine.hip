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
//
// Fused decode step (APPEND): each sequence's new last token arrives as fp16
// K/V rows instead of being in the cache.  The partial kernels take it in
// the range that ends at the sequence's last cached token; only a sequence
// whose context is the new token alone reaches the merge without a partial
// state.  For it the merge wave rotates and quantizes the rows with the
// append's arithmetic (the same fp32 operations in the same order, so the
// same codes and scale bit for bit), stores them in the cache (the unit of
// the first query head of each KV head writes), and takes the token as the
// only state: max = its score, sum = 1, output = its dequantized value row.
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

// The two results of v_permlane16_swap (SPAN 16) or v_permlane32_swap
// (SPAN 32) applied to x: lo = the value x holds in the lower row (rows 0,
// 2) or half of the lane's pair, hi = the upper one's.  (Copied to scalars
// before any bit cast: a bit cast applied directly to an element of the
// builtin's two-element vector reads element 0 for both.)
template <int SPAN>
__device__ __forceinline__ void swap_pair(float x, float &lo, float &hi) {
    const uint32_t a = __builtin_bit_cast(uint32_t, x);
    const auto r = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(a, a, false, false)
                              : __builtin_amdgcn_permlane32_swap(a, a, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}

// Value of lane t ^ M (M = 1, 2, 4, ..., 32) without going through LDS:
// DPP within rows of 16 lanes (quad permutes, and the row mirrors: lane i
// of a row takes lane 15 - i, or 7 - i within each half row, so two of
// them compose to xor 4 or xor 8), v_permlane16_swap across the two rows of
// each half, v_permlane32_swap across the halves.
template <int M>
__device__ __forceinline__ float xor_lane(float v, int t) {
    const int x = __builtin_bit_cast(int, v);
    if constexpr (M == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
    } else if constexpr (M == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
    } else if constexpr (M == 4) {   // xor 7 (half-row mirror), then xor 3
        const int y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, true));
    } else if constexpr (M == 8) {   // xor 15 (row mirror), then xor 7
        const int y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, true));
    } else {
        static_assert(M == 16 || M == 32, "lane distance is a power of two below 64");
        float lo, hi;
        swap_pair<M>(v, lo, hi);
        return (t & M) ? lo : hi;
    }
}

// One butterfly stage of span 2M between lanes t and t ^ M on the pairs
// (2t, 2t+1): the lower entry gets u + v, the upper one u - v (u the lower
// entry's value), one fp32 rounding each.
template <int M>
__device__ __forceinline__ void lane_butterfly(float &y0, float &y1, int t) {
    const bool upper = (t & M) != 0;
    const float p0 = xor_lane<M>(y0, t);
    const float p1 = xor_lane<M>(y1, t);
    y0 = upper ? (p0 - y0) : (y0 + p0);
    y1 = upper ? (p1 - y1) : (y1 + p1);
}

// The unnormalised block transform (spans 1 .. bh/2 in ascending order) of
// 128 values held as (2t, 2t+1) by lane t; bh = 0 leaves them alone.
__device__ __forceinline__ void fwht_pairs(float &y0, float &y1, int bh, int t) {
#pragma clang fp contract(off)
    if (bh <= 0) return;
    const float u = y0 + y1, v = y0 - y1;   // span 1: inside the lane
    y0 = u;
    y1 = v;
    if (bh > 2) lane_butterfly<1>(y0, y1, t);
    if (bh > 4) lane_butterfly<2>(y0, y1, t);
    if (bh > 8) lane_butterfly<4>(y0, y1, t);
    if (bh > 16) lane_butterfly<8>(y0, y1, t);
    if (bh > 32) lane_butterfly<16>(y0, y1, t);
    if (bh > 64) lane_butterfly<32>(y0, y1, t);
}

// Inverse rotation of 128 values held as (2t, 2t+1) by lane t (S R: the
// block rotation, then the sign mask), then store.
__device__ __forceinline__ void rotate_back_and_store(float o0, float o1, int bh, int t, const uint32_t (&mask)[4],
                                                      float *out) {
    if (bh > 0) {
        fwht_pairs(o0, o1, bh, t);
        const float c = rsqrtf(static_cast<float>(bh));
        o0 *= c;
        o1 *= c;
    }
    const uint32_t bits = (mask[t >> 4] >> (2 * (t & 15))) & 3u;   // channels 2t, 2t + 1
    o0 = (bits & 1u) ? -o0 : o0;
    o1 = (bits & 2u) ? -o1 : o1;
    *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(o0, o1);
}

// ---- fused decode step: the new token ----

// Wave-wide max and sum: rows of 16 by DPP, then across rows by the
// permlane swaps (no LDS).  The max is exact in any order.
__device__ __forceinline__ float wave_max(float v) {
    float lo, hi;
    swap_pair<16>(dec::row_max16(v), lo, hi);
    swap_pair<32>(fmaxf(lo, hi), lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float wave_sum(float v) {
    float lo, hi;
    swap_pair<16>(dec::row_sum16(v), lo, hi);
    swap_pair<32>(lo + hi, lo, hi);
    return lo + hi;
}

// fp32 nearest 1/sqrt(bh) for the supported blocks.
__device__ __forceinline__ float block_scale(int bh) {
    return __builtin_bit_cast(float, bh == 32 ? 0x3E3504F3u : bh == 64 ? 0x3E000000u : 0x3DB504F3u);
}

// Block rotation (transform, then the product with the fp32 nearest
// 1/sqrt(bh)) of a 128-entry fp16 vector held as entries (2t, 2t+1) by lane
// t, the entries widened exactly to fp32 first.
__device__ __forceinline__ void rotate_pair(uint32_t w, int bh, int t, float &y0, float &y1) {
#pragma clang fp contract(off)
    y0 = dec::half_to_float(w);
    y1 = dec::half_to_float(w >> 16);
    if (bh <= 0) return;
    fwht_pairs(y0, y1, bh, t);
    const float c = block_scale(bh);
    y0 = y0 * c;
    y1 = y1 * c;
}

// Token-wise INT4 of the rotated entries (y0, y1) of lane t: m = max |y| over
// the wave (exact), s = fp16(m / 7) (IEEE quotient, then round to nearest
// even), code = clamp(rint(y / s), -8, 7) with the IEEE quotient (0 when s =
// 0).  Gives the code byte of entries 2t (low nibble) and 2t + 1, the
// dequantized entries code * s (exact) and the fp16 scale bits.
struct NewRow {
    uint32_t byte;
    float d0, d1;
    uint16_t s16;
};
__device__ __forceinline__ NewRow quantize_pair(float y0, float y1) {
#pragma clang fp contract(off)
    const float m = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    float s32 = m / 7.0f;
    asm("" : "+v"(s32));   // two roundings (fp32, then fp16), as written
    const _Float16 h = static_cast<_Float16>(s32);
    const float s = static_cast<float>(h);
    float c0 = 0.0f, c1 = 0.0f;
    if (s > 0.0f) {
        c0 = fminf(fmaxf(rintf(y0 / s), -8.0f), 7.0f);
        c1 = fminf(fmaxf(rintf(y1 / s), -8.0f), 7.0f);
    }
    NewRow r;
    r.byte = (static_cast<uint32_t>(static_cast<int>(c0)) & 15u) |
             ((static_cast<uint32_t>(static_cast<int>(c1)) & 15u) << 4);
    r.d0 = c0 * s;
    r.d1 = c1 * s;
    r.s16 = __builtin_bit_cast(uint16_t, h);
    return r;
}

// The new token of one (sequence, query head): its K and V rows quantized,
// and its score against the query (log2 units).
struct NewToken {
    NewRow k, v;
    float z;
};
__device__ __forceinline__ NewToken new_token(uint32_t kw, uint32_t vw, uint32_t qw, int bh, float score_scale,
                                              int t) {
    float k0, k1, v0, v1, q0, q1;
    rotate_pair(kw, bh, t, k0, k1);
    rotate_pair(vw, bh, t, v0, v1);
    rotate_pair(qw, bh, t, q0, q1);
    NewToken n;
    n.k = quantize_pair(k0, k1);
    n.v = quantize_pair(v0, v1);
    n.z = wave_sum(fmaf(q0, n.k.d0, q1 * n.k.d1)) * score_scale;
    return n;
}

// Folds the new token into (M, lsum, o0, o1) as one more partial state:
// max z, sum 1, output its value row.
__device__ __forceinline__ void fold(const NewToken &n, float &M, float &lsum, float &o0, float &o1) {
    const float Mn = fmaxf(M, n.z);
    const float corr = M == -INFINITY ? 0.0f : dec::fast_exp2(M - Mn);
    const float w = dec::fast_exp2(n.z - Mn);
    lsum = fmaf(lsum, corr, w);
    o0 = fmaf(o0, corr, n.v.d0 * w);
    o1 = fmaf(o1, corr, n.v.d1 * w);
    M = Mn;
}

// Stores the new token's codes and scales at slot `slot` of page `page` for
// KV head hk (the append's page layout).
__device__ __forceinline__ void store_new_token(const DecodeArgs &a, const NewToken &n, int32_t page, int slot,
                                                int hk, int t) {
    const int64_t page_off = (int64_t)page * a.num_kv_heads * a.tile_bytes;
    const int64_t row = (int64_t)hk * a.page_size + slot;
    const int64_t scale_off = (int64_t)a.num_kv_heads * a.page_size * kCodeBytesPerRow + row * 2;
    uint8_t *kp = static_cast<uint8_t *>(const_cast<void *>(a.k_pool)) + page_off;
    uint8_t *vp = static_cast<uint8_t *>(const_cast<void *>(a.v_pool)) + page_off;
    kp[row * kCodeBytesPerRow + t] = static_cast<uint8_t>(n.k.byte);
    vp[row * kCodeBytesPerRow + t] = static_cast<uint8_t>(n.v.byte);
    if (t == 0) {
        *reinterpret_cast<uint16_t *>(kp + scale_off) = n.k.s16;
        *reinterpret_cast<uint16_t *>(vp + scale_off) = n.v.s16;
    }
}

// NW = 1: 4 units per block, one wave each.  NW = 4 or 16: one unit per block,
// NW waves each merging every NW-th split.
template <int NW, bool APPEND>
__global__ __launch_bounds__(NW == 1 ? kThreads : 64 * NW) void combine_kernel(DecodeArgs a, int rotate_back) {
    constexpr bool WIDE = NW > 1;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loads below
    const int t = threadIdx.x & 63;
    // The launch parameters the first addresses depend on, fetched at once
    // (one wait, instead of one per branch that needs the next of them).
    const int nq = a.num_q_heads, gshift = a.group_shift, group = a.group, skg = a.sk_groups, B = a.batch;
    const int32_t *skp = a.sk_prefix;
    asm volatile("" ::"s"(nq), "s"(gshift), "s"(group), "s"(skg), "s"(B), "s"(skp));
    // grid: x = sequence, y = query head (NW > 1) or quad of query heads
    const int b = blockIdx.x;
    const int qh = WIDE ? (int)blockIdx.y : (int)blockIdx.y * kWaves + wave;
    if (qh >= nq) return;
    const int64_t unit = (int64_t)b * nq + qh;
    float *out = a.out + unit * kHeadDim;
    const int hk = gshift >= 0 ? (qh >> gshift) : qh / group;
    const int s0 = WIDE ? wave : 0, step = WIDE ? NW : 1;
    const int bh = rotate_back ? a.had_block : 0;

    // Balanced schedule: the chunk prefix sums this unit's state addresses
    // depend on.
    int tot = 0, pb = 0, pb1 = 0;
    if (skg > 0) {
        tot = skp[B];
        pb = skp[b];
        pb1 = skp[b + 1];
    }

    // Fused step: a sequence whose context is the new token alone has no
    // partial state (the partial kernels take each sequence's new token in
    // the range that ends at its last cached token); its rows and slot are
    // loaded first.  In the balanced schedule only a sequence without chunks
    // can be one, so only such a sequence waits for its context length.
    int Lnew = 0;
    uint32_t kw = 0, vw = 0, qw = 0;
    int32_t page = 0;
    if constexpr (APPEND) {
        if (a.sk_groups == 0 || pb1 == pb) Lnew = full_len(a, b);
        if (Lnew == 1) {
            kw = reinterpret_cast<const uint32_t *>(a.k_new + ((int64_t)b * a.num_kv_heads + hk) * kHeadDim)[t];
            vw = reinterpret_cast<const uint32_t *>(a.v_new + ((int64_t)b * a.num_kv_heads + hk) * kHeadDim)[t];
            qw = reinterpret_cast<const uint32_t *>(a.q + ((int64_t)b * a.num_q_heads + qh) * kHeadDim)[t];
            page = a.page_table[(int64_t)b * a.max_pages_per_seq + ((Lnew - 1) >> a.page_shift)];
        }
    }

    int nsplit = 0, limit = 1;
    Round r0;   // the first round of this wave's states
    const float *ml = a.ws_ml, *po = a.ws_o;
    if (a.sk_groups > 0) {
        // Balanced decode: the partial states of (b, qh) come from the ranges
        // g_first .. g_last that meet sequence b, at positions
        // ((quad * 4 + wave) * 4 + head) * (sk_groups + batch) + g + b.  A
        // sequence with no chunks has none.
        if (pb1 > pb && tot > 0) {   // (tot > 0 whenever pb1 > pb: the test only orders the loads)
            const int G = balanced_groups(a.sk_min, a.sk_target, tot);
            int g_first, g_last;
            if (a.sk_div32) {
                g_first = (int)(((uint32_t)(pb + 1) * (uint32_t)G - 1u) / (uint32_t)tot);
                g_last = (int)(((uint32_t)pb1 * (uint32_t)G - 1u) / (uint32_t)tot);
            } else {
                g_first = (int)((((int64_t)pb + 1) * G - 1) / tot);
                g_last = (int)(((int64_t)pb1 * G - 1) / tot);
            }
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
        }
    } else {
        // Split mode: the unit owns num_splits positions, the first nsplit of
        // them written (none if the context is empty); the first round of
        // loads is issued before the context length is known.
        const int64_t first = unit * a.num_splits;
        ml = a.ws_ml + first * 2;
        po = a.ws_o + first * kHeadDim;
        limit = a.num_splits;
        r0 = load_round(ml, po, s0, step, limit, t);
        const int L = decode_len(a, b);
        const int npages = (L + a.page_size - 1) >> a.page_shift;
        nsplit = L > 0 ? (npages + a.pages_per_split - 1) / a.pages_per_split : 0;
    }
    NewToken nt{};
    if constexpr (APPEND) {
        if (Lnew == 1) nt = new_token(kw, vw, qw, a.had_block, a.score_scale, t);
    }

    float M = -INFINITY, lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    if (nsplit > 0) {
        add_round(r0, s0, step, nsplit, M, lsum, o0, o1);
        for (int base = s0 + kRound * step; base < nsplit; base += kRound * step)
            add_round(load_round(ml, po, base, step, limit, t), base, step, nsplit, M, lsum, o0, o1);
    }
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
    bool empty = nsplit == 0;
    if constexpr (APPEND) {
        if (Lnew == 1) {
            fold(nt, M, lsum, o0, o1);
            if (qh % a.group == 0) store_new_token(a, nt, page, 0, hk, t);
            empty = false;
        }
    }
    if (empty) {   // no context: a zero row
        *reinterpret_cast<float2 *>(out + 2 * t) = make_float2(0.0f, 0.0f);
        return;
    }
    const float inv = 1.0f / lsum;
    rotate_back_and_store(o0 * inv, o1 * inv, bh, t, a.sign_mask, out);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, bool rotate_back, hipStream_t stream) {
    const int rb = rotate_back ? 1 : 0;
    // Many splits per sequence (long context, small batch): spread each unit's
    // splits over 4 or 16 waves, so that a wave merges about one round
    // (kRound states); otherwise one wave per unit.  Grid: x = sequence,
    // y = query head, or quad of query heads with one wave per unit.
    const int per_unit = a.sk_groups > 0 ? a.sk_groups / a.batch + 2 : a.num_splits;
    const dim3 one_grid((unsigned)a.batch, (unsigned)((a.num_q_heads + kWaves - 1) / kWaves));
    const dim3 wide_grid((unsigned)a.batch, (unsigned)a.num_q_heads);
    if (a.k_new) {
        if (per_unit > 4 * kRound)
            hipLaunchKernelGGL((combine_kernel<kWideWaves, true>), wide_grid, dim3(64 * kWideWaves), 0, stream, a, rb);
        else if (per_unit > kRound)
            hipLaunchKernelGGL((combine_kernel<kWaves, true>), wide_grid, dim3(kThreads), 0, stream, a, rb);
        else
            hipLaunchKernelGGL((combine_kernel<1, true>), one_grid, dim3(kThreads), 0, stream, a, rb);
    } else {
        if (per_unit > 4 * kRound)
            hipLaunchKernelGGL((combine_kernel<kWideWaves, false>), wide_grid, dim3(64 * kWideWaves), 0, stream, a, rb);
        else if (per_unit > kRound)
            hipLaunchKernelGGL((combine_kernel<kWaves, false>), wide_grid, dim3(kThreads), 0, stream, a, rb);
        else
            hipLaunchKernelGGL((combine_kernel<1, false>), one_grid, dim3(kThreads), 0, stream, a, rb);
    }
    return hipGetLastError();
}

}  // namespace kvq
