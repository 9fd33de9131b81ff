// Fused rotate -> quantize -> paged append (INT4), and the fp16 baseline append.
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "システムこそが設計である — 融合カーネル" (figure: K,V fp16 -> block
// Hadamard rotation -> token-wise INT4 -> append into the paged KV block, no
// revisiting of past tokens); token-wise scales from "素朴なINT4はなぜ崩れるのか";
// rotation within blocks from "回転のトリック — ブロック対角アダマール".
//
// The result must equal, bit for bit, the arithmetic stated in include/kvq.h:
// fp32 butterflies in ascending span order, multiply by the fp32 nearest
// 1/sqrt(Bh), absmax, s = fp16(m / 7), code = clamp(rint(y / s), -8, 7).
// This file is therefore compiled with -ffp-contract=off, and the pragma below
// repeats it: no multiply-add may be fused unless written as fmaf.
//
// Mapping: a quad of lanes owns one 128-entry vector (one token, one KV head,
// K or V); lane q holds the 8-entry chunks 4 i + q (four 16-byte loads).  A
// 256-thread block takes 64 consecutive tokens of one (KV head, K or V): when
// those are consecutive positions of one sequence (a prefill append) their
// rows land in consecutive slots of the same pages, so the block's code and
// scale stores cover whole cache lines.  Page layout (include/kvq.h): the
// code rows of KV heads 0..Hkv-1 ([P][64] bytes each), then the scales of
// heads 0..Hkv-1 ([P] fp16 each).  Butterfly span 1 is done while the
// fp16 input is widened, spans 2, 4, 32, 64 inside a lane, spans 8 and 16
// between lanes of the quad with DPP operands; the absmax is a DPP quad
// reduction.  The quad's code words are regrouped through LDS so that each
// lane stores 16 contiguous bytes of its row.
//
// Scale.  s32 = m / 7 is computed as q0 = m * r7, e = fma(-q0, 7, m),
// q = fma(e, r7, q0) with r7 the fp32 value nearest 1/7; this equals the IEEE
// quotient for every non-negative finite fp32 m (checked exhaustively, all
// 2^31 - 2^23 values, zero mismatches).
//
// Division.  The quotient y / s must be the IEEE-rounded one, because rint of
// it decides the code.  One correctly rounded reciprocal r = 1 / s is computed
// per vector; then q0 = y * r, e = fma(-q0, s, y) (exact remainder),
// q = fma(e, r, q0).  For a divisor s carrying at most 11 significant bits (an
// fp16 value) this q equals the IEEE quotient y / s: checked exhaustively over
// every 10-bit divisor fraction, every 23-bit dividend fraction and every
// quotient exponent in [2^-5, 2^5) (77 G cases, zero mismatches); smaller
// quotients round to code 0 and larger ones clamp either way.  (Markstein's
// correction step; the check replaces the general theorem's preconditions.)
// Rounding to an integer is done by adding 1.5 * 2^23 + 8 (round-half-even at
// unit spacing); the low byte of the sum's bits is then code + 8.
#pragma clang fp contract(off)

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kLanesPerVec = 16;
constexpr int kVecsPerBlock = 16;
constexpr int kBlockThreads = kLanesPerVec * kVecsPerBlock;
constexpr int kTokensPerBlock = kBlockThreads / 4;   // INT4 append: one token per quad

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

__device__ __forceinline__ float xor_lane16(float v, int mask) {
    return __shfl_xor(v, mask, kLanesPerVec);
}

// fp32 value nearest 1/sqrt(bh) for the supported block sizes.
template <int BH>
__device__ __forceinline__ float inv_sqrt_block() {
    static_assert(BH == 32 || BH == 64 || BH == 128, "unsupported Hadamard block");
    if constexpr (BH == 32) return __builtin_bit_cast(float, 0x3E3504F3u);
    else if constexpr (BH == 64) return __builtin_bit_cast(float, 0x3E000000u);
    else return __builtin_bit_cast(float, 0x3DB504F3u);
}

// Quad exchange: the value of lane (i ^ MASK), MASK = 1 or 2, of this quad.
template <int MASK>
__device__ __forceinline__ float quad_xor(float v) {
    constexpr int ctrl = (MASK == 1) ? 0xB1 : 0x4E;    // quad_perm [1,0,3,2] / [2,3,0,1]
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), ctrl, 0xF, 0xF, true));
}

// Span-1 butterfly of two fp16 entries packed in one word, straight from the
// fp16 bits: (x0 + x1, x0 - x1) in fp32 with one rounding each, via the
// mixed-precision fma (fp16 operands widened exactly, x0 * 1 + x1 and
// x1 * -1 + x0): two instructions instead of two conversions and two adds.
__device__ __forceinline__ void widen_span1(uint32_t w, float &y0, float &y1) {
    asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(y0) : "v"(w));
    asm("v_fma_mix_f32 %0, %1, -1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(y1) : "v"(w));
}

// Butterfly across lanes q and q ^ MASK of the quad, as y += c * y_partner
// with c = +1 in the lower lane and -1 in the upper one: one fused
// multiply-add with a DPP operand per entry (the product is exact, so it is
// the same single rounding as the add or the subtraction).  The upper lane
// gets the negated result, y_upper - y_lower = -(y_lower - y_upper); the
// caller tracks that sign per lane.  (The s_nop gives the two wait states a
// DPP read of a just-written register needs.)
template <int MASK>
__device__ __forceinline__ void quad_butterfly8(float &y0, float &y1, float &y2, float &y3, float &y4, float &y5,
                                                float &y6, float &y7, float c) {
    if constexpr (MASK == 1) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(y0), "+v"(y1), "+v"(y2), "+v"(y3), "+v"(y4), "+v"(y5), "+v"(y6), "+v"(y7)
            : "v"(c));
    } else {
        static_assert(MASK == 2, "quad lane distance 1 or 2");
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "+v"(y0), "+v"(y1), "+v"(y2), "+v"(y3), "+v"(y4), "+v"(y5), "+v"(y6), "+v"(y7)
            : "v"(c));
    }
}

// One 128-entry vector (token, KV head, K or V) per quad of lanes.  Lane q of
// the quad holds the 8-entry chunks c = 4 i + q, i = 0..3 (entries 8c..8c+7)
// in y[8 i + k]: the quad's four 16-byte loads i cover 64 contiguous bytes
// each, and butterfly spans 1, 2, 4 (inside a chunk) and 32, 64 (chunk bits
// 2, 3 = i) stay in the lane; spans 8, 16 (chunk bits 0, 1 = q) pair lanes
// q ^ 1, q ^ 2 of the quad.  Span 1 is done while widening the fp16 input.
// Returns the sign F (+1 or -1) of this lane's results: y holds F times the
// transform (the lane-pair butterflies leave the upper lane's values negated;
// every later step is linear, so one sign per lane describes them all).
template <int BH>
__device__ __forceinline__ float rotate_chunks(const uint4 (&raw)[4], float (&y)[32], int q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        widen_span1(raw[i].x, y[8 * i + 0], y[8 * i + 1]);
        widen_span1(raw[i].y, y[8 * i + 2], y[8 * i + 3]);
        widen_span1(raw[i].z, y[8 * i + 4], y[8 * i + 5]);
        widen_span1(raw[i].w, y[8 * i + 6], y[8 * i + 7]);
    }
    // Spans 2, 4 inside each chunk.
#pragma unroll
    for (int span = 2; span < 8; span <<= 1) {
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            if (r & span) continue;
            const float u = y[r];
            const float v = y[r + span];
            y[r] = u + v;
            y[r + span] = u - v;
        }
    }
    // Spans 8 (lanes q, q ^ 1), then 16 (lanes q, q ^ 2).  After the first,
    // lanes with q & 1 hold negated values; in the second both partners carry
    // the same sign, so c = -1 again marks the upper lane, which flips its sign.
    static_assert(BH >= 32, "the lane-pair spans 8 and 16 are always part of the transform");
    const float c1 = (q & 1) ? -1.0f : 1.0f;
    const float c2 = (q & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; i += 8)
        quad_butterfly8<1>(y[i], y[i + 1], y[i + 2], y[i + 3], y[i + 4], y[i + 5], y[i + 6], y[i + 7], c1);
#pragma unroll
    for (int i = 0; i < 32; i += 8)
        quad_butterfly8<2>(y[i], y[i + 1], y[i + 2], y[i + 3], y[i + 4], y[i + 5], y[i + 6], y[i + 7], c2);
    // Spans 32, 64: chunk index bits 2, 3 are the register index bits 3, 4.
#pragma unroll
    for (int span = 8; span < 32; span <<= 1) {
        if (4 * span >= BH) break;
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            if (r & span) continue;
            const float u = y[r];
            const float v = y[r + span];
            y[r] = u + v;
            y[r + span] = u - v;
        }
    }
    return c1 * c2;
}

// Randomized Hadamard: the entries of chunk c (8 fp16 values, one 16-byte
// load) whose bits are set in byte c of the 128-bit sign mask are negated
// before the rotation, by flipping their fp16 sign bits (exact).
__device__ __forceinline__ uint4 sign_flip_words(uint4 w, const uint32_t (&mask)[4], int chunk) {
    const uint32_t b = (mask[chunk >> 2] >> (8 * (chunk & 3))) & 0xFFu;
    w.x ^= ((b & 1u) << 15) | ((b & 2u) << 30);
    w.y ^= ((b & 4u) << 13) | ((b & 8u) << 28);
    w.z ^= ((b & 16u) << 11) | ((b & 32u) << 26);
    w.w ^= ((b & 64u) << 9) | ((b & 128u) << 24);
    return w;
}

// Block b of the launch covers 64 consecutive tokens of one (KV head, K or
// V): token block b / (2 Hkv), then K heads 0 .. Hkv - 1 and V heads 0 ..
// Hkv - 1 in turn, so consecutive blocks read the adjacent 256-byte rows of
// the same tokens and write the adjacent code rows of the same pages
// (measured against blocks ordered head by head over the whole call: 52.7 ->
// 48.7 us for 65,536 tokens without rotation, 52.0 -> 50.6 us at Bh 64);
// quad g takes token base + g, so consecutive quads write consecutive slots
// of a page.
struct AppendBlock {
    int32_t token0, h;
    bool is_v;
};
__device__ __forceinline__ AppendBlock append_block(const AppendArgs &a) {
    const int32_t per_tokens = 2 * a.num_kv_heads;
    const int32_t bid = (int32_t)blockIdx.x;
    const int32_t tb = bid / per_tokens;
    const int32_t r = bid - tb * per_tokens;
    AppendBlock ab;
    ab.token0 = tb * kTokensPerBlock;
    ab.is_v = r >= a.num_kv_heads;
    ab.h = ab.is_v ? r - a.num_kv_heads : r;
    return ab;
}

template <int BH, bool SIGNS>
__global__ __launch_bounds__(kBlockThreads) void quant_append_kernel(AppendArgs a) {
    const int q = threadIdx.x & 3;
    const AppendBlock ab = append_block(a);
    const int32_t t = ab.token0 + (int32_t)(threadIdx.x >> 2);
    if (t >= a.num_tokens) return;  // the whole quad leaves together
    const int32_t h = ab.h;
    const bool is_v = ab.is_v;

    // Issue the address loads first; their latency overlaps the arithmetic.
    const int32_t seq = a.token_seq[t];
    const int32_t pos = a.token_pos[t];
    const int32_t page = a.page_table[(int64_t)seq * a.max_pages_per_seq + (pos >> a.page_shift)];
    const int32_t slot = pos & (a.page_size - 1);

    const uint4 *src = reinterpret_cast<const uint4 *>((is_v ? a.v_new : a.k_new) +
                                                       ((int64_t)t * a.num_kv_heads + h) * kHeadDim) + q;
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[4 * i];
    if constexpr (SIGNS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = sign_flip_words(raw[i], a.sign_mask, 4 * i + q);
    }

    float y[32];
    // 1/sqrt(Bh) is a power of two for Bh = 64: then y * c is exact, and
    // scaling the absmax and the divisor instead of the 128 entries gives the
    // same numbers (the quotient y c / s equals y / (s / c) exactly).
    constexpr bool kExactScale = (BH == 64);
    float sign = 1.0f;   // y holds sign times the rotated vector
    if constexpr (BH == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[8 * i + 0] = half_bits_to_float(raw[i].x);
            y[8 * i + 1] = half_bits_to_float(raw[i].x >> 16);
            y[8 * i + 2] = half_bits_to_float(raw[i].y);
            y[8 * i + 3] = half_bits_to_float(raw[i].y >> 16);
            y[8 * i + 4] = half_bits_to_float(raw[i].z);
            y[8 * i + 5] = half_bits_to_float(raw[i].z >> 16);
            y[8 * i + 6] = half_bits_to_float(raw[i].w);
            y[8 * i + 7] = half_bits_to_float(raw[i].w >> 16);
        }
    } else {
        sign = rotate_chunks<BH>(raw, y, q);
        if constexpr (!kExactScale) {
            const float c = inv_sqrt_block<BH>();
#pragma unroll
            for (int r = 0; r < 32; ++r) y[r] = y[r] * c;
        }
    }

    // Token-wise absmax over the 128 entries (exact): lane, then quad.
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) m = fmaxf(m, fabsf(y[r]));
    {
        // non-negative floats order like their bit patterns: integer max
        int k = __builtin_bit_cast(int, m);
        k = max(k, __builtin_amdgcn_mov_dpp(k, 0xB1, 0xF, 0xF, true));
        k = max(k, __builtin_amdgcn_mov_dpp(k, 0x4E, 0xF, 0xF, true));
        m = __builtin_bit_cast(float, k);
    }
    if constexpr (kExactScale) m = m * inv_sqrt_block<BH>();

    const float r7 = __builtin_bit_cast(float, 0x3E124925u);   // fp32 nearest 1/7
    const float m0 = m * r7;
    float s32 = __builtin_fmaf(__builtin_fmaf(-m0, 7.0f, m), r7, m0);   // == m / 7 (see header)
    // The empty asm keeps the compiler from folding the fp16 conversion into
    // the fma (one rounding to fp16 instead of fp32 then fp16: not the same).
    asm("" : "+v"(s32));
    const _Float16 s16 = static_cast<_Float16>(s32);  // round to nearest even
    const float s = static_cast<float>(s16);
    float sd = 0.0f;     // divisor (zero scale: every code is 0)
    float rcp = 0.0f;
    if (s > 0.0f && s <= 65504.0f) {
        // Correctly rounded 1/s: hardware reciprocal (1 ulp) and one Newton
        // step; equal to IEEE 1/s for every positive finite fp16 s (checked
        // on the device for all of them).
        const float r0 = __builtin_amdgcn_rcpf(s);
        rcp = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
        sd = s;
        if constexpr (kExactScale) {
            sd = s * 8.0f;              // s / c, exact
            rcp = rcp * 0.125f;         // 1 / (s / c), exact
        }
        // Dividing the sign-carrying entries by the sign-carrying divisor
        // gives the quotients of the true ones, exactly (IEEE division and
        // these steps are odd in the divisor).
        sd *= sign;
        rcp *= sign;
    }
    // With s a normal fp16 value (or 0) |y / s| <= 7 (1 + 2^-11) < 7.5, so
    // every code lies in [-7, 7] without clamping; only a subnormal scale
    // (an absmax below 7 * 2^-14) needs the clamp, and a wave takes the
    // clamping path only if one of its vectors has one.
    const bool no_clamp = __all(!(s > 0.0f && s < 6.103515625e-05f));

    uint8_t *pool = static_cast<uint8_t *>(is_v ? a.v_pool : a.k_pool);
    uint8_t *page_base = pool + (int64_t)page * a.num_kv_heads * a.tile_bytes;
    uint8_t *code_row = page_base + ((int64_t)h * a.page_size + slot) * kCodeBytesPerRow;
    uint8_t *scale_at = page_base + (int64_t)a.num_kv_heads * a.page_size * kCodeBytesPerRow +
                        ((int64_t)h * a.page_size + slot) * 2;
    // The quad's code words pass through LDS so that each lane stores 16
    // contiguous bytes of the row: lane q holds words q, q + 4, q + 8, q + 12
    // (chunks 4 i + q) and stores words 4 q .. 4 q + 3, and a wave's store
    // covers its 16 rows as whole cache lines.
    __shared__ __attribute__((aligned(16))) uint32_t words[kTokensPerBlock][kCodeBytesPerRow / 4];
    uint32_t *my_words = words[threadIdx.x >> 2];
    auto quantize_store = [&](auto clamp) {
        constexpr bool kClamp = decltype(clamp)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // Codes of chunk 4 i + q: exact quotient, clamp, round half to even
            // by adding 1.5 * 2^23 + 8 (the low byte of the sum is code + 8);
            // nibble pairs, then bytes, then xor 0x88 gives two's complement
            // nibbles.
            uint32_t u[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float yv = y[8 * i + k];
                const float q0 = yv * rcp;
                const float e = __builtin_fmaf(-q0, sd, yv);
                float qt = __builtin_fmaf(e, rcp, q0);  // == y / s (see header)
                // Clamping to integer bounds commutes with rounding to an integer.
                if constexpr (kClamp) qt = __builtin_amdgcn_fmed3f(qt, -8.0f, 7.0f);
                u[k] = __builtin_bit_cast(uint32_t, qt + 12582920.0f);
            }
            uint32_t b[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) b[k] = (u[2 * k + 1] << 4) | u[2 * k];   // low byte: the code pair
            const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);   // bytes b0.0, b1.0
            const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);   // b2.0, b3.0 at bytes 2, 3
            my_words[4 * i + q] = (lo | hi) ^ 0x88888888u;
        }
        // the quad's lanes are in one wave: a wave-level LDS ordering suffices
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // Non-temporal store: the codes are not read again in this pass (the
        // decode streams them later); measured 63 -> 53.5 us for 65,536
        // tokens, where normally cached stores disturb the input stream.
        const uint4 w4 = *reinterpret_cast<const uint4 *>(&my_words[4 * q]);
        __builtin_nontemporal_store(v4u{w4.x, w4.y, w4.z, w4.w},
                                    reinterpret_cast<v4u *>(code_row + 16 * q));
    };
    if (no_clamp) quantize_store(std::false_type{});
    else quantize_store(std::true_type{});
    if (q == 0) {
        __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, s16),   // non-temporal, as the codes
                                    reinterpret_cast<uint16_t *>(scale_at));
    }
}

// ---------------------------------------------------------------------------
// Quantizer variants: one scale per group of G channels (INT4, optionally
// chosen by a search over clipping ratios) or MXFP4 (E2M1 codes, one E8M0
// scale per 32 channels).  Source: "BitDecoding-FP4:FP4 KVキャッシュのネイティブ
// 復号", section 深掘り分析 (a scale chosen per group by scale search, after a
// Hadamard rotation) and its opening summary (4-bit microscaling formats).
// The arithmetic is bit-exact with the definition in include/kvq.h
// (kv_quant_append_cfg).  The mapping is the token-wise kernel's: a quad of
// lanes per vector, lane q holding chunks 4 i + q in y[8 i .. 8 i + 7], so
// group g of G channels is registers y[R g .. R g + R - 1] (R = G / 4) of
// every lane of the quad.
// ---------------------------------------------------------------------------

// m / 7 as the IEEE quotient (Markstein, see the file header).
__device__ __forceinline__ float div7(float m) {
    const float r7 = __builtin_bit_cast(float, 0x3E124925u);
    const float m0 = m * r7;
    float s32 = __builtin_fmaf(__builtin_fmaf(-m0, 7.0f, m), r7, m0);
    asm("" : "+v"(s32));   // keeps the fp16 conversion from folding into the fma
    return s32;
}

// Correctly rounded 1 / s for a positive finite fp16 value s (see the header).
__device__ __forceinline__ float rcp_fp16(float s) {
    const float r0 = __builtin_amdgcn_rcpf(s);
    return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// IEEE y / s for an fp16 divisor s given rcp = 1 / s (see the header; both
// may carry the lane's sign, the quotient is odd in the divisor).
__device__ __forceinline__ float div_fp16(float y, float s, float rcp) {
    const float q0 = y * rcp;
    const float e = __builtin_fmaf(-q0, s, y);
    return __builtin_fmaf(e, rcp, q0);
}

__device__ __forceinline__ float quad_max_nonneg(float v) {
    int k = __builtin_bit_cast(int, v);
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0xB1, 0xF, 0xF, true));
    k = max(k, __builtin_amdgcn_mov_dpp(k, 0x4E, 0xF, 0xF, true));
    return __builtin_bit_cast(float, k);
}

__device__ __forceinline__ uint32_t quad_sum_u32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
    v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
    return v;
}

// Exponent E with m < 2^E for a normal positive fp32 m (frexp's exponent).
__device__ __forceinline__ int frexp_exp(float m) {
    return (int)((__builtin_bit_cast(uint32_t, m) >> 23) & 0xFFu) - 126;
}

// Error of INT4 candidate scale s (fp16 value; this lane's R registers):
// sum of D^2, D = round-half-even((y - s c) 2^(12 - E)) with the candidate's
// codes c; |D| <= 2^12, so the quad's sum over up to 128 channels fits in 32
// bits.  y carries the lane's sign, which D^2 does not see.
template <int R>
__device__ __forceinline__ uint32_t int4_candidate_err(const float *y, float s, float sign, float scl) {
    uint32_t err = 0;
    if (s > 0.0f) {
        const float sd = s * sign, rcp = rcp_fp16(s) * sign;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float c = __builtin_rintf(__builtin_amdgcn_fmed3f(div_fp16(y[r], sd, rcp), -8.0f, 7.0f));
            const float res = __builtin_fmaf(-sd, c, y[r]);   // s c is exact: one rounding, as y - s c
            const int D = (int)__builtin_rintf(res * scl);
            const uint32_t a = (uint32_t)(D < 0 ? -D : D);
            err += __umul24(a, a);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int D = (int)__builtin_rintf(y[r] * scl);
            const uint32_t a = (uint32_t)(D < 0 ? -D : D);
            err += __umul24(a, a);
        }
    }
    return err;
}

template <int FMT, int G, bool SEARCH>
__global__ __launch_bounds__(kBlockThreads) void quant_append_grouped_kernel(AppendArgs a) {
    constexpr int NG = kHeadDim / G;       // scale groups per vector
    constexpr int R = G / 4;               // registers of one group in each lane of the quad
    constexpr int SB = FMT == KVQ_FMT_MXFP4 ? 1 : 2;   // bytes per scale
    const int q = threadIdx.x & 3;
    const AppendBlock ab = append_block(a);
    const int32_t t = ab.token0 + (int32_t)(threadIdx.x >> 2);
    if (t >= a.num_tokens) return;  // the whole quad leaves together
    const int32_t h = ab.h;
    const bool is_v = ab.is_v;

    const int32_t seq = a.token_seq[t];
    const int32_t pos = a.token_pos[t];
    const int32_t page = a.page_table[(int64_t)seq * a.max_pages_per_seq + (pos >> a.page_shift)];
    const int32_t slot = pos & (a.page_size - 1);

    const uint4 *src = reinterpret_cast<const uint4 *>((is_v ? a.v_new : a.k_new) +
                                                       ((int64_t)t * a.num_kv_heads + h) * kHeadDim) + q;
    uint4 raw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[i] = src[4 * i];
    if ((a.sign_mask[0] | a.sign_mask[1] | a.sign_mask[2] | a.sign_mask[3]) != 0u) {   // uniform
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[i] = sign_flip_words(raw[i], a.sign_mask, 4 * i + q);
    }

    // y = R (S x), times the lane's sign (see rotate_chunks)
    float y[32];
    float sign = 1.0f;
    auto scale_entries = [&](float c) {
#pragma unroll
        for (int r = 0; r < 32; ++r) y[r] = y[r] * c;
    };
    switch (a.had_block) {
        case 32: sign = rotate_chunks<32>(raw, y, q); scale_entries(inv_sqrt_block<32>()); break;
        case 64: sign = rotate_chunks<64>(raw, y, q); scale_entries(inv_sqrt_block<64>()); break;
        case 128: sign = rotate_chunks<128>(raw, y, q); scale_entries(inv_sqrt_block<128>()); break;
        default:
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w4[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[8 * i + 2 * e] = half_bits_to_float(w4[e]);
                    y[8 * i + 2 * e + 1] = half_bits_to_float(w4[e] >> 16);
                }
            }
            break;
    }

    uint32_t nib[32];          // stored nibble of each entry
    uint32_t sbits[NG];        // stored scale of each group (fp16 bits or E8M0 byte), same in the quad
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        float *yg = &y[R * gi];
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) m = fmaxf(m, fabsf(yg[r]));
        m = quad_max_nonneg(m);
        if constexpr (FMT == KVQ_FMT_INT4) {
            _Float16 s16 = static_cast<_Float16>(div7(m));
            if constexpr (SEARCH) {
                // candidates fp16(fp32(m a_k) / 7), a_k = (16 - k) / 16: the
                // smallest integer error wins, ties to the smaller k
                const float scl = ldexpf(1.0f, 12 - (m > 0.0f ? frexp_exp(m) : 0));
                uint32_t best = 0xFFFFFFFFu;
#pragma unroll 1
                for (int k = 0; k < 8; ++k) {
                    const _Float16 c16 = static_cast<_Float16>(div7(m * (static_cast<float>(16 - k) * 0.0625f)));
                    const uint32_t err = quad_sum_u32(int4_candidate_err<R>(yg, static_cast<float>(c16), sign, scl));
                    if (err < best) {
                        best = err;
                        s16 = c16;
                    }
                }
            }
            const float s = static_cast<float>(s16);
            sbits[gi] = __builtin_bit_cast(uint16_t, s16);
            // zero scale: every code is 0 (divisor and reciprocal 0)
            float sd = 0.0f, rcp = 0.0f;
            if (s > 0.0f) {
                sd = s * sign;
                rcp = rcp_fp16(s) * sign;
            }
            // With the plain scale fp16(m / 7), normal, |y / s| <= 7 (1 +
            // 2^-11) < 7.5, so the codes need no clamp; a wave clamps only if
            // one of its groups has a subnormal scale (the token-wise
            // kernel's argument).  A searched scale clips: always clamp.
            auto codes = [&](auto clamp) {
                constexpr bool kClamp = decltype(clamp)::value;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    float qt = div_fp16(yg[r], sd, rcp);
                    if constexpr (kClamp) qt = __builtin_amdgcn_fmed3f(qt, -8.0f, 7.0f);
                    // round half to even, low nibble = code + 8; xor 8: two's complement
                    nib[R * gi + r] = (__builtin_bit_cast(uint32_t, qt + 12582920.0f) & 0xFu) ^ 8u;
                }
            };
            if (!SEARCH && __all(!(s > 0.0f && s < 6.103515625e-05f))) codes(std::false_type{});
            else codes(std::true_type{});
        } else {
            // MXFP4: X = floor(log2 m) - 2, element = nearest E2M1 value to
            // y / 2^X (ties to the even code, saturating at 6), sign bit set
            // iff the value is negative.  gfx950's v_cvt_scalef32_pk_fp4_f32
            // converts two fp32 values divided by a power-of-two scale to
            // E2M1 exactly so (round to nearest even, saturating, sign of the
            // quotient), which a probe over every multiple of 1/64 in
            // [-10, 10] (all ties) and +-0, tiny, subnormal and large inputs
            // confirmed for scales 2^-3 .. 2^3; the one difference, -0 giving
            // the sign bit, is removed by adding +0 (-0 + 0 = +0, every other
            // value unchanged).  It takes the entries' true signs: y times the
            // lane's sign (exact).  |X| stays far inside the normal range
            // (rotated fp16 inputs), so 2^X is a normal fp32.
            if (m > 0.0f) {
                int X = frexp_exp(m) - 3;
                X = X < -127 ? -127 : (X > 127 ? 127 : X);
                sbits[gi] = (uint32_t)(X + 127);
                const float scale = ldexpf(1.0f, X);
#pragma unroll
                for (int r = 0; r < R; r += 2) {
                    const float v0 = yg[r] * sign + 0.0f, v1 = yg[r + 1] * sign + 0.0f;
                    const uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, scale, 0) & 0xFFu;
                    nib[R * gi + r] = b & 0xFu;
                    nib[R * gi + r + 1] = b >> 4;
                }
            } else {
                sbits[gi] = 0u;
#pragma unroll
                for (int r = 0; r < R; ++r) nib[R * gi + r] = 0u;
            }
        }
    }

    uint8_t *pool = static_cast<uint8_t *>(is_v ? a.v_pool : a.k_pool);
    uint8_t *page_base = pool + (int64_t)page * a.num_kv_heads * a.tile_bytes;
    uint8_t *code_row = page_base + ((int64_t)h * a.page_size + slot) * kCodeBytesPerRow;
    uint8_t *scale_at = page_base + (int64_t)a.num_kv_heads * a.page_size * kCodeBytesPerRow +
                        ((int64_t)h * a.page_size + slot) * (NG * SB);
    __shared__ __attribute__((aligned(16))) uint32_t words[kTokensPerBlock][kCodeBytesPerRow / 4];
    uint32_t *my_words = words[threadIdx.x >> 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= nib[8 * i + k] << (4 * k);
        my_words[4 * i + q] = w;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const uint4 w4 = *reinterpret_cast<const uint4 *>(&my_words[4 * q]);
    __builtin_nontemporal_store(v4u{w4.x, w4.y, w4.z, w4.w}, reinterpret_cast<v4u *>(code_row + 16 * q));
    if (q == 0) {
        if constexpr (NG * SB == 8) {   // non-temporal, as the codes
            typedef unsigned int v2u __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(v2u{sbits[0] | (sbits[1] << 16), sbits[2] | (sbits[3] << 16)},
                                        reinterpret_cast<v2u *>(scale_at));
        } else if constexpr (NG * SB == 4) {
            const uint32_t v1 = SB == 2 ? (sbits[0] | (sbits[NG - 1] << 16))
                                        : (sbits[0] | (sbits[NG > 1 ? 1 : 0] << 8) | (sbits[NG > 2 ? 2 : 0] << 16) |
                                           (sbits[NG > 3 ? 3 : 0] << 24));
            __builtin_nontemporal_store(v1, reinterpret_cast<uint32_t *>(scale_at));
        } else {
            static_assert(NG * SB == 2, "scale bytes per vector");
            __builtin_nontemporal_store(static_cast<uint16_t>(sbits[0]), reinterpret_cast<uint16_t *>(scale_at));
        }
    }
}

// fp16 baseline: copy one 256-byte row per 16 lanes.
__global__ __launch_bounds__(kBlockThreads) void append_fp16_kernel(AppendArgs a) {
    const int lane = threadIdx.x & (kLanesPerVec - 1);
    const int64_t vec = (int64_t)blockIdx.x * kVecsPerBlock + (threadIdx.x / kLanesPerVec);
    const int64_t per_tensor = (int64_t)a.num_tokens * a.num_kv_heads;
    if (vec >= 2 * per_tensor) return;
    const bool is_v = vec >= per_tensor;
    const int64_t row = is_v ? vec - per_tensor : vec;
    const int32_t t = (int32_t)(row / a.num_kv_heads);
    const int32_t h = (int32_t)(row - (int64_t)t * a.num_kv_heads);
    const int32_t seq = a.token_seq[t];
    const int32_t pos = a.token_pos[t];
    const int32_t page = a.page_table[(int64_t)seq * a.max_pages_per_seq + (pos >> a.page_shift)];
    const int32_t slot = pos & (a.page_size - 1);
    const uint4 raw = *reinterpret_cast<const uint4 *>((is_v ? a.v_new : a.k_new) + row * kHeadDim + lane * 8);
    uint16_t *pool = static_cast<uint16_t *>(is_v ? a.v_pool : a.k_pool);
    uint16_t *dst = pool + (((int64_t)page * a.num_kv_heads + h) * a.page_size + slot) * kHeadDim + lane * 8;
    __builtin_nontemporal_store(v4u{raw.x, raw.y, raw.z, raw.w}, reinterpret_cast<v4u *>(dst));   // as the INT4 codes
}

dim3 grid_for(const AppendArgs &a) {
    const int64_t vecs = 2 * (int64_t)a.num_tokens * a.num_kv_heads;
    return dim3((unsigned)((vecs + kVecsPerBlock - 1) / kVecsPerBlock));
}

}  // namespace

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream) {
    // one dimension: (token block, K or V, head), see append_block
    const int64_t blocks = (int64_t)((a.num_tokens + kTokensPerBlock - 1) / kTokensPerBlock) * 2 * a.num_kv_heads;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks, 1, 1);
    const bool signs = (a.sign_mask[0] | a.sign_mask[1] | a.sign_mask[2] | a.sign_mask[3]) != 0;
    if (a.format != KVQ_FMT_INT4 || a.scale_group != kHeadDim || a.scale_search) {
        // per-group scales, scale search, MXFP4
#define KVQ_GROUPED(FMT, G, S) hipLaunchKernelGGL((quant_append_grouped_kernel<FMT, G, S>), grid, dim3(kBlockThreads), 0, stream, a)
        if (a.format == KVQ_FMT_MXFP4) {
            if (a.scale_group != 32 || a.scale_search) return hipErrorInvalidValue;
            KVQ_GROUPED(KVQ_FMT_MXFP4, 32, false);
        } else if (a.scale_group == 32) {
            if (a.scale_search) KVQ_GROUPED(KVQ_FMT_INT4, 32, true); else KVQ_GROUPED(KVQ_FMT_INT4, 32, false);
        } else if (a.scale_group == 64) {
            if (a.scale_search) KVQ_GROUPED(KVQ_FMT_INT4, 64, true); else KVQ_GROUPED(KVQ_FMT_INT4, 64, false);
        } else if (a.scale_group == 128) {
            KVQ_GROUPED(KVQ_FMT_INT4, 128, true);
        } else {
            return hipErrorInvalidValue;
        }
#undef KVQ_GROUPED
        return hipGetLastError();
    }
#define KVQ_TOKEN(BHV) \
    do { \
        if (signs) hipLaunchKernelGGL((quant_append_kernel<BHV, true>), grid, dim3(kBlockThreads), 0, stream, a); \
        else hipLaunchKernelGGL((quant_append_kernel<BHV, false>), grid, dim3(kBlockThreads), 0, stream, a); \
    } while (0)
    switch (a.had_block) {
        case 0: KVQ_TOKEN(0); break;
        case 32: KVQ_TOKEN(32); break;
        case 64: KVQ_TOKEN(64); break;
        case 128: KVQ_TOKEN(128); break;
        default: return hipErrorInvalidValue;
    }
#undef KVQ_TOKEN
    return hipGetLastError();
}

hipError_t launch_append_fp16(const AppendArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(append_fp16_kernel, grid_for(a), dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
