// Paged decode attention over the INT4 cache on the int8 matrix cores
// (v_mfma_i32_16x16x64_i8): split-K partial kernel.
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// sections "KVキャッシュこそが本当のボトルネックである理由" (every decode step
// streams the whole paged cache, with fused attention) and
// "回転のトリック — ブロック対角アダマール" (R = H/sqrt(Bh) is orthogonal and its
// own inverse: the query is rotated once, (R q).(R k) = q.k, and the merged
// output is rotated back by the combine kernel).
//
// Why matrix cores: for each (token, KV head) the four query heads of a GQA
// group need 4 x 128 multiply-adds for q.k and 4 x 128 for p.v against only
// 132 bytes of cache.  On the vector ALUs that work, plus unpacking, bounds
// the kernel far below the HBM roofline (measured: ~3,300 lane operations per
// token-head).  Both products are exact integer contractions once the fp32
// operand is written in fixed point, so they map onto int8 MFMA:
//
//   q.k : the rotated, pre-scaled query of head hq is written as a 28-bit
//         fixed-point integer X = round(q' 2^(27-E)), E the exponent of
//         max|q'| of that head, split into limbs
//         X = L0 2^21 + L1 2^14 + L2 2^7 + L3 (L0 signed, L1..L3 in
//         [0,127]).  One MFMA row per (head, limb): 4 heads x 4 limbs fill
//         the 16 rows.  Keys enter as offset-binary nibbles u = c + 8 in
//         [0, 15]; the accumulator starts at -8 sum_d L (per row), so the
//         integer result is exactly sum_d L_d c_d.
//   p.v : the unnormalised weight times the value scale, P = p s_V, is
//         written as a 21-bit unsigned fixed-point integer F relative to the
//         largest P of the head in the 64-token chunk, split the same way
//         into three 7-bit limbs (again one row per (head, limb)).  Values
//         also enter as offset-binary nibbles u = c + 8; the MFMA gives
//         sum_t F_t u_t exactly, and 8 sum_t F_t (one number per head and
//         chunk) is subtracted in fp32.
// Limbs are recombined with integer shifts (exact, below 2^31) and fp32
// conversions.  The approximations are the 2^-28 relative rounding of q' and
// the 2^-21 one of P (each relative to the largest element of its vector),
// and fp32 rounding of the accumulation and of the offset subtraction.  (With
// a 21-bit query the query's rounding dominated the error: scores are sums of
// 128 products with keys up to 7 scale units, and a sharp softmax turns their
// absolute error into a relative weight error.)
//
// Work decomposition: one wave owns one work item (sequence, KV head, 4 of
// its query heads, a page range of at most 2048 tokens) and walks it in
// chunks of 64 tokens.  A block holds the 4 waves of 4 KV heads of the same
// sequence and page range: they read adjacent tiles of the same pages (DRAM
// locality) and share nothing but LDS space.  The grid is ordered
// page-range-major (blockIdx.y).  A sequence's chunks are shared out evenly
// over its ranges (no short remainder range), so the work items of a launch
// have similar sizes and the launch does not end on a few long ones.  Ranges are long because every partial result
// written back costs far more than its size in lost read bandwidth (writes
// interleaved with the streaming reads).
//
// Layout of one wave (64 lanes, g = lane / 16, j = lane % 16), per chunk
// (4 groups t of 16 tokens; a group is one page of 16 tokens or half a page
// of 32):
//   q.k  A (query limbs): lane row j = (head j/4, limb j%4), k-slots of lane
//        group g = dims 32g + 2e (MFMA 0) and 32g + 2e + 1 (MFMA 1), e < 16.
//        B (keys): lane column j = token j of the group; the lane's 16-byte
//        load of the token's codes (bytes 16g..16g+15 = dims 32g..32g+31)
//        splits into low nibbles (MFMA 0) and high nibbles (MFMA 1).
//        D: lane (g, j) gets rows (head g, limbs 0..3) for token j, i.e. the
//        score of head g for one token: no replicated softmax work.
//   softmax: the running max of head g lives in row g (16 lanes), which is
//        also where head g's output accumulates below, so rescaling needs no
//        cross-lane traffic.
//   P hand-off: each lane writes its fixed-point P (one dword per token) to
//        1 KiB of LDS; lane (g, j) reads back the 16 tokens of group g for
//        head j/4 and keeps limb j%4 (A operand of p.v).
//   p.v  B (values): lane column j = dim 16m + j of MFMA m, k-slots = the
//        16 tokens of group g.  Values go from HBM straight into LDS
//        (global_load_lds_dwordx4, 1 KiB per instruction) and are read back
//        with gfx950's transposed 4-bit LDS read (ds_read_b64_tr_b4): one read
//        gives a lane one dim of 16 tokens as 16 nibbles, which split into
//        the operand's bytes with two bit operations each.
//        D: lane (g, j) gets rows (head g, limbs) for dim 16m + j.
//   Pipelining: chunk c + 1 loads while chunk c computes, its values into
//        the second LDS buffer, its keys and scales into registers once chunk
//        c's have been used.
//   All cache bytes are read with non-temporal 16-byte loads.
#include <type_traits>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dec;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int kChunk = kChunkTokens;  // 64 tokens per chunk

// Low / high nibbles of 8 two's-complement codes as offset-binary bytes
// (c + 8 = c xor 8 on 4 bits).  Each is one 3-input bitwise op on gfx950
// (v_bitop3), plus one shift for the high nibbles.
__device__ __forceinline__ void split_offset(uint32_t w, uint32_t &lo, uint32_t &hi) {
    lo = (w ^ 0x08080808u) & 0x0F0F0F0Fu;
    hi = ((w >> 4) ^ 0x08080808u) & 0x0F0F0F0Fu;
}

// 4x4 byte transpose: out[k] byte r = in[r] byte k.
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t &o0,
                                           uint32_t &o1, uint32_t &o2, uint32_t &o3) {
    // v_perm_b32(x, y, sel): selector bytes 0-3 pick bytes of y, 4-7 bytes of x.
    const uint32_t ab02 = __builtin_amdgcn_perm(b, a, 0x06020400u);  // a0 b0 a2 b2
    const uint32_t ab13 = __builtin_amdgcn_perm(b, a, 0x07030501u);  // a1 b1 a3 b3
    const uint32_t cd02 = __builtin_amdgcn_perm(d, c, 0x06020400u);  // c0 d0 c2 d2
    const uint32_t cd13 = __builtin_amdgcn_perm(d, c, 0x07030501u);  // c1 d1 c3 d3
    o0 = __builtin_amdgcn_perm(cd02, ab02, 0x05040100u);             // a0 b0 c0 d0
    o2 = __builtin_amdgcn_perm(cd02, ab02, 0x07060302u);             // a2 b2 c2 d2
    o1 = __builtin_amdgcn_perm(cd13, ab13, 0x05040100u);             // a1 b1 c1 d1
    o3 = __builtin_amdgcn_perm(cd13, ab13, 0x07060302u);             // a3 b3 c3 d3
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// D0 2^21 + D1 2^14 + D2 2^7 + D3 of one (head, limbs 0..3) row group of
// q.k: |D0| <= 2^16 and |D1..D3| < 2^17, so the halves D0 2^7 + D1 (below
// 2^24: exact in fp32) and D2 2^7 + D3 (below 2^25) are exact in int32, and
// the sum takes one fma (one rounding, plus at most one in the low half's
// conversion, both relative 2^-24 to the largest term).
__device__ __forceinline__ float limbs4_to_float(v4i d) {
    const int hi = (d[0] << 7) + d[1];
    const int lo = (d[2] << 7) + d[3];
    return fmaf(static_cast<float>(hi), 16384.0f, static_cast<float>(lo));
}
// D0 2^14 + D1 2^7 + D2 of one (head, limbs 0..2) row group of p.v, exact in
// 32 bits (0 <= D0 < 64*127*15), then one rounding.  (Two shift-and-add
// instructions; the empty asm keeps the compiler from re-associating them
// into three.)
__device__ __forceinline__ float ulimbs_to_float(v4i d) {
    uint32_t s = (static_cast<uint32_t>(d[0]) << 7) + static_cast<uint32_t>(d[1]);
    asm("" : "+v"(s));
    s = (s << 7) + static_cast<uint32_t>(d[2]);
    return static_cast<float>(s);
}

// Value codes go from HBM straight to LDS (global_load_lds_dwordx4: lane l
// of the instruction deposits its 16 bytes at 16 l of a 1 KiB block) and are
// read back transposed; a chunk's reads come first in its compute step, so
// the next chunk's values can load into the same buffer right after them.  One 16-token group is one 1 KiB
// block: 16 rows of 64 code bytes, row n's 16-byte piece p stored in slot
// 4n + (p ^ ((n >> 2) & 3)).  A transposed read (one 8-byte word from each of
// the group's 16 rows) then touches 32 distinct banks; the groups start at
// 0, 1152, 2176 and 3328 bytes, so that the two groups read in the same pass
// (0 and 1, 2 and 3) lie 128 bytes apart modulo 256 and use the other 32.
constexpr int kVGroupBytes = 1024;
__host__ __device__ constexpr int vgroup_off(int t) { return t * kVGroupBytes + 128 * ((t + 1) >> 1); }
constexpr int kVBufBytes = vgroup_off(3) + kVGroupBytes;     // 4352
static_assert(vgroup_off(1) >= kVGroupBytes && vgroup_off(2) >= vgroup_off(1) + kVGroupBytes &&
              vgroup_off(3) >= vgroup_off(2) + kVGroupBytes, "value groups overlap");
constexpr int kPfixPitch = kChunk + 4;                          // dwords per head row

// LDS of one wave, in arrays of their own so that the compiler can tell the
// value loads' destination apart from the rest (and waits for the value
// loads only before reading values):
//   value space: one chunk of value codes, vbuf[kVBufBytes];
//   query space: the query limbs, qlimb[kH][4][2][4][4]
//                ([head][limb][parity][lane group][dword]), written and read
//                at set-up while the range's first chunk already loads;
//   P space:     fixed-point P of the current chunk, pfix[kH][kPfixPitch];
//   held state:  (balanced decode) one partial state kept back until the end
//                of the wave's range, lane-private: 8 output floats, max, sum.
struct alignas(16) WaveValues {
    uint8_t vbuf[kVBufBytes];
};
typedef uint32_t QLimbs[kH][4][2][4][4];
struct alignas(16) WaveQuery {
    QLimbs qlimb;
};
struct alignas(16) WavePfix {
    uint32_t pfix[kH][kPfixPitch];
};
struct alignas(16) WaveHeld {
    float4 o[2][64];     // [half][lane]: o[4 h .. 4 h + 3]
    float2 ml[64];       // [lane]: (max, sum)
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Streaming 16-byte load that does not allocate in the L1 cache: the cache is
// read once per step, and on gfx950 this is the load shape that keeps enough
// requests in flight to approach the HBM roofline on scattered 1 KiB tiles.
__device__ __forceinline__ uint4 stream_load16(const uint8_t *p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw cache bytes of one chunk, as loaded.
struct ChunkData {
    uint4 k[4];          // keys: group t, token j, dims 32g..32g+31
    uint32_t ks;         // key scale (fp16 bits) of group g, token j
    uint32_t vs;         // value scale (fp16 bits) of group g, token j
};

// x held by lane (row r, j) of each row of 16 lanes -> y[t] = x of lane
// (t, j), in every row: one v_permlane16_swap pairs rows (0,1) and (2,3),
// two v_permlane32_swap pair the halves.
__device__ __forceinline__ void rows_broadcast(uint32_t x, uint32_t (&y)[4]) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);       // rows r & ~1, r | 1
    const auto e = __builtin_amdgcn_permlane32_swap(r[0], r[0], false, false);  // rows 0, 2
    const auto o = __builtin_amdgcn_permlane32_swap(r[1], r[1], false, false);  // rows 1, 3
    y[0] = e[0];
    y[1] = o[0];
    y[2] = e[1];
    y[3] = o[1];
}

// Address of tile (page phys) in a pool: base + phys * stride (wave-uniform).
__device__ __forceinline__ const uint8_t *tile_addr(const uint8_t *base, uint32_t phys, uint32_t stride) {
    return base + (uint64_t)phys * stride;
}

// Value of lane j ^ M of the same row of 16 (M = 1, 2, 4, 8) by DPP: quad
// permutes, and the row mirrors (lane i takes lane 15 - i, or 7 - i within
// each half row), two of which compose to xor 4 or xor 8.
template <int M>
__device__ __forceinline__ float row_xor(float v) {
    const int x = __builtin_bit_cast(int, v);
    if constexpr (M == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true));
    } else if constexpr (M == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true));
    } else if constexpr (M == 4) {
        const int y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(y, 0x1B, 0xF, 0xF, true));
    } else {
        static_assert(M == 8, "lane distance inside a row of 16");
        const int y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, true));
    }
}

// Butterflies of spans 8 .. BH/2 over 8 entries per lane (dims 8j .. 8j + 7)
// between lanes j and j ^ span/8, in ascending order: the lower entry gets
// u + v, the upper one u - v (u the lower entry's value).
template <int M, int BH>
__device__ __forceinline__ void row_butterflies(float (&y)[8], int j) {
    if constexpr (M < BH / 8) {
        const bool upper = (j & M) != 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float p = row_xor<M>(y[r]);
            y[r] = upper ? (p - y[r]) : (y[r] + p);
        }
        row_butterflies<2 * M, BH>(y, j);
    }
}

// Rotated query of lane (g, j): dims 8j .. 8j + 7 of one head from its fp16
// words (zero if !live), with the sign mask of the randomized Hadamard
// (byte j of the mask) applied first: R (S q) in fp32.
template <int BH>
__device__ __forceinline__ void rotate_query(uint4 raw, const uint32_t (&mask)[4], int j, bool live,
                                             float (&qv)[8]) {
    const uint4 rs = sign_flip_query(raw, mask, j);
    if (live) {
        qv[0] = half_to_float(rs.x); qv[1] = half_to_float(rs.x >> 16);
        qv[2] = half_to_float(rs.y); qv[3] = half_to_float(rs.y >> 16);
        qv[4] = half_to_float(rs.z); qv[5] = half_to_float(rs.z >> 16);
        qv[6] = half_to_float(rs.w); qv[7] = half_to_float(rs.w >> 16);
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) qv[r] = 0.0f;
    }
    if constexpr (BH > 0) {
#pragma unroll
        for (int span = 1; span < 8; span <<= 1) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r & span) continue;
                const float u = qv[r], v = qv[r + span];
                qv[r] = u + v;
                qv[r + span] = u - v;
            }
        }
        row_butterflies<1, BH>(qv, j);
        const float c = rsqrtf(static_cast<float>(BH));
#pragma unroll
        for (int r = 0; r < 8; ++r) qv[r] *= c;
    }
}

// ---- fused decode step: the sequence's new token ----
//
// Rotation and token-wise INT4 of one fp16 row (K or V of the new token),
// held as lane (g, j) = dims 8j .. 8j + 7 (every row g of 16 lanes holds the
// whole vector, the layout of the query set-up), with the append's
// arithmetic: fp32 butterflies of ascending span (spans 1, 2, 4 inside the
// lane, 8 .. Bh/2 between lanes j and j ^ span/8; lower entry u + v, upper
// u - v), the product with the fp32 nearest 1/sqrt(Bh), m = max |y| (exact),
// s = fp16(m / 7) (IEEE quotient, then round to nearest even), code =
// clamp(rint(y / s), -8, 7) with the IEEE quotient and rint rounding half
// to even.  Gives the lane's four
// code bytes (dims 8j + 2i in the low nibble of byte i), the dequantized
// entries and the scale.
struct NewRow {
    uint32_t bytes;
    float d[8];
    float s;
    uint16_t s16;
};
template <int BH>
__device__ __forceinline__ NewRow quantize_new_row(uint4 w, int j) {
#pragma clang fp contract(off)
    float y[8] = {half_to_float(w.x), half_to_float(w.x >> 16), half_to_float(w.y), half_to_float(w.y >> 16),
                  half_to_float(w.z), half_to_float(w.z >> 16), half_to_float(w.w), half_to_float(w.w >> 16)};
    if constexpr (BH > 0) {
#pragma unroll
        for (int span = 1; span < 8; span <<= 1) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r & span) continue;
                const float u = y[r], v = y[r + span];
                y[r] = u + v;
                y[r + span] = u - v;
            }
        }
        row_butterflies<1, BH>(y, j);
        const float c = __builtin_bit_cast(float, BH == 32 ? 0x3E3504F3u : BH == 64 ? 0x3E000000u : 0x3DB504F3u);
#pragma unroll
        for (int r = 0; r < 8; ++r) y[r] = y[r] * c;
    }
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(y[r]));
    m = row_max16(m);
    // m / 7 and y / s as the IEEE quotients without a division: q0 = x r,
    // e = fma(-q0, d, x), q = fma(e, r, q0), with r the fp32 nearest 1/7 for
    // m / 7 (exact for every non-negative finite m) and the correctly
    // rounded 1/s for y / s (exact for every fp16 divisor s over the
    // quotients that decide a code; smaller ones give code 0, larger ones
    // clamp either way) -- the append kernel's arithmetic.
    const float r7 = __builtin_bit_cast(float, 0x3E124925u);
    const float m0 = m * r7;
    float s32 = __builtin_fmaf(__builtin_fmaf(-m0, 7.0f, m), r7, m0);
    asm("" : "+v"(s32));   // two roundings (fp32, then fp16), as written
    const _Float16 h = static_cast<_Float16>(s32);
    NewRow nr;
    nr.s = static_cast<float>(h);
    nr.s16 = __builtin_bit_cast(uint16_t, h);
    float sd = 0.0f, rcp = 0.0f;   // zero scale: every code is 0
    if (nr.s > 0.0f && nr.s <= 65504.0f) {
        const float r0 = __builtin_amdgcn_rcpf(nr.s);
        rcp = __builtin_fmaf(__builtin_fmaf(-nr.s, r0, 1.0f), r0, r0);
        sd = nr.s;
    }
    nr.bytes = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float q0 = y[r] * rcp;
        const float e = __builtin_fmaf(-q0, sd, y[r]);
        const float qt = __builtin_amdgcn_fmed3f(__builtin_fmaf(e, rcp, q0), -8.0f, 7.0f);
        // round half to even at unit spacing: the low byte of the sum is code + 8
        const uint32_t u = __builtin_bit_cast(uint32_t, qt + 12582920.0f) & 15u;
        nr.d[r] = static_cast<float>(static_cast<int>(u) - 8) * nr.s;
        nr.bytes |= (u ^ 8u) << (4 * r);
    }
    return nr;
}

// One work range: tokens [p0 P, min(p1 P, L)) of sequence b (p0 on a chunk
// boundary) for head slot (KV head hk, query-head chunk chunk_id); returns
// its partial softmax state.  In the fused decode step (a.k_new set) the
// range that ends at the sequence's last cached token also takes the new
// token at position L: it quantizes the token's K and V rows, stores them
// (head chunk 0 of the KV head), and starts its online softmax from that
// token (max = its score, sum = 1, output = its value row).
template <int BH, int P>
__device__ __forceinline__ PartialState decode_range(const DecodeArgs &a, WaveValues &sv, WavePfix &sp,
                                                     WaveQuery &sq, const int lane, const int b, const int hk,
                                                     const int chunk_id, const int L, const int p0, const int p1) {
    const int g = lane >> 4;
    const int j = lane & 15;
    const int tok_begin = p0 * P;
    const int tok_end = min(p1 * P, L);
    const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
    const int qh0 = hk * a.group + chunk_id * kH;
    const int nheads = min(kH, a.group - chunk_id * kH);

    // The query (lane (g, j) holds dims 8j..8j+7 of head g) loads first, ahead
    // of the first chunk's loads: the counter of loads in flight drains in
    // order, so the set-up's wait for it leaves those alone.
    // (Unconditional, from a valid head, so that the wait for it is exact;
    // rows beyond the group's heads are zeroed below.)
    const uint4 raw = *reinterpret_cast<const uint4 *>(
        a.q + ((int64_t)b * a.num_q_heads + qh0 + min(g, nheads - 1)) * kHeadDim + 8 * j);

    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    // A page holds the code rows of every KV head ([P][64] bytes each), then
    // every head's scales ([P] fp16 each); all fit in 32 bits (the host
    // checks num_kv_heads * tile_bytes < 2^31).
    const uint32_t page_stride = (uint32_t)a.num_kv_heads * (uint32_t)a.tile_bytes;
    const uint32_t code_off = (uint32_t)hk * (uint32_t)(P * kCodeBytesPerRow);
    const uint32_t scale_off = (uint32_t)a.num_kv_heads * (uint32_t)(P * kCodeBytesPerRow) + (uint32_t)hk * (2 * P);
    const uint8_t *kbase = kpool + code_off;
    const uint8_t *vbase = vpool + code_off;
    const uint8_t *ksbase = kpool + scale_off;
    const uint8_t *vsbase = vpool + scale_off;
    const int last_rel = p1 - 1 - p0;
    // Page numbers of the range, read with scalar loads (the table is not
    // written during the call), one chunk ahead of the loads that use them.
    const __attribute__((address_space(4))) int32_t *pages =
        (const __attribute__((address_space(4))) int32_t *)(a.page_table + (int64_t)b * a.max_pages_per_seq + p0);
    struct PageSet { int32_t p[4]; };   // physical page of each 16-token group of a chunk
    auto fetch_pages = [&](int c) {
        PageSet ps;
#pragma unroll
        for (int t = 0; t < 4; ++t) ps.p[t] = pages[min(c * (kChunk / P) + (16 * t) / P, last_rel)];   // clamp past the end
        return ps;
    };

    // Per-lane byte offsets inside a 16-token group: key row j, part g;
    // value piece for LDS slot lane (row lane / 4, swizzled piece); scale of
    // token j of group g (the scales of a chunk are two loads, one per
    // tensor, of 64 distinct tokens, then broadcast across the lane rows).
    const uint32_t koff = j * kCodeBytesPerRow + 16 * g;
    const uint32_t voff = 64 * (lane >> 2) + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t soff = 2 * ((16 * g) % P + j);
    struct TileAddrs {
        const uint8_t *kt[4], *vt[4];   // tile of group t (wave-uniform)
        const uint8_t *ks, *vs;         // this lane's scale (group g, token j)
    };
    // Chunk c starts at page p0 + c * 64 / P (ranges start on chunk boundaries).
    auto addrs = [&](const PageSet &ps, TileAddrs &ta) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ta.kt[t] = tile_addr(kbase, (uint32_t)ps.p[t], page_stride);
            ta.vt[t] = tile_addr(vbase, (uint32_t)ps.p[t], page_stride);
        }
        // page of group g, selected with bit masks (an indexed pick would go
        // through scratch memory)
        int32_t m1 = -(g & 1), m2 = -((g >> 1) & 1);
        uint32_t so = soff;
        asm("" : "+v"(so), "+v"(m1), "+v"(m2));
        const int32_t p01 = ps.p[0] ^ (m1 & (ps.p[0] ^ ps.p[1]));
        const int32_t p23 = ps.p[2] ^ (m1 & (ps.p[2] ^ ps.p[3]));
        const int32_t mine = p01 ^ (m2 & (p01 ^ p23));
        ta.ks = tile_addr(ksbase, (uint32_t)mine, page_stride) + so;
        ta.vs = tile_addr(vsbase, (uint32_t)mine, page_stride) + so;
    };
    // Opaque copies of the lane offsets: they are then extended next to the
    // loads, which lets them take the scalar-base + 32-bit-offset form.
    auto load_v = [&](const TileAddrs &ta) {
        uint32_t vo = voff;
        asm("" : "+v"(vo));
#pragma unroll
        for (int t = 0; t < 4; ++t)
            __builtin_amdgcn_global_load_lds((const void *)(ta.vt[t] + ((16 * t) % P) * kCodeBytesPerRow + vo),
                                             (__attribute__((address_space(3))) void *)&sv.vbuf[vgroup_off(t)],
                                             16, 0, 2 /* nt */);
    };
    auto load_k = [&](const TileAddrs &ta, ChunkData &cd) {
        uint32_t ko = koff;
        asm("" : "+v"(ko));
#pragma unroll
        for (int t = 0; t < 4; ++t) cd.k[t] = stream_load16(ta.kt[t] + ((16 * t) % P) * kCodeBytesPerRow + ko);
        cd.ks = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(ta.ks));
    };
    auto load_vs = [&](const TileAddrs &ta, ChunkData &cd) {
        cd.vs = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(ta.vs));
    };

    // The range's first chunk starts loading before the set-up below, whose
    // latency (query load, rotation, LDS round trip) it then hides.
    const int nfull = (tok_end - tok_begin) / kChunk;   // chunks with no masked token
    ChunkData buf;
    PageSet pages_next;   // pages of the chunk whose loads are issued next
    if (nchunks > 0) {
        TileAddrs ta;
        addrs(fetch_pages(0), ta);
        pages_next = fetch_pages(1);
        // Wait for the query here, with the page numbers: once value loads
        // into LDS are in flight the compiler waits for every load before
        // using any.
        asm volatile("" ::"v"(raw.x), "v"(raw.y), "v"(raw.z), "v"(raw.w));
        load_v(ta);
        load_k(ta, buf);
        load_vs(ta, buf);
    }

    // ---- setup: rotated query as fixed-point limbs; row g = head g ----
    float qv[8];
    rotate_query<BH>(raw, a.sign_mask, j, g < nheads, qv);
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) amax = fmaxf(amax, fabsf(qv[r]));
    amax = row_max16(amax);
    int qexp = 0;
    if (amax > 0.0f) (void)frexpf(amax, &qexp);      // amax < 2^qexp
    const float qmul = ldexpf(1.0f, 27 - qexp);
    int lsum[4] = {0, 0, 0, 0};
    QLimbs &qlimb = sq.qlimb;
    {
        uint32_t w[4][2] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};   // [limb][parity]
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // |X| <= 2^27 (exact in fp32 before the conversion)
            const int X = static_cast<int>(rintf(qv[k] * qmul));
            const int limb[4] = {X >> 21, (X >> 14) & 127, (X >> 7) & 127, X & 127};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lsum[r] += limb[r];
                w[r][k & 1] |= (static_cast<uint32_t>(limb[r]) & 0xFFu) << (8 * (k >> 1));
            }
        }
        // dim 8j + k sits at lane group j/4, slot 4 (j%4) + k/2 of parity k%2
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            qlimb[g][r][0][j >> 2][j & 3] = w[r][0];
            qlimb[g][r][1][j >> 2][j & 3] = w[r][1];
        }
    }
    v4i qk_init;    // rows (head g, limbs 0..3): -8 sum_d L, offset-binary keys
#pragma unroll
    for (int r = 0; r < 4; ++r) qk_init[r] = -8 * row_sum16_i(lsum[r]);
    const float score_mul = ldexpf(a.score_scale, qexp - 27);   // head g
    wave_lds_sync();
    v4i qa0, qa1;   // A operands: row (head j/4, limb j%4), k-slots of group g
    {
        const uint4 e0 = *reinterpret_cast<const uint4 *>(&qlimb[j >> 2][j & 3][0][g][0]);
        const uint4 e1 = *reinterpret_cast<const uint4 *>(&qlimb[j >> 2][j & 3][1][g][0]);
        qa0 = v4i{(int)e0.x, (int)e0.y, (int)e0.z, (int)e0.w};
        qa1 = v4i{(int)e1.x, (int)e1.y, (int)e1.z, (int)e1.w};
    }
    // Fused step: this range ends at the sequence's last cached token, so it
    // also takes the new token (position L) at its end.  The rotated query
    // then waits in the query space (free once the A operands are built) and
    // the new K/V rows load during the last chunk, by direct-to-LDS loads
    // into the value buffer the next chunk's values would use.
    const bool take_new = a.k_new != nullptr && tok_end == L && nchunks > 0;
    float *qstash = reinterpret_cast<float *>(&sq.qlimb[0][0][0][0][0]);
    if (take_new) {
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < 8; ++r) qstash[128 * g + 8 * j + r] = qv[r];
    }
    int32_t new_page = 0;

    // ---- main loop state ----
    float m_run = -INFINITY;     // running max (log2 units) of head g, uniform in row g
    float l_lane = 0.0f;         // this lane's part of the running sum
    float o_acc[8];              // head g, dims 16m + j
#pragma unroll
    for (int m = 0; m < 8; ++m) o_acc[m] = 0.0f;

    // TAIL: the chunk may extend past the range's last token (masked).
    auto compute = [&](int c, ChunkData &cd, auto tail, auto pf) {
        constexpr bool TAIL = decltype(tail)::value;
        constexpr bool PF = decltype(pf)::value;   // prefetch chunk c + 1
        const int T0 = tok_begin + c * kChunk;
        // This chunk's values were loaded into the buffer by DMA, which the
        // vector-memory counter tracks; wait for it explicitly (vmcnt(0))
        // rather than trust the compiler to see the DMA write and these reads
        // as the same memory (it does not always).
        __builtin_amdgcn_s_waitcnt(0x0F70);
        // Value columns by transposed 4-bit LDS reads: lane (g, n) points at
        // the 8-byte word m (dims 16m..16m+15) of token n of group g, and lane
        // (g, i) receives dim 16m + i of the 16 tokens (token n in nibble n).
        uint2 vt[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const v2i r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(
                &sv.vbuf[vgroup_off(g) + 16 * (4 * j + ((m >> 1) ^ ((j >> 2) & 3))) + 8 * (m & 1)]));
            vt[m] = make_uint2(static_cast<uint32_t>(r.x), static_cast<uint32_t>(r.y));
        }

        // The next chunk's values then load into the same buffer: once these
        // reads have completed (they also come first because the compiler
        // waits for every value load in flight before any read of the buffer).
        TileAddrs ta;
        if constexpr (PF) {
            addrs(pages_next, ta);
            pages_next = fetch_pages(c + 2);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the reads above are done
            load_v(ta);
        }

        // q.k: z[t] = score of head g, token 16t + j (log2 units)
        uint32_t ks[4];   // key scale of token 16t + j
        rows_broadcast(cd.ks, ks);
        float z[4];
        float zmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t lo[4], hi[4];
            split_offset(cd.k[t].x, lo[0], hi[0]);
            split_offset(cd.k[t].y, lo[1], hi[1]);
            split_offset(cd.k[t].z, lo[2], hi[2]);
            split_offset(cd.k[t].w, lo[3], hi[3]);
            v4i d = mfma(qa0, v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]}, qk_init);
            d = mfma(qa1, v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}, d);
            const float sc = limbs4_to_float(d) * score_mul * half_to_float(ks[t]);
            z[t] = (!TAIL || T0 + 16 * t + j < tok_end) ? sc : -INFINITY;
            zmax = fmaxf(zmax, z[t]);
        }
        if constexpr (PF) {
            load_k(ta, cd);
        } else if (take_new) {
            // lanes 0-15: the K row's 16-byte pieces, 16-31: the V row's (bytes
            // 0-255 and 256-511 of the buffer); lanes 32-63 repeat them
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the value reads above are done
            const uint16_t *src = (lane & 16) ? a.v_new : a.k_new;
            __builtin_amdgcn_global_load_lds(
                (const void *)(src + ((int64_t)b * a.num_kv_heads + hk) * kHeadDim + 8 * (lane & 15)),
                (__attribute__((address_space(3))) void *)&sv.vbuf[0], 16, 0, 0);
            new_page = a.page_table[(int64_t)b * a.max_pages_per_seq + (L >> a.page_shift)];
        }

        // online softmax for head g (row g)
        zmax = row_max16_fast(zmax);
        if (zmax > m_run) {
            const float alpha = fast_exp2(m_run - zmax);
            l_lane *= alpha;
#pragma unroll
            for (int m = 0; m < 8; ++m) o_acc[m] *= alpha;
            m_run = zmax;
        }
        uint32_t vs[4];   // value scale of token 16t + j
        rows_broadcast(cd.vs, vs);
        float pv[4];
        float pmax = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float p = fast_exp2(z[t] - m_run);      // 0 for masked tokens
            l_lane += p;
            // masked tokens: p = 0, but their scales may be garbage
            pv[t] = (!TAIL || T0 + 16 * t + j < tok_end) ? p * half_to_float(vs[t]) : 0.0f;
            pmax = fmaxf(pmax, pv[t]);
        }
        if constexpr (PF) load_vs(ta, cd);
        pmax = row_max16_nonneg(pmax);
        int pexp = 0;
        if (pmax > 0.0f) (void)frexpf(pmax, &pexp);        // pv < 2^pexp
        const float pmul = ldexpf(1.0f, 20 - pexp);
        const float pback = ldexpf(1.0f, pexp - 20);
        int fsum = 0;   // sum of this lane's fixed-point P (exact: < 2^23)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t F = static_cast<uint32_t>(fmaf(pv[t], pmul, 0.5f));
            sp.pfix[g][16 * t + j] = F;
            fsum += static_cast<int>(F);
        }
        // Values enter as offset-binary codes u = c + 8, so sum_t F_t c_t =
        // sum_t F_t u_t - 8 sum_t F_t; the second term is one number per head
        // (its integer sum is exact: 64 values below 2^21).
        const float corr = 8.0f * pback * static_cast<float>(row_sum16_i(fsum));
        wave_lds_sync();
        // A operand of p.v: row (head j/4, limb j%4; limb 3 is zero), tokens
        // of group g in the k-slot order of the transposed value words:
        // dword 0 = tokens 0,2,4,6; 1 = 1,3,5,7; 2 = 8,10,12,14; 3 = 9,11,13,15.
        v4i pa;
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(&sp.pfix[j >> 2][16 * g]);
            const uint4 f0 = src[0], f1 = src[1], f2 = src[2], f3 = src[3];
            const int limb = j & 3;
            const uint32_t shift = (limb == 3) ? 0u : 14u - 7u * limb;
            const uint32_t width = (limb == 3) ? 0u : 7u;   // the zero row
            auto L = [&](uint32_t f) { return __builtin_amdgcn_ubfe(f, shift, width); };
            pa[0] = (int)(L(f0.x) | (L(f0.z) << 8) | (L(f1.x) << 16) | (L(f1.z) << 24));
            pa[1] = (int)(L(f0.y) | (L(f0.w) << 8) | (L(f1.y) << 16) | (L(f1.w) << 24));
            pa[2] = (int)(L(f2.x) | (L(f2.z) << 8) | (L(f3.x) << 16) | (L(f3.z) << 24));
            pa[3] = (int)(L(f2.y) | (L(f2.w) << 8) | (L(f3.y) << 16) | (L(f3.w) << 24));
        }
        wave_lds_sync();
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            // nibble n = token n -> bytes: tokens (0,2,4,6) (1,3,5,7) (8,..,14) (9,..,15)
            uint32_t e0, o0, e1, o1;
            split_offset(vt[m].x, e0, o0);
            split_offset(vt[m].y, e1, o1);
            const v4i d = mfma(pa, v4i{(int)e0, (int)o0, (int)e1, (int)o1}, zero);
            o_acc[m] = fmaf(ulimbs_to_float(d), pback, o_acc[m]) - corr;
        }
    };

    // Chunk c + 1 loads while chunk c computes: values into the same LDS
    // buffer once chunk c's have been read back, keys and scales into
    // registers once chunk c's have been used.  Every chunk before the last
    // is full.
    int c = 0;
    for (; c + 1 < nchunks; ++c) compute(c, buf, std::false_type{}, std::true_type{});
    if (c < nfull) compute(c, buf, std::false_type{}, std::false_type{});
    else if (c < nchunks) compute(c, buf, std::true_type{}, std::false_type{});

    if (take_new) {
        // Fused step: quantize and store the new token's K and V rows (lane
        // (g, j): dims 8j..8j+7), score it against head g's rotated query,
        // move its value row to the output layout (dims 16m + j) through the
        // P buffer, and fold it into the running state.  (Lane indices go
        // through an opaque copy, so that nothing derived from them is
        // computed ahead of the loop and kept live through it.)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int gg = ln >> 4, jj = ln & 15;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the rows are in LDS
        const uint4 kraw = *reinterpret_cast<const uint4 *>(&sv.vbuf[16 * jj]);
        const uint4 vraw = *reinterpret_cast<const uint4 *>(&sv.vbuf[256 + 16 * jj]);
        const NewRow kr = quantize_new_row<BH>(kraw, jj);
        const NewRow vr = quantize_new_row<BH>(vraw, jj);
        if (chunk_id == 0) {
            const uint32_t slot = (uint32_t)(L & (P - 1));
            uint8_t *kt = const_cast<uint8_t *>(tile_addr(kbase, (uint32_t)new_page, page_stride));
            uint8_t *vt = const_cast<uint8_t *>(tile_addr(vbase, (uint32_t)new_page, page_stride));
            if (gg == 0) {
                *reinterpret_cast<uint32_t *>(kt + slot * kCodeBytesPerRow + 4 * jj) = kr.bytes;
                *reinterpret_cast<uint32_t *>(vt + slot * kCodeBytesPerRow + 4 * jj) = vr.bytes;
            }
            if (ln == 0) {
                *reinterpret_cast<uint16_t *>(
                    const_cast<uint8_t *>(tile_addr(ksbase, (uint32_t)new_page, page_stride)) + 2 * slot) = kr.s16;
                *reinterpret_cast<uint16_t *>(
                    const_cast<uint8_t *>(tile_addr(vsbase, (uint32_t)new_page, page_stride)) + 2 * slot) = vr.s16;
            }
        }
        float dot = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) dot = fmaf(qstash[128 * gg + 8 * jj + r], kr.d[r], dot);
        const float z = row_sum16(dot) * a.score_scale;
        float *vbuf = reinterpret_cast<float *>(&sp.pfix[0][0]);
        wave_lds_sync();
        if (gg == 0) {
#pragma unroll
            for (int r = 0; r < 8; ++r) vbuf[8 * jj + r] = vr.d[r];
        }
        wave_lds_sync();
        const float mn = fmaxf(m_run, z);
        const float corr = fast_exp2(m_run - mn);
        const float w = fast_exp2(z - mn);
        l_lane = fmaf(l_lane, corr, jj == 0 ? w : 0.0f);
#pragma unroll
        for (int m = 0; m < 8; ++m) o_acc[m] = fmaf(o_acc[m], corr, vbuf[16 * m + jj] * w);
        m_run = mn;
        wave_lds_sync();
    }

    PartialState st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.o[m] = o_acc[m];
    st.m = m_run;
    st.l = row_sum16(l_lane);
    return st;
}


// Split mode: one page range of one sequence per wave (dec::split_item).
template <int BH, int P>
__global__ __launch_bounds__(kThreads) void decode_int4_mfma_kernel(DecodeArgs a) {
    // The wave index is uniform across the wave; saying so keeps everything
    // derived from it (head, tile addresses) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const SplitItem it = split_item<P>(a, wave);
    if (!it.live) return;
    __shared__ WaveValues values[kWaves];
    __shared__ WavePfix pfix[kWaves];
    __shared__ WaveQuery query[kWaves];
    const int qh0 = it.hk * a.group + it.chunk_id * kH;
    const PartialState st = decode_range<BH, P>(a, values[wave], pfix[wave], query[wave], lane, it.b, it.hk,
                                                it.chunk_id, it.L, it.p0, it.p1);
    write_partial(a, st, lane, min(kH, a.group - it.chunk_id * kH),
                  ((int64_t)it.b * a.num_q_heads + qh0) * a.num_splits + it.s, a.num_splits);
}

// Split mode with few work items (small batches, long contexts): each page
// range is shared by WPR waves of one block, each taking a consecutive part
// of its chunks, and their partial states are merged in LDS before the one
// write to the workspace.  A range's chunks then stream in parallel instead
// of one after another behind a single wave (with one wave per SIMD, every
// chunk of a range exposed a whole memory latency), while the number of
// partial states the merge kernel reads stays that of the plain split.
template <int BH, int P, int WPR>
__global__ __launch_bounds__(kThreads * WPR) void decode_int4_wide_kernel(DecodeArgs a) {
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave = wid % kWaves;        // head slot of the block's quad
    const int part = wid / kWaves;        // part of the range
    const int lane = threadIdx.x & 63;
    const SplitItem it = split_item<P>(a, wave);
    struct WideDecode {
        WaveValues values[kWaves * WPR];
    };
    struct WideMerge {
        float o[kWaves * WPR][8][64];
        float ml[kWaves * WPR][2][64];
    };
    union WideShared {
        WideDecode dec;
        WideMerge mrg;
    };
    __shared__ WideShared sh;
    __shared__ WavePfix pfix[kWaves * WPR];
    __shared__ WaveQuery query[kWaves * WPR];
    constexpr int kChunkPages = kChunk / P;
    PartialState st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.o[m] = 0.0f;
    st.m = -INFINITY;
    st.l = 0.0f;
    if (it.live) {
        const int nch = (it.p1 - it.p0 + kChunkPages - 1) / kChunkPages;
        const int c0 = part * nch / WPR, c1 = (part + 1) * nch / WPR;
        if (c0 < c1)
            st = decode_range<BH, P>(a, sh.dec.values[wid], pfix[wid], query[wid], lane, it.b, it.hk, it.chunk_id,
                                     it.L, it.p0 + c0 * kChunkPages, min(it.p0 + c1 * kChunkPages, it.p1));
    }
    __syncthreads();   // every wave is done with its value buffer: the merge space overlays them
#pragma unroll
    for (int m = 0; m < 8; ++m) sh.mrg.o[wid][m][lane] = st.o[m];
    sh.mrg.ml[wid][0][lane] = st.m;
    sh.mrg.ml[wid][1][lane] = st.l;
    __syncthreads();
    if (part != 0 || !it.live) return;
    // merge the WPR parts of this head slot (a part with no chunk has max -inf)
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPR; ++w) M = fmaxf(M, sh.mrg.ml[w * kWaves + wave][0][lane]);
    PartialState r;
    r.m = M;
    r.l = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) r.o[m] = 0.0f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) {
        const int src = w * kWaves + wave;
        const float mw = sh.mrg.ml[src][0][lane];
        const float f = mw == -INFINITY ? 0.0f : fast_exp2(mw - M);
        r.l = fmaf(sh.mrg.ml[src][1][lane], f, r.l);
#pragma unroll
        for (int m = 0; m < 8; ++m) r.o[m] = fmaf(sh.mrg.o[src][m][lane], f, r.o[m]);
    }
    const int qh0 = it.hk * a.group + it.chunk_id * kH;
    write_partial<true>(a, r, lane, min(kH, a.group - it.chunk_id * kH),
                  ((int64_t)it.b * a.num_q_heads + qh0) * a.num_splits + it.s, a.num_splits);
}

// Balanced mode (batch 16..4096): equal ranges of the batch's concatenated
// chunks (dec::balanced_range); the block walks every sequence its range
// meets, so every block streams the same amount of cache whatever the mix of
// context lengths, and the launch neither waits on a few long work items nor
// dispatches a second round of them.
template <int BH, int P>
__global__ __launch_bounds__(kThreads) void decode_int4_balanced_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int B = a.batch;
    union Shared {
        ScanSpace scan;
        WaveValues waves[kWaves];
    };
    __shared__ Shared sm;
    __shared__ WavePfix pfix[kWaves];
    __shared__ WaveQuery query[kWaves];
    __shared__ WaveHeld held[kWaves];

    const BlockRange r = balanced_range(a, sm.scan, wave, lane);
    if (r.tot == 0 || r.gi >= r.G) return;
    const int qd = r.qd, gi = r.gi, start = r.start, end = r.end, b0 = r.b0, pb0 = r.pb0;

    const int head_slots = a.num_kv_heads * a.head_chunks;
    const int slot = qd * kWaves + wave;
    if (slot >= head_slots) return;
    const int hk = slot / a.head_chunks;
    const int chunk_id = slot - hk * a.head_chunks;
    constexpr int kChunkPages = kChunk / P;
    // A range's first partial state, when more pieces follow it, is held in
    // LDS and written back with the last one at the end of the range: a write
    // in the middle of the stream of cache reads was measured to cost several
    // times its size in lost read bandwidth.  (A third piece of one range, rare,
    // is written at once.)
    const int nheads = min(kH, a.group - chunk_id * kH);
    const int64_t per_head = (int64_t)a.sk_groups + B;   // partial states per head
    const int64_t unit_base = ((int64_t)(qd * kWaves + wave) * kH) * per_head + gi;
    int64_t held_u0 = -1;
    WaveHeld &hw = held[wave];
    int pb = pb0;
    for (int b = b0; b < B && pb < end; ++b) {
        const int L = decode_len(a, b);
        const int nch = L > 0 ? (L + kChunk - 1) / kChunk : 0;
        const int pb1 = pb + nch;
        const int c0 = max(start, pb) - pb;
        const int c1 = min(end, pb1) - pb;
        if (c0 < c1) {
            const int npages = (L + P - 1) / P;
            const PartialState st = decode_range<BH, P>(a, sm.waves[wave], pfix[wave], query[wave], lane, b, hk, chunk_id, L,
                                                        c0 * kChunkPages, min(c1 * kChunkPages, npages));
            if (pb1 < end && held_u0 < 0) {
                // lane-private slots: the lane that writes one reads it back
                hw.o[0][lane] = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
                hw.o[1][lane] = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
                hw.ml[lane] = make_float2(st.m, st.l);
                held_u0 = unit_base + b;
            } else {
                write_partial(a, st, lane, nheads, unit_base + b, per_head);
            }
        }
        pb = pb1;
    }
    if (held_u0 >= 0) {
        PartialState st;
        const float4 o0 = hw.o[0][lane], o1 = hw.o[1][lane];
        const float2 ml = hw.ml[lane];
        st.o[0] = o0.x; st.o[1] = o0.y; st.o[2] = o0.z; st.o[3] = o0.w;
        st.o[4] = o1.x; st.o[5] = o1.y; st.o[6] = o1.z; st.o[7] = o1.w;
        st.m = ml.x;
        st.l = ml.y;
        write_partial(a, st, lane, nheads, held_u0, per_head);
    }
}

}  // namespace

hipError_t launch_decode_int4_mfma(const DecodeArgs &a, hipStream_t stream) {
    const int quads = (a.num_kv_heads * a.head_chunks + kWaves - 1) / kWaves;
    const bool balanced = a.sk_groups > 0;
    const dim3 grid = balanced ? dim3((unsigned)(quads * a.sk_groups), 1, 1)
                               : dim3((unsigned)(a.batch * quads), (unsigned)a.num_splits, 1);
    const dim3 block(kThreads);
#define KVQ_LAUNCH(BHV, PV)                                                                                  \
    do {                                                                                                     \
        if (balanced)                                                                                        \
            hipLaunchKernelGGL((decode_int4_balanced_kernel<BHV, PV>), grid, block, 0, stream, a);            \
        else if (a.range_waves == 4)                                                                         \
            hipLaunchKernelGGL((decode_int4_wide_kernel<BHV, PV, 4>), grid, dim3(4 * kThreads), 0, stream, a); \
        else if (a.range_waves == 2)                                                                         \
            hipLaunchKernelGGL((decode_int4_wide_kernel<BHV, PV, 2>), grid, dim3(2 * kThreads), 0, stream, a); \
        else                                                                                                 \
            hipLaunchKernelGGL((decode_int4_mfma_kernel<BHV, PV>), grid, block, 0, stream, a);                \
    } while (0)
    if (a.page_size == 16) {
        switch (a.had_block) {
            case 0: KVQ_LAUNCH(0, 16); break;
            case 32: KVQ_LAUNCH(32, 16); break;
            case 64: KVQ_LAUNCH(64, 16); break;
            case 128: KVQ_LAUNCH(128, 16); break;
            default: return hipErrorInvalidValue;
        }
    } else if (a.page_size == 32) {
        switch (a.had_block) {
            case 0: KVQ_LAUNCH(0, 32); break;
            case 32: KVQ_LAUNCH(32, 32); break;
            case 64: KVQ_LAUNCH(64, 32); break;
            case 128: KVQ_LAUNCH(128, 32); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
#undef KVQ_LAUNCH
    return hipGetLastError();
}

}  // namespace kvq
