// Paged decode attention over a quantizer variant's cache: INT4 codes with
// one fp16 scale per group of G channels (G = 32 or 64), or MXFP4 (E2M1
// codes, one E8M0 scale per 32 channels); split-K partial kernel.  INT4 on
// the int8 matrix cores (v_mfma_i32_16x16x64_i8); MXFP4's q.k on gfx950's
// scaled FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4: keys straight
// from the cache with their E8M0 scales), its p.v on the int8 ones.
//
// Method sources: "BitDecoding-FP4:FP4 KVキャッシュのネイティブ復号", section
// 深掘り分析 (scales chosen per group after a Hadamard rotation) and its
// opening summary (4-bit microscaling KV formats); "KVキャッシュを4ビットへ —
// SAW-INT4...", section 回転のトリック (R = H/sqrt(Bh) orthogonal: the query is
// rotated, R S q with the sign mask S, and the output brought back with S R
// by the merge kernel).
//
// The schedule, the partial-state layout and the value staging are the
// token-wise kernel's (decode_mfma.hip); what differs is that a key's score
// is a sum over its scale groups, score = sum_g s_g (q'_g . c_g), and a
// value's dims carry the scale of their group.
//
//   q.k : the rotated, pre-scaled query of each head is a 24-bit fixed-point
//         integer X = round(q' 2^(23-E)) (E chosen with max|q'| < 2^E (1 -
//         2^-7)) in balanced signed 8-bit digits X = D0 2^16 + D1 2^8 + D2.
//         The A operand of digit d has one row per (head, scale group): lane
//         (g', j) holds, for row j = (head j/4, group j%4), the digits of the
//         dims of lane group g' (dims 32g'..32g'+31) if those belong to group
//         j%4, else zeros.  So one MFMA pair (even / odd dims) per digit gives
//         every group's partial dot product for 4 heads at once, and lane
//         (g, j) receives rows (head g, groups 0..3) for token j.  INT4 keys
//         enter as offset-binary nibbles (c + 8) with -8 sum(digits) per row
//         as the accumulator's start.  Per group: (D0 2^8 + D1) exact in
//         int32, then one fma with D2, times the group's fp16 key scale.
//         MXFP4: see the set-up below (4-bit query digits as exact E4M3
//         integers against the E2M1 keys, all scales in the instruction).
//   p.v : values as INT4 offset-binary bytes, or MXFP4's signed bytes 2 v
//         (v the E2M1 value, 2 v an integer in [-12, 12], by a byte table,
//         with the scale 2^(X-1)); per value group, P = p (value scale of
//         the group) in 21-bit fixed
//         point relative to the group's largest P of the head in the chunk,
//         three 7-bit limbs as in the token-wise kernel; groups are handed
//         through LDS one after another.  The dims of MFMA m (16m..16m+15)
//         lie in one group.
#include <type_traits>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dec;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kChunk = kChunkTokens;

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// INT4 key or value bytes of 4 nibbles (one per byte, in the low 4 bits of
// each byte of n) as MFMA operands: offset binary c + 8 (c xor 8).
__device__ __forceinline__ uint32_t nib_bytes_int4(uint32_t n) { return (n ^ 0x08080808u) & 0x0F0F0F0Fu; }

// Even / odd dims of 8 packed codes (one word) as two operand words.
// MXFP4: the magnitudes by table from the low 3 bits of each nibble, the
// sign (bit 3 of the nibble) as a 0xFF byte mask straight from v_perm_b32's
// sign-fill selectors (8, 9 replicate bit 15, 31 of the second source; 10,
// 11 bit 15, 31 of the first), fed with shifted copies of w that put each
// nibble's sign bit at one of those positions, and one bitwise select
// between the negative and the positive table entry: 14 instructions per
// word instead of 21.
template <int FMT>
__device__ __forceinline__ void split_codes(uint32_t w, uint32_t &lo, uint32_t &hi) {
    if constexpr (FMT == KVQ_FMT_INT4) {
        lo = nib_bytes_int4(w & 0x0F0F0F0Fu);
        hi = nib_bytes_int4((w >> 4) & 0x0F0F0F0Fu);
    } else {
        const uint32_t sl = w & 0x07070707u;
        const uint32_t sh = (w >> 4) & 0x07070707u;
        const uint32_t ml = __builtin_amdgcn_perm(w << 12, w << 4, 0x090B080Au);   // w bits 3, 11, 19, 27
        const uint32_t mh = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);         // w bits 7, 15, 23, 31
        const uint32_t pl = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sl);
        const uint32_t nl = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sl);
        const uint32_t ph = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, sh);
        const uint32_t nh = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, sh);
        lo = (nl & ml) | (pl & ~ml);
        hi = (nh & mh) | (ph & ~mh);
    }
}

__device__ __forceinline__ float ulimbs_to_float(v4i d) {
    uint32_t s = (static_cast<uint32_t>(d[0]) << 7) + static_cast<uint32_t>(d[1]);
    asm("" : "+v"(s));
    s = (s << 7) + static_cast<uint32_t>(d[2]);
    return static_cast<float>(s);
}

// Value staging (as the token-wise kernel): one 16-token group per 1 KiB,
// row n's 16-byte piece p in slot 4n + (p ^ ((n >> 2) & 3)).
constexpr int kVGroupBytes = 1024;
__host__ __device__ constexpr int vgroup_off(int t) { return t * kVGroupBytes + 128 * ((t + 1) >> 1); }
constexpr int kVBufBytes = vgroup_off(3) + kVGroupBytes;
constexpr int kPfixPitch = kChunk + 4;

struct alignas(16) WaveValues {
    uint8_t vbuf[kVBufBytes];
};
typedef uint32_t QDigits[kH][3][2][4][4];   // [head][digit][parity][lane group][dword]
struct alignas(16) WaveQuery {
    union {
        QDigits qd;                 // INT4 groups: 8-bit digits in the A-operand order
        int32_t qx[kH][kHeadDim];   // MXFP4: the fixed-point query X per (head, dim)
    };
};
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// E4M3 bytes of 4 integers 0..15 held one per byte: 0 -> 0x00, 1 -> 0x38,
// 2 -> 0x40, 3 -> 0x44, 4 -> 0x48, 5 -> 0x4A, 6 -> 0x4C, 7 -> 0x4E, 8 -> 0x50,
// 9 .. 15 -> 0x51 .. 0x57 (exact: at most 4 significant bits).
__device__ __forceinline__ uint32_t e4m3_of_small(uint32_t b) {
    const uint32_t sel = b & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(0x4E4C4A48u, 0x44403800u, sel);
    const uint32_t hi = __builtin_amdgcn_perm(0x57565554u, 0x53525150u, sel);
    const uint32_t t = b & 0x08080808u;
    const uint32_t m = (t << 5) - (t >> 3);   // 0xFF where the value is 8 or more
    return (hi & m) | (lo & ~m);
}
struct alignas(16) WavePfix {
    uint32_t pfix[kH][kPfixPitch];
};
struct alignas(16) WaveHeld {
    float4 o[2][64];
    float2 ml[64];
};

__device__ __forceinline__ uint4 stream_load16(const uint8_t *p) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void rows_broadcast(uint32_t x, uint32_t (&y)[4]) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const auto e = __builtin_amdgcn_permlane32_swap(r[0], r[0], false, false);
    const auto o = __builtin_amdgcn_permlane32_swap(r[1], r[1], false, false);
    y[0] = e[0];
    y[1] = o[0];
    y[2] = e[1];
    y[3] = o[1];
}

// Scale traits: bytes per (token, head) and the scale of group gg from the
// token's scale words (w0: bytes 0..3, w1: bytes 4..7).
template <int FMT, int G>
struct Scales {
    static constexpr int kGroups = kHeadDim / G;
    static constexpr int kBytes = FMT == KVQ_FMT_MXFP4 ? kGroups : 2 * kGroups;   // 8 or 4
    static constexpr int kWords = kBytes / 4;
    __device__ static __forceinline__ float get(uint32_t w0, uint32_t w1, int gg) {
        if constexpr (FMT == KVQ_FMT_MXFP4) {
            // 2^(X - 1): the operand bytes are 2 v
            const int byte = (int)((w0 >> (8 * gg)) & 0xFFu);
            return ldexpf(1.0f, byte - 128);
        } else {
            const uint32_t w = gg < 2 ? w0 : w1;
            return half_to_float(w >> (16 * (gg & 1)));
        }
    }
};

struct ChunkData {
    uint4 k[4];
    uint32_t ks[2];      // this lane's token's key scale bytes (group g, token j)
    uint32_t vs[2];
};

template <int FMT, int G, int P>
__device__ __forceinline__ PartialState decode_range_grouped(const DecodeArgs &a, WaveValues &sv, WavePfix &sp,
                                                             WaveQuery &sq, const int lane, const int b,
                                                             const int hk, const int chunk_id, const int L,
                                                             const int p0, const int p1) {
    using S = Scales<FMT, G>;
    constexpr int NG = S::kGroups;
    constexpr int SBT = S::kBytes;
    constexpr int kLaneGroupsPerGroup = G / 32;   // lane groups (32 dims each) per scale group
    const int g = lane >> 4;
    const int j = lane & 15;
    const int tok_begin = p0 * P;
    const int tok_end = min(p1 * P, L);
    const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;
    const int qh0 = hk * a.group + chunk_id * kH;
    const int nheads = min(kH, a.group - chunk_id * kH);

    const uint4 raw = *reinterpret_cast<const uint4 *>(
        a.q + ((int64_t)b * a.num_q_heads + qh0 + min(g, nheads - 1)) * kHeadDim + 8 * j);

    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    const uint32_t page_stride = (uint32_t)a.num_kv_heads * (uint32_t)a.tile_bytes;
    const uint32_t code_off = (uint32_t)hk * (uint32_t)(P * kCodeBytesPerRow);
    const uint32_t scale_off = (uint32_t)a.num_kv_heads * (uint32_t)(P * kCodeBytesPerRow) + (uint32_t)hk * (SBT * P);
    const uint8_t *kbase = kpool + code_off;
    const uint8_t *vbase = vpool + code_off;
    const uint8_t *ksbase = kpool + scale_off;
    const uint8_t *vsbase = vpool + scale_off;
    const int last_rel = p1 - 1 - p0;
    const __attribute__((address_space(4))) int32_t *pages =
        (const __attribute__((address_space(4))) int32_t *)(a.page_table + (int64_t)b * a.max_pages_per_seq + p0);
    struct PageSet { int32_t p[4]; };
    auto fetch_pages = [&](int c) {
        PageSet ps;
#pragma unroll
        for (int t = 0; t < 4; ++t) ps.p[t] = pages[min(c * (kChunk / P) + (16 * t) / P, last_rel)];
        return ps;
    };
    const uint32_t koff = j * kCodeBytesPerRow + 16 * g;
    const uint32_t voff = 64 * (lane >> 2) + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t soff = SBT * ((16 * g) % P + j);
    struct TileAddrs {
        const uint8_t *kt[4], *vt[4];
        const uint8_t *ks, *vs;
    };
    auto addrs = [&](const PageSet &ps, TileAddrs &ta) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ta.kt[t] = kbase + (uint64_t)(uint32_t)ps.p[t] * page_stride;
            ta.vt[t] = vbase + (uint64_t)(uint32_t)ps.p[t] * page_stride;
        }
        int32_t m1 = -(g & 1), m2 = -((g >> 1) & 1);
        uint32_t so = soff;
        asm("" : "+v"(so), "+v"(m1), "+v"(m2));
        const int32_t p01 = ps.p[0] ^ (m1 & (ps.p[0] ^ ps.p[1]));
        const int32_t p23 = ps.p[2] ^ (m1 & (ps.p[2] ^ ps.p[3]));
        const int32_t mine = p01 ^ (m2 & (p01 ^ p23));
        ta.ks = ksbase + (uint64_t)(uint32_t)mine * page_stride + so;
        ta.vs = vsbase + (uint64_t)(uint32_t)mine * page_stride + so;
    };
    auto load_v = [&](const TileAddrs &ta) {
        uint32_t vo = voff;
        asm("" : "+v"(vo));
#pragma unroll
        for (int t = 0; t < 4; ++t)
            __builtin_amdgcn_global_load_lds((const void *)(ta.vt[t] + ((16 * t) % P) * kCodeBytesPerRow + vo),
                                             (__attribute__((address_space(3))) void *)&sv.vbuf[vgroup_off(t)],
                                             16, 0, 2 /* nt */);
    };
    auto load_scales = [&](const uint8_t *p, uint32_t (&w)[2]) {
        if constexpr (SBT == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            w[0] = v.x;
            w[1] = v.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
            w[1] = 0u;
        }
    };
    auto load_k = [&](const TileAddrs &ta, ChunkData &cd) {
        uint32_t ko = koff;
        asm("" : "+v"(ko));
#pragma unroll
        for (int t = 0; t < 4; ++t) cd.k[t] = stream_load16(ta.kt[t] + ((16 * t) % P) * kCodeBytesPerRow + ko);
        load_scales(ta.ks, cd.ks);
    };
    auto load_vs = [&](const TileAddrs &ta, ChunkData &cd) { load_scales(ta.vs, cd.vs); };

    const int nfull = (tok_end - tok_begin) / kChunk;
    ChunkData buf;
    PageSet pages_next;
    if (nchunks > 0) {
        TileAddrs ta;
        addrs(fetch_pages(0), ta);
        pages_next = fetch_pages(1);
        asm volatile("" ::"v"(raw.x), "v"(raw.y), "v"(raw.z), "v"(raw.w));
        load_v(ta);
        load_k(ta, buf);
        load_vs(ta, buf);
    }

    // ---- set-up: R S q for each head (row g), 24-bit balanced digits ----
    float qv[8];
    {
        const uint4 rs = sign_flip_query(raw, a.sign_mask, j);
        if (g < nheads) {
            qv[0] = half_to_float(rs.x); qv[1] = half_to_float(rs.x >> 16);
            qv[2] = half_to_float(rs.y); qv[3] = half_to_float(rs.y >> 16);
            qv[4] = half_to_float(rs.z); qv[5] = half_to_float(rs.z >> 16);
            qv[6] = half_to_float(rs.w); qv[7] = half_to_float(rs.w >> 16);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) qv[r] = 0.0f;
        }
        const int bh = a.had_block;
        if (bh > 0) {
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
            for (int m = 1; m < bh / 8; m <<= 1) {
                const bool upper = (j & m) != 0;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const float p = __shfl_xor(qv[r], m, 16);
                    qv[r] = upper ? (p - qv[r]) : (qv[r] + p);
                }
            }
            const float c = rsqrtf(static_cast<float>(bh));
#pragma unroll
            for (int r = 0; r < 8; ++r) qv[r] *= c;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) amax = fmaxf(amax, fabsf(qv[r]));
    amax = row_max16(amax);
    int qexp = 0;
    if (amax > 0.0f) (void)frexpf(amax * 1.0078125f, &qexp);   // |X| < 127 (2^16 + 2^8 + 1)
    const float qmul = ldexpf(1.0f, 23 - qexp);
    int dsum[3] = {0, 0, 0};   // this lane's digit sums (its 8 dims lie in one scale group)
    if constexpr (FMT == KVQ_FMT_MXFP4) {
        // the fixed-point query to LDS, per (head, dim)
        int4 xv0, xv1;
        xv0.x = static_cast<int>(rintf(qv[0] * qmul)); xv0.y = static_cast<int>(rintf(qv[1] * qmul));
        xv0.z = static_cast<int>(rintf(qv[2] * qmul)); xv0.w = static_cast<int>(rintf(qv[3] * qmul));
        xv1.x = static_cast<int>(rintf(qv[4] * qmul)); xv1.y = static_cast<int>(rintf(qv[5] * qmul));
        xv1.z = static_cast<int>(rintf(qv[6] * qmul)); xv1.w = static_cast<int>(rintf(qv[7] * qmul));
        *reinterpret_cast<int4 *>(&sq.qx[g][8 * j]) = xv0;
        *reinterpret_cast<int4 *>(&sq.qx[g][8 * j + 4]) = xv1;
    } else {
        uint32_t w[3][2] = {{0, 0}, {0, 0}, {0, 0}};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int X = static_cast<int>(rintf(qv[k] * qmul));
            const int d2 = static_cast<int>(static_cast<int8_t>(X & 0xFF));
            const int x1 = (X - d2) >> 8;
            const int d1 = static_cast<int>(static_cast<int8_t>(x1 & 0xFF));
            const int d0 = (x1 - d1) >> 8;
            const int dig[3] = {d0, d1, d2};
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                dsum[d] += dig[d];
                w[d][k & 1] |= (static_cast<uint32_t>(dig[d]) & 0xFFu) << (8 * (k >> 1));
            }
        }
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            sq.qd[g][d][0][j >> 2][j & 3] = w[d][0];
            sq.qd[g][d][1][j >> 2][j & 3] = w[d][1];
        }
    }
    // accumulator start of rows (head g, group gg): -8 sum of the group's
    // digits for INT4's offset-binary keys; 0 for MXFP4's signed bytes.
    v4i qk_init[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        // sum over the lanes of one group: G/8 consecutive lanes of the row
        int s = dsum[d];
        s += __shfl_xor(s, 1, 16);
        s += __shfl_xor(s, 2, 16);
        if constexpr (G == 64) s += __shfl_xor(s, 4, 16);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const int v = gg < NG ? __shfl(s, (G / 8) * (gg < NG ? gg : 0), 16) : 0;
            qk_init[d][gg] = FMT == KVQ_FMT_INT4 ? -8 * v : 0;
        }
    }
    const float score_mul = ldexpf(a.score_scale, qexp - 23);
    wave_lds_sync();
    // MXFP4: q.k on the scaled FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4):
    // B = the keys' E2M1 codes as stored (lane (g, j): token j, dims 32g ..
    // 32g + 31) with their E8M0 block scales; A = the query's 24-bit X in six
    // 4-bit digits, X = sum_{d<5} u_d 2^(4d) + t 2^20 (u_d in [0, 15], t in
    // [-8, 7]), one row per (head, digit), each digit an exact E4M3 integer and
    // its weight 2^(4d + E - 23) in the row's E8M0 scale; A's byte order
    // (established by a layout probe): bytes 0-15 are dims 16g .. 16g + 15,
    // bytes 16-31 dims 64 + 16g .. 64 + 16g + 15.  MFMA u holds digits 4u +
    // (j % 4) of head j / 4 (rows with digit 6 or 7 are zero); the scores are
    // the sums of a head's digit rows.
    v8i qf[2];
    int qsa[2];
    if constexpr (FMT == KVQ_FMT_MXFP4) {
        const int hh = j >> 2;
        const int eh = __shfl(qexp, 16 * hh);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int d = 4 * u + (j & 3);
            qsa[u] = d < 6 ? 127 + 4 * d + eh - 23 : 127;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int4 *src = reinterpret_cast<const int4 *>(&sq.qx[hh][64 * half + 16 * g]);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int4 x = src[q4];
                    const int xs[4] = {x.x, x.y, x.z, x.w};
                    uint32_t mag = 0, neg = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        int v = d < 5 ? ((xs[e] >> (4 * d)) & 15) : (d == 5 ? (xs[e] >> 20) : 0);
                        neg |= (v < 0 ? 0x80u : 0u) << (8 * e);
                        mag |= static_cast<uint32_t>(v < 0 ? -v : v) << (8 * e);
                    }
                    qf[u][4 * half + q4] = static_cast<int>(e4m3_of_small(mag) | neg);
                }
            }
        }
    }
    // INT4 groups: A operands with row j = (head j/4, group j%4); lane group
    // g's dims belong to group g / (G/32)
    v4i qa[3][2];
    if constexpr (FMT == KVQ_FMT_INT4) {
        const bool mine = (j & 3) == g / kLaneGroupsPerGroup;
#pragma unroll
        for (int d = 0; d < 3; ++d)
#pragma unroll
            for (int par = 0; par < 2; ++par) {
                const uint4 e = *reinterpret_cast<const uint4 *>(&sq.qd[j >> 2][d][par][g][0]);
                qa[d][par] = mine ? v4i{(int)e.x, (int)e.y, (int)e.z, (int)e.w} : v4i{0, 0, 0, 0};
            }
    }

    float m_run = -INFINITY;
    float l_lane = 0.0f;
    float o_acc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o_acc[m] = 0.0f;

    auto compute = [&](int c, ChunkData &cd, auto tail, auto pf) {
        constexpr bool TAIL = decltype(tail)::value;
        constexpr bool PF = decltype(pf)::value;
        const int T0 = tok_begin + c * kChunk;
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this chunk's value DMA has landed
        uint2 vt[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const v2i r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(
                &sv.vbuf[vgroup_off(g) + 16 * (4 * j + ((m >> 1) ^ ((j >> 2) & 3))) + 8 * (m & 1)]));
            vt[m] = make_uint2(static_cast<uint32_t>(r.x), static_cast<uint32_t>(r.y));
        }
        TileAddrs ta;
        if constexpr (PF) {
            addrs(pages_next, ta);
            pages_next = fetch_pages(c + 2);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            load_v(ta);
        }

        // q.k
        uint32_t ks[2][4];
        rows_broadcast(cd.ks[0], ks[0]);
        if constexpr (S::kWords == 2) rows_broadcast(cd.ks[1], ks[1]);
        float z[4];
        float zmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (FMT == KVQ_FMT_MXFP4) {
                const v8i bk = {(int)cd.k[t].x, (int)cd.k[t].y, (int)cd.k[t].z, (int)cd.k[t].w, 0, 0, 0, 0};
                const int sb = (int)__builtin_amdgcn_ubfe(ks[0][t], 8 * g, 8);   // E8M0 of (token j, block g)
                const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f d0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[0], bk, zero4, 0, 4, 0, qsa[0], 0, sb);
                const v4f d1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[1], bk, zero4, 0, 4, 0, qsa[1], 0, sb);
                const float sc = (((d0[0] + d0[1]) + (d0[2] + d0[3])) + (d1[0] + d1[1])) * a.score_scale;
                z[t] = (!TAIL || T0 + 16 * t + j < tok_end) ? sc : -INFINITY;
                zmax = fmaxf(zmax, z[t]);
                continue;
            }
            uint32_t lo[4], hi[4];
            split_codes<FMT>(cd.k[t].x, lo[0], hi[0]);
            split_codes<FMT>(cd.k[t].y, lo[1], hi[1]);
            split_codes<FMT>(cd.k[t].z, lo[2], hi[2]);
            split_codes<FMT>(cd.k[t].w, lo[3], hi[3]);
            const v4i bl = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
            const v4i bhv = {(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            v4i dd[3];
#pragma unroll
            for (int d = 0; d < 3; ++d) dd[d] = mfma(qa[d][1], bhv, mfma(qa[d][0], bl, qk_init[d]));
            float sc = 0.0f;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                // |D| <= 128 * 15 * 32 < 2^16: D0 2^8 + D1 exact in int32
                const float dot = fmaf(static_cast<float>((dd[0][gg] << 8) + dd[1][gg]), 256.0f,
                                       static_cast<float>(dd[2][gg]));
                sc = fmaf(dot, S::get(ks[0][t], S::kWords == 2 ? ks[1][t] : 0u, gg), sc);
            }
            sc *= score_mul;
            z[t] = (!TAIL || T0 + 16 * t + j < tok_end) ? sc : -INFINITY;
            zmax = fmaxf(zmax, z[t]);
        }
        if constexpr (PF) load_k(ta, cd);

        zmax = row_max16_fast(zmax);
        if (zmax > m_run) {
            const float alpha = fast_exp2(m_run - zmax);
            l_lane *= alpha;
#pragma unroll
            for (int m = 0; m < 8; ++m) o_acc[m] *= alpha;
            m_run = zmax;
        }
        uint32_t vs[2][4];
        rows_broadcast(cd.vs[0], vs[0]);
        if constexpr (S::kWords == 2) rows_broadcast(cd.vs[1], vs[1]);
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            p[t] = fast_exp2(z[t] - m_run);
            l_lane += p[t];
        }
        if constexpr (PF) load_vs(ta, cd);

        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int gv = 0; gv < NG; ++gv) {
            float pv[4];
            float pmax = 0.0f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float s = S::get(vs[0][t], S::kWords == 2 ? vs[1][t] : 0u, gv);
                pv[t] = (!TAIL || T0 + 16 * t + j < tok_end) ? p[t] * s : 0.0f;   // masked: any scale bytes
                pmax = fmaxf(pmax, pv[t]);
            }
            pmax = row_max16_nonneg(pmax);
            int pexp = 0;
            if (pmax > 0.0f) (void)frexpf(pmax, &pexp);
            const float pmul = ldexpf(1.0f, 20 - pexp);
            const float pback = ldexpf(1.0f, pexp - 20);
            int fsum = 0;
            if (gv > 0) wave_lds_sync();   // the previous group's reads are done
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t F = static_cast<uint32_t>(fmaf(pv[t], pmul, 0.5f));
                sp.pfix[g][16 * t + j] = F;
                fsum += static_cast<int>(F);
            }
            const float corr = FMT == KVQ_FMT_INT4 ? 8.0f * pback * static_cast<float>(row_sum16_i(fsum)) : 0.0f;
            wave_lds_sync();
            v4i pa;
            {
                const uint4 *src = reinterpret_cast<const uint4 *>(&sp.pfix[j >> 2][16 * g]);
                const uint4 f0 = src[0], f1 = src[1], f2 = src[2], f3 = src[3];
                const int limb = j & 3;
                const uint32_t shift = (limb == 3) ? 0u : 14u - 7u * limb;
                const uint32_t width = (limb == 3) ? 0u : 7u;
                auto Lb = [&](uint32_t f) { return __builtin_amdgcn_ubfe(f, shift, width); };
                pa[0] = (int)(Lb(f0.x) | (Lb(f0.z) << 8) | (Lb(f1.x) << 16) | (Lb(f1.z) << 24));
                pa[1] = (int)(Lb(f0.y) | (Lb(f0.w) << 8) | (Lb(f1.y) << 16) | (Lb(f1.w) << 24));
                pa[2] = (int)(Lb(f2.x) | (Lb(f2.z) << 8) | (Lb(f3.x) << 16) | (Lb(f3.z) << 24));
                pa[3] = (int)(Lb(f2.y) | (Lb(f2.w) << 8) | (Lb(f3.y) << 16) | (Lb(f3.w) << 24));
            }
            constexpr int kTilesPerGroup = G / 16;
#pragma unroll
            for (int mm = 0; mm < kTilesPerGroup; ++mm) {
                const int m = gv * kTilesPerGroup + mm;
                // nibble n = token n -> bytes: tokens (0,2,4,6) (1,3,5,7) (8,..,14) (9,..,15)
                uint32_t e0, o0, e1, o1;
                split_codes<FMT>(vt[m].x, e0, o0);
                split_codes<FMT>(vt[m].y, e1, o1);
                const v4i d = mfma(pa, v4i{(int)e0, (int)o0, (int)e1, (int)o1}, zero);
                if constexpr (FMT == KVQ_FMT_INT4) {
                    o_acc[m] = fmaf(ulimbs_to_float(d), pback, o_acc[m]) - corr;
                } else {
                    // signed bytes: |D0| <= 127 * 12 * 64, so the sum is exact in int32
                    const int s = d[0] * 16384 + d[1] * 128 + d[2];
                    o_acc[m] = fmaf(static_cast<float>(s), pback, o_acc[m]);
                }
            }
        }
        wave_lds_sync();   // the P reads are done before the next chunk writes
    };

    int c = 0;
    for (; c + 1 < nchunks; ++c) compute(c, buf, std::false_type{}, std::true_type{});
    if (c < nfull) compute(c, buf, std::false_type{}, std::false_type{});
    else if (c < nchunks) compute(c, buf, std::true_type{}, std::false_type{});

    PartialState st;
#pragma unroll
    for (int m = 0; m < 8; ++m) st.o[m] = o_acc[m];
    st.m = m_run;
    st.l = row_sum16(l_lane);
    return st;
}

template <int FMT, int G, int P>
__global__ __launch_bounds__(kThreads) void decode_grouped_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const SplitItem it = split_item<P>(a, wave);
    if (!it.live) return;
    __shared__ WaveValues values[kWaves];
    __shared__ WavePfix pfix[kWaves];
    __shared__ WaveQuery query[kWaves];
    const int qh0 = it.hk * a.group + it.chunk_id * kH;
    const PartialState st = decode_range_grouped<FMT, G, P>(a, values[wave], pfix[wave], query[wave], lane, it.b,
                                                            it.hk, it.chunk_id, it.L, it.p0, it.p1);
    write_partial(a, st, lane, min(kH, a.group - it.chunk_id * kH),
                  ((int64_t)it.b * a.num_q_heads + qh0) * a.num_splits + it.s, a.num_splits);
}

template <int FMT, int G, int P>
__global__ __launch_bounds__(kThreads) void decode_grouped_balanced_kernel(DecodeArgs a) {
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
    const int nheads = min(kH, a.group - chunk_id * kH);
    const int64_t per_head = (int64_t)a.sk_groups + B;
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
            const PartialState st = decode_range_grouped<FMT, G, P>(a, sm.waves[wave], pfix[wave], query[wave], lane,
                                                                    b, hk, chunk_id, L, c0 * kChunkPages,
                                                                    min(c1 * kChunkPages, npages));
            if (pb1 < end && held_u0 < 0) {
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

hipError_t launch_decode_grouped(const DecodeArgs &a, hipStream_t stream) {
    const int quads = (a.num_kv_heads * a.head_chunks + kWaves - 1) / kWaves;
    const bool balanced = a.sk_groups > 0;
    const dim3 grid = balanced ? dim3((unsigned)(quads * a.sk_groups), 1, 1)
                               : dim3((unsigned)(a.batch * quads), (unsigned)a.num_splits, 1);
    const dim3 block(kThreads);
#define KVQ_LAUNCH(FMT, G, PV)                                                                          \
    do {                                                                                                \
        if (balanced)                                                                                   \
            hipLaunchKernelGGL((decode_grouped_balanced_kernel<FMT, G, PV>), grid, block, 0, stream, a); \
        else                                                                                            \
            hipLaunchKernelGGL((decode_grouped_kernel<FMT, G, PV>), grid, block, 0, stream, a);          \
    } while (0)
#define KVQ_BY_P(FMT, G)                                    \
    do {                                                    \
        if (a.page_size == 16) KVQ_LAUNCH(FMT, G, 16);      \
        else if (a.page_size == 32) KVQ_LAUNCH(FMT, G, 32); \
        else return hipErrorInvalidValue;                   \
    } while (0)
    if (a.format == KVQ_FMT_MXFP4) {
        if (a.scale_group != 32) return hipErrorInvalidValue;
        KVQ_BY_P(KVQ_FMT_MXFP4, 32);
    } else if (a.scale_group == 32) {
        KVQ_BY_P(KVQ_FMT_INT4, 32);
    } else if (a.scale_group == 64) {
        KVQ_BY_P(KVQ_FMT_INT4, 64);
    } else {
        return hipErrorInvalidValue;
    }
#undef KVQ_BY_P
#undef KVQ_LAUNCH
    return hipGetLastError();
}

}  // namespace kvq
