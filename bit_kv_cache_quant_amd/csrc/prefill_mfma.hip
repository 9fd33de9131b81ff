// Causal prefill attention over the INT4 paged cache (int8 matrix cores for
// q.k, v_mfma_i32_16x16x64_i8; fp16 ones for p.v, v_mfma_f32_16x16x32_f16).
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "KVキャッシュこそが本当のボトルネックである理由" (the cache is written on
// arrival and attention reads the paged INT4 blocks; the prompt's tokens are
// appended by the same fused kernel as decode tokens) and
// "回転のトリック — ブロック対角アダマール" (R = H/sqrt(Bh) is orthogonal and its own
// inverse: queries are rotated, outputs rotated back).
//
// Query row i of sequence b (the last q_len_b positions of its cached
// context) attends to the cached tokens 0 .. position(i): the same
// computation as one decode step per query position, with the keys and
// values reused across 16 query positions and the 4 query heads of a GQA
// group, so the work is bound by the chip's arithmetic rather than by HBM.
//
// Block = 4 waves = the 4 query heads of one head slot (KV head, chunk of 4
// of its query heads) x 16 consecutive query positions of one sequence; it
// walks the keys in chunks of 64, staged once in LDS for the 4 waves: key
// codes pre-split into the two signed-byte operands below, values converted
// once to fp16.  Everything is computed transposed (keys or dims as rows,
// query positions as columns), so that the weights leave the score MFMA in
// exactly the lanes and registers the p.v MFMA takes them from.
//   q.k  S^T = K Q^T, exact integer products on v_mfma_i32_16x16x64_i8, as in
//        the decode: the rotated query of each position is a 24-bit
//        fixed-point integer X = round(q' 2^(23-E)) (E chosen with max |q'| <
//        2^E (1 - 2^-7)) written in balanced signed 8-bit digits
//        X = D0 2^16 + D1 2^8 + D2, each in [-128, 127], one MFMA per digit
//        and nibble half.  A (keys): row j = key 16t + j, its 16 code
//        bytes (dims 32g .. 32g + 31) with the even dims' nibbles moved to the
//        top of each byte, or the odd dims' kept there: signed bytes 16 c.
//        B (digit): column j = query position j, the dims 32g + 2e (even half)
//        or 32g + 2e + 1 (odd half).  The digit results are exact in int32
//        (below 2^21 in magnitude); D0 and D1 are combined in int32, the
//        rest in fp32, then the key's scale.  D: lane (g, j) holds keys
//        16t + 4g + i (i = 0..3) of query position j.  (fp16 products summed
//        in fp32 were measurably less accurate here: with the rotation every
//        code is nonzero and the softmax of large scores amplifies their
//        rounding.  So was a 21-bit query: its rounding, relative 2^-21 to
//        the largest element, dominated the error at sharp softmax scales.)
//   softmax: online per query position; a position's 64 scores of a chunk
//        are 16 registers in each of the 4 lanes j, j + 16, j + 32, j + 48
//        (two lane-swap steps reduce across them); the position's factor
//        2^(E-20) / 16 times the softmax scale goes into the exponent's fma.
//   p.v  O^T = V^T P^T.  B (weights): column j = query position j, k = 8g + e
//        is key 32h + 4g + e (e < 4) or 32h + 16 + 4g + e - 4: exactly the
//        scores lane (g, j) holds for key groups t = 2h and 2h + 1, so
//        P = p * (value scale), split into fp16 hi + lo (two MFMAs, ~22
//        bits), needs no data movement.  A (values): row j = dim 16m + j, the
//        same 8 keys, read from the fp16 value rows with the transposed
//        16-bit LDS read (ds_read_b64_tr_b16: in each group of 16 lanes,
//        lane i's element e is element i & 3 of the word lane 4e + i/4
//        points at).  D: lane (g, j) holds dims 16m + 4g + i of position j.
//   Output: divided by the sums, rotated back (spans 1, 2 between a lane's
//   registers i, 4, 8 between lane groups, 16..64 between registers m),
//   stored as 16-byte rows of 4 dims.
#include <type_traits>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dec;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kQRows = 16;        // query positions per block
constexpr int kKeys = kChunkTokens;   // keys per step
constexpr int kVRow = 2 * kHeadDim;   // bytes per fp16 value row

// LDS of one chunk.  Every access but the transposed value reads is
// lane-contiguous (lane l at 16 l of a 1 KiB block): measured, the earlier
// row-major key layout (80-byte rows, read as lane (g, j) = row 16t + j,
// piece g) and value stores of one 16-byte piece per row for 16 rows each
// cost as many LDS bank-conflict cycles as they had instructions.
struct alignas(16) PrefillShared {
    // key codes as the q.k A operand wants them: key 16t + j, 16-byte piece g
    // (dims 32g .. 32g + 31) at 16 ((4t + g) 16 + j); even dims' nibbles at the
    // top of each byte, or the odd dims' kept there (low nibble 0)
    uint8_t kev[kKeys * kCodeBytesPerRow];
    uint8_t kod[kKeys * kCodeBytesPerRow];
    // values as fp16; row T's 16-byte piece p (dims 8p .. 8p + 7, in the
    // order 8p + 0, 2, 4, 6, 1, 3, 5, 7) at piece slot p ^ vswz(T)
    uint8_t v[kKeys * kVRow];
    float ks[kKeys], vs[kKeys];          // scales
};

// Piece swizzle of value row T (16-byte piece p of the row at slot
// p ^ vswz(T)).  Bits 1-3 (2 (T & 7)) give the 8 rows a half-wave reads
// transposed 8 different 32-byte piece pairs (all 64 banks once).  Bit 0
// makes vswz a permutation of 0..15 over any 16 consecutive rows whose low
// 3 bits are also distinct over any 8 of them: the staging stores (lane
// (j, g) writes piece 4g + s of row 16w + j) then hit 8 or 16 distinct slots
// in every group of 8 or 16 lanes.
__host__ __device__ constexpr int vswz(int T) { return (2 * (T & 7)) | (((T >> 2) ^ (T >> 3)) & 1); }

__device__ __forceinline__ v4f mfma(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 8 two's-complement nibbles (nibble e = element e) -> 8 fp16 values in the
// order e = 0, 2, 4, 6, 1, 3, 5, 7: the offset-binary nibble u = c + 8 goes
// into the mantissa of 1024 (fp16 1024 + u, exact; the exponent byte 0x64 is
// taken from a constant by the byte permute itself) and 1032 is subtracted
// (exact).  Pairing each byte's low nibbles (or its high nibbles) in one
// word is what lets the permute draw the exponent bytes from one source.
__device__ __forceinline__ v8h nibbles_to_half_eo(uint32_t w) {
    const uint32_t x = w ^ 0x88888888u;
    const uint32_t lo = x & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6 (one per byte)
    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
    const uint32_t e64 = 0x64646464u;
    // v_perm_b32(a, b, sel): selector bytes 0-3 pick bytes of b, 4-7 bytes of a
    uint32_t d[4];
    d[0] = __builtin_amdgcn_perm(e64, lo, 0x04010400u);   // (element 0, element 2)
    d[1] = __builtin_amdgcn_perm(e64, lo, 0x04030402u);   // (4, 6)
    d[2] = __builtin_amdgcn_perm(e64, hi, 0x04010400u);   // (1, 3)
    d[3] = __builtin_amdgcn_perm(e64, hi, 0x04030402u);   // (5, 7)
    const v8h biased = __builtin_bit_cast(v8h, make_uint4(d[0], d[1], d[2], d[3]));
    const _Float16 off = static_cast<_Float16>(1032.0f);
    return biased - v8h{off, off, off, off, off, off, off, off};
}

// Lane-row exchanges over the 4 lanes j, j + 16, j + 32, j + 48 (the rows
// of 16 lanes).  swap_rows<1> is v_permlane16_swap of x with itself: lo = the
// value of the even row of the lane's row pair (0, 1) or (2, 3), hi = the odd
// row's; swap_rows<2> is v_permlane32_swap: lo = the lower half's value
// (rows 0, 1), hi = the upper half's.  (The results are copied to scalars
// before the bit cast: a bit cast applied directly to an element of the
// builtin's two-element vector read element 0 for both.)
template <int SPAN>
__device__ __forceinline__ void swap_rows(float x, float &lo, float &hi) {
    const uint32_t a = __builtin_bit_cast(uint32_t, x);
    const auto r = SPAN == 1 ? __builtin_amdgcn_permlane16_swap(a, a, false, false)
                             : __builtin_amdgcn_permlane32_swap(a, a, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float rows_max4(float x) {
    float lo, hi;
    swap_rows<1>(x, lo, hi);
    swap_rows<2>(fmaxf(lo, hi), lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ float rows_sum4(float x) {
    float lo, hi;
    swap_rows<1>(x, lo, hi);
    swap_rows<2>(lo + hi, lo, hi);
    return lo + hi;
}
// Butterfly between lane rows r and r ^ SPAN (SPAN 1 or 2): the lower row
// gets a + b, the upper a - b (a the lower row's value).
template <int SPAN>
__device__ __forceinline__ float rows_butterfly(float x, const int g) {
    float lo, hi;
    swap_rows<SPAN>(x, lo, hi);
    return (g & SPAN) ? lo - hi : lo + hi;
}

// Which sequence b and which of its 16-row query tiles global tile t is
// (tiles of one sequence are consecutive); false past the last tile.
__device__ __forceinline__ bool find_tile(const int32_t *q_start, const int B, const int t, const int lane, int &b_out,
                                          int &tile_out) {
    int acc = 0;
    for (int base = 0; base < B; base += 64) {
        const int b = base + lane;
        int nt = 0;
        if (b < B) {
            const int ql = q_start[b + 1] - q_start[b];
            nt = ql > 0 ? (ql + kQRows - 1) / kQRows : 0;
        }
        int incl = nt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off);
            if (lane >= off) incl += v;
        }
        const unsigned long long hit = __ballot(acc + incl > t);
        if (hit) {
            const int first = __builtin_ctzll(hit);
            b_out = base + first;
            tile_out = t - acc - __shfl(incl - nt, first);
            return true;
        }
        acc += __shfl(incl, 63);
    }
    return false;
}

template <int BH, int P>
__global__ __launch_bounds__(kThreads, 3) void prefill_int4_kernel(PrefillArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int j = lane & 15;
    // longest tiles (latest positions) first: reversed order
    const int t_global = (int)gridDim.x - 1 - (int)blockIdx.x;
    int b = 0, tile = 0;
    if (!find_tile(a.q_start, a.batch, t_global, lane, b, tile)) return;   // the same for the whole block
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);

    const int slot = blockIdx.y;
    const int hk = slot / a.head_chunks;
    const int chunk_id = slot - hk * a.head_chunks;
    const int qh_local = chunk_id * kH + wave;
    const bool live = qh_local < a.group;
    const int qh = hk * a.group + min(qh_local, a.group - 1);

    const int q0 = a.q_start[b];
    const int qlen = a.q_start[b + 1] - q0;
    const int L = prefill_len(a, b);
    const int rows = min(kQRows, qlen - kQRows * tile);
    const int row0 = q0 + kQRows * tile;
    const int pos0 = L - qlen + kQRows * tile;   // position of row 0
    const int last_pos = pos0 + rows - 1;
    const int nchunks = last_pos / kKeys + 1;
    const int my_pos = pos0 + j;                 // this lane's query position

    // Out of contract (more queries than cached tokens, which includes an
    // empty context): the rows get zeros and no page is read.
    if (qlen > L) {
        if (live && j < rows) {
            float *dst = a.out + ((int64_t)(row0 + j) * a.num_q_heads + qh) * kHeadDim + 4 * g;
#pragma unroll
            for (int m = 0; m < 8; ++m) *reinterpret_cast<float4 *>(dst + 16 * m) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }

    __shared__ PrefillShared sh;

    // ---- the rotated query of head qh: lane (g, j) holds position j, dims 32g .. 32g + 31 ----
    float x[32];
    {
        uint4 raw[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                        make_uint4(0, 0, 0, 0)};
        if (j < rows) {
            const uint4 *src = reinterpret_cast<const uint4 *>(a.q + ((int64_t)(row0 + j) * a.num_q_heads + qh) *
                                                                         kHeadDim + 32 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) raw[s] = src[s];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t w4[4] = {raw[s].x, raw[s].y, raw[s].z, raw[s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[8 * s + 2 * e] = half_to_float(w4[e]);
                x[8 * s + 2 * e + 1] = half_to_float(w4[e] >> 16);
            }
        }
        if constexpr (BH > 0) {
#pragma unroll
            for (int span = 1; span < 32 && span < BH; span <<= 1) {
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    if (r & span) continue;
                    const float u = x[r], v = x[r + span];
                    x[r] = u + v;
                    x[r + span] = u - v;
                }
            }
#pragma unroll
            for (int m = 16; m < 64; m <<= 1) {     // spans 32, 64: lane groups g ^ 1, g ^ 2
                if (32 * (m / 16) >= BH) break;
                const bool upper = (lane & m) != 0;
#pragma unroll
                for (int r = 0; r < 32; ++r) {
                    const float p = __shfl_xor(x[r], m);
                    x[r] = upper ? (p - x[r]) : (x[r] + p);
                }
            }
            const float c = rsqrtf(static_cast<float>(BH));
#pragma unroll
            for (int r = 0; r < 32; ++r) x[r] *= c;
        }
    }
    // 24-bit fixed point per (position, head): the position's 128 dims are in
    // lanes j, j + 16, j + 32, j + 48
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(x[r]));
    amax = rows_max4(amax);
    int qexp = 0;
    // amax (1 + 2^-7) < 2^qexp, so |X| <= 2^23 / (1 + 2^-7) < 127 (2^16 +
    // 2^8 + 1): the top digit stays in [-128, 127]
    if (amax > 0.0f) (void)frexpf(amax * 1.0078125f, &qexp);
    const float qmul = ldexpf(1.0f, 23 - qexp);
    v4i qb[3][2];   // [digit][even / odd dims]: byte e of dword w = dim 32g + 2 (4w + e) + half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t wd[3][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int X = static_cast<int>(rintf(x[2 * e + h] * qmul));
            // balanced digits: D2 = X mod 256 in [-128, 127], then the same on
            // (X - D2) / 256; the bytes of X - D2 2^0 - D1 2^8 are D0's
            const int d2 = static_cast<int>(static_cast<int8_t>(X & 0xFF));
            const int x1 = (X - d2) >> 8;
            const int d1 = static_cast<int>(static_cast<int8_t>(x1 & 0xFF));
            const int d0 = (x1 - d1) >> 8;
            const int dig[3] = {d0, d1, d2};
#pragma unroll
            for (int l = 0; l < 3; ++l) wd[l][e >> 2] |= (static_cast<uint32_t>(dig[l]) & 0xFFu) << (8 * (e & 3));
        }
#pragma unroll
        for (int l = 0; l < 3; ++l) qb[l][h] = v4i{(int)wd[l][0], (int)wd[l][1], (int)wd[l][2], (int)wd[l][3]};
    }
    // score factor of this position (log2 units): 2^(E-23), 1/16 for the
    // nibble position, the softmax scale (positive)
    const float rm = ldexpf(a.score_scale * 0.0625f, qexp - 23);

    // ---- loads of one chunk: wave w takes keys 16w .. 16w + 15 ----
    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    const int64_t page_stride = (int64_t)a.num_kv_heads * a.tile_bytes;
    const int64_t code_off = (int64_t)hk * (P * kCodeBytesPerRow);
    const int64_t scale_off = (int64_t)a.num_kv_heads * (P * kCodeBytesPerRow) + (int64_t)hk * (2 * P);
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages_per_seq;
    const int last_page = (L - 1) / P;
    // Wave w stages keys 16w .. 16w + 15 of a chunk: lane l loads the
    // 16-byte piece l / 16 (dims 32 (l / 16) .. + 31) of key 16w + l % 16, of
    // the key and of the value codes.  Its key bytes land at 16 l of the
    // wave's 1 KiB block, its values as fp16 pieces 4 (l / 16) .. + 3 of row
    // 16w + l % 16.
    const int kj = lane & 15, kg = lane >> 4;
    struct Raw { uint4 k, v; uint32_t s; };
    auto load = [&](int c, Raw &r) {
        const int key0 = kKeys * c + 16 * wave;
        const int64_t page = pt[min(key0 / P, last_page)];
        const int slot0 = key0 % P;
        const uint8_t *tile_k = kpool + page * page_stride + code_off + (int64_t)slot0 * kCodeBytesPerRow;
        const uint8_t *tile_v = vpool + page * page_stride + code_off + (int64_t)slot0 * kCodeBytesPerRow;
        r.k = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                            reinterpret_cast<const v4u *>(tile_k + kj * kCodeBytesPerRow + 16 * kg)));
        r.v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                            reinterpret_cast<const v4u *>(tile_v + kj * kCodeBytesPerRow + 16 * kg)));
        const uint8_t *sp = (lane < 16 ? kpool : vpool) + page * page_stride + scale_off + 2 * (slot0 + kj);
        r.s = lane < 32 ? *reinterpret_cast<const uint16_t *>(sp) : 0u;
    };
    auto stage = [&](const Raw &r) {
        const uint32_t kw[4] = {r.k.x, r.k.y, r.k.z, r.k.w};
        uint32_t ev[4], od[4];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            ev[s4] = (kw[s4] << 4) & 0xF0F0F0F0u;
            od[s4] = kw[s4] & 0xF0F0F0F0u;
        }
        *reinterpret_cast<uint4 *>(&sh.kev[1024 * wave + 16 * lane]) = make_uint4(ev[0], ev[1], ev[2], ev[3]);
        *reinterpret_cast<uint4 *>(&sh.kod[1024 * wave + 16 * lane]) = make_uint4(od[0], od[1], od[2], od[3]);
        const uint32_t vw[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
        const int T = 16 * wave + kj;
        const int vx = vswz(T);
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
            *reinterpret_cast<v8h *>(&sh.v[T * kVRow + 16 * ((4 * kg + s4) ^ vx)]) = nibbles_to_half_eo(vw[s4]);
        if (lane < 16) sh.ks[16 * wave + lane] = half_to_float(r.s);
        else if (lane < 32) sh.vs[16 * wave + lane - 16] = half_to_float(r.s);
    };

    float m_run = -INFINITY, l_lane = 0.0f;   // this lane's position
    // o[m][i]: position j, value slot 16m + 4g + i, which holds dim
    // 16m + 8 (g >> 1) + 2i + (g & 1) (the staging's element order)
    v4f o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // transposed-read address of value slots 16m + 4 (j & 3) of key row 4g + j / 4
    // (+ 32 h for half h, + 16 for its second read): piece 2m + (j & 3) / 2
    const int tr_key = 4 * g + (j >> 2);
    const uint32_t tr_base = tr_key * kVRow + 8 * (j & 1);
    const int tr_piece = (j & 3) >> 1;
    const int tr_x = vswz(tr_key);          // the row's piece swizzle (rows + 16, + 32 share it)
    const uint32_t tr_b = tr_base + 16u * (uint32_t)(tr_piece ^ (tr_x & 1));
    const uint32_t tr_c = 32u * (uint32_t)(tr_x >> 1);

    // -1 as the multiplier operand of the weight split's mixed-precision fmas
    float neg_one = -1.0f;
    asm("" : "+v"(neg_one));

    auto compute = [&](int c, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        // q.k: z[t][i] = score of key 16t + 4g + i before the position's factor
        float z[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4i ke = *reinterpret_cast<const v4i *>(&sh.kev[1024 * t + 16 * lane]);
            const v4i ko = *reinterpret_cast<const v4i *>(&sh.kod[1024 * t + 16 * lane]);
            const v4i zero = {0, 0, 0, 0};
            v4i dl[3];
#pragma unroll
            for (int l = 0; l < 3; ++l) dl[l] = mfma_i8(ko, qb[l][1], mfma_i8(ke, qb[l][0], zero));
            const float4 sk = *reinterpret_cast<const float4 *>(&sh.ks[16 * t + 4 * g]);
            const float skv[4] = {sk.x, sk.y, sk.z, sk.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // |D . k| <= 128 * 128 * 128 = 2^21 for each digit, so
                // D0 . k 2^8 + D1 . k is exact in int32
                const float dot = fmaf(static_cast<float>((dl[0][i] << 8) + dl[1][i]), 256.0f,
                                       static_cast<float>(dl[2][i]));
                const float sc = dot * skv[i];
                z[t][i] = (!MASK || kKeys * c + 16 * t + 4 * g + i <= my_pos) ? sc : -INFINITY;
            }
        }
        // online softmax of this position (its 64 scores: 16 here, 48 in lanes j + 16 k)
        float zm = z[0][0];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) zm = fmaxf(zm, z[t][i]);
        // rescale only when some position of the wave has a new maximum (a
        // wave-uniform branch; alpha is exactly 1 for the others).  A
        // position's maximum is over its 4 lanes, and it exceeds m_run
        // exactly when one of those lanes' own maxima does (rm > 0), so the
        // lane exchange is needed only inside the branch.
        if (__builtin_amdgcn_ballot_w64(zm * rm > m_run)) {
            const float m_new = fmaxf(m_run, rows_max4(zm) * rm);   // finite from the first chunk on (key 0 is visible)
            const float alpha = fast_exp2(m_run - m_new);
            l_lane *= alpha;
#pragma unroll
            for (int m = 0; m < 8; ++m) o[m] *= alpha;
            m_run = m_new;
        }
        // weights times the value scale, split hi / lo: the p.v B operands,
        // built a pair of keys at a time (v_cvt_pk_f16_f32)
        v2h ph[4][2], pl[4][2];   // [t][i / 2]
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float4 sv = *reinterpret_cast<const float4 *>(&sh.vs[16 * t + 4 * g]);
            const float svv[4] = {sv.x, sv.y, sv.z, sv.w};
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(fmaf(z[t][i], rm, -m_run));   // 0 for masked keys
                l_lane += p;
                // masked keys past the context may have any scale bytes (0 * NaN)
                pv[i] = (!MASK || kKeys * c + 16 * t + 4 * g + i <= my_pos) ? p * svv[i] : 0.0f;
                // hi and lo must both derive from this rounded product: left
                // free, the compiler fuses the product into lo's conversion
                // but not into hi's, and where the product lies within one
                // fp32 rounding of an fp16 midpoint hi + lo then misses it by
                // a whole fp16 ulp
                asm("" : "+v"(pv[i]));
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const v2h hi = __builtin_convertvector((v2f){pv[2 * u], pv[2 * u + 1]}, v2h);
                ph[t][u] = hi;
                // lo = fp16(pv - hi): pv - hi is exact in fp32 (|pv - hi| is at
                // most half an fp16 ulp of pv), so one mixed-precision fma that
                // rounds straight to fp16 gives the same bits as an fp32 fma
                // and a conversion; mixlo / mixhi fill the two halves of the
                // pair (the fp16 operand is hi's low or high half, widened
                // inside the instruction)
                const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
                uint32_t lb;
                asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]"
                    : "=v"(lb) : "v"(hb), "v"(neg_one), "v"(pv[2 * u]));
                asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                    : "+v"(lb) : "v"(hb), "v"(neg_one), "v"(pv[2 * u + 1]));
                pl[t][u] = __builtin_bit_cast(v2h, lb);
            }
        }
        v8h pb_hi[2], pb_lo[2];   // element 4 (t & 1) + i of half t / 2
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            pb_hi[h] = __builtin_shufflevector(__builtin_shufflevector(ph[2 * h][0], ph[2 * h][1], 0, 1, 2, 3),
                                               __builtin_shufflevector(ph[2 * h + 1][0], ph[2 * h + 1][1], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
            pb_lo[h] = __builtin_shufflevector(__builtin_shufflevector(pl[2 * h][0], pl[2 * h][1], 0, 1, 2, 3),
                                               __builtin_shufflevector(pl[2 * h + 1][0], pl[2 * h + 1][1], 0, 1, 2, 3),
                                               0, 1, 2, 3, 4, 5, 6, 7);
        }
        // p.v: dim tile m, both key halves h; tile m + 1's values are read
        // while tile m's products run.  Piece (2m + tr_piece) ^ tr_x of the
        // row is 2 (m ^ (tr_x >> 1)) + (tr_piece ^ (tr_x & 1)).
        auto read_tile = [&](const int m, v8h (&va)[2]) {
            const uint32_t addr = tr_b + (tr_c ^ (32u * (uint32_t)m));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s *)&sh.v[addr + 32 * h * kVRow]);
                const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4s *)&sh.v[addr + 32 * h * kVRow + 16 * kVRow]);
                va[h] = __builtin_bit_cast(
                    v8h, make_uint4(__builtin_bit_cast(uint2, r0).x, __builtin_bit_cast(uint2, r0).y,
                                    __builtin_bit_cast(uint2, r1).x, __builtin_bit_cast(uint2, r1).y));
            }
        };
        // (scheduling barriers that only vector and scalar ALU work may
        // cross keep each tile's reads ahead of the previous tile's products)
        v8h va[2][2];
        read_tile(0, va[0]);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (m + 1 < 8) read_tile(m + 1, va[(m + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0x6);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                o[m] = mfma(va[m & 1][h], pb_hi[h], o[m]);
                o[m] = mfma(va[m & 1][h], pb_lo[h], o[m]);
            }
            __builtin_amdgcn_sched_barrier(0x6);
        }
    };

    // chunks below n_full hold only keys every position of the tile sees
    // (64 c + 63 <= pos0); the rest need the causal mask.  Two loops, one
    // per variant, keep the accumulators in place (one loop choosing per
    // chunk made the compiler copy them around).
    const int n_full = min((pos0 + 1) / kKeys, nchunks);
    Raw raw;
    load(0, raw);
    auto run = [&](int c0, int c1, auto masked) {
        for (int c = c0; c < c1; ++c) {
            __syncthreads();          // every wave is done with the previous chunk's LDS
            stage(raw);
            __syncthreads();
            if (c + 1 < nchunks) load(c + 1, raw);
            if (live) compute(c, masked);
        }
    };
    run(0, n_full, std::false_type{});
    run(n_full, nchunks, std::true_type{});
    if (!live) return;

    // ---- normalise, rotate back, store ----
    const float inv = 1.0f / rows_sum4(l_lane);
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] *= inv;
    if constexpr (BH > 0) {
        // the spans in increasing order, each where its dim bit lives
#pragma unroll
        for (int m = 0; m < 8; ++m)                                // span 1: lane rows g ^ 1
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m][i] = rows_butterfly<1>(o[m][i], g);
#pragma unroll
        for (int s = 1; s < 4; s <<= 1) {                          // spans 2, 4: registers i ^ s
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i & s) continue;
                    const float u = o[m][i], v = o[m][i + s];
                    o[m][i] = u + v;
                    o[m][i + s] = u - v;
                }
        }
#pragma unroll
        for (int m = 0; m < 8; ++m)                                // span 8: lane rows g ^ 2
#pragma unroll
            for (int i = 0; i < 4; ++i) o[m][i] = rows_butterfly<2>(o[m][i], g);
#pragma unroll
        for (int s = 1; s < 8 && 16 * s < BH; s <<= 1) {           // spans 16, 32, 64: registers m ^ s
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                if (m & s) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float u = o[m][i], v = o[m + s][i];
                    o[m][i] = u + v;
                    o[m + s][i] = u - v;
                }
            }
        }
        const float cb = rsqrtf(static_cast<float>(BH));
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m] *= cb;
    }
    // Regroup lane rows g and g ^ 1 so that lane (g, j) holds dims
    // 16m + 4g .. 16m + 4g + 3: the even row (dims 8h + 0, 2, 4, 6) keeps
    // 0, 2 and takes the odd row's 1, 3; the odd row (8h + 1, 3, 5, 7) keeps
    // 5, 7 and takes the even row's 4, 6.
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        float lo0, hi0, lo1, hi1;
        swap_rows<1>(odd ? o[m][0] : o[m][2], lo0, hi0);   // even gets the odd row's dim 1, odd the even row's 4
        swap_rows<1>(odd ? o[m][1] : o[m][3], lo1, hi1);   // dims 3 and 6
        const float r0 = odd ? lo0 : hi0, r1 = odd ? lo1 : hi1;
        o[m] = odd ? v4f{r0, o[m][2], r1, o[m][3]} : v4f{o[m][0], r0, o[m][1], r1};
    }
    if (j < rows) {
        float *dst = a.out + ((int64_t)(row0 + j) * a.num_q_heads + qh) * kHeadDim + 4 * g;
#pragma unroll
        for (int m = 0; m < 8; ++m) *reinterpret_cast<float4 *>(dst + 16 * m) = make_float4(o[m][0], o[m][1], o[m][2], o[m][3]);
    }
}

}  // namespace

hipError_t launch_prefill_int4(const PrefillArgs &a, hipStream_t stream) {
    // every sequence adds at most one partly filled tile
    const int64_t tiles = (int64_t)a.num_q / kQRows + a.batch;
    const dim3 grid((unsigned)tiles, (unsigned)(a.num_kv_heads * a.head_chunks), 1);
    const dim3 block(kThreads);
#define KVQ_LAUNCH(BHV, PV) hipLaunchKernelGGL((prefill_int4_kernel<BHV, PV>), grid, block, 0, stream, a)
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
