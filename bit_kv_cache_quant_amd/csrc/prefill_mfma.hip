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
// group, so the work is bound by the matrix cores rather than by HBM.
//
// Block = 4 waves = the 4 query heads of one head slot (KV head, chunk of 4
// of its query heads) x 16 consecutive query positions of one sequence; it
// walks the keys in chunks of 64 staged once in LDS for the 4 waves.
//   q.k  exact integer products on v_mfma_i32_16x16x64_i8, as in the
//        decode: the rotated query of each row is a 21-bit fixed-point
//        integer X = round(q' 2^(20-E)) (E the exponent of the row's max
//        |q'|) split into limbs X = L0 2^14 + L1 2^7 + L2, one MFMA per limb
//        and nibble half.  A (limb): row j = query position j; the lanes of
//        k-group g hold dims 32g + 2e (even half) or 32g + 2e + 1 (odd half).
//        B (keys): column j = key 16t + j, its 16 code bytes (dims 32g ..
//        32g + 31) with the even dims' nibbles moved to the top of each byte
//        and the odd dims' kept there: signed bytes 16 c, no offset term.
//        The three limb results are exact in int32 and are recombined in
//        fp32; the row's scale, 1/16 and the key's scale follow.  D: lane
//        (g, j) holds rows 4g..4g+3 (query positions) for key j: scores,
//        masked causally.  (fp16 products summed in fp32 were measurably less
//        accurate here: with the rotation every code is nonzero and the
//        softmax of large scores amplifies their rounding.)
//   softmax: online per query row; a row's 16 keys of a group are the 16
//        lanes of one lane row (DPP reductions), its 4 rows per lane are
//        rescaled lane-locally.
//   p.v  A (weights): row j = query position j, k = keys 16g + 8h .. 16g + 8h +
//        7 (MFMA half h), P = p * (value scale) split into fp16 hi + lo and
//        passed through LDS.  B (values): the value codes of dim 16m + j of
//        the same keys, read with the transposed 4-bit LDS read
//        (ds_read_b64_tr_b4) from the decode's swizzled layout and converted
//        to fp16.  D: lane (g, j) holds rows 4g..4g+3 of output dim 16m + j.
//   Output: divided by the row sums, rotated back (spans below 16 between
//   the lanes of a row, 16..64 between a lane's registers), stored in fp32.
#include <type_traits>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dec;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kQRows = 16;        // query positions per block
constexpr int kKeys = kChunkTokens;   // keys per step
constexpr int kKPitch = 80;       // LDS bytes per key row of codes (64 + 16: conflict-free 16-byte reads)
constexpr int kVGroup = 1024;     // value codes of 16 keys, swizzled slots
__host__ __device__ constexpr int vgroup(int t) { return t * kVGroup + 128 * ((t + 1) >> 1); }
constexpr int kVBytes = vgroup(3) + kVGroup;
constexpr int kPPitch = kKeys + 8;    // halves per weight row (16-byte aligned rows, spread banks)

struct alignas(16) PrefillShared {
    uint8_t k[kKeys * kKPitch];            // key codes, row n at n * kKPitch
    uint8_t v[kVBytes];                    // value codes, 4 swizzled groups
    float ks[kKeys], vs[kKeys];            // scales
    _Float16 p[kWaves][2][kQRows][kPPitch];   // per wave: weights hi / lo [query row][key]
};

__device__ __forceinline__ v4f mfma(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 8 two's-complement nibbles (nibble e = element e) -> 8 fp16 values: the
// offset-binary nibble u = c + 8 goes into the mantissa of 1024 (fp16 1024 + u,
// exact) and 1032 is subtracted (exact).
__device__ __forceinline__ v8h nibbles_to_half(uint32_t w) {
    const uint32_t x = w ^ 0x88888888u;
    const uint32_t lo = x & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6 (one per byte)
    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
    // v_perm_b32(a, b, sel): selector bytes 0-3 pick bytes of b, 4-7 bytes of a, 0x0c gives 0
    uint32_t d[4];
    d[0] = __builtin_amdgcn_perm(hi, lo, 0x0c040c00u) | 0x64006400u;   // (lo byte 0, hi byte 0)
    d[1] = __builtin_amdgcn_perm(hi, lo, 0x0c050c01u) | 0x64006400u;
    d[2] = __builtin_amdgcn_perm(hi, lo, 0x0c060c02u) | 0x64006400u;
    d[3] = __builtin_amdgcn_perm(hi, lo, 0x0c070c03u) | 0x64006400u;
    const v8h biased = __builtin_bit_cast(v8h, make_uint4(d[0], d[1], d[2], d[3]));
    const _Float16 off = static_cast<_Float16>(1032.0f);
    return biased - v8h{off, off, off, off, off, off, off, off};
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
__global__ __launch_bounds__(kThreads) void prefill_int4_kernel(PrefillArgs a) {
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
    const int L = a.context_lens[b];
    const int rows = min(kQRows, qlen - kQRows * tile);
    const int row0 = q0 + kQRows * tile;
    const int pos0 = L - qlen + kQRows * tile;   // position of row 0
    const int last_pos = pos0 + rows - 1;
    const int nchunks = last_pos / kKeys + 1;

    __shared__ PrefillShared sh;

    // ---- the rotated, scaled query of head qh: lane (row j, group g), dims 32g .. 32g + 31 ----
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
        }
        if constexpr (BH > 0) {
            const float c = rsqrtf(static_cast<float>(BH));
#pragma unroll
            for (int r = 0; r < 32; ++r) x[r] *= c;
        }
    }
    // 21-bit fixed point per (row, head): the row's 128 dims are in lanes
    // j, j + 16, j + 32, j + 48
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(x[r]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int qexp = 0;
    if (amax > 0.0f) (void)frexpf(amax, &qexp);     // amax < 2^qexp
    const float qmul = ldexpf(1.0f, 20 - qexp);
    v4i qa[3][2];   // [limb][even / odd dims]: byte e of dword w = dim 32g + 2 (4w + e) + half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t wd[3][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int X = static_cast<int>(rintf(x[2 * e + h] * qmul));
            const int limb[3] = {X >> 14, (X >> 7) & 127, X & 127};
#pragma unroll
            for (int l = 0; l < 3; ++l) wd[l][e >> 2] |= (static_cast<uint32_t>(limb[l]) & 0xFFu) << (8 * (e & 3));
        }
#pragma unroll
        for (int l = 0; l < 3; ++l) qa[l][h] = v4i{(int)wd[l][0], (int)wd[l][1], (int)wd[l][2], (int)wd[l][3]};
    }
    // the score factor of rows 4g + i (this lane's result rows): 2^(E-20) of
    // that row, 1/16 for the nibble position, the softmax scale (log2 units)
    float row_mul[4];
    {
        const float mine = ldexpf(a.score_scale * 0.0625f, qexp - 20);
#pragma unroll
        for (int i = 0; i < 4; ++i) row_mul[i] = __shfl(mine, 4 * g + i);
    }

    // ---- loads of one chunk: wave w takes key group w (16 keys) ----
    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    const int64_t page_stride = (int64_t)a.num_kv_heads * a.tile_bytes;
    const int64_t code_off = (int64_t)hk * (P * kCodeBytesPerRow);
    const int64_t scale_off = (int64_t)a.num_kv_heads * (P * kCodeBytesPerRow) + (int64_t)hk * (2 * P);
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages_per_seq;
    const int last_page = (L - 1) / P;
    const int ln = lane >> 2, lp = lane & 3;   // key row, 16-byte piece of this lane's loads
    struct Raw { uint4 k, v; uint32_t s; };
    auto load = [&](int c, Raw &r) {
        const int key0 = kKeys * c + 16 * wave;                      // first key of group `wave`
        const int64_t page = pt[min(key0 / P, last_page)];
        const int slot0 = key0 % P;
        const uint8_t *kt = kpool + page * page_stride + code_off + (int64_t)(slot0 + ln) * kCodeBytesPerRow + 16 * lp;
        const uint8_t *vt = vpool + page * page_stride + code_off + (int64_t)(slot0 + ln) * kCodeBytesPerRow + 16 * lp;
        r.k = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u *>(kt)));
        r.v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4u *>(vt)));
        const uint8_t *sp = (lane < 16 ? kpool : vpool) + page * page_stride + scale_off + 2 * (slot0 + (lane & 15));
        r.s = lane < 32 ? *reinterpret_cast<const uint16_t *>(sp) : 0u;
    };
    auto stage = [&](const Raw &r) {
        *reinterpret_cast<uint4 *>(&sh.k[(16 * wave + ln) * kKPitch + 16 * lp]) = r.k;
        *reinterpret_cast<uint4 *>(&sh.v[vgroup(wave) + 16 * (4 * ln + (lp ^ ((ln >> 2) & 3)))]) = r.v;
        if (lane < 16) sh.ks[16 * wave + lane] = half_to_float(r.s);
        else if (lane < 32) sh.vs[16 * wave + lane - 16] = half_to_float(r.s);
    };

    float m_run[4], l_lane[4];      // query rows 4g + i
    v4f o[8];                       // output dims 16m + j, rows 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_run[i] = -INFINITY;
        l_lane[i] = 0.0f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) o[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int c, auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        // q.k and the causal mask
        float z[4][4];   // [key group t][row i]
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 kr = *reinterpret_cast<const uint4 *>(&sh.k[(16 * t + j) * kKPitch + 16 * g]);
            // signed bytes 16 c: even dims (low nibbles) shifted up, odd dims in place
            const v4i kev = {(int)((kr.x << 4) & 0xF0F0F0F0u), (int)((kr.y << 4) & 0xF0F0F0F0u),
                             (int)((kr.z << 4) & 0xF0F0F0F0u), (int)((kr.w << 4) & 0xF0F0F0F0u)};
            const v4i kod = {(int)(kr.x & 0xF0F0F0F0u), (int)(kr.y & 0xF0F0F0F0u), (int)(kr.z & 0xF0F0F0F0u),
                             (int)(kr.w & 0xF0F0F0F0u)};
            const v4i zero = {0, 0, 0, 0};
            v4i dl[3];
#pragma unroll
            for (int l = 0; l < 3; ++l) dl[l] = mfma_i8(qa[l][1], kod, mfma_i8(qa[l][0], kev, zero));
            const float sk = sh.ks[16 * t + j];
            const int kp = kKeys * c + 16 * t + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dot = fmaf(static_cast<float>(dl[0][i]), 16384.0f,
                                       fmaf(static_cast<float>(dl[1][i]), 128.0f, static_cast<float>(dl[2][i])));
                const float sc = dot * row_mul[i] * sk;
                z[t][i] = (!MASK || kp <= pos0 + 4 * g + i) ? sc : -INFINITY;
            }
        }
        // online softmax per row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float zm = fmaxf(fmaxf(z[0][i], z[1][i]), fmaxf(z[2][i], z[3][i]));
            zm = row_max16_fast(zm);
            if (zm > m_run[i]) {
                const float alpha = fast_exp2(m_run[i] - zm);
                l_lane[i] *= alpha;
#pragma unroll
                for (int m = 0; m < 8; ++m) o[m][i] *= alpha;
                m_run[i] = zm;
            }
        }
        // weights times the value scale, hi / lo, into LDS [row][key]
        _Float16(*pw)[kQRows][kPPitch] = sh.p[wave];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float sv = sh.vs[16 * t + j];
            const int kp = kKeys * c + 16 * t + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(z[t][i] - m_run[i]);   // 0 for masked keys
                l_lane[i] += p;
                // masked keys past the context may have any scale bytes (0 * NaN)
                const float pv = (!MASK || kp <= pos0 + 4 * g + i) ? p * sv : 0.0f;
                const _Float16 h = static_cast<_Float16>(pv);
                pw[0][4 * g + i][16 * t + j] = h;
                pw[1][4 * g + i][16 * t + j] = static_cast<_Float16>(pv - static_cast<float>(h));
            }
        }
        wave_lds_sync();
        v8h pa_hi[2], pa_lo[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            pa_hi[h] = *reinterpret_cast<const v8h *>(&pw[0][j][16 * g + 8 * h]);
            pa_lo[h] = *reinterpret_cast<const v8h *>(&pw[1][j][16 * g + 8 * h]);
        }
        wave_lds_sync();
        // p.v: dim tile m, keys 16g + 8h + e of the lane group
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const v2i r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(
                &sh.v[vgroup(g) + 16 * (4 * j + ((m >> 1) ^ ((j >> 2) & 3))) + 8 * (m & 1)]));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const v8h vb = nibbles_to_half(static_cast<uint32_t>(h == 0 ? r.x : r.y));
                o[m] = mfma(pa_hi[h], vb, o[m]);
                o[m] = mfma(pa_lo[h], vb, o[m]);
            }
        }
    };

    Raw raw;
    load(0, raw);
    for (int c = 0; c < nchunks; ++c) {
        __syncthreads();          // every wave is done with the previous chunk's LDS
        stage(raw);
        __syncthreads();
        if (c + 1 < nchunks) load(c + 1, raw);
        if (live) {
            if (kKeys * c + kKeys - 1 > pos0) compute(c, std::true_type{});
            else compute(c, std::false_type{});
        }
    }
    if (!live) return;

    // ---- normalise, rotate back, store ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float inv = 1.0f / row_sum16(l_lane[i]);
#pragma unroll
        for (int m = 0; m < 8; ++m) o[m][i] *= inv;
    }
    if constexpr (BH > 0) {
#pragma unroll
        for (int span = 1; span < 16 && span < BH; span <<= 1) {   // partner lane j ^ span of the row
            const bool upper = (j & span) != 0;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __shfl_xor(o[m][i], span, 16);
                    o[m][i] = upper ? (p - o[m][i]) : (o[m][i] + p);
                }
        }
#pragma unroll
        for (int s = 1; s < 8 && 16 * s < BH; s <<= 1) {          // spans 16, 32, 64: registers m ^ s
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        if (r < rows) {
            float *dst = a.out + ((int64_t)(row0 + r) * a.num_q_heads + qh) * kHeadDim + j;
#pragma unroll
            for (int m = 0; m < 8; ++m) dst[16 * m] = o[m][i];
        }
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
