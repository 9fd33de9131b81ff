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
//         max|q'| of that head, split into limbs X = L0 2^21 + L1 2^14 +
//         L2 2^7 + L3 (L0 signed, L1..L3 in [0,127]).  One MFMA row per
//         (head, limb): 4 heads x 4 limbs fill the 16 rows.  Keys enter as
//         offset-binary nibbles u = c + 8 in [0, 15]; the accumulator starts
//         at -8 sum_d L (per row), so the integer result is exactly
//         sum_d L_d c_d.
//   p.v : the unnormalised weight times the value scale, P = p s_V, is
//         written as a 28-bit unsigned fixed-point integer relative to the
//         largest P of the head in the 64-token chunk, split the same way
//         into four 7-bit limbs (again one row per (head, limb)); values
//         enter as sign-extended int8 codes.
// Limbs are recombined with integer shifts (exact) and one fp32 fma.  The
// only approximations are the 2^-28 relative roundings of q' and P and fp32
// accumulation, far inside the 2e-3 tolerance.
//
// Layout of one wave (64 lanes, g = lane / 16, j = lane % 16), per chunk of
// 64 tokens (4 groups t of 16 tokens; a group is one page of 16 tokens or
// half a page of 32):
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
//   p.v  B (values): lane column j = dims 8j..8j+7 of MFMA m (dim 8j+m),
//        k-slots = the 16 tokens of group g: one dword load per token,
//        sign-extended to bytes and byte-transposed in registers.
//        D: lane (g, j) gets rows (head g, limbs 0..3) for dim 8j+m.
// A block of 4 waves owns one work item (sequence, KV head, 4 query heads,
// page range); waves take chunks round-robin and merge through LDS at the end.
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 64;            // tokens per chunk
constexpr int kH = kHeadsPerChunk;    // 4 query heads

__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// All-reduce inside each row of 16 lanes; every lane of the row gets the result.
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_f<0x140>(v));   // row_mirror
    return v;
}

__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Low / high nibbles of 8 two's-complement codes as offset-binary bytes (c + 8).
__device__ __forceinline__ void split_offset(uint32_t w, uint32_t &lo, uint32_t &hi) {
    const uint32_t x = w ^ 0x88888888u;
    lo = x & 0x0F0F0F0Fu;
    hi = (x >> 4) & 0x0F0F0F0Fu;
}

// Low / high nibbles of 8 two's-complement codes as sign-extended bytes.
// For u = c + 8 in [0, 15]: (u + 0x78) stays below 0x100 per byte, and
// xor 0x80 then gives u - 8 = c modulo 256.
__device__ __forceinline__ void split_signed(uint32_t w, uint32_t &lo, uint32_t &hi) {
    uint32_t l, h;
    split_offset(w, l, h);
    lo = (l + 0x78787878u) ^ 0x80808080u;
    hi = (h + 0x78787878u) ^ 0x80808080u;
}

// 4x4 byte transpose: out[k] byte r = in[r] byte k.
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, uint32_t &o0,
                                           uint32_t &o1, uint32_t &o2, uint32_t &o3) {
    // v_perm_b32(x, y, sel): bytes 0-3 of the selector pick from y (0..3) and x (4..7).
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

// Exact value of a (head, *) row group of 4 limb results: sum_r 2^(21-7r) D_r,
// returned as fp32 (one rounding).
__device__ __forceinline__ float limbs_to_float(v4i d) {
    const int hi = (d[0] << 7) + d[1];
    const int lo = (d[2] << 7) + d[3];
    return fmaf(static_cast<float>(hi), 16384.0f, static_cast<float>(lo));
}

struct Shared {
    float q[kWaves][kH][kHeadDim];        // rotated queries (per wave, setup)
    uint32_t pfix[kWaves][kH][kChunk];     // fixed-point P hand-off
    float mo[kWaves][kH][kHeadDim];        // merge: unnormalised outputs
    float mm[kWaves][kH];
    float ml[kWaves][kH];
};

template <int BH, int P>
__global__ __launch_bounds__(kThreads) void decode_int4_mfma_kernel(DecodeArgs a) {
    const int s = blockIdx.x;
    const int hk = blockIdx.y / a.head_chunks;
    const int chunk_id = blockIdx.y - hk * a.head_chunks;
    const int b = blockIdx.z;
    const int L = a.context_lens[b];
    if (L <= 0) return;
    const int npages = (L + P - 1) / P;
    const int p0 = s * a.pages_per_split;
    if (p0 >= npages) return;
    const int p1 = min(p0 + a.pages_per_split, npages);
    const int tok_begin = p0 * P;
    const int tok_end = min(p1 * P, L);
    const int nchunks = (tok_end - tok_begin + kChunk - 1) / kChunk;

    __shared__ Shared sh;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int qh0 = hk * a.group + chunk_id * kH;
    const int nheads = min(kH, a.group - chunk_id * kH);

    // ---- setup: rotated query, fixed-point limbs, per-head score scale ----
    {
        // lane loads 8 dims of one head: head lane/16, dims 8*(lane%16)..+7
        const int hq = lane >> 4, d0 = (lane & 15) * 8;
        float x[8];
        if (hq < nheads) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(a.q + ((int64_t)b * a.num_q_heads + qh0 + hq) * kHeadDim + d0);
            x[0] = half_to_float(raw.x); x[1] = half_to_float(raw.x >> 16);
            x[2] = half_to_float(raw.y); x[3] = half_to_float(raw.y >> 16);
            x[4] = half_to_float(raw.z); x[5] = half_to_float(raw.z >> 16);
            x[6] = half_to_float(raw.w); x[7] = half_to_float(raw.w >> 16);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) x[r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) sh.q[wave][hq][d0 + r] = x[r];
        if constexpr (BH > 0) {
            // butterflies over the 128 dims of each head: 64 per head and stage,
            // each lane doing 4 (one per head)
            for (int span = 1; span < BH; span <<= 1) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                const int i = ((lane / span) * 2 * span) + (lane % span);
                float u[kH], v[kH];
#pragma unroll
                for (int h = 0; h < kH; ++h) { u[h] = sh.q[wave][h][i]; v[h] = sh.q[wave][h][i + span]; }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int h = 0; h < kH; ++h) { sh.q[wave][h][i] = u[h] + v[h]; sh.q[wave][h][i + span] = u[h] - v[h]; }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // Lane (g, j): row (head j/4, limb j%4); dims 32g..32g+31.
    const int arow_head = j >> 2;
    const int arow_limb = j & 3;
    float qv[32];
    float amax = 0.0f;
    const float rot_scale = (BH > 0) ? rsqrtf(static_cast<float>(BH)) : 1.0f;
#pragma unroll
    for (int d = 0; d < 32; ++d) {
        qv[d] = sh.q[wave][arow_head][32 * g + d] * rot_scale;
        amax = fmaxf(amax, fabsf(qv[d]));
    }
    // max over the head's 128 dims: lanes j, j+16, j+32, j+48 hold its 4 quarters
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    int qexp = 0;
    if (amax > 0.0f) (void)frexpf(amax, &qexp);      // amax < 2^qexp
    const float qmul = ldexpf(1.0f, 27 - qexp);
    v4i qa0, qa1;        // A operands: MFMA 0 (even dims), MFMA 1 (odd dims)
    int limb_sum = 0;    // sum over this lane's 32 dims of its limb
    {
        uint32_t w0[4] = {0, 0, 0, 0}, w1[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int X = static_cast<int>(rintf(qv[2 * e + t] * qmul));
                int limb;
                if (arow_limb == 0) limb = X >> 21;
                else limb = (X >> (21 - 7 * arow_limb)) & 127;
                limb_sum += limb;
                const uint32_t byte = static_cast<uint32_t>(limb) & 0xFFu;
                if (t == 0) w0[e >> 2] |= byte << (8 * (e & 3));
                else w1[e >> 2] |= byte << (8 * (e & 3));
            }
        }
        qa0 = v4i{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3]};
        qa1 = v4i{(int)w1[0], (int)w1[1], (int)w1[2], (int)w1[3]};
    }
    // Sum of each row's limbs over all 128 dims (4 lane groups).
    limb_sum += __shfl_xor(limb_sum, 16);
    limb_sum += __shfl_xor(limb_sum, 32);
    // Accumulator init for q.k: lane (g, j) holds rows (head g, limbs 0..3);
    // row (g, r) is A-row 4g + r, whose total sits in lane 4g + r.
    v4i qk_init;
#pragma unroll
    for (int r = 0; r < 4; ++r) qk_init[r] = -8 * __shfl(limb_sum, 4 * g + r);
    // Score scale of head g (this lane's D rows): 2^(E_g - 27) * softmax_scale * log2(e)
    const int qexp_g = __shfl(qexp, 4 * g);
    const float score_mul = ldexpf(a.score_scale, qexp_g - 27);

    // ---- main loop over chunks ----
    float m_run = -INFINITY;     // running max (log2 units) of head g, uniform in row g
    float l_lane = 0.0f;         // this lane's part of the running sum
    float o_acc[8];              // head g, dims 8j + m
#pragma unroll
    for (int m = 0; m < 8; ++m) o_acc[m] = 0.0f;

    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages_per_seq;
    const uint8_t *kpool = static_cast<const uint8_t *>(a.k_pool);
    const uint8_t *vpool = static_cast<const uint8_t *>(a.v_pool);
    const int64_t head_off = (int64_t)hk * a.tile_bytes;
    const int64_t page_stride = (int64_t)a.num_kv_heads * a.tile_bytes;

    for (int c = wave; c < nchunks; c += kWaves) {
        const int T0 = tok_begin + c * kChunk;
        // physical pages of the 4 groups (clamped to a valid page past the end)
        int64_t tile_off[4];
        int slot0[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tok = T0 + 16 * t;
            const int lp = min(tok / P, npages - 1);
            slot0[t] = tok % P;
            const int32_t phys = (int32_t)uniform((uint32_t)pt[lp]);
            tile_off[t] = (int64_t)phys * page_stride + head_off;
        }
        // loads: keys (16 B per lane and group), key and value scales, values
        uint4 kraw[4];
        float ks[4], vs[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t *kt = kpool + tile_off[t];
            const uint8_t *vt = vpool + tile_off[t];
            kraw[t] = *reinterpret_cast<const uint4 *>(kt + (slot0[t] + j) * kCodeBytesPerRow + 16 * g);
            ks[t] = half_to_float(*reinterpret_cast<const uint16_t *>(kt + P * kCodeBytesPerRow + 2 * (slot0[t] + j)));
            vs[t] = half_to_float(*reinterpret_cast<const uint16_t *>(vt + P * kCodeBytesPerRow + 2 * (slot0[t] + j)));
        }
        uint32_t vraw[16];
        {
            // lane (g, j): group g's 16 tokens, dims 8j..8j+7 (dword j of each row)
            int64_t toff = 0;
            int sl = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (g == t) { toff = tile_off[t]; sl = slot0[t]; }
            }
            const uint8_t *vt = vpool + toff + sl * kCodeBytesPerRow + 4 * j;
#pragma unroll
            for (int e = 0; e < 16; ++e) vraw[e] = *reinterpret_cast<const uint32_t *>(vt + e * kCodeBytesPerRow);
        }

        // q.k for the 4 groups: z[t] = score of head g, token 16t + j (log2 units)
        float z[4];
        float zmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t lo[4], hi[4];
            split_offset(kraw[t].x, lo[0], hi[0]);
            split_offset(kraw[t].y, lo[1], hi[1]);
            split_offset(kraw[t].z, lo[2], hi[2]);
            split_offset(kraw[t].w, lo[3], hi[3]);
            v4i d = mfma(qa0, v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]}, qk_init);
            d = mfma(qa1, v4i{(int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}, d);
            const int tok = T0 + 16 * t + j;
            const float sc = limbs_to_float(d) * score_mul * ks[t];
            z[t] = (tok < tok_end) ? sc : -INFINITY;
            zmax = fmaxf(zmax, z[t]);
        }
        // online softmax for head g (row g)
        zmax = row_max16(zmax);
        if (zmax > m_run) {
            const float alpha = exp2f(m_run - zmax);
            l_lane *= alpha;
#pragma unroll
            for (int m = 0; m < 8; ++m) o_acc[m] *= alpha;
            m_run = zmax;
        }
        float pv[4];
        float pmax = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float p = exp2f(z[t] - m_run);          // 0 for masked tokens
            l_lane += p;
            const int tok = T0 + 16 * t + j;
            pv[t] = (tok < tok_end) ? p * vs[t] : 0.0f;   // masked scales may be garbage
            pmax = fmaxf(pmax, pv[t]);
        }
        pmax = row_max16(pmax);
        int pexp = 0;
        if (pmax > 0.0f) (void)frexpf(pmax, &pexp);        // pv < 2^pexp
        const float pmul = ldexpf(1.0f, 27 - pexp);
        const float pback = ldexpf(1.0f, pexp - 27);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t F = static_cast<uint32_t>(fmaf(pv[t], pmul, 0.5f));
            sh.pfix[wave][g][16 * t + j] = F;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A operand of p.v: row (head j/4, limb j%4), tokens of group g
        v4i pa;
        {
            const uint4 *src = reinterpret_cast<const uint4 *>(&sh.pfix[wave][arow_head][16 * g]);
            const int shift = 21 - 7 * arow_limb;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const uint4 f = src[q4];
                const uint32_t b0 = (f.x >> shift) & 127u, b1 = (f.y >> shift) & 127u;
                const uint32_t b2 = (f.z >> shift) & 127u, b3 = (f.w >> shift) & 127u;
                pa[q4] = (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // B operands of p.v: sign-extended value codes, transposed to
        // (dim 8j + m) x (16 tokens of group g)
        uint32_t lo[16], hi[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) split_signed(vraw[e], lo[e], hi[e]);
        // lo[e] bytes: dims 8j+0, +2, +4, +6 of token e; hi[e]: +1, +3, +5, +7
        v4i vb[8];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t t0, t1, t2, t3;
            transpose4(lo[4 * q4], lo[4 * q4 + 1], lo[4 * q4 + 2], lo[4 * q4 + 3], t0, t1, t2, t3);
            vb[0][q4] = (int)t0; vb[2][q4] = (int)t1; vb[4][q4] = (int)t2; vb[6][q4] = (int)t3;
            transpose4(hi[4 * q4], hi[4 * q4 + 1], hi[4 * q4 + 2], hi[4 * q4 + 3], t0, t1, t2, t3);
            vb[1][q4] = (int)t0; vb[3][q4] = (int)t1; vb[5][q4] = (int)t2; vb[7][q4] = (int)t3;
        }
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const v4i d = mfma(pa, vb[m], zero);
            o_acc[m] = fmaf(limbs_to_float(d), pback, o_acc[m]);
        }
    }

    // ---- merge the 4 waves' states of this block ----
    const float l_row = row_sum16(l_lane);
    if (j == 0) {
        sh.mm[wave][g] = m_run;
        sh.ml[wave][g] = l_row;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) sh.mo[wave][g][8 * j + m] = o_acc[m];
    __syncthreads();
    for (int idx = threadIdx.x; idx < kH * kHeadDim; idx += kThreads) {
        const int h = idx / kHeadDim;
        const int d = idx - h * kHeadDim;
        if (h >= nheads) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sh.mm[w][h]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (sh.mm[w][h] == -INFINITY) ? 0.0f : exp2f(sh.mm[w][h] - M);
            acc = fmaf(sh.mo[w][h][d], f, acc);
            lsum = fmaf(sh.ml[w][h], f, lsum);
        }
        const int64_t unit = ((int64_t)b * a.num_q_heads + qh0 + h) * a.num_splits + s;
        a.ws_o[unit * kHeadDim + d] = acc;
        if (d == 0) {
            a.ws_ml[unit * 2 + 0] = M;
            a.ws_ml[unit * 2 + 1] = lsum;
        }
    }
}

}  // namespace

hipError_t launch_decode_int4_mfma(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)a.num_splits, (unsigned)(a.num_kv_heads * a.head_chunks), (unsigned)a.batch);
    const dim3 block(kThreads);
#define KVQ_LAUNCH(BHV, PV) hipLaunchKernelGGL((decode_int4_mfma_kernel<BHV, PV>), grid, block, 0, stream, a)
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
