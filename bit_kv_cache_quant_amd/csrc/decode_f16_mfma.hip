// Paged decode attention over the fp16 baseline cache on the fp16 matrix
// cores (v_mfma_f32_16x16x32_f16): split-K partial kernel.
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "KVキャッシュこそが本当のボトルネックである理由" (every decode step
// streams the whole paged cache, with fused attention over the paged blocks).
// The baseline cache holds unrotated fp16 keys and values, so there is no
// rotation here; the work schedule (balanced ranges over the batch, or even
// splits per sequence), the partial-state layout and the merge are those of
// the INT4 kernel, so one merge kernel serves both.
//
// Per (token, KV head) this cache is 512 bytes against 132 for INT4, and the
// four query heads of a GQA group need the same 2 x 512 multiply-adds: on the
// matrix cores that is a few percent of their rate at the HBM roofline.
//
// Layout of one wave (64 lanes, g = lane / 16, j = lane % 16), per step of 32
// tokens (token groups tg = 0, 1 of 16):
//   q.k  A (query): row j = (head j/4, quarter j%4); the lanes of k-group g
//        hold dims 32s + 8g .. 32s + 8g + 7 of MFMA s (s < 4) for rows whose
//        quarter is g, zero otherwise.  B (keys): column j = token 16 tg + j,
//        the same dims, one 16-byte load per lane and MFMA.  So row
//        (head h, quarter u) of the result is the dot product over the dims
//        {32 s + 8 u + e}; lane (g, j) holds the four quarters of head g for
//        token j, and their sum is the score: every lane holds one
//        (head, token) score, and the rows of head g are the lanes where its
//        output accumulates below (the online-softmax rescale is lane-local).
//   p.v  A (weights): row j = (head j/4, quarter j%4), k-group g = tokens
//        8g .. 8g + 7, nonzero only where the quarter is g; the fp32 weight p
//        is split into fp16 hi + lo (p - hi), two MFMAs per output tile, so
//        the products keep ~22 bits.  B (values): column j = dim 16 nt + j of
//        output tile nt, k = the 8 tokens of group g, read transposed from
//        LDS.  Rows (head g, quarter u) of the result accumulate across the
//        range and are summed at its end.
//   Values go from HBM straight to LDS (global_load_lds_dwordx4, 1 KiB per
//   instruction, lane l's 16 bytes at 16 l), token row T's 16-byte piece p at
//   slot 16 T + (p ^ 2 ((T & 3) | ((T >> 3 & 1) << 2))).  gfx950's transposed
//   16-bit LDS read (ds_read_b64_tr_b16: in each group of 16 lanes, lane i's
//   element e is element i & 3 of the word lane 4 e + i / 4 points at) then
//   hands lane (g, j) dim 16 nt + j of 4 consecutive tokens, and each pass of
//   32 lanes covers all 64 banks once.
//   Pipelining: a step first reads its values back from LDS, then issues the
//   next step's value loads into the same buffer, and its keys into
//   registers once this step's keys have been used.
#include <type_traits>

#include "decode_common.h"

namespace kvq {
namespace {

using namespace dec;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kStep = 32;                    // tokens per compute step
constexpr int kRowBytes = kHeadDim * 2;      // 256 bytes per token row
static_assert(kChunkTokens % kStep == 0, "a schedule chunk is a whole number of steps");

// LDS of one wave: one step's values (32 rows of 256 bytes), and the fp16
// hi / lo parts of the step's weights (head, token).
struct alignas(16) F16Values {
    uint8_t vbuf[kStep * kRowBytes];
};
struct alignas(16) F16Weights {
    _Float16 hi[kH][kStep];
    _Float16 lo[kH][kStep];
};

__device__ __forceinline__ v4f mfma(v8h a, v8h b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v8h as_v8h(uint4 u) { return __builtin_bit_cast(v8h, u); }

// One work range: tokens [p0 P, min(p1 P, L)) of sequence b (p0 on a
// schedule-chunk boundary) for head slot (KV head hk, query-head chunk
// chunk_id); returns its partial softmax state.
template <int P>
__device__ __forceinline__ PartialState f16_range(const DecodeArgs &a, F16Values &sv, F16Weights &sw, const int lane,
                                                  const int b, const int hk, const int chunk_id, const int L,
                                                  const int p0, const int p1) {
    static_assert(P == 16 || P == 32, "page size");
    const int g = lane >> 4;
    const int j = lane & 15;
    const int qh0 = hk * a.group + chunk_id * kH;
    const int nheads = min(kH, a.group - chunk_id * kH);

    // Query operands (from a valid head always; dead rows are zeroed).
    const int qh = j >> 2;
    const bool qlive = (g == (j & 3)) && (qh < nheads);
    const uint16_t *qsrc = a.q + ((int64_t)b * a.num_q_heads + qh0 + min(qh, nheads - 1)) * kHeadDim + 8 * g;
    uint4 qraw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const uint4 *>(qsrc + 32 * s);

    const int64_t tile_bytes = a.tile_bytes;                       // P * 256
    const uint32_t page_stride = (uint32_t)(a.num_kv_heads * tile_bytes);
    const uint8_t *kbase = static_cast<const uint8_t *>(a.k_pool) + hk * tile_bytes;
    const uint8_t *vbase = static_cast<const uint8_t *>(a.v_pool) + hk * tile_bytes;
    const int last_rel = p1 - 1 - p0;
    const __attribute__((address_space(4))) int32_t *pages =
        (const __attribute__((address_space(4))) int32_t *)(a.page_table + (int64_t)b * a.max_pages_per_seq + p0);
    // Physical pages of the two 16-token groups of step c (clamped to the
    // range's last page past its end: those tokens are masked).
    struct PageSet { int32_t p[2]; };
    auto fetch_pages = [&](int c) {
        PageSet ps;
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) ps.p[tg] = pages[min((kStep * c + 16 * tg) / P, last_rel)];
        return ps;
    };
    struct StepAddrs { const uint8_t *k[2], *v[2]; };   // row 16 tg of the step
    auto addrs = [&](const PageSet &ps, StepAddrs &sa) {
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
            const int64_t row0 = ((16 * tg) % P) * kRowBytes;
            sa.k[tg] = kbase + (uint64_t)(uint32_t)ps.p[tg] * page_stride + row0;
            sa.v[tg] = vbase + (uint64_t)(uint32_t)ps.p[tg] * page_stride + row0;
        }
    };
    // Lane offsets: keys (token j of a group, dims 32 s + 8 g: +64 s); values
    // (DMA instruction i of a group: row i * 4 + g, piece j ^ f, with f's high
    // bit set for instructions 2, 3 of each group, i.e. rows 8..15).
    // (Opaque copies are taken where they are used, so that the compiler
    // keeps each address as a scalar tile base plus this 32-bit offset.)
    const uint32_t koff = j * kRowBytes + 16 * g;
    const uint32_t voff0 = g * kRowBytes + 16 * (j ^ (2 * g));
    const uint32_t voff1 = g * kRowBytes + 16 * (j ^ (2 * g + 8));

    const int tok_begin = p0 * P;
    const int tok_end = min(p1 * P, L);
    const int nsteps = (tok_end - tok_begin + kStep - 1) / kStep;
    const int nfull = (tok_end - tok_begin) / kStep;

    auto load_v = [&](const StepAddrs &sa) {
        // rows 4 i' .. 4 i' + 3 of a group (i' = i & 3): offset 1024 i' in the
        // lane offset, so that the tile base stays the scalar operand
        uint32_t off[4] = {voff0, voff0 + 1024, voff1 + 2048, voff1 + 3072};
        asm("" : "+v"(off[0]), "+v"(off[1]), "+v"(off[2]), "+v"(off[3]));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tg = i >> 2;
            __builtin_amdgcn_global_load_lds((const void *)(sa.v[tg] + off[i & 3]),
                                             (__attribute__((address_space(3))) void *)&sv.vbuf[1024 * i], 16, 0,
                                             /*nt*/ 2);
        }
    };
    auto load_k = [&](const StepAddrs &sa, uint4 (&kr)[2][4]) {
        uint32_t ko = koff;
        asm("" : "+v"(ko));
#pragma unroll
        for (int tg = 0; tg < 2; ++tg)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kr[tg][s] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                                          reinterpret_cast<const v4u *>(sa.k[tg] + ko + 64 * s)));
    };

    uint4 kr[2][4];
    PageSet pages_next;
    if (nsteps > 0) {
        StepAddrs sa;
        addrs(fetch_pages(0), sa);
        pages_next = fetch_pages(1);
        asm volatile("" ::"v"(qraw[0].x), "v"(qraw[1].x), "v"(qraw[2].x), "v"(qraw[3].x));
        load_v(sa);
        load_k(sa, kr);
    }
    v8h qa[4];
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = as_v8h(qlive ? qraw[s] : zero4);

    // Transposed-read addresses: row T = 8 g + j / 4 (+4 for the second
    // read), piece 2 (nt ^ w) + (j & 3) / 2 with w = (j / 4) | ((g & 1) << 2).
    const int tw = (j >> 2) | ((g & 1) << 2);
    const uint32_t tr_row = (8 * g + (j >> 2)) * kRowBytes + 8 * (j & 3);

    v4f acc[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;
    float l_lane = 0.0f;

    auto step = [&](int c, auto tail, auto pf) {
        constexpr bool TAIL = decltype(tail)::value;
        constexpr bool PF = decltype(pf)::value;
        const int T0 = tok_begin + kStep * c;
        // This step's values were loaded into the buffer by DMA (counted by
        // the vector-memory counter): wait for them explicitly.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        v8h vb[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const uint32_t addr = tr_row + 32 * (nt ^ tw);
            const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s *)&sv.vbuf[addr]);
            const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s *)&sv.vbuf[addr + 4 * kRowBytes]);
            vb[nt] = __builtin_bit_cast(v8h, make_uint4(__builtin_bit_cast(uint2, r0).x, __builtin_bit_cast(uint2, r0).y,
                                                        __builtin_bit_cast(uint2, r1).x, __builtin_bit_cast(uint2, r1).y));
        }
        StepAddrs sa;   // step c + 1
        if constexpr (PF) {
            addrs(pages_next, sa);
            pages_next = fetch_pages(c + 2);
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the reads above are done
            load_v(sa);
        }

        // q.k: score of head g, token 16 tg + j (log2 units)
        float z[2];
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
            v4f d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) d = mfma(qa[s], as_v8h(kr[tg][s]), d);
            const float sc = ((d[0] + d[1]) + (d[2] + d[3])) * a.score_scale;
            z[tg] = (!TAIL || T0 + 16 * tg + j < tok_end) ? sc : -INFINITY;
        }
        if constexpr (PF) load_k(sa, kr);   // this step's keys are used
        const float zmax = row_max16(fmaxf(z[0], z[1]));
        if (zmax > m_run) {
            const float alpha = fast_exp2(m_run - zmax);
            l_lane *= alpha;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[nt] *= alpha;
            m_run = zmax;
        }
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
            const float p = fast_exp2(z[tg] - m_run);   // 0 for masked tokens
            l_lane += p;
            const _Float16 hi = static_cast<_Float16>(p);
            const _Float16 lo = static_cast<_Float16>(p - static_cast<float>(hi));
            sw.hi[g][16 * tg + j] = hi;
            sw.lo[g][16 * tg + j] = lo;
        }
        wave_lds_sync();
        const bool plive = g == (j & 3);
        const uint4 phi = *reinterpret_cast<const uint4 *>(&sw.hi[j >> 2][8 * g]);
        const uint4 plo = *reinterpret_cast<const uint4 *>(&sw.lo[j >> 2][8 * g]);
        wave_lds_sync();
        const v8h pa_hi = as_v8h(plive ? phi : zero4);
        const v8h pa_lo = as_v8h(plive ? plo : zero4);
        if constexpr (TAIL) {
            // masked tokens have p = 0, but their cache bytes may be anything
            // (an fp16 NaN or infinity would poison the products)
            const int nvalid = tok_end - T0;
            uint32_t mk[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int t0 = 8 * g + 2 * w;
                mk[w] = (t0 < nvalid ? 0x0000FFFFu : 0u) | (t0 + 1 < nvalid ? 0xFFFF0000u : 0u);
            }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                uint4 u = __builtin_bit_cast(uint4, vb[nt]);
                u.x &= mk[0]; u.y &= mk[1]; u.z &= mk[2]; u.w &= mk[3];
                vb[nt] = as_v8h(u);
            }
        }
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            acc[nt] = mfma(pa_hi, vb[nt], acc[nt]);
            acc[nt] = mfma(pa_lo, vb[nt], acc[nt]);
        }
    };

    int c = 0;
    for (; c + 1 < nsteps; ++c) step(c, std::false_type{}, std::true_type{});
    if (c < nfull) step(c, std::false_type{}, std::false_type{});
    else if (c < nsteps) step(c, std::true_type{}, std::false_type{});

    PartialState st;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.o[nt] = (acc[nt][0] + acc[nt][1]) + (acc[nt][2] + acc[nt][3]);
    st.m = m_run;
    st.l = row_sum16(l_lane);
    return st;
}

// Split mode: one page range of one sequence per wave (dec::split_item).
template <int P>
__global__ __launch_bounds__(kThreads) void decode_f16_mfma_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const SplitItem it = split_item<P>(a, wave);
    if (!it.live) return;
    __shared__ F16Values values[kWaves];
    __shared__ F16Weights weights[kWaves];
    const int qh0 = it.hk * a.group + it.chunk_id * kH;
    const PartialState st = f16_range<P>(a, values[wave], weights[wave], lane, it.b, it.hk, it.chunk_id, it.L,
                                         it.p0, it.p1);
    write_partial(a, st, lane, min(kH, a.group - it.chunk_id * kH),
                  ((int64_t)it.b * a.num_q_heads + qh0) * a.num_splits + it.s, a.num_splits);
}

// Balanced mode (batch 16..4096): equal ranges of the batch's concatenated
// chunks (dec::balanced_range); the block walks every sequence its range
// meets and writes one partial state per (sequence, head).
template <int P>
__global__ __launch_bounds__(kThreads) void decode_f16_balanced_kernel(DecodeArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int B = a.batch;
    union Shared {
        ScanSpace scan;
        F16Values waves[kWaves];
    };
    __shared__ Shared sm;
    __shared__ F16Weights weights[kWaves];

    const BlockRange r = balanced_range(a, sm.scan, wave, lane);
    if (r.tot == 0 || r.gi >= r.G) return;
    const int qd = r.qd, gi = r.gi, start = r.start, end = r.end, b0 = r.b0, pb0 = r.pb0;

    const int head_slots = a.num_kv_heads * a.head_chunks;
    const int slot = qd * kWaves + wave;
    if (slot >= head_slots) return;
    const int hk = slot / a.head_chunks;
    const int chunk_id = slot - hk * a.head_chunks;
    constexpr int kChunkPages = kChunkTokens / P;
    const int nheads = min(kH, a.group - chunk_id * kH);
    const int64_t per_head = (int64_t)a.sk_groups + B;
    const int64_t unit_base = ((int64_t)(qd * kWaves + wave) * kH) * per_head + gi;
    int pb = pb0;
    for (int b = b0; b < B && pb < end; ++b) {
        const int L = decode_len(a, b);
        const int nch = L > 0 ? (L + kChunkTokens - 1) / kChunkTokens : 0;
        const int pb1 = pb + nch;
        const int c0 = max(start, pb) - pb;
        const int c1 = min(end, pb1) - pb;
        if (c0 < c1) {
            const int npages = (L + P - 1) / P;
            const PartialState st = f16_range<P>(a, sm.waves[wave], weights[wave], lane, b, hk, chunk_id, L,
                                                 c0 * kChunkPages, min(c1 * kChunkPages, npages));
            write_partial(a, st, lane, nheads, unit_base + b, per_head);
        }
        pb = pb1;
    }
}

}  // namespace

hipError_t launch_decode_fp16(const DecodeArgs &a, hipStream_t stream) {
    const int quads = (a.num_kv_heads * a.head_chunks + kWaves - 1) / kWaves;
    const bool balanced = a.sk_groups > 0;
    const dim3 grid = balanced ? dim3((unsigned)(quads * a.sk_groups), 1, 1)
                               : dim3((unsigned)(a.batch * quads), (unsigned)a.num_splits, 1);
    const dim3 block(kThreads);
    if (a.page_size == 16) {
        if (balanced) hipLaunchKernelGGL(decode_f16_balanced_kernel<16>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(decode_f16_mfma_kernel<16>, grid, block, 0, stream, a);
    } else if (a.page_size == 32) {
        if (balanced) hipLaunchKernelGGL(decode_f16_balanced_kernel<32>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(decode_f16_mfma_kernel<32>, grid, block, 0, stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kvq
