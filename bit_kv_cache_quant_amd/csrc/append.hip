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
// Mapping: 16 lanes own one 128-entry vector (one token, one KV head, K or V),
// 8 consecutive entries per lane, loaded with one 16-byte load; 16 vectors per
// 256-thread block, consecutive vectors being consecutive (token, head) rows,
// so a wave reads 1 KiB of contiguous input.  Butterfly spans 1, 2, 4 are done
// inside a lane, spans 8..64 between lanes (lane distance span/8).  Each lane
// then produces exactly one 32-bit word of packed codes (its 8 nibbles), so
// the 16 lanes write the 64 code bytes of the slot with one coalesced store.
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
#pragma clang fp contract(off)

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kLanesPerVec = 16;
constexpr int kVecsPerBlock = 16;
constexpr int kBlockThreads = kLanesPerVec * kVecsPerBlock;

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

template <int BH>
__global__ __launch_bounds__(kBlockThreads) void quant_append_kernel(AppendArgs a) {
    const int lane = threadIdx.x & (kLanesPerVec - 1);
    const int64_t vec = (int64_t)blockIdx.x * kVecsPerBlock + (threadIdx.x / kLanesPerVec);
    const int64_t per_tensor = (int64_t)a.num_tokens * a.num_kv_heads;
    if (vec >= 2 * per_tensor) return;  // the whole 16-lane group leaves together
    const bool is_v = vec >= per_tensor;
    const int64_t row = is_v ? vec - per_tensor : vec;
    const int32_t t = (int32_t)(row / a.num_kv_heads);
    const int32_t h = (int32_t)(row - (int64_t)t * a.num_kv_heads);

    // Issue the address loads first; their latency overlaps the arithmetic.
    const int32_t seq = a.token_seq[t];
    const int32_t pos = a.token_pos[t];
    const int32_t page = a.page_table[(int64_t)seq * a.max_pages_per_seq + (pos >> a.page_shift)];
    const int32_t slot = pos & (a.page_size - 1);

    const uint16_t *src = (is_v ? a.v_new : a.k_new) + row * kHeadDim + lane * 8;
    const uint4 raw = *reinterpret_cast<const uint4 *>(src);

    float y[8];
    y[0] = half_bits_to_float(raw.x);
    y[1] = half_bits_to_float(raw.x >> 16);
    y[2] = half_bits_to_float(raw.y);
    y[3] = half_bits_to_float(raw.y >> 16);
    y[4] = half_bits_to_float(raw.z);
    y[5] = half_bits_to_float(raw.z >> 16);
    y[6] = half_bits_to_float(raw.w);
    y[7] = half_bits_to_float(raw.w >> 16);

    if constexpr (BH > 0) {
        // Spans 1, 2, 4: both entries of a butterfly live in this lane.
#pragma unroll
        for (int span = 1; span < 8; span <<= 1) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (r & span) continue;
                const float u = y[r];
                const float v = y[r + span];
                y[r] = u + v;
                y[r + span] = u - v;
            }
        }
        // Spans 8 .. BH/2: the partner entry sits in lane ^ (span / 8).  The
        // lane holding the lower index keeps u + v, the other keeps u - v,
        // where u is the lower-index entry (the partner's value there).
#pragma unroll
        for (int m = 1; m < BH / 8; m <<= 1) {
            const bool upper = (lane & m) != 0;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float p = xor_lane16(y[r], m);
                y[r] = upper ? (p - y[r]) : (y[r] + p);
            }
        }
        const float c = inv_sqrt_block<BH>();
#pragma unroll
        for (int r = 0; r < 8; ++r) y[r] = y[r] * c;
    }

    // Token-wise absmax over the 128 entries (exact).
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(y[r]));
#pragma unroll
    for (int k = 1; k < kLanesPerVec; k <<= 1) m = fmaxf(m, xor_lane16(m, k));

    const float s32 = m / 7.0f;                       // IEEE division
    const _Float16 s16 = static_cast<_Float16>(s32);  // round to nearest even
    const float s = static_cast<float>(s16);
    float sd = s;
    float rcp = 0.0f;
    if (s > 0.0f && s <= 65504.0f) {
        rcp = 1.0f / s;                               // correctly rounded
    } else {
        sd = 0.0f;                                    // zero scale: every code is 0
    }

    uint32_t word = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float q0 = y[r] * rcp;
        const float e = __builtin_fmaf(-q0, sd, y[r]);
        const float q = __builtin_fmaf(e, rcp, q0);  // == y / s (see header)
        // Clamping to integer bounds commutes with rounding to an integer.
        const float qc = fminf(fmaxf(q, -8.0f), 7.0f);
        const int code = static_cast<int>(rintf(qc));
        word |= (static_cast<uint32_t>(code) & 0xFu) << (4 * r);
    }

    uint8_t *pool = static_cast<uint8_t *>(is_v ? a.v_pool : a.k_pool);
    uint8_t *tile = pool + ((int64_t)page * a.num_kv_heads + h) * a.tile_bytes;
    *reinterpret_cast<uint32_t *>(tile + slot * kCodeBytesPerRow + lane * 4) = word;
    if (lane == 0) {
        *reinterpret_cast<uint16_t *>(tile + a.page_size * kCodeBytesPerRow + 2 * slot) =
            __builtin_bit_cast(uint16_t, s16);
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
    *reinterpret_cast<uint4 *>(dst) = raw;
}

dim3 grid_for(const AppendArgs &a) {
    const int64_t vecs = 2 * (int64_t)a.num_tokens * a.num_kv_heads;
    return dim3((unsigned)((vecs + kVecsPerBlock - 1) / kVecsPerBlock));
}

}  // namespace

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream) {
    const dim3 grid = grid_for(a);
    switch (a.had_block) {
        case 0: hipLaunchKernelGGL(quant_append_kernel<0>, grid, dim3(kBlockThreads), 0, stream, a); break;
        case 32: hipLaunchKernelGGL(quant_append_kernel<32>, grid, dim3(kBlockThreads), 0, stream, a); break;
        case 64: hipLaunchKernelGGL(quant_append_kernel<64>, grid, dim3(kBlockThreads), 0, stream, a); break;
        case 128: hipLaunchKernelGGL(quant_append_kernel<128>, grid, dim3(kBlockThreads), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_append_fp16(const AppendArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(append_fp16_kernel, grid_for(a), dim3(kBlockThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
