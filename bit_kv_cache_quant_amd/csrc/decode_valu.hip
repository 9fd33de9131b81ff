// Paged decode attention on the vector ALUs over the fp16 baseline cache:
// split-K partial kernel.  (The INT4 cache has its own matrix-core kernel,
// decode_mfma.hip; this file's earlier INT4 variant was retired.)
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "KVキャッシュこそが本当のボトルネックである理由" (attention reads the
// whole paged cache each decode step; fused attention over paged blocks).  The
// baseline cache holds unrotated fp16 keys and values, so there is no
// rotation here.
//
// Work item: (split s, KV head h and a chunk of up to 4 of its query heads,
// sequence b); 256 threads = 4 waves; wave w walks pages p0+w, p0+w+4, ...
// Inside a wave, each 16-lane row takes one token per step (tokens row,
// row+4, ... of the page); lane l of a row holds dims 8l..8l+7.  Each row
// keeps its own online-softmax state (running max in log2 units, running
// sum, 8 output dims per head); the 16 row states of the block are merged
// through LDS and written as one partial state per (b, query head, split).
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = kThreads / 16;   // 16 token streams per block
constexpr int kH = kHeadsPerChunk;

__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xFFFFu)));
}

// Sum over the 16 lanes of a row; every lane gets the same total.
__device__ __forceinline__ float row_sum16(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ float xor16(float v, int mask) { return __shfl_xor(v, mask, 16); }

__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeArgs a) {
    const int s = blockIdx.x;
    const int hk = blockIdx.y / a.head_chunks;
    const int chunk = blockIdx.y - hk * a.head_chunks;
    const int b = blockIdx.z;
    const int L = a.context_lens[b];
    if (L <= 0) return;
    const int npages = (L + a.page_size - 1) >> a.page_shift;
    const int p0 = s * a.pages_per_split;
    if (p0 >= npages) return;
    const int p1 = min(p0 + a.pages_per_split, npages);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int row = (tid >> 4) & 3;
    const int lane = tid & 15;
    const int qh0 = hk * a.group + chunk * kH;
    const int nheads = min(kH, a.group - chunk * kH);

    // Rotated, pre-scaled query: q'[i][r] for dims 8*lane + r.
    float qr[kH][8];
#pragma unroll
    for (int i = 0; i < kH; ++i) {
        if (i < nheads) {
            const uint4 raw = *reinterpret_cast<const uint4 *>(
                a.q + ((int64_t)b * a.num_q_heads + qh0 + i) * kHeadDim + lane * 8);
            qr[i][0] = half_to_float(raw.x); qr[i][1] = half_to_float(raw.x >> 16);
            qr[i][2] = half_to_float(raw.y); qr[i][3] = half_to_float(raw.y >> 16);
            qr[i][4] = half_to_float(raw.z); qr[i][5] = half_to_float(raw.z >> 16);
            qr[i][6] = half_to_float(raw.w); qr[i][7] = half_to_float(raw.w >> 16);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) qr[i][r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) qr[i][r] *= a.score_scale;
    }

    float m_run[kH], l_run[kH], o[kH][8];
#pragma unroll
    for (int i = 0; i < kH; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; ++r) o[i][r] = 0.0f;
    }

    const int P = a.page_size;
    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages_per_seq;
    for (int p = p0 + wave; p < p1; p += 4) {
        const int64_t phys = pt[p];
        const int ntok = min(P, L - p * P);
        const uint8_t *ktile = static_cast<const uint8_t *>(a.k_pool) + (phys * a.num_kv_heads + hk) * a.tile_bytes;
        const uint8_t *vtile = static_cast<const uint8_t *>(a.v_pool) + (phys * a.num_kv_heads + hk) * a.tile_bytes;
        for (int j = row; j < ntok; j += 4) {
            float kx[8], vx[8];
            const uint4 kr = *reinterpret_cast<const uint4 *>(ktile + ((int64_t)j * kHeadDim + lane * 8) * 2);
            const uint4 vr = *reinterpret_cast<const uint4 *>(vtile + ((int64_t)j * kHeadDim + lane * 8) * 2);
            kx[0] = half_to_float(kr.x); kx[1] = half_to_float(kr.x >> 16);
            kx[2] = half_to_float(kr.y); kx[3] = half_to_float(kr.y >> 16);
            kx[4] = half_to_float(kr.z); kx[5] = half_to_float(kr.z >> 16);
            kx[6] = half_to_float(kr.w); kx[7] = half_to_float(kr.w >> 16);
            vx[0] = half_to_float(vr.x); vx[1] = half_to_float(vr.x >> 16);
            vx[2] = half_to_float(vr.y); vx[3] = half_to_float(vr.y >> 16);
            vx[4] = half_to_float(vr.z); vx[5] = half_to_float(vr.z >> 16);
            vx[6] = half_to_float(vr.w); vx[7] = half_to_float(vr.w >> 16);
#pragma unroll
            for (int i = 0; i < kH; ++i) {
                float dot = 0.0f;
#pragma unroll
                for (int r = 0; r < 8; ++r) dot = fmaf(qr[i][r], kx[r], dot);
                const float z = row_sum16(dot);
                if (z > m_run[i]) {
                    const float alpha = exp2f(m_run[i] - z);
                    l_run[i] *= alpha;
#pragma unroll
                    for (int r = 0; r < 8; ++r) o[i][r] *= alpha;
                    m_run[i] = z;
                }
                const float pw = exp2f(z - m_run[i]);
                l_run[i] += pw;
                #pragma unroll
                for (int r = 0; r < 8; ++r) o[i][r] = fmaf(pw, vx[r], o[i][r]);
            }
        }
    }

    // Merge the 16 row states of the block.
    __shared__ float sh_o[kRows][kH][kHeadDim];
    __shared__ float sh_m[kRows][kH];
    __shared__ float sh_l[kRows][kH];
    const int grow = tid >> 4;
#pragma unroll
    for (int i = 0; i < kH; ++i) {
#pragma unroll
        for (int r = 0; r < 8; ++r) sh_o[grow][i][lane * 8 + r] = o[i][r];
        if (lane == 0) {
            sh_m[grow][i] = m_run[i];
            sh_l[grow][i] = l_run[i];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kH * kHeadDim; idx += kThreads) {
        const int i = idx / kHeadDim;
        const int d = idx - i * kHeadDim;
        if (i >= nheads) continue;
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < kRows; ++g) M = fmaxf(M, sh_m[g][i]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int g = 0; g < kRows; ++g) {
            const float f = exp2f(sh_m[g][i] - M);   // 0 for rows that saw no token
            acc = fmaf(sh_o[g][i][d], f, acc);
            lsum = fmaf(sh_l[g][i], f, lsum);
        }
        const int64_t unit = ((int64_t)b * a.num_q_heads + qh0 + i) * a.num_splits + s;
        a.ws_o[unit * kHeadDim + d] = acc;
        if (d == 0) {
            a.ws_ml[unit * 2 + 0] = M;
            a.ws_ml[unit * 2 + 1] = lsum;
        }
    }
}

dim3 decode_grid(const DecodeArgs &a) {
    return dim3((unsigned)a.num_splits, (unsigned)(a.num_kv_heads * a.head_chunks), (unsigned)a.batch);
}

}  // namespace

hipError_t launch_decode_fp16(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(decode_partial_kernel, decode_grid(a), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace kvq
