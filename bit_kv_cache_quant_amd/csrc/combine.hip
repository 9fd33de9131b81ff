// Split-K merge of partial softmax states and inverse rotation of the output.
//
// Method source: "KVキャッシュを4ビットへ — SAW-INT4とシステムを踏まえたINT4量子化",
// section "回転のトリック — ブロック対角アダマール": the rotation R = H/sqrt(Bh)
// is orthogonal and its own inverse, so the attention output computed in the
// rotated basis is brought back by applying R once more.  That is done after
// the merge, since merging (a weighted sum) commutes with R.
//
// One 64-thread block per (sequence, query head); thread t owns dims t and
// t + 64.  Partial state of split s: running max M_s (log2 units), running sum
// l_s, unnormalised output o_s.  Merge: M = max M_s, l = sum l_s 2^(M_s - M),
// o = sum o_s 2^(M_s - M) / l.
#include "kvq_internal.h"

namespace kvq {
namespace {

__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a, int rotate_back) {
    const int unit = blockIdx.x;                 // b * num_q_heads + qh
    const int b = unit / a.num_q_heads;
    const int t = threadIdx.x;
    float *out = a.out + (int64_t)unit * kHeadDim;
    const int L = a.context_lens[b];
    if (L <= 0) {
        out[t] = 0.0f;
        out[t + 64] = 0.0f;
        return;
    }
    const int npages = (L + a.page_size - 1) >> a.page_shift;
    const int nsplit = (npages + a.pages_per_split - 1) / a.pages_per_split;
    const float *ml = a.ws_ml + (int64_t)unit * a.num_splits * 2;
    const float *po = a.ws_o + (int64_t)unit * a.num_splits * kHeadDim;

    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
    float lsum = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int s = 0; s < nsplit; ++s) {
        const float f = exp2f(ml[2 * s] - M);
        lsum = fmaf(ml[2 * s + 1], f, lsum);
        o0 = fmaf(po[(int64_t)s * kHeadDim + t], f, o0);
        o1 = fmaf(po[(int64_t)s * kHeadDim + t + 64], f, o1);
    }
    const float inv = 1.0f / lsum;
    __shared__ float x[kHeadDim];
    x[t] = o0 * inv;
    x[t + 64] = o1 * inv;
    const int bh = rotate_back ? a.had_block : 0;
    if (bh > 0) {
        __syncthreads();
        for (int span = 1; span < bh; span <<= 1) {
            // butterfly number t: lower index i has bit `span` clear
            const int i = ((t / span) * 2 * span) + (t % span);
            const float u = x[i], v = x[i + span];
            __syncthreads();
            x[i] = u + v;
            x[i + span] = u - v;
            __syncthreads();
        }
        const float c = rsqrtf(static_cast<float>(bh));
        out[t] = x[t] * c;
        out[t + 64] = x[t + 64] * c;
    } else {
        out[t] = x[t];
        out[t + 64] = x[t + 64];
    }
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, bool rotate_back, hipStream_t stream) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(a.batch * a.num_q_heads)), dim3(64), 0, stream,
                       a, rotate_back ? 1 : 0);
    return hipGetLastError();
}

}  // namespace kvq
