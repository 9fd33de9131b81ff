// Internal launch interface between the C ABI (kvq_api.hip) and the kernels.
// Not installed; the public interface is include/kvq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;          // the only supported head dimension
constexpr int kCodeBytesPerRow = kHeadDim / 2;
constexpr int kHeadsPerChunk = 4;      // query heads handled together per KV head
constexpr int kChunkTokens = 64;       // decode processes tokens in chunks of 64
constexpr int kMaxSplitTokens = 2048;  // longest page range one decode wave takes (split mode)
constexpr int kMaxScanBatch = 4096;    // balanced decode: largest batch one block scans
constexpr int kMaxRangeChunks = 64;    // balanced decode: longest work range, in chunks
constexpr int KVQ_FMT_INT4 = 0;        // quantizer formats (KVQ_FORMAT_* in include/kvq.h)
constexpr int KVQ_FMT_MXFP4 = 1;

struct AppendArgs {
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *token_seq;
    const int32_t *token_pos;
    const int32_t *page_table;
    void *k_pool;
    void *v_pool;
    int64_t tile_bytes;        // INT4: bytes per (page, head) tile; fp16: P*D*2
    int32_t num_tokens;
    int32_t max_pages_per_seq;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t page_shift;        // log2(page_size)
    int32_t had_block;
    // Quantizer variant (kv_quant_append_cfg): KVQ_FORMAT_*, channels per
    // scale, scale search, and the sign mask applied before the rotation
    // (bit i: channel i negated).  The plain method is INT4, 128, 0, no signs.
    int32_t format;
    int32_t scale_group;
    int32_t scale_search;
    uint32_t sign_mask[4];
};

struct DecodeArgs {
    const uint16_t *q;
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    const int32_t *context_lens;
    float *out;
    float *ws_o;               // [batch][num_q_heads][num_splits][kHeadDim]
    float *ws_ml;              // [batch][num_q_heads][num_splits][2]  (max in log2 units, sum)
    int64_t tile_bytes;
    int32_t max_pages_per_seq;
    int32_t max_context_len;   // every context length read is clamped to this
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;             // num_q_heads / num_kv_heads
    int32_t head_chunks;       // ceil(group / kHeadsPerChunk)
    int32_t page_size;
    int32_t page_shift;
    int32_t had_block;
    int32_t pages_per_split;
    int32_t num_splits;
    int32_t range_waves;       // split mode: waves sharing one page range in a block (1, 2 or 4)
    float score_scale;         // softmax_scale * log2(e): scores are kept in log2 units
    // Quantizer variant of the cache: KVQ_FMT_*, channels per scale, and the
    // sign mask of the randomized Hadamard (bit i: channel i negated before
    // the rotation; the query gets it too, the output gets it back).
    int32_t format;
    int32_t scale_group;
    uint32_t sign_mask[4];
    // Balanced decode (sk_groups > 0): the concatenated chunk list of all
    // sequences is cut into equal ranges, one per block group; partial states
    // are indexed by (head quad, range + sequence, wave, head).
    int32_t *sk_prefix;        // [batch + 1] chunk prefix sums (written by the partial kernel)
    int32_t sk_groups;         // block groups launched per head quad (0: split mode)
    int32_t sk_min;            // block groups wanted for parallelism
    int32_t sk_target;         // most block groups wanted
    int32_t quads;             // head quads (groups of kHeadsPerChunk head slots) per sequence
    // Fused decode step (k_new != nullptr): sequence b's last context token
    // (position context_lens[b] - 1) arrives here as fp16 K/V rows
    // [batch][num_kv_heads][kHeadDim].  The partial kernel then covers the
    // positions before it (len_offset = 1), and the merge kernel quantizes
    // the new rows into the cache and folds them into the output.
    const uint16_t *k_new;
    const uint16_t *v_new;
    int32_t len_offset;        // 0, or 1 in the fused step
    // Merge-kernel shortcuts set by the host: log2(group) when group is a
    // power of two (else -1), and whether the balanced schedule's range
    // arithmetic ((chunk + 1) * groups) fits 31 bits (32-bit divisions).
    int32_t group_shift;
    int32_t sk_div32;
};

// Number of ranges the balanced decode cuts `tot` chunks into: ranges of
// about kPreferredRangeChunks (few partial states to write and merge), but at
// least gmin ranges (parallelism) and at most gmax, never a range longer than
// kMaxRangeChunks, never an empty one.  Monotonic in tot.
constexpr int kPreferredRangeChunks = 32;
__host__ __device__ inline int32_t balanced_groups(int32_t gmin, int32_t gmax, int32_t tot) {
    int32_t g = (tot + kPreferredRangeChunks - 1) / kPreferredRangeChunks;
    if (g < gmin) g = gmin;
    if (g > gmax) g = gmax;
    const int32_t gcap = (tot + kMaxRangeChunks - 1) / kMaxRangeChunks;
    if (g < gcap) g = gcap;
    if (g > tot) g = tot;
    return g < 1 ? 1 : g;
}

// Causal prefill attention over the INT4 cache: query row i of sequence b
// (rows q_start[b] .. q_start[b + 1] - 1, the last q_len_b positions of its
// context) attends to the cached tokens 0 .. context_lens[b] - q_len_b + i.
struct PrefillArgs {
    const uint16_t *q;         // fp16 [num_q][num_q_heads][kHeadDim]
    const int32_t *q_start;    // [batch + 1]
    const void *k_pool;
    const void *v_pool;
    const int32_t *page_table;
    const int32_t *context_lens;
    float *out;                // fp32 [num_q][num_q_heads][kHeadDim]
    int64_t tile_bytes;
    int32_t max_pages_per_seq;
    int32_t batch;
    int32_t num_q;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t head_chunks;
    int32_t page_size;
    int32_t had_block;
    float score_scale;         // softmax_scale * log2(e)
};

// Context length of sequence b as the kernels use it: context_lens[b]
// clamped to the largest length the caller sized the page table and the
// workspace for, so a length past that contract can give a wrong row but
// never an access outside the buffers.
__device__ __forceinline__ int32_t full_len(const DecodeArgs &a, int b) {
    return min(a.context_lens[b], a.max_context_len);
}
// Tokens the partial kernels read from the cache: all of them, or (fused
// step) all but the new last one.
__device__ __forceinline__ int32_t decode_len(const DecodeArgs &a, int b) {
    return full_len(a, b) - a.len_offset;
}
__device__ __forceinline__ int32_t prefill_len(const PrefillArgs &a, int b) {
    return min(a.context_lens[b], a.max_pages_per_seq * a.page_size);
}

hipError_t launch_quant_append(const AppendArgs &a, hipStream_t stream);
hipError_t launch_prefill_int4(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_append_fp16(const AppendArgs &a, hipStream_t stream);
hipError_t launch_decode_int4_mfma(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_fp16(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_grouped(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_combine(const DecodeArgs &a, bool rotate_back, hipStream_t stream);

}  // namespace kvq
