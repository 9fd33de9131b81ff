// C ABI of the INT4 KV-cache library: argument validation, split choice and
// kernel launches.  The contract of every entry point is documented in
// include/kvq.h.
#include <cmath>
#include <mutex>
#include <stdlib.h>
#include <string.h>

#include "../../include/kvq.h"
#include "kvq_internal.h"

// Static split-K scratch of paged_decode_attn_int4_noalloc (one copy per
// GPU, held until the process ends).  Host code never uses this name as an
// address: kernels get the device address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[KVQ_SCRATCH_BYTES];

namespace {

using kvq::kHeadDim;

// Device address of the current GPU's scratch, looked up once per GPU (with
// that GPU current) and kept; nullptr if the runtime lookup fails.
constexpr int kMaxDevices = 64;
void *scratch_of_current_device() {
    static std::mutex mu;
    static void *ptrs[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}

static_assert(kvq::KVQ_FMT_INT4 == KVQ_FORMAT_INT4 && kvq::KVQ_FMT_MXFP4 == KVQ_FORMAT_MXFP4, "format codes");

bool valid_page_size(int32_t p) { return p == 16 || p == 32; }
bool valid_had_block(int32_t bh) { return bh == 0 || bh == 32 || bh == 64 || bh == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int log2i(int32_t v) { int s = 0; while ((1 << s) < v) ++s; return s; }

bool valid_cfg(const kvq_quant_config *c) {
    if (!c || !valid_had_block(c->had_block)) return false;
    if (c->format == KVQ_FORMAT_INT4)
        return (c->scale_group == 32 || c->scale_group == 64 || c->scale_group == 128) &&
               (c->scale_search == 0 || c->scale_search == 1);
    if (c->format == KVQ_FORMAT_MXFP4) return c->scale_group == 32 && c->scale_search == 0;
    return false;
}

bool grouped_cfg(const kvq_quant_config *c) {
    return c && (c->format != KVQ_FORMAT_INT4 || c->scale_group != kHeadDim);
}

size_t scale_bytes_cfg(const kvq_quant_config *c) {
    return (size_t)(kHeadDim / c->scale_group) * (c->format == KVQ_FORMAT_MXFP4 ? 1 : 2);
}

// Split-K choice shared by the workspace query and the decode calls.  One
// split is one wave's work item.  Aim for about 2048 of them (two per SIMD)
// when the batch alone does not provide that many; a split is a whole number
// of 64-token chunks and at most 2048 tokens (a wave holds its range's
// page-table entries in two registers, one entry per lane each).  Splits are
// not made shorter than needed: each one writes a partial result, and those
// writes, interleaved with the cache reads, cost far more read bandwidth
// than their size.  A caller's pages_per_split is rounded and capped the
// same way.
constexpr int64_t kSplitItems = 1024;

void choose_split(int32_t batch, int32_t num_kv_heads, int32_t head_chunks, int32_t max_context_len,
                  int32_t page_size, int32_t pages_per_split, int32_t *pps, int32_t *nsplit) {
    const int32_t npages = max_context_len > 0 ? (max_context_len + page_size - 1) / page_size : 1;
    int32_t p = pages_per_split;
    if (p <= 0) {
        // about 1024 work items (one wave each) over the GPU: with more, the
        // ranges get so short (batch 1, 32K context: 2 chunks at 2048 items)
        // that per-range set-up and the merge of the extra partial states cost
        // more than the parallelism gains (measured 18.4 -> 16.6 us per layer)
        const int64_t items = (int64_t)batch * num_kv_heads * head_chunks;
        const int64_t want = items >= kSplitItems ? 1 : (kSplitItems + items - 1) / items;
        p = (int32_t)((npages + want - 1) / want);
    }
    const int32_t cap = kvq::kMaxSplitTokens / page_size;
    if (p > cap) p = cap;
    if (p < 1) p = 1;
    const int32_t chunk_pages = kvq::kChunkTokens / page_size;
    p = ((p + chunk_pages - 1) / chunk_pages) * chunk_pages;
    *pps = p;
    *nsplit = (npages + p - 1) / p;
}

int32_t head_chunks_of(int32_t num_q_heads, int32_t num_kv_heads) {
    const int32_t group = num_q_heads / num_kv_heads;
    return (group + kvq::kHeadsPerChunk - 1) / kvq::kHeadsPerChunk;
}

size_t workspace_bytes_for(int32_t batch, int32_t num_q_heads, int32_t nsplit) {
    return (size_t)batch * num_q_heads * nsplit * (kHeadDim + 2) * sizeof(float);
}

// Balanced decode plan (batch <= kMaxScanBatch).  The chunk total is
// only known on the device; tot_max = batch * ceil(max_context_len / 64)
// bounds it, and the launch has enough block groups for any total up to it.
// Default: between 512 and 1024 blocks over all head quads (two to four per
// CU), ranges of about 32 chunks in between.  A caller's pages_per_split
// fixes the number of ranges so that a range holds about that many pages.
constexpr int32_t kBalancedMinBatch = 16;

struct BalancedPlan {
    int32_t quads = 0, gmin = 0, gmax = 0, groups = 0;
    size_t partial_units = 0;   // partial states in the workspace
};

bool balanced_plan(int32_t batch, int32_t num_kv_heads, int32_t head_chunks, int32_t max_context_len,
                   int32_t page_size, int32_t pages_per_split, BalancedPlan *pl) {
    // Few sequences: the split mode already cuts each into equal ranges
    // (mostly full-length ones), without the scan, the range lookup in the
    // merge and the balanced kernel's larger register footprint (measured:
    // 3% slower at batch 8 x 131,072, 8% at batch 1 x 32,768).
    if (batch < kBalancedMinBatch || batch > kvq::kMaxScanBatch) return false;
    const int64_t heads_per_quad = (int64_t)kvq::kHeadsPerChunk * 4;   // 4 waves x 4 query heads
    const int64_t quads = ((int64_t)num_kv_heads * head_chunks + 3) / 4;
    int64_t tot_max = (int64_t)batch * ((max_context_len + kvq::kChunkTokens - 1) / kvq::kChunkTokens);
    if (tot_max < 1) tot_max = 1;
    if (tot_max >= (1ll << 30)) return false;
    int64_t gmin, gmax;
    if (pages_per_split <= 0) {
        gmax = 1024 / quads;
        if (gmax < 1) gmax = 1;
        gmin = gmax / 2;
        if (gmin < 1) gmin = 1;
    } else {
        int64_t cpr = ((int64_t)pages_per_split * page_size + kvq::kChunkTokens - 1) / kvq::kChunkTokens;
        if (cpr < 1) cpr = 1;
        gmax = gmin = (tot_max + cpr - 1) / cpr;
    }
    if (gmax > (1 << 24)) gmax = gmin = 1 << 24;
    const int64_t groups = kvq::balanced_groups((int32_t)gmin, (int32_t)gmax, (int32_t)tot_max);
    if (groups * quads > (1ll << 31) - 1) return false;
    pl->quads = (int32_t)quads;
    pl->gmin = (int32_t)gmin;
    pl->gmax = (int32_t)gmax;
    pl->groups = (int32_t)groups;
    pl->partial_units = (size_t)quads * (size_t)(groups + batch) * (size_t)heads_per_quad;
    return true;
}

size_t balanced_workspace_bytes(const BalancedPlan &pl, int32_t batch) {
    const size_t floats = pl.partial_units * (kHeadDim + 2);
    return floats * sizeof(float) + (((size_t)batch + 1) * sizeof(int32_t) + 15) / 16 * 16;
}

// Optional debug mode (environment variable KVQ_CHECK=1, read at each call):
// copy the page table and lengths to the host (this synchronises the stream)
// and range-check them.
bool debug_checks_enabled() {
    const char *e = getenv("KVQ_CHECK");
    return e && e[0] == '1';
}

int check_append_indices(const int32_t *token_seq, const int32_t *token_pos, int32_t num_tokens,
                         const int32_t *page_table, int32_t max_pages_per_seq, int64_t num_pages,
                         int32_t page_size, hipStream_t stream) {
    int32_t *seq = (int32_t *)malloc(sizeof(int32_t) * num_tokens);
    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * num_tokens);
    int32_t *pt = nullptr;
    int rc = KVQ_OK;
    if (!seq || !pos) { free(seq); free(pos); return KVQ_ERR_INVALID_ARG; }
    if (hipMemcpyAsync(seq, token_seq, sizeof(int32_t) * num_tokens, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(pos, token_pos, sizeof(int32_t) * num_tokens, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        rc = KVQ_ERR_HIP;
    }
    // the page-table rows the call addresses (0 .. largest sequence), in one copy on the stream
    int32_t rows = 0;
    for (int32_t t = 0; rc == KVQ_OK && t < num_tokens; ++t) {
        if (seq[t] < 0 || pos[t] < 0 || pos[t] / page_size >= max_pages_per_seq) rc = KVQ_ERR_INVALID_ARG;
        else if (seq[t] + 1 > rows) rows = seq[t] + 1;
    }
    if (rc == KVQ_OK) {
        const size_t n = (size_t)rows * max_pages_per_seq;
        pt = (int32_t *)malloc(sizeof(int32_t) * n);
        if (!pt) rc = KVQ_ERR_INVALID_ARG;
        else if (hipMemcpyAsync(pt, page_table, sizeof(int32_t) * n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
                 hipStreamSynchronize(stream) != hipSuccess)
            rc = KVQ_ERR_HIP;
    }
    for (int32_t t = 0; rc == KVQ_OK && t < num_tokens; ++t) {
        const int32_t page = pt[(size_t)seq[t] * max_pages_per_seq + pos[t] / page_size];
        if (page < 0 || page >= num_pages) rc = KVQ_ERR_INVALID_ARG;
    }
    free(seq);
    free(pos);
    free(pt);
    return rc;
}

int check_decode_indices(const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                         int32_t batch, int32_t max_context_len, int64_t num_pages, int32_t page_size,
                         hipStream_t stream) {
    const size_t n = (size_t)batch * max_pages_per_seq;
    int32_t *pt = (int32_t *)malloc(sizeof(int32_t) * n);
    int32_t *cl = (int32_t *)malloc(sizeof(int32_t) * batch);
    int rc = KVQ_OK;
    if (!pt || !cl) { free(pt); free(cl); return KVQ_ERR_INVALID_ARG; }
    if (hipMemcpyAsync(pt, page_table, sizeof(int32_t) * n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(cl, context_lens, sizeof(int32_t) * batch, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess) {
        rc = KVQ_ERR_HIP;
    }
    for (int32_t b = 0; rc == KVQ_OK && b < batch; ++b) {
        if (cl[b] > max_context_len || (int64_t)cl[b] > (int64_t)max_pages_per_seq * page_size) { rc = KVQ_ERR_INVALID_ARG; break; }
        for (int32_t p = 0; p < (cl[b] + page_size - 1) / page_size; ++p) {
            const int32_t v = pt[(size_t)b * max_pages_per_seq + p];
            if (v < 0 || v >= num_pages) { rc = KVQ_ERR_INVALID_ARG; break; }
        }
    }
    free(pt);
    free(cl);
    return rc;
}

// Debug check of a prefill call (KVQ_CHECK=1): q_start starts at 0, never
// decreases and ends at num_q; every context length fits the page table;
// every page entry a sequence's context reads lies in [0, num_pages).
int check_prefill_indices(const int32_t *q_start, int32_t num_q, const int32_t *page_table, int32_t max_pages_per_seq,
                          const int32_t *context_lens, int32_t batch, int64_t num_pages, int32_t page_size,
                          hipStream_t stream) {
    int32_t *qs = (int32_t *)malloc(sizeof(int32_t) * ((size_t)batch + 1));
    int rc = qs ? KVQ_OK : KVQ_ERR_INVALID_ARG;
    if (rc == KVQ_OK && (hipMemcpyAsync(qs, q_start, sizeof(int32_t) * ((size_t)batch + 1), hipMemcpyDeviceToHost,
                                        stream) != hipSuccess ||
                         hipStreamSynchronize(stream) != hipSuccess))
        rc = KVQ_ERR_HIP;
    if (rc == KVQ_OK && (qs[0] != 0 || qs[batch] != num_q)) rc = KVQ_ERR_INVALID_ARG;
    for (int32_t b = 0; rc == KVQ_OK && b < batch; ++b)
        if (qs[b + 1] < qs[b]) rc = KVQ_ERR_INVALID_ARG;
    free(qs);
    if (rc != KVQ_OK) return rc;
    // the decode's check with the largest length the page table holds
    const int64_t cap = (int64_t)max_pages_per_seq * page_size;
    return check_decode_indices(page_table, max_pages_per_seq, context_lens, batch,
                                cap > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int32_t)cap, num_pages, page_size, stream);
}

int validate_append(const void *k_new, const void *v_new, const int32_t *token_seq, const int32_t *token_pos,
                    int32_t num_tokens, const int32_t *page_table, int32_t max_pages_per_seq,
                    const void *k_pool, const void *v_pool, int64_t num_pages, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size) {
    if (num_tokens < 0 || num_kv_heads <= 0 || max_pages_per_seq <= 0 || num_pages <= 0)
        return KVQ_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || !valid_page_size(page_size)) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens == 0) return KVQ_OK;
    if (!k_new || !v_new || !token_seq || !token_pos || !page_table || !k_pool || !v_pool)
        return KVQ_ERR_INVALID_ARG;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return KVQ_ERR_INVALID_ARG;
    if ((int64_t)num_tokens * num_kv_heads * 2 / 16 + 1 >= 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
    // the INT4 appends launch one block per (64 tokens, K or V, KV head)
    if ((int64_t)((num_tokens + 63) / 64) * 2 * num_kv_heads > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

int validate_decode(const void *q, const void *k_pool, const void *v_pool, int64_t num_pages,
                    const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                    int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t page_size, const float *out) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages_per_seq <= 0 ||
        num_pages <= 0 || max_context_len < 0)
        return KVQ_ERR_INVALID_ARG;
    if (num_q_heads % num_kv_heads) return KVQ_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || !valid_page_size(page_size)) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)max_context_len > (int64_t)max_pages_per_seq * page_size) return KVQ_ERR_INVALID_ARG;
    if (batch == 0) return KVQ_OK;
    if (!q || !k_pool || !v_pool || !page_table || !context_lens || !out) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return KVQ_ERR_INVALID_ARG;
    if ((int64_t)batch * num_kv_heads > (1ll << 30)) return KVQ_ERR_UNSUPPORTED;
    return KVQ_OK;
}

int decode_common(bool int4, const uint16_t *q, const void *k_pool, const void *v_pool, int64_t num_pages,
                  const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                  int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t page_size, int32_t had_block, float softmax_scale, float *out,
                  void *workspace, size_t workspace_bytes, int32_t pages_per_split, void *phase_event,
                  void *stream, bool use_scratch = false, const kvq_quant_config *cfg = nullptr,
                  const uint16_t *k_new = nullptr, const uint16_t *v_new = nullptr) {
    int rc = validate_decode(q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                             max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, out);
    if (rc != KVQ_OK) return rc;
    if (int4 && !valid_had_block(had_block)) return KVQ_ERR_UNSUPPORTED;
    if (cfg && !valid_cfg(cfg)) return KVQ_ERR_UNSUPPORTED;
    if (pages_per_split < 0) return KVQ_ERR_INVALID_ARG;
    if (batch == 0) return KVQ_OK;
    const int32_t chunks = head_chunks_of(num_q_heads, num_kv_heads);
    int32_t pps = 0, nsplit = 0;
    choose_split(batch, num_kv_heads, chunks, max_context_len, page_size, pages_per_split, &pps, &nsplit);
    if (nsplit > 65535 || (int64_t)num_kv_heads * chunks > 65535 || num_q_heads > 65535) return KVQ_ERR_UNSUPPORTED;
    BalancedPlan bp;
    const bool balanced = balanced_plan(batch, num_kv_heads, chunks, max_context_len, page_size, pages_per_split, &bp);
    const size_t need = balanced ? balanced_workspace_bytes(bp, batch) : workspace_bytes_for(batch, num_q_heads, nsplit);
    if (use_scratch) {
        // the static scratch stands in for the workspace; sizes are checked
        // before anything touches the device
        if (need > KVQ_SCRATCH_BYTES) return KVQ_ERR_TOO_LARGE;
        workspace = scratch_of_current_device();
        if (!workspace) return KVQ_ERR_HIP;
        workspace_bytes = KVQ_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return KVQ_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_checks_enabled()) {
        rc = check_decode_indices(page_table, max_pages_per_seq, context_lens, batch, max_context_len, num_pages,
                                  page_size, st);
        if (rc != KVQ_OK) return rc;
    }
    kvq::DecodeArgs a{};
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.context_lens = context_lens;
    a.out = out;
    a.ws_o = static_cast<float *>(workspace);
    if (balanced) {
        a.ws_ml = a.ws_o + bp.partial_units * kHeadDim;
        a.sk_prefix = reinterpret_cast<int32_t *>(a.ws_ml + bp.partial_units * 2);
        a.sk_groups = bp.groups;
        a.sk_min = bp.gmin;
        a.sk_target = bp.gmax;
        a.quads = bp.quads;
    } else {
        a.ws_ml = a.ws_o + (size_t)batch * num_q_heads * nsplit * kHeadDim;
    }
    a.tile_bytes = !int4 ? (int64_t)page_size * head_dim * 2
                         : cfg ? (int64_t)kvq_page_tile_bytes_cfg(head_dim, page_size, cfg)
                               : (int64_t)kvq_page_tile_bytes(head_dim, page_size);
    a.format = cfg ? cfg->format : KVQ_FORMAT_INT4;
    a.scale_group = cfg ? cfg->scale_group : kHeadDim;
    for (int i = 0; i < 4; ++i) a.sign_mask[i] = cfg ? cfg->sign_mask[i] : 0u;
    a.max_pages_per_seq = max_pages_per_seq;
    a.max_context_len = max_context_len;
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.head_chunks = chunks;
    a.page_size = page_size;
    a.page_shift = log2i(page_size);
    a.had_block = int4 ? had_block : 0;
    a.pages_per_split = pps;
    a.num_splits = nsplit;
    // Split mode with few work items (at most two 8-wave blocks per CU): a
    // range of 4 chunks or more is shared by 2 waves of a block, each taking
    // half of its chunks; shorter ranges stay with one wave.  Measured in HIP
    // graphs, batch 1-12, contexts 2K-128K: 2 waves beat one by 7-13% once a
    // range has 4 chunks or more and lose with 1-3 (the second wave then
    // idles or gets a single chunk); 4 waves per range were never the
    // fastest (each wave's set-up then serves one chunk).  The INT4
    // token-wise kernel only.  KVQ_RANGE_WAVES=1/2/4 overrides (measurement).
    a.range_waves = 1;
    if (!balanced && int4 && !grouped_cfg(cfg)) {
        const int64_t blocks = (int64_t)batch * ((num_kv_heads * chunks + 3) / 4) * nsplit;
        const int32_t range_chunks = pps / (kvq::kChunkTokens / page_size);
        a.range_waves = (blocks <= 512 && range_chunks >= 4) ? 2 : 1;
        const char *e = getenv("KVQ_RANGE_WAVES");
        if (e && (e[0] == '1' || e[0] == '2' || e[0] == '4') && e[1] == 0) a.range_waves = e[0] - '0';
    }
    a.score_scale = softmax_scale * 1.4426950408889634f;
    a.k_new = k_new;
    a.v_new = v_new;
    a.len_offset = k_new ? 1 : 0;
    a.group_shift = -1;
    if ((a.group & (a.group - 1)) == 0) a.group_shift = log2i(a.group);
    a.sk_div32 = balanced && ((int64_t)batch * ((max_context_len + kvq::kChunkTokens - 1) / kvq::kChunkTokens) + 1) *
                                     (int64_t)bp.gmax < (1ll << 31);
    const bool grouped = int4 && (a.format != KVQ_FORMAT_INT4 || a.scale_group != kHeadDim);
    hipError_t e = !int4 ? kvq::launch_decode_fp16(a, st)
                         : grouped ? kvq::launch_decode_grouped(a, st) : kvq::launch_decode_int4_mfma(a, st);
    if (e != hipSuccess) return KVQ_ERR_HIP;
    if (phase_event && hipEventRecord(static_cast<hipEvent_t>(phase_event), st) != hipSuccess)
        return KVQ_ERR_HIP;
    e = kvq::launch_combine(a, int4 && a.had_block > 0, st);
    return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char *kvq_status_string(int status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_INVALID_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported head_dim, page_size, had_block or size";
        case KVQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case KVQ_ERR_HIP: return "HIP runtime error";
        case KVQ_ERR_TOO_LARGE: return "request needs more than the library's static scratch";
        default: return "unknown status";
    }
}

size_t kvq_page_tile_bytes(int32_t head_dim, int32_t page_size) {
    if (head_dim != kHeadDim || !valid_page_size(page_size)) return 0;
    return (size_t)page_size * (head_dim / 2) + 2 * (size_t)page_size;
}

int kv_quant_append(const uint16_t *k_new, const uint16_t *v_new, const int32_t *token_seq,
                    const int32_t *token_pos, int32_t num_tokens, const int32_t *page_table,
                    int32_t max_pages_per_seq, uint8_t *k_pool, uint8_t *v_pool, int64_t num_pages,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t had_block,
                    void *stream) {
    int rc = validate_append(k_new, v_new, token_seq, token_pos, num_tokens, page_table, max_pages_per_seq,
                             k_pool, v_pool, num_pages, num_kv_heads, head_dim, page_size);
    if (rc != KVQ_OK) return rc;
    if (!valid_had_block(had_block)) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens == 0) return KVQ_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_checks_enabled()) {
        rc = check_append_indices(token_seq, token_pos, num_tokens, page_table, max_pages_per_seq, num_pages,
                                  page_size, st);
        if (rc != KVQ_OK) return rc;
    }
    kvq::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.token_seq = token_seq;
    a.token_pos = token_pos;
    a.page_table = page_table;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tile_bytes = (int64_t)kvq_page_tile_bytes(head_dim, page_size);
    a.num_tokens = num_tokens;
    a.max_pages_per_seq = max_pages_per_seq;
    a.num_kv_heads = num_kv_heads;
    a.page_size = page_size;
    a.page_shift = log2i(page_size);
    a.had_block = had_block;
    a.format = KVQ_FORMAT_INT4;
    a.scale_group = kHeadDim;
    return kvq::launch_quant_append(a, st) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t kvq_page_tile_bytes_cfg(int32_t head_dim, int32_t page_size, const kvq_quant_config *cfg) {
    if (head_dim != kHeadDim || !valid_page_size(page_size) || !valid_cfg(cfg)) return 0;
    return (size_t)page_size * (head_dim / 2) + (size_t)page_size * scale_bytes_cfg(cfg);
}

int kv_quant_append_cfg(const uint16_t *k_new, const uint16_t *v_new, const int32_t *token_seq,
                        const int32_t *token_pos, int32_t num_tokens, const int32_t *page_table,
                        int32_t max_pages_per_seq, uint8_t *k_pool, uint8_t *v_pool, int64_t num_pages,
                        int32_t num_kv_heads, int32_t head_dim, int32_t page_size, const kvq_quant_config *cfg,
                        void *stream) {
    int rc = validate_append(k_new, v_new, token_seq, token_pos, num_tokens, page_table, max_pages_per_seq,
                             k_pool, v_pool, num_pages, num_kv_heads, head_dim, page_size);
    if (rc != KVQ_OK) return rc;
    if (!cfg) return KVQ_ERR_INVALID_ARG;
    if (!valid_cfg(cfg)) return KVQ_ERR_UNSUPPORTED;
    if (num_tokens == 0) return KVQ_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_checks_enabled()) {
        rc = check_append_indices(token_seq, token_pos, num_tokens, page_table, max_pages_per_seq, num_pages,
                                  page_size, st);
        if (rc != KVQ_OK) return rc;
    }
    kvq::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.token_seq = token_seq;
    a.token_pos = token_pos;
    a.page_table = page_table;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tile_bytes = (int64_t)kvq_page_tile_bytes_cfg(head_dim, page_size, cfg);
    a.num_tokens = num_tokens;
    a.max_pages_per_seq = max_pages_per_seq;
    a.num_kv_heads = num_kv_heads;
    a.page_size = page_size;
    a.page_shift = log2i(page_size);
    a.had_block = cfg->had_block;
    a.format = cfg->format;
    a.scale_group = cfg->scale_group;
    a.scale_search = cfg->scale_search;
    for (int i = 0; i < 4; ++i) a.sign_mask[i] = cfg->sign_mask[i];
    return kvq::launch_quant_append(a, st) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int kv_append_fp16(const uint16_t *k_new, const uint16_t *v_new, const int32_t *token_seq,
                   const int32_t *token_pos, int32_t num_tokens, const int32_t *page_table,
                   int32_t max_pages_per_seq, uint16_t *k_pool, uint16_t *v_pool, int64_t num_pages,
                   int32_t num_kv_heads, int32_t head_dim, int32_t page_size, void *stream) {
    int rc = validate_append(k_new, v_new, token_seq, token_pos, num_tokens, page_table, max_pages_per_seq,
                             k_pool, v_pool, num_pages, num_kv_heads, head_dim, page_size);
    if (rc != KVQ_OK) return rc;
    if (num_tokens == 0) return KVQ_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (debug_checks_enabled()) {
        rc = check_append_indices(token_seq, token_pos, num_tokens, page_table, max_pages_per_seq, num_pages,
                                  page_size, st);
        if (rc != KVQ_OK) return rc;
    }
    kvq::AppendArgs a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.token_seq = token_seq;
    a.token_pos = token_pos;
    a.page_table = page_table;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tile_bytes = (int64_t)page_size * head_dim * 2;
    a.num_tokens = num_tokens;
    a.max_pages_per_seq = max_pages_per_seq;
    a.num_kv_heads = num_kv_heads;
    a.page_size = page_size;
    a.page_shift = log2i(page_size);
    a.had_block = 0;
    return kvq::launch_append_fp16(a, st) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_context_len, int32_t page_size,
                                         int32_t pages_per_split) {
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
        head_dim != kHeadDim || !valid_page_size(page_size) || pages_per_split < 0 || max_context_len < 0)
        return 0;
    int32_t pps = 0, nsplit = 0;
    const int32_t chunks = head_chunks_of(num_q_heads, num_kv_heads);
    choose_split(batch, num_kv_heads, chunks, max_context_len, page_size, pages_per_split, &pps, &nsplit);
    size_t need = workspace_bytes_for(batch, num_q_heads, nsplit);   // split mode
    BalancedPlan bp;
    if (balanced_plan(batch, num_kv_heads, chunks, max_context_len, page_size, pages_per_split, &bp)) {
        const size_t nb = balanced_workspace_bytes(bp, batch);
        if (nb > need) need = nb;
    }
    return need;
}

int paged_prefill_attn_int4(const uint16_t *q, const int32_t *q_start, int32_t num_q, const uint8_t *k_pool,
                            const uint8_t *v_pool, int64_t num_pages, const int32_t *page_table,
                            int32_t max_pages_per_seq, const int32_t *context_lens, int32_t batch,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                            int32_t had_block, float softmax_scale, float *out, void *stream) {
    if (num_q < 0 || batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_pages_per_seq <= 0 ||
        num_pages <= 0 || num_q_heads % num_kv_heads || !(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
        return KVQ_ERR_INVALID_ARG;
    if (head_dim != kHeadDim || !valid_page_size(page_size) || !valid_had_block(had_block))
        return KVQ_ERR_UNSUPPORTED;
    if (num_q == 0 || batch == 0) return KVQ_OK;
    if (!q || !q_start || !k_pool || !v_pool || !page_table || !context_lens || !out) return KVQ_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return KVQ_ERR_INVALID_ARG;
    if ((int64_t)num_q / 16 + batch > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
    if ((int64_t)max_pages_per_seq * page_size > 0x7FFFFFFFLL) return KVQ_ERR_UNSUPPORTED;
    const int32_t chunks = head_chunks_of(num_q_heads, num_kv_heads);
    if ((int64_t)num_kv_heads * chunks > 65535) return KVQ_ERR_UNSUPPORTED;
    if (debug_checks_enabled()) {
        const int rc = check_prefill_indices(q_start, num_q, page_table, max_pages_per_seq, context_lens, batch,
                                             num_pages, page_size, static_cast<hipStream_t>(stream));
        if (rc != KVQ_OK) return rc;
    }
    kvq::PrefillArgs a{};
    a.q = q;
    a.q_start = q_start;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_table = page_table;
    a.context_lens = context_lens;
    a.out = out;
    a.tile_bytes = (int64_t)kvq_page_tile_bytes(head_dim, page_size);
    a.max_pages_per_seq = max_pages_per_seq;
    a.batch = batch;
    a.num_q = num_q;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_q_heads / num_kv_heads;
    a.head_chunks = chunks;
    a.page_size = page_size;
    a.had_block = had_block;
    a.score_scale = softmax_scale * 1.4426950408889634f;
    return kvq::launch_prefill_int4(a, static_cast<hipStream_t>(stream)) == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}

int paged_decode_attn_int4(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool, int64_t num_pages,
                           const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                           int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t page_size, int32_t had_block, float softmax_scale,
                           float *out, void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                           void *phase_event, void *stream) {
    return decode_common(true, q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                         max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, had_block,
                         softmax_scale, out, workspace, workspace_bytes, pages_per_split, phase_event, stream);
}

int paged_decode_step_int4(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new, uint8_t *k_pool,
                           uint8_t *v_pool, int64_t num_pages, const int32_t *page_table, int32_t max_pages_per_seq,
                           const int32_t *context_lens, int32_t batch, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t had_block,
                           float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                           int32_t pages_per_split, void *phase_event, void *stream) {
    if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVQ_ERR_INVALID_ARG;
    return decode_common(true, q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                         max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, had_block,
                         softmax_scale, out, workspace, workspace_bytes, pages_per_split, phase_event, stream, false,
                         nullptr, k_new, v_new);
}

int paged_decode_attn_cfg(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool, int64_t num_pages,
                          const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                          int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t page_size, const kvq_quant_config *cfg, float softmax_scale,
                          float *out, void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                          void *phase_event, void *stream) {
    if (!cfg) return KVQ_ERR_INVALID_ARG;
    return decode_common(true, q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                         max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, cfg->had_block,
                         softmax_scale, out, workspace, workspace_bytes, pages_per_split, phase_event, stream, false,
                         cfg);
}

int paged_decode_attn_int4_noalloc(const uint16_t *q, const uint8_t *k_pool, const uint8_t *v_pool, int64_t num_pages,
                                   const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                                   int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t page_size, int32_t had_block, float softmax_scale,
                                   float *out, int32_t pages_per_split, void *phase_event, void *stream) {
    return decode_common(true, q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                         max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, had_block,
                         softmax_scale, out, nullptr, 0, pages_per_split, phase_event, stream, true);
}

int paged_decode_attn_fp16(const uint16_t *q, const uint16_t *k_pool, const uint16_t *v_pool, int64_t num_pages,
                           const int32_t *page_table, int32_t max_pages_per_seq, const int32_t *context_lens,
                           int32_t batch, int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t page_size, float softmax_scale, float *out,
                           void *workspace, size_t workspace_bytes, int32_t pages_per_split,
                           void *phase_event, void *stream) {
    return decode_common(false, q, k_pool, v_pool, num_pages, page_table, max_pages_per_seq, context_lens, batch,
                         max_context_len, num_q_heads, num_kv_heads, head_dim, page_size, 0, softmax_scale, out,
                         workspace, workspace_bytes, pages_per_split, phase_event, stream);
}

}  // extern "C"
