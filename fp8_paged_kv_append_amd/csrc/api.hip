// Host side of the C ABI declared in include/kvfp8.h: argument checks, the
// split heuristic, scalar pre-computation, launches.  No allocation, no
// synchronisation, no printing.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/kvfp8.h"
#include "kvfp8_internal.h"

using namespace kvfp8;

static_assert(KVFP8_READ_SINK_WORDS == kReadSinkWords, "checksum words of the read-rate kernels");

namespace {

constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// An attention workspace opens with one uint32 count per (request, query head) -- the GQA kernel uses one
// per (request, KV head) -- padded to 256 bytes; the split partials follow.
// GQA split counts up to this are merged inside the attention launch (by the last split block of each
// (request, KV head)); more are merged by a launch of their own.  Measured on MI355X: one request of 8192
// tokens in a 61-layer step, 16 splits, 14.2 against 15.3 us per layer; 8 requests, 4 splits, 30.3 against
// 30.7; 4 x 131072 tokens at 32 splits 167.0 us with the separate merge, 182.5 with the merge inside.
constexpr int32_t kMergeInLaunchMaxSplits = 16;

// The split counts at the head of an attention workspace: a 128-byte line per (request, query head), so
// that the GQA counts (one per (request, KV head), a line apart) never share one.
inline size_t attn_count_bytes(int32_t batch, int32_t num_q_heads) {
  return ((size_t)batch * num_q_heads * 128 + 255) / 256 * 256;
}
inline bool good_scale(float s) { return isfinite(s) && s > 0.f; }
// The softmax scale a caller passes, with 0 standing for the usual 1/sqrt(score dim).
inline float softmax_scale(float sm_scale, int32_t score_dim) {
  return sm_scale == 0.f ? 1.0f / sqrtf((float)score_dim) : sm_scale;
}

int check_pool(const kvfp8_pool_desc* d, bool need_v_dim_eq, int elt_bytes) {
  if (d == nullptr) return KVFP8_ERR_NULL;
  if (d->num_pages < 1 || d->page_size < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->v_dim < 0)
    return KVFP8_ERR_SHAPE;
  // a power of two from 16 to 256: the kernels find a token's page and slot by shift and mask
  if (d->page_size < 16 || d->page_size > 256 || (d->page_size & (d->page_size - 1)) != 0) return KVFP8_ERR_UNSUPPORTED;
  // K rows are cut into 64-byte slices (the chunk-reordered K layout)
  if ((d->head_dim * elt_bytes) % 64 != 0 || d->v_dim % 16 != 0) return KVFP8_ERR_UNSUPPORTED;
  if (need_v_dim_eq && (d->head_dim != kHeadDim || d->v_dim != kHeadDim)) return KVFP8_ERR_UNSUPPORTED;
  return KVFP8_OK;
}

int32_t n_tiles_of(int32_t max_ctx) { return (int32_t)(((int64_t)max_ctx + kAttnTileTokens - 1) / kAttnTileTokens); }

// Blocks (4 waves each) the split heuristic aims for: one per CU.  Measured on MI355X, a block
// over a whole 8192-token context is cheaper than splitting it further once every CU has a
// block (each extra split costs its block set-up, partial writes and the merge launch); below
// that, splits add the parallelism that short batches lack.
constexpr int64_t kTargetBlocks = 256;

int32_t auto_splits(int32_t batch, int32_t num_kv_heads, int32_t max_ctx) {
  const int64_t items = (int64_t)batch * num_kv_heads;
  const int32_t tiles = n_tiles_of(max_ctx);
  if (items <= 0 || tiles <= 0) return 1;
  int64_t s = (kTargetBlocks + items - 1) / items;
  int64_t cap = tiles / 8;  // at least two tiles per wave
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int32_t)s;
}

int append_common(const kvfp8_pool_desc* desc, void* k_pool, void* v_pool, const uint16_t* k_new,
                  const uint16_t* v_new, const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens,
                  const int32_t* page_table, int32_t batch, int32_t pt_stride, const uint32_t* flags,
                  bool fp8, float k_scale, float v_scale, hipStream_t stream) {
  int st = check_pool(desc, false, fp8 ? 1 : 2);
  if (st) return st;
  if (n_tokens < 0 || batch < 0 || pt_stride < 1) return KVFP8_ERR_SHAPE;
  if (n_tokens == 0) return KVFP8_OK;
  if (!k_pool || !k_new || !tok_req || !tok_pos || !page_table) return KVFP8_ERR_NULL;
  if ((v_pool == nullptr) != (v_new == nullptr)) return KVFP8_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(k_new) || (v_pool && (!aligned16(v_pool) || !aligned16(v_new))))
    return KVFP8_ERR_ALIGN;
  if (fp8 && (!good_scale(k_scale) || (v_pool && !good_scale(v_scale)))) return KVFP8_ERR_VALUE;
  if ((int64_t)n_tokens * desc->num_kv_heads > ((int64_t)1 << 33)) return KVFP8_ERR_SHAPE;
  AppendArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.tok_req = tok_req;
  a.tok_pos = tok_pos;
  a.page_table = page_table;
  a.flags = flags;
  a.n_tokens = n_tokens;
  a.batch = batch;
  a.pt_stride = pt_stride;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.v_dim = desc->v_dim;
  a.k_inv = fp8 ? 1.0f / k_scale : 1.0f;  // fl32(1/scale): one IEEE fp32 division
  a.v_inv = fp8 && v_pool ? 1.0f / v_scale : 1.0f;
  return launch_append(a, fp8, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

int gather_common(const kvfp8_pool_desc* desc, const void* k_pool, const void* v_pool, const int32_t* tok_req,
                  const int32_t* tok_pos, int32_t n_tokens, const int32_t* page_table, int32_t batch,
                  int32_t pt_stride, void* k_out, void* v_out, bool fp8, hipStream_t stream) {
  int st = check_pool(desc, false, fp8 ? 1 : 2);
  if (st) return st;
  if (n_tokens < 0 || batch < 0 || pt_stride < 1) return KVFP8_ERR_SHAPE;
  if (n_tokens == 0) return KVFP8_OK;
  if (!k_pool || !tok_req || !tok_pos || !page_table || !k_out) return KVFP8_ERR_NULL;
  if ((v_out != nullptr) && v_pool == nullptr) return KVFP8_ERR_NULL;
  GatherArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tok_req = tok_req;
  a.tok_pos = tok_pos;
  a.page_table = page_table;
  a.k_out = k_out;
  a.v_out = v_out;
  a.n_tokens = n_tokens;
  a.batch = batch;
  a.pt_stride = pt_stride;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.v_dim = desc->v_dim;
  return launch_gather(a, fp8, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

int attn_common(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads, const void* k_pool,
                const void* v_pool, const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens,
                int32_t batch, int32_t max_ctx_len, const uint32_t* flags, bool fp8, float k_scale,
                float v_scale, float sm_scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
                uint16_t* out, hipStream_t stream, bool launch = true, const uint16_t* k_new = nullptr,
                const uint16_t* v_new = nullptr, const uint32_t* page_tags = nullptr,
                const uint32_t* expected_tags = nullptr, uint32_t* flags_out = nullptr) {
  int st = check_pool(desc, true, fp8 ? 1 : 2);
  if (st) return st;
  if (batch < 0 || num_q_heads < 1 || pt_stride < 1 || num_splits < 0) return KVFP8_ERR_SHAPE;
  if (batch == 0) return KVFP8_OK;
  if (!q || !k_pool || !v_pool || !page_table || !ctx_lens || !out) return KVFP8_ERR_NULL;
  if (num_q_heads % desc->num_kv_heads != 0) return KVFP8_ERR_SHAPE;
  const int32_t group = num_q_heads / desc->num_kv_heads;
  if (group > 16) return KVFP8_ERR_UNSUPPORTED;
  if (max_ctx_len < 1) return KVFP8_ERR_SHAPE;
  if ((int64_t)pt_stride * desc->page_size < max_ctx_len) return KVFP8_ERR_SHAPE;
  if (batch > 65535 || desc->num_kv_heads > 65535) return KVFP8_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out)) return KVFP8_ERR_ALIGN;
  sm_scale = softmax_scale(sm_scale, desc->head_dim);
  if (!good_scale(k_scale) || !good_scale(v_scale) || !good_scale(sm_scale)) return KVFP8_ERR_VALUE;
  const int32_t tiles = n_tiles_of(max_ctx_len);
  int32_t splits = num_splits == 0 ? auto_splits(batch, desc->num_kv_heads, max_ctx_len) : num_splits;
  if (splits > tiles) return KVFP8_ERR_SHAPE;
  const int32_t chunk_tiles = (tiles + splits - 1) / splits;
  splits = (tiles + chunk_tiles - 1) / chunk_tiles;  // drop splits that would start past max_ctx_len
  AttnArgs a;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.count = nullptr;
  a.merge_here = 0;
  if (splits > 1) {
    const size_t need = paged_decode_attn_workspace_bytes(batch, num_q_heads, kHeadDim, splits);
    if (workspace == nullptr) return KVFP8_ERR_NULL;
    if (workspace_bytes < need) return KVFP8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVFP8_ERR_ALIGN;
    // the merge's rows are addressed with 32-bit buffer offsets: at most 2^31 bytes per (request, KV head)
    if ((int64_t)group * splits * kHeadDim * 4 >= ((int64_t)1 << 31)) return KVFP8_ERR_UNSUPPORTED;
    const size_t rows = (size_t)batch * num_q_heads * splits;
    a.count = reinterpret_cast<uint32_t*>(workspace);
    a.merge_here = splits <= kMergeInLaunchMaxSplits ? 1 : 0;
    a.o_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + attn_count_bytes(batch, num_q_heads));
    a.lse_part = a.o_part + rows * kHeadDim;
  }
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.flags = flags;
  a.out = out;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = group;
  a.num_q_heads = num_q_heads;
  a.pt_stride = pt_stride;
  a.chunk_tiles = chunk_tiles;
  a.num_splits = splits;
  a.max_ctx = max_ctx_len;
  a.qk_scale_log2 = fp8 ? sm_scale * k_scale * kLog2e : sm_scale * kLog2e;
  a.v_scale = fp8 ? v_scale : 1.0f;
  // the step's token, written and folded in by the attention launch itself
  if ((k_new == nullptr) != (v_new == nullptr)) return KVFP8_ERR_NULL;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return KVFP8_ERR_ALIGN;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_inv = fp8 ? 1.0f / k_scale : 1.0f;  // fl32(1/scale), as the append computes it
  a.v_inv = fp8 ? 1.0f / v_scale : 1.0f;
  // the tag check in the same launch: it writes the flags instead of reading them
  if (page_tags && (!expected_tags || !flags_out)) return KVFP8_ERR_NULL;
  a.page_tags = page_tags;
  a.expected = expected_tags;
  a.flags_out = flags_out;
  if (page_tags) a.flags = nullptr;
  if (!launch) return KVFP8_OK;
  return launch_attn_gqa(a, fp8, batch, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

int check_append_common(const kvfp8_pool_desc* desc, void* k_pool, void* v_pool, const uint16_t* k_new,
                        const uint16_t* v_new, const int32_t* page_table, int32_t pt_stride,
                        const int32_t* ctx_lens, int32_t batch, const uint32_t* page_tags,
                        const uint32_t* expected_tags, uint32_t* abort_flags, bool fp8, float k_scale,
                        float v_scale, hipStream_t stream, bool launch = true, int32_t max_ctx = 0) {
  // page_tags null: no check, abort_flags (may be null) only read -- see check_append_kernel
  int st = check_pool(desc, false, fp8 ? 1 : 2);
  if (st) return st;
  if (batch < 0 || pt_stride < 1) return KVFP8_ERR_SHAPE;
  if (batch == 0) return KVFP8_OK;
  if (!k_pool || !k_new || !page_table || !ctx_lens) return KVFP8_ERR_NULL;
  if (page_tags && (!expected_tags || !abort_flags)) return KVFP8_ERR_NULL;
  if ((v_pool == nullptr) != (v_new == nullptr)) return KVFP8_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(k_new) || (v_pool && (!aligned16(v_pool) || !aligned16(v_new))))
    return KVFP8_ERR_ALIGN;
  if (fp8 && (!good_scale(k_scale) || (v_pool && !good_scale(v_scale)))) return KVFP8_ERR_VALUE;
  if ((int64_t)desc->num_kv_heads * desc->head_dim / 2 > kCheckAppendMaxPairs ||
      (int64_t)desc->num_kv_heads * desc->v_dim / 2 > kCheckAppendMaxPairs)
    return KVFP8_ERR_UNSUPPORTED;
  TagArgs c;
  c.page_tags = page_tags;
  c.page_table = page_table;
  c.expected = expected_tags;
  c.ctx_lens = ctx_lens;
  c.flags = abort_flags;
  c.num_pages = desc->num_pages;
  c.pt_stride = pt_stride;
  c.batch = batch;
  c.page_size = desc->page_size;
  c.max_ctx = max_ctx;
  AppendArgs a;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = k_new;
  a.v_new = v_new;
  a.tok_req = nullptr;
  a.tok_pos = nullptr;
  a.page_table = page_table;
  a.flags = nullptr;
  a.n_tokens = batch;
  a.batch = batch;
  a.pt_stride = pt_stride;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.v_dim = desc->v_dim;
  a.k_inv = fp8 ? 1.0f / k_scale : 1.0f;
  a.v_inv = fp8 && v_pool ? 1.0f / v_scale : 1.0f;
  if (!launch) return KVFP8_OK;
  return launch_check_append(c, a, fp8, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

// Heads per block: 128 for attn_latent_split_kernel, 64 for the FP8 wave-pair kernel
// (attn_latent_pairs.hip).
constexpr int32_t kLatentPairHeads = 64;
int32_t latent_head_groups(int32_t num_q_heads, bool pairs) {
  const int32_t hpb = pairs ? kLatentPairHeads : kLatentHeadsPerBlock;
  return (num_q_heads + hpb - 1) / hpb;
}

int32_t latent_auto_splits(int32_t batch, int32_t num_q_heads, int32_t max_ctx, bool pairs) {
  const int64_t items = (int64_t)batch * latent_head_groups(num_q_heads, pairs);
  const int32_t tiles = (int32_t)(((int64_t)max_ctx + kLatentTileTokens - 1) / kLatentTileTokens);
  if (items <= 0 || tiles <= 0) return 1;
  int64_t s = (kTargetBlocks + items - 1) / items;
  // at least four 32-token tiles per split: below that a block's fixed traffic (the q of its heads,
  // 147 KB in bf16 for 128, and its fp32 partials, 256 KB) costs more than the added parallelism
  // (one request of 4096 tokens: 32 splits 31.4 us per step against 34.3 us at 64)
  int64_t cap = tiles / 4;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  return (int32_t)s;
}

// FP8: the wave-pair kernel while its splits are at most 1024 tokens.  Measured at 4096 tokens per
// request, pair kernel against 128-head kernel, each at its own split count: B=1 (32 splits) 31.4
// against 35.7 us, B=8 (16 against 32) 43.6 against 56.5, B=16 (8 against 16) 57.7 against 67.0,
// B=32 (4 against 8) 83.5-84.0 against 87.2-88.0; at B=64 (2048-token splits against 4 splits of the
// 128-head kernel) 143-145 against 130-134 us, where each of the two head-group blocks copying every
// tile into its own LDS costs more than the second wave per SIMD gains.
constexpr int32_t kPairMaxSplitTokens = 1024;
bool latent_use_pairs(bool fp8, int32_t max_ctx, int32_t pair_splits) {
  return fp8 && pair_splits > 0 && ((int64_t)max_ctx + pair_splits - 1) / pair_splits <= kPairMaxSplitTokens;
}

int latent_common(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads, const void* pool,
                  const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                  int32_t max_ctx_len, const uint32_t* flags, bool fp8, float scale, float sm_scale,
                  int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* out, hipStream_t stream,
                  bool launch = true, const uint16_t* c_new = nullptr, const uint32_t* page_tags = nullptr,
                  const uint32_t* expected_tags = nullptr, uint32_t* flags_out = nullptr) {
  int st = check_pool(desc, false, fp8 ? 1 : 2);
  if (st) return st;
  if (desc->num_kv_heads != 1 || desc->head_dim != kLatentDim || desc->v_dim != kLatentVDim)
    return KVFP8_ERR_UNSUPPORTED;
  if (batch < 0 || num_q_heads < 1 || pt_stride < 1 || num_splits < 0) return KVFP8_ERR_SHAPE;
  if (batch == 0) return KVFP8_OK;
  if (!q || !pool || !page_table || !ctx_lens || !out) return KVFP8_ERR_NULL;
  if (num_q_heads % 16 != 0) return KVFP8_ERR_UNSUPPORTED;
  if (max_ctx_len < 1) return KVFP8_ERR_SHAPE;
  if ((int64_t)pt_stride * desc->page_size < max_ctx_len) return KVFP8_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(pool) || !aligned16(out)) return KVFP8_ERR_ALIGN;
  sm_scale = softmax_scale(sm_scale, desc->head_dim);
  if (!good_scale(scale) || !good_scale(sm_scale)) return KVFP8_ERR_VALUE;
  const int32_t tiles = (int32_t)(((int64_t)max_ctx_len + kLatentTileTokens - 1) / kLatentTileTokens);
  // FP8: the wave-pair kernel while its splits stay short (latent_use_pairs), else the 128-head
  // kernel; each with its own split count unless the caller gives one
  const int32_t sp = num_splits == 0 ? latent_auto_splits(batch, num_q_heads, max_ctx_len, true) : num_splits;
  const bool pairs = latent_use_pairs(fp8, max_ctx_len, sp);
  int32_t splits = pairs ? sp : (num_splits == 0 ? latent_auto_splits(batch, num_q_heads, max_ctx_len, false)
                                                 : num_splits);
  if (splits > tiles) return KVFP8_ERR_SHAPE;
  const int32_t chunk_tiles = (tiles + splits - 1) / splits;
  splits = (tiles + chunk_tiles - 1) / chunk_tiles;
  const int32_t n_hg = latent_head_groups(num_q_heads, pairs);
  if ((((int64_t)batch * splits + 7) / 8) * 8 * n_hg > 2147483647LL) return KVFP8_ERR_SHAPE;
  LatentArgs a;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  if (splits > 1) {
    const size_t need = paged_decode_attn_workspace_bytes(batch, num_q_heads, kLatentVDim, splits);
    if (workspace == nullptr) return KVFP8_ERR_NULL;
    if (workspace_bytes < need) return KVFP8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVFP8_ERR_ALIGN;
    a.o_part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + attn_count_bytes(batch, num_q_heads));
    a.lse_part = a.o_part + (size_t)batch * num_q_heads * splits * kLatentVDim;
  }
  a.q = q;
  a.pool = pool;
  a.page_table = page_table;
  a.ctx_lens = ctx_lens;
  a.flags = flags;
  a.out = out;
  a.num_pages = desc->num_pages;
  a.page_size = desc->page_size;
  a.num_q_heads = num_q_heads;
  a.pt_stride = pt_stride;
  a.chunk_tiles = chunk_tiles;
  a.num_splits = splits;
  a.max_ctx = max_ctx_len;
  a.batch = batch;
  a.n_hg = n_hg;
  a.qk_scale_log2 = (fp8 ? sm_scale * scale : sm_scale) * kLog2e;
  a.v_scale = fp8 ? scale : 1.0f;
  if (c_new && !aligned16(c_new)) return KVFP8_ERR_ALIGN;
  a.c_new = c_new;
  a.c_inv = fp8 ? 1.0f / scale : 1.0f;  // fl32(1/scale), as the append computes it
  // the tag check in the same launch: it writes the flags instead of reading them (FP8 only; for the
  // BF16 cache the check is a launch of its own)
  if (page_tags && (!expected_tags || !flags_out)) return KVFP8_ERR_NULL;
  if (page_tags && !fp8) return KVFP8_ERR_UNSUPPORTED;
  a.page_tags = page_tags;
  a.expected = expected_tags;
  a.flags_out = flags_out;
  if (page_tags) a.flags = nullptr;
  if (!launch) return KVFP8_OK;
  return launch_attn_latent(a, fp8, pairs, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

// One decode step over a layer stack: every argument of every layer is checked (a dry pass of the
// per-layer checks) before the first launch, so an error launches nothing.  With page_tags given, the
// tag check is its own batched launch before anything reads the cache (the agentlenshq summary,
// section "KV Cache 完整性检查", and the xujun.org note, section "一个不能出错的共享缓存", keep it out
// of the attention kernel): layer 0's check + write launch, then layer 0's attention reading the
// flags it left.  Every later layer (and layer 0 without the tracker) is one attention launch (plus
// the merge when split) that also writes the layer's token: GQA, the block whose split holds position
// L - 1 writes it and adds it to its softmax from registers; latent, the block(s) holding it store it
// before copying any tile and read it back.  With KVFP8_STEP_FUSED_CHECK layer 0's check runs inside
// its attention launch instead (GQA and FP8 latent: in every block, before it reads any page; BF16
// latent keeps its check + write launch).  Stream order carries the layer-to-layer dependency.
int decode_step_common(const kvfp8_pool_desc* desc, const kvfp8_layer_stack* layers, int32_t num_q_heads,
                       const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                       int32_t max_ctx_len, const uint32_t* page_tags, const uint32_t* expected_tags,
                       uint32_t* abort_flags, bool fp8, float sm_scale, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (desc == nullptr || layers == nullptr) return KVFP8_ERR_NULL;
  const kvfp8_layer_stack& ls = *layers;
  if (ls.num_layers < 1 || batch < 0 || num_q_heads < 1) return KVFP8_ERR_SHAPE;
  if ((ls.options & ~KVFP8_STEP_FUSED_CHECK) != 0u) return KVFP8_ERR_VALUE;
  const bool fused = (ls.options & KVFP8_STEP_FUSED_CHECK) != 0u;
  if (!ls.k_pools || !ls.q || !ls.k_new || !ls.out) return KVFP8_ERR_NULL;
  const bool latent = ls.v_pools == nullptr;
  if (latent != (ls.v_new == nullptr)) return KVFP8_ERR_NULL;
  if (fp8 && (!ls.k_scales || (!latent && !ls.v_scales))) return KVFP8_ERR_NULL;
  if (page_tags && (!expected_tags || !abort_flags)) return KVFP8_ERR_NULL;
  if (desc->num_pages < 1 || desc->page_size < 1 || desc->num_kv_heads < 1 || desc->head_dim < 1 || desc->v_dim < 0)
    return KVFP8_ERR_SHAPE;
  const int64_t elt = fp8 ? 1 : 2;
  const int64_t slots = (int64_t)desc->num_pages * desc->page_size * desc->num_kv_heads;
  const int64_t kpool_b = slots * desc->head_dim * elt, vpool_b = slots * desc->v_dim * elt;
  const int64_t q_n = (int64_t)batch * num_q_heads * desc->head_dim;
  const int64_t kn_n = (int64_t)batch * desc->num_kv_heads * desc->head_dim;
  const int64_t vn_n = (int64_t)batch * desc->num_kv_heads * desc->v_dim;
  const int64_t out_n = (int64_t)batch * num_q_heads * desc->v_dim;
  for (int pass = 0; pass < 2; ++pass) {
    const bool launch = pass == 1;
    for (int32_t l = 0; l < ls.num_layers; ++l) {
      void* kp = static_cast<uint8_t*>(ls.k_pools) + l * kpool_b;
      void* vp = latent ? nullptr : static_cast<uint8_t*>(ls.v_pools) + l * vpool_b;
      const uint16_t* q = ls.q + l * q_n;
      const uint16_t* kn = ls.k_new + l * kn_n;
      const uint16_t* vn = latent ? nullptr : ls.v_new + l * vn_n;
      uint16_t* out = ls.out + l * out_n;
      const float ks = fp8 ? ls.k_scales[l] : 1.f;
      const float vs = fp8 && !latent ? ls.v_scales[l] : 1.f;
      const uint32_t* tags = l == 0 ? page_tags : nullptr;
      // layer 0 with the tracker: the check (and the layer's write) as a launch of its own, unless the
      // caller asks for the fused form -- which the BF16 latent cache does not take (measured slower
      // at 64 x 4096: 135.0-136.1 us per single-layer step with the check in its 128-head blocks
      // against 132.5-132.9 with the separate launch)
      const bool own_write = tags != nullptr && (!fused || (latent && !fp8));
      int st = KVFP8_OK;
      if (!launch || own_write)  // the dry pass checks the write's arguments for every layer
        st = check_append_common(desc, kp, vp, kn, vn, page_table, pt_stride, ctx_lens, batch, tags, expected_tags,
                                 abort_flags, fp8, ks, vs, stream, launch, max_ctx_len);
      if (st) return st;
      if (own_write) tags = nullptr;
      st = latent ? latent_common(desc, q, num_q_heads, kp, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                                  tags ? nullptr : abort_flags, fp8, ks, sm_scale, num_splits, workspace,
                                  workspace_bytes, out, stream, launch, own_write ? nullptr : kn, tags,
                                  expected_tags, tags ? abort_flags : nullptr)
                  : attn_common(desc, q, num_q_heads, kp, vp, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                                tags ? nullptr : abort_flags, fp8, ks, vs, sm_scale, num_splits, workspace,
                                workspace_bytes, out, stream, launch, own_write ? nullptr : kn,
                                own_write ? nullptr : vn, tags, expected_tags, tags ? abort_flags : nullptr);
      if (st) return st;
    }
  }
  return KVFP8_OK;
}

// ---- the attention scratch of the allocation-free entry point
// Split partials (fp32 o and lse) of paged_decode_attn_fp8_noalloc live in this file-scope array
// instead of a caller's workspace.  Host code never uses its name as an address: each device's copy is
// found once with hipGetSymbolAddress (that device current) and that pointer is what the kernels get.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

}  // namespace

static __device__ __align__(256) float scratch[KVFP8_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

int scratch_of_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KVFP8_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return KVFP8_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVFP8_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVFP8_OK;
}

}  // namespace

extern "C" {

int kvfp8_abi_version(void) { return KVFP8_ABI_VERSION; }

const char* kvfp8_status_string(int s) {
  switch (s) {
    case KVFP8_OK: return "ok";
    case KVFP8_ERR_NULL: return "null pointer";
    case KVFP8_ERR_SHAPE: return "bad shape";
    case KVFP8_ERR_UNSUPPORTED: return "unsupported size";
    case KVFP8_ERR_WORKSPACE: return "workspace too small";
    case KVFP8_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KVFP8_ERR_HIP: return "HIP launch error";
    case KVFP8_ERR_VALUE: return "invalid scalar argument";
    case KVFP8_ERR_NOSPACE: return "not enough free pages";
    default: return "unknown status";
  }
}

int kv_absmax_bf16(const uint16_t* x, int64_t n, uint32_t* absmax_bits, hipStream_t stream) {
  if (n < 0) return KVFP8_ERR_SHAPE;
  if (n == 0) return KVFP8_OK;
  if (!x || !absmax_bits) return KVFP8_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(absmax_bits) & 3u)) return KVFP8_ERR_ALIGN;
  return launch_absmax(x, n, absmax_bits, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

float kv_scale_from_absmax(uint32_t absmax_bits) {
  float a;
  memcpy(&a, &absmax_bits, sizeof a);
  return a / 448.0f;
}

int kv_append_fp8(const kvfp8_pool_desc* desc, uint8_t* k_pool, uint8_t* v_pool, const uint16_t* k_new,
                  const uint16_t* v_new, const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens,
                  const int32_t* page_table, int32_t batch, int32_t pt_stride, const uint32_t* abort_flags,
                  float k_scale, float v_scale, hipStream_t stream) {
  return append_common(desc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, n_tokens, page_table, batch,
                       pt_stride, abort_flags, true, k_scale, v_scale, stream);
}

int kv_append_bf16(const kvfp8_pool_desc* desc, uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new,
                   const uint16_t* v_new, const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens,
                   const int32_t* page_table, int32_t batch, int32_t pt_stride, const uint32_t* abort_flags,
                   hipStream_t stream) {
  return append_common(desc, k_pool, v_pool, k_new, v_new, tok_req, tok_pos, n_tokens, page_table, batch,
                       pt_stride, abort_flags, false, 1.f, 1.f, stream);
}

int kv_tag_check(const uint32_t* page_tags, int32_t num_pages, const int32_t* page_table,
                 const uint32_t* expected_tags, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                 int32_t page_size, uint32_t* abort_flags, hipStream_t stream) {
  if (batch < 0 || num_pages < 0 || pt_stride < 1 || page_size < 1) return KVFP8_ERR_SHAPE;
  if (batch == 0) return KVFP8_OK;
  if (!page_table || !expected_tags || !ctx_lens || !abort_flags || (num_pages > 0 && !page_tags))
    return KVFP8_ERR_NULL;
  TagArgs a;
  a.page_tags = page_tags;
  a.page_table = page_table;
  a.expected = expected_tags;
  a.ctx_lens = ctx_lens;
  a.flags = abort_flags;
  a.num_pages = num_pages;
  a.pt_stride = pt_stride;
  a.batch = batch;
  a.page_size = page_size;
  a.max_ctx = 0;
  return launch_tag_check(a, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

int kv_tag_check_append_fp8(const kvfp8_pool_desc* desc, uint8_t* k_pool, uint8_t* v_pool, const uint16_t* k_new,
                            const uint16_t* v_new, const int32_t* page_table, int32_t pt_stride,
                            const int32_t* ctx_lens, int32_t batch, const uint32_t* page_tags,
                            const uint32_t* expected_tags, uint32_t* abort_flags, float k_scale, float v_scale,
                            hipStream_t stream) {
  if (page_tags == nullptr) return KVFP8_ERR_NULL;
  return check_append_common(desc, k_pool, v_pool, k_new, v_new, page_table, pt_stride, ctx_lens, batch, page_tags,
                             expected_tags, abort_flags, true, k_scale, v_scale, stream);
}

int kv_tag_check_append_bf16(const kvfp8_pool_desc* desc, uint16_t* k_pool, uint16_t* v_pool, const uint16_t* k_new,
                             const uint16_t* v_new, const int32_t* page_table, int32_t pt_stride,
                             const int32_t* ctx_lens, int32_t batch, const uint32_t* page_tags,
                             const uint32_t* expected_tags, uint32_t* abort_flags, hipStream_t stream) {
  if (page_tags == nullptr) return KVFP8_ERR_NULL;
  return check_append_common(desc, k_pool, v_pool, k_new, v_new, page_table, pt_stride, ctx_lens, batch, page_tags,
                             expected_tags, abort_flags, false, 1.f, 1.f, stream);
}

int kv_decode_step_fp8(const kvfp8_pool_desc* desc, const kvfp8_layer_stack* layers, int32_t num_q_heads,
                       const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                       int32_t max_ctx_len, const uint32_t* page_tags, const uint32_t* expected_tags,
                       uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return decode_step_common(desc, layers, num_q_heads, page_table, pt_stride, ctx_lens, batch, max_ctx_len, page_tags,
                            expected_tags, abort_flags, true, sm_scale, num_splits, workspace, workspace_bytes, stream);
}

int kv_decode_step_bf16(const kvfp8_pool_desc* desc, const kvfp8_layer_stack* layers, int32_t num_q_heads,
                        const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                        int32_t max_ctx_len, const uint32_t* page_tags, const uint32_t* expected_tags,
                        uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return decode_step_common(desc, layers, num_q_heads, page_table, pt_stride, ctx_lens, batch, max_ctx_len, page_tags,
                            expected_tags, abort_flags, false, sm_scale, num_splits, workspace, workspace_bytes,
                            stream);
}

size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t v_dim, int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || v_dim <= 0 || num_splits <= 1) return 0;
  const size_t rows = (size_t)batch * num_q_heads * num_splits;
  // the split counters, then the partials (fp32; the FP8 kernels store fp16 in the first half of the same
  // region) and lse of every (request, head, split)
  return attn_count_bytes(batch, num_q_heads) + rows * (size_t)v_dim * sizeof(float) + rows * sizeof(float);
}

int32_t paged_decode_attn_auto_splits(int32_t batch, int32_t num_kv_heads, int32_t max_ctx_len) {
  return auto_splits(batch, num_kv_heads, max_ctx_len);
}

int paged_decode_attn_fp8(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                          const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* page_table,
                          int32_t pt_stride, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                          const uint32_t* abort_flags, float k_scale, float v_scale, float sm_scale,
                          int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* out,
                          hipStream_t stream) {
  return attn_common(desc, q, num_q_heads, k_pool, v_pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                     abort_flags, true, k_scale, v_scale, sm_scale, num_splits, workspace, workspace_bytes, out,
                     stream);
}

int paged_decode_attn_bf16(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                           const uint16_t* k_pool, const uint16_t* v_pool, const int32_t* page_table,
                           int32_t pt_stride, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                           const uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return attn_common(desc, q, num_q_heads, k_pool, v_pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                     abort_flags, false, 1.f, 1.f, sm_scale, num_splits, workspace, workspace_bytes, out, stream);
}

int paged_decode_attn_fp8_noalloc(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                  const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* page_table,
                                  int32_t pt_stride, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                  const uint32_t* abort_flags, float k_scale, float v_scale, float sm_scale,
                                  int32_t num_splits, uint16_t* out, hipStream_t stream) {
  // every argument checked (with the scratch as the workspace: a split count whose partials exceed it
  // fails with KVFP8_ERR_WORKSPACE) before the scratch address is looked up or anything launched
  static char probe alignas(256);
  int st = attn_common(desc, q, num_q_heads, k_pool, v_pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                       abort_flags, true, k_scale, v_scale, sm_scale, num_splits, &probe,
                       KVFP8_NOALLOC_SCRATCH_BYTES, out, stream, false);
  if (st || batch == 0) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  return attn_common(desc, q, num_q_heads, k_pool, v_pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len,
                     abort_flags, true, k_scale, v_scale, sm_scale, num_splits, ws, KVFP8_NOALLOC_SCRATCH_BYTES, out,
                     stream);
}

int32_t paged_decode_attn_latent_auto_splits(int32_t batch, int32_t num_q_heads, int32_t max_ctx_len) {
  // the larger of the two caches' choices, so that a workspace sized with it fits either
  const int32_t b = latent_auto_splits(batch, num_q_heads, max_ctx_len, false);
  const int32_t p = latent_auto_splits(batch, num_q_heads, max_ctx_len, true);
  const int32_t f = latent_use_pairs(true, max_ctx_len, p) ? p : b;
  return f > b ? f : b;
}

int paged_decode_attn_latent_fp8(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                 const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                 const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                 const uint32_t* abort_flags, float scale, float sm_scale, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return latent_common(desc, q, num_q_heads, pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len, abort_flags,
                       true, scale, sm_scale, num_splits, workspace, workspace_bytes, out, stream);
}

int paged_decode_attn_latent_bf16(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                  const uint16_t* pool, const int32_t* page_table, int32_t pt_stride,
                                  const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                  const uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                                  size_t workspace_bytes, uint16_t* out, hipStream_t stream) {
  return latent_common(desc, q, num_q_heads, pool, page_table, pt_stride, ctx_lens, batch, max_ctx_len, abort_flags,
                       false, 1.f, sm_scale, num_splits, workspace, workspace_bytes, out, stream);
}

int kv_read_stream(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return KVFP8_OK;
  if (!src || !sink) return KVFP8_ERR_NULL;
  if (bytes % 4 != 0) return KVFP8_ERR_SHAPE;
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3u)) return KVFP8_ERR_ALIGN;
  // at most 2^40 16-byte vectors, 2^29 thread blocks of 2048 vectors: inside the grid's 2^31 - 1
  if (bytes / 16 > ((uint64_t)1 << 40)) return KVFP8_ERR_SHAPE;
  return launch_read_stream(src, bytes, sink, stream) == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

int kv_read_blocks(const void* base, int64_t num_blocks, int64_t block_bytes, const int32_t* ids, int64_t n_ids,
                   uint32_t* sink, hipStream_t stream) {
  if (n_ids < 0 || num_blocks < 0 || block_bytes <= 0 || block_bytes % 16 != 0) return KVFP8_ERR_SHAPE;
  if (n_ids == 0) return KVFP8_OK;
  if (!base || !ids || !sink) return KVFP8_ERR_NULL;
  if (!aligned16(base) || (reinterpret_cast<uintptr_t>(ids) & 3u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return KVFP8_ERR_ALIGN;
  const int64_t pieces = (block_bytes / 16 + 63) / 64;  // 1 KiB pieces per block
  // at most 2^35 pieces, 2^30 thread blocks of 32 pieces: inside the grid's 2^31 - 1
  if (n_ids > ((int64_t)1 << 35) / pieces) return KVFP8_ERR_SHAPE;
  return launch_read_blocks(base, num_blocks, ids, n_ids, block_bytes, sink, stream) == hipSuccess ? KVFP8_OK
                                                                                                    : KVFP8_ERR_HIP;
}

int kv_gather_fp8(const kvfp8_pool_desc* desc, const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* tok_req,
                  const int32_t* tok_pos, int32_t n_tokens, const int32_t* page_table, int32_t batch,
                  int32_t pt_stride, uint8_t* k_out, uint8_t* v_out, hipStream_t stream) {
  return gather_common(desc, k_pool, v_pool, tok_req, tok_pos, n_tokens, page_table, batch, pt_stride, k_out,
                       v_out, true, stream);
}

int kv_gather_bf16(const kvfp8_pool_desc* desc, const uint16_t* k_pool, const uint16_t* v_pool,
                   const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens, const int32_t* page_table,
                   int32_t batch, int32_t pt_stride, uint16_t* k_out, uint16_t* v_out, hipStream_t stream) {
  return gather_common(desc, k_pool, v_pool, tok_req, tok_pos, n_tokens, page_table, batch, pt_stride, k_out,
                       v_out, false, stream);
}

}  // extern "C"
