/*
 * kvfp8.h -- C ABI of the MI355X (gfx950) library for decode attention over a
 * paged KV cache stored as FP8 e4m3 (or BF16), its write path and its batched
 * page-tag integrity check.
 *
 * What the operations compute comes from these pages:
 *  [Q] Cloudflare blog, "Smaller, faster, safer: running Kimi and GLM at
 *      scale", section "Quantized KV cache": K and V are cached as FP8 e4m3
 *      instead of BF16 (half the bytes); the attention kernel converts the
 *      stored values as it reads them; BF16 and FP8 caches are compared.
 *  [T] agentlenshq summary "Cloudflare Workers AI: 大规模优化 Kimi 和 GLM 推理",
 *      section "KV Cache 完整性检查", and the xujun.org note on the same post,
 *      section "一个不能出错的共享缓存": every physical cache page carries a
 *      tag that changes on reallocation; each request's expected (page, tag)
 *      list is validated before decode reads the cache; a mismatch aborts the
 *      request; the check runs as a separate batched pass, not inside the
 *      attention kernel; deployments that do not want it use a no-op tracker.
 * Readings where the pages are silent (OCP E4M3, round-to-nearest-even,
 * saturation, per-tensor scale, layouts, flag bits) are stated per call.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked (host).  The library never
 *    allocates, frees, synchronises or prints; the caller owns all memory,
 *    including the attention workspace.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and returns
 *    a status: KVFP8_OK or a negative KVFP8_ERR_*.  A call that returns an
 *    error has enqueued nothing.  KVFP8_ERR_HIP means a launch failed.
 *  - Data faults that live in device memory (stale tags, bad page ids, bad
 *    context lengths) never become status codes: they surface through the
 *    abort flags and, in attention, as all-zero output rows.
 *  - bf16 values travel as uint16_t bit patterns; e4m3 codes as uint8_t.
 *  - Pools and q/out/new-row buffers must be 16-byte aligned.
 *
 * Page pool layout (element = 1 byte e4m3 or 2 bytes bf16).  Every (page,
 * head) block is contiguous.
 *    V pool  [P][Hkv][Dv][S]   element (page, kv head, d, slot): each
 *                              (page, head) block of V is stored transposed.
 *    K pool  [P][Hkv][S/16][16 tokens x D]: each 16-token sub-page block is
 *            kept as 16-byte chunks in a fixed order: token t = 4s + i of the
 *            sub-page (s, i in 0..3) and chunk c of its row (c = q*NI + k,
 *            NI = D*bytes/64, q in 0..3) sit at chunk position
 *            ((s*NI + k)*4 + q)*4 + i.  (A wave reading one chunk of four
 *            tokens from each of four pages then reads four contiguous
 *            256-byte runs per instruction.)  D*bytes must be a multiple of 64.
 *    latent  [P][Hkv][S][Dl] row-major (Hkv = 1): a pool written or read with
 *            no V pool (v_pool NULL) is a latent pool; the tokens of a page
 *            are consecutive Dl-element rows.
 * Page table: int32 [B][pt_stride]; entry i of request r is the physical page
 * of its tokens [i*S, (i+1)*S).  Entries at or past ceil(L_r/S) are never read.
 * Context length L_r counts the token appended in the current step.
 */
#ifndef KVFP8_H
#define KVFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define KVFP8_ABI_VERSION 2

#define KVFP8_OK 0
#define KVFP8_ERR_NULL (-1)        /* a required pointer is NULL                       */
#define KVFP8_ERR_SHAPE (-2)       /* sizes inconsistent or out of range               */
#define KVFP8_ERR_UNSUPPORTED (-3) /* a size outside the compiled set                  */
#define KVFP8_ERR_WORKSPACE (-4)   /* workspace smaller than the query says            */
#define KVFP8_ERR_ALIGN (-5)       /* a pointer is not 16-byte aligned                 */
#define KVFP8_ERR_HIP (-6)         /* the HIP runtime reported a launch error          */
#define KVFP8_ERR_VALUE (-7)       /* a scalar argument is invalid (scale <= 0, NaN)   */
#define KVFP8_ERR_NOSPACE (-8)     /* the page allocator has fewer free pages than asked */

/* Abort-flag bits written by kv_tag_check (uint32 per request). */
#define KVFP8_FLAG_TAG_MISMATCH 1u /* a used entry's page tag != the expected tag      */
#define KVFP8_FLAG_BAD_PAGE 2u     /* a used page id outside [0,P), or ceil(L/S) > pt_stride */

/* Shape of a page pool (host struct). */
typedef struct kvfp8_pool_desc {
  int32_t num_pages;    /* P                                                   */
  int32_t page_size;    /* S tokens per page: 16, 32, 64, 128 or 256          */
  int32_t num_kv_heads; /* Hkv (1 for the latent cache)                        */
  int32_t head_dim;     /* D: K width (the latent width Dl for the latent cache) */
  int32_t v_dim;        /* Dv: V width (for the latent cache: the value part)  */
} kvfp8_pool_desc;

int kvfp8_abi_version(void);
/* Static string naming a status code. */
const char* kvfp8_status_string(int status);

/* ---------------------------------------------------------------- scale calibration
 * Per-tensor scale = fl32(max|x| / 448) (448 = largest finite e4m3).  The
 * pages give no scale rule; this per-tensor max-abs reading is recorded with
 * the tests.  kv_absmax_bf16 max-accumulates max|x| over n bf16 values into
 * *absmax_bits (device, float32 bit pattern, NaN inputs ignored, +inf
 * counts): zero it first, or call repeatedly to calibrate over chunks.
 * kv_scale_from_absmax is a host function: fl32(absmax / 448). */
int kv_absmax_bf16(const uint16_t* x, int64_t n, uint32_t* absmax_bits, hipStream_t stream);
float kv_scale_from_absmax(uint32_t absmax_bits);

/* ---------------------------------------------------------------- write path  [Q]
 * For each new token n (request tok_req[n], position tok_pos[n]) and KV head
 * h: store its K row and V row at page page_table[r][pos / S], slot pos % S.
 * kv_append_fp8 first quantises: code = E4M3(fl32(x * fl32(1/scale))), with
 * OCP E4M3 round-to-nearest-even, |value| > 448 saturating to +-448, NaN ->
 * 0x7F with the input's sign.  kv_append_bf16 copies the bf16 bits.
 *   k_new [N][Hkv][D], v_new [N][Hkv][Dv] (bf16).  v_pool/v_new may both be
 *   NULL: the pool is then a latent pool (row-major layout above).
 *   abort_flags [B] or NULL (NULL = no-op tracker): tokens of a request whose
 *   flag is non-zero are skipped [T].  Tokens whose request is outside [0,B),
 *   whose position is outside [0, pt_stride*S) or whose page id is outside
 *   [0,P) are skipped (memory safety; the tag check reports such pages).
 *   Two tokens aimed at the same slot: which one lands is unspecified.
 *   Scales must be finite and > 0 (KVFP8_ERR_VALUE otherwise). */
int kv_append_fp8(const kvfp8_pool_desc* desc, uint8_t* k_pool, uint8_t* v_pool,
                  const uint16_t* k_new, const uint16_t* v_new, const int32_t* tok_req,
                  const int32_t* tok_pos, int32_t n_tokens, const int32_t* page_table,
                  int32_t batch, int32_t pt_stride, const uint32_t* abort_flags, float k_scale,
                  float v_scale, hipStream_t stream);
int kv_append_bf16(const kvfp8_pool_desc* desc, uint16_t* k_pool, uint16_t* v_pool,
                   const uint16_t* k_new, const uint16_t* v_new, const int32_t* tok_req,
                   const int32_t* tok_pos, int32_t n_tokens, const int32_t* page_table,
                   int32_t batch, int32_t pt_stride, const uint32_t* abort_flags,
                   hipStream_t stream);

/* ---------------------------------------------------------------- integrity check  [T]
 * abort_flags[r] = OR over the used entries i < ceil(L_r/S) of request r of
 *   KVFP8_FLAG_BAD_PAGE      if page_table[r][i] is outside [0, num_pages),
 *   KVFP8_FLAG_TAG_MISMATCH  else if page_tags[page] != expected_tags[r][i];
 * plus KVFP8_FLAG_BAD_PAGE when ceil(L_r/S) > pt_stride.  L_r <= 0 gives 0.
 * Rewritten on every call (flags are not sticky).  One batched launch;
 * attention and append read the flags it leaves, in stream order.
 *   page_tags uint32 [P]; page_table int32 [B][pt_stride];
 *   expected_tags uint32 [B][pt_stride]; ctx_lens int32 [B]; abort_flags out [B]. */
int kv_tag_check(const uint32_t* page_tags, int32_t num_pages, const int32_t* page_table,
                 const uint32_t* expected_tags, int32_t pt_stride, const int32_t* ctx_lens,
                 int32_t batch, int32_t page_size, uint32_t* abort_flags, hipStream_t stream);

/* ---------------------------------------------------------------- check + write, one launch  [T][Q]
 * The decode step's first two passes for the usual case of one new token per
 * request: token r of k_new/v_new [B][Hkv][D|Dv] belongs to request r at
 * position ctx_lens[r] - 1.  Writes abort_flags exactly as kv_tag_check does
 * (page tags uint32 [desc->num_pages]) and then writes each request's token
 * exactly as kv_append_* would with those flags; the check of a request
 * still completes before its write.  Same result as kv_tag_check followed by
 * kv_append_* with tok_req[n] = n, tok_pos[n] = ctx_lens[n] - 1, in one
 * launch.  Hkv*D and Hkv*Dv at most 4096 (KVFP8_ERR_UNSUPPORTED otherwise). */
int kv_tag_check_append_fp8(const kvfp8_pool_desc* desc, uint8_t* k_pool, uint8_t* v_pool,
                            const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table,
                            int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                            const uint32_t* page_tags, const uint32_t* expected_tags,
                            uint32_t* abort_flags, float k_scale, float v_scale, hipStream_t stream);
int kv_tag_check_append_bf16(const kvfp8_pool_desc* desc, uint16_t* k_pool, uint16_t* v_pool,
                             const uint16_t* k_new, const uint16_t* v_new, const int32_t* page_table,
                             int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                             const uint32_t* page_tags, const uint32_t* expected_tags,
                             uint32_t* abort_flags, hipStream_t stream);

/* ---------------------------------------------------------------- decode attention  [Q]
 * For request r, query head h (KV head g = h / (Hq/Hkv)), over positions t < L_r:
 *   s_t = sm_scale * <q_h, K^_t>,  o_h = sum_t softmax(s)_t V^_t,
 * with K^ = dec(K)*k_scale, V^ = dec(V)*v_scale for the FP8 cache (e4m3
 * decoded in registers as pages are read) and K^ = K, V^ = V for BF16.  The
 * fp32 result is rounded to bf16 (RNE).  Long contexts are cut into
 * num_splits chunks whose partial softmax states are merged by log-sum-exp.
 *   q bf16 [B][Hq][D]; out bf16 [B][Hq][Dv].  D = Dv = 128; Hq/Hkv <= 16.
 *   ctx_lens int32 [B]; max_ctx_len (host) bounds every L_r and sizes the
 *   grid: a request with L_r > max_ctx_len, L_r > pt_stride*S or L_r <= 0
 *   gets zero rows.
 *   abort_flags [B] or NULL (no-op tracker).  A flagged request reads no
 *   pages and gets zero rows [T].  A page id outside [0,P) met while reading
 *   also zeroes the request's rows (memory safety when the tracker is off).
 *   num_splits: 0 = chosen by the library; otherwise at most
 *   ceil(max_ctx_len/64).  workspace (device, 16-byte aligned): at least
 *   paged_decode_attn_workspace_bytes(...) bytes for the split count used
 *   (0 when it is 1; then workspace may be NULL).  It opens with B*Hq
 *   128-byte lines of uint32 counters (padded to 256 bytes; counters that
 *   shared a line would make the split blocks queue on it) that must be zero
 *   before the first call that uses the workspace (allocate it zeroed once); every call
 *   leaves them zero, so a workspace serves any sequence of ordered calls,
 *   GQA or latent, of any shape it is large enough for.  With 2..16 splits
 *   the GQA launch merges them itself (the last split block of each
 *   (request, KV head) does the log-sum-exp merge); more splits, and the
 *   latent cache, add a merge launch.  Calls that share a workspace must be
 *   ordered (one stream).
 *   sm_scale: the softmax scale; 0 selects 1/sqrt(D) (the pages give none).
 *   k_scale, v_scale and a non-zero sm_scale must be finite and > 0. */
size_t paged_decode_attn_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t v_dim,
                                         int32_t num_splits);
/* The split count that num_splits = 0 selects for this shape (host only). */
int32_t paged_decode_attn_auto_splits(int32_t batch, int32_t num_kv_heads, int32_t max_ctx_len);

int paged_decode_attn_fp8(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                          const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* page_table,
                          int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                          int32_t max_ctx_len, const uint32_t* abort_flags, float k_scale,
                          float v_scale, float sm_scale, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, uint16_t* out, hipStream_t stream);
int paged_decode_attn_bf16(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                           const uint16_t* k_pool, const uint16_t* v_pool,
                           const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens,
                           int32_t batch, int32_t max_ctx_len, const uint32_t* abort_flags,
                           float sm_scale, int32_t num_splits, void* workspace,
                           size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/* ---------------------------------------------------------------- attention with no workspace
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation, arguments, kernels and results as paged_decode_attn_fp8, with
 * the split partials kept in a scratch array of KVFP8_NOALLOC_SCRATCH_BYTES
 * that the library holds in device memory (one per GPU it runs on, for the
 * life of the process) instead of a caller's workspace.  The call allocates
 * nothing.  The current device must be the one `stream` belongs to; the first
 * call on a device looks the array up there (hipGetSymbolAddress).  A split
 * count whose partials would exceed the array
 * (paged_decode_attn_workspace_bytes(B, Hq, 128, splits) bytes) is rejected
 * with KVFP8_ERR_WORKSPACE before anything is enqueued.  Every call on a
 * device shares that device's array: calls that overlap on one GPU (other
 * streams, other threads) race on it; calls in one stream's order do not.
 * The array's split counters start at zero (it is zero-initialised when the
 * library loads) and every call leaves them zero, so nothing in it needs
 * clearing between calls. */
#define KVFP8_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int paged_decode_attn_fp8_noalloc(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                  const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* page_table,
                                  int32_t pt_stride, const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                  const uint32_t* abort_flags, float k_scale, float v_scale, float sm_scale,
                                  int32_t num_splits, uint16_t* out, hipStream_t stream);

/* ---------------------------------------------------------------- latent (MLA-style) cache  [Q]
 * One cached vector c_t of width Dl = 576 per token, shared by every query
 * head (the pool: latent layout, num_kv_heads = 1, head_dim = 576,
 * v_dim = 512, written by kv_append_* with v_pool = v_new = NULL).  For
 * request r, head h:
 *   s_t = sm_scale * <q_h, c^_t>,  o_h = sum_t softmax(s)_t c^_t[0:512],
 * with c^ = dec(c) * scale for the FP8 cache (one per-tensor scale) and
 * c^ = c for BF16; fp32 result rounded to bf16.
 *   q bf16 [B][Hq][576]; out bf16 [B][Hq][512]; Hq a multiple of 16.
 *   Page ids, lengths, abort flags, splits and workspace behave as for
 *   paged_decode_attn_fp8 (with 32-token tiles: num_splits at most
 *   ceil(max_ctx_len/32); workspace from
 *   paged_decode_attn_workspace_bytes(B, Hq, 512, splits)).  With
 *   num_splits = 0 each cache type picks its own count (the FP8 kernel works
 *   on 64 heads per block, the BF16 one on 128);
 *   paged_decode_attn_latent_auto_splits returns the larger of the two, so a
 *   workspace sized with it fits either.  sm_scale 0 selects 1/sqrt(576). */
int32_t paged_decode_attn_latent_auto_splits(int32_t batch, int32_t num_q_heads, int32_t max_ctx_len);
int paged_decode_attn_latent_fp8(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                 const uint8_t* pool, const int32_t* page_table, int32_t pt_stride,
                                 const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                 const uint32_t* abort_flags, float scale, float sm_scale, int32_t num_splits,
                                 void* workspace, size_t workspace_bytes, uint16_t* out, hipStream_t stream);
int paged_decode_attn_latent_bf16(const kvfp8_pool_desc* desc, const uint16_t* q, int32_t num_q_heads,
                                  const uint16_t* pool, const int32_t* page_table, int32_t pt_stride,
                                  const int32_t* ctx_lens, int32_t batch, int32_t max_ctx_len,
                                  const uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                                  size_t workspace_bytes, uint16_t* out, hipStream_t stream);

/* ---------------------------------------------------------------- one decode step over a layer stack  [T][Q]
 * The attention part of a decode step for num_layers layers that share one
 * page table, one set of page tags, the context lengths and the abort flags
 * (a page id names the same logical slot in every layer's pool).  Layer l's
 * buffers are the l-th blocks of contiguous stacks:
 *   k_pools  [layers][K pool] (the latent pool for the latent cache);
 *   v_pools  [layers][V pool], or NULL for the latent cache (then v_new NULL);
 *   q        bf16 [layers][B][Hq][D];   out bf16 [layers][B][Hq][Dv];
 *   k_new    bf16 [layers][B][Hkv][D];  v_new bf16 [layers][B][Hkv][Dv];
 *   k_scales, v_scales (host) float [layers]: per-tensor scales of each
 *   layer's FP8 cache (the latent cache uses k_scales; both ignored, may be
 *   NULL, for BF16).
 * Each layer writes request r's token at position ctx_lens[r] - 1 and
 * attends.  With page_tags given, the tag check runs ONCE per step, as its
 * own batched launch before anything reads the cache [T]: layer 0's
 * kv_tag_check_append_* launch (check, then layer 0's write of every clean
 * request), then layer 0's attention reading the flags it left.  Every later
 * layer honours those flags (read, not rewritten) and is one attention launch
 * (plus the merge when split) that also writes the layer's token: GQA, the
 * block whose split holds position ctx_lens[r] - 1 quantises the token as
 * kv_append_fp8 does, stores it and adds it to its softmax from the values it
 * holds; latent, the block(s) holding it store it before copying any tile and
 * read it back with the rest.  With page_tags NULL (no-op tracker) there is
 * no check and layer 0 is such a launch too; abort_flags, when given, are
 * only read.
 * options (in the struct): KVFP8_STEP_FUSED_CHECK moves layer 0's check into
 * its attention launch (GQA and FP8 latent: every block checks all pages of
 * its request before it reads any, block (split 0, first head group) stores
 * the flag; the BF16 latent cache keeps the separate launch).  Same flags,
 * pools and outputs; one launch fewer.  Other bits: KVFP8_ERR_VALUE.
 * A request with ctx_lens[r] > max_ctx_len is a caller error: its flag is
 * computed as usual, its rows are zero and no layer writes its token.
 * Every layer's arguments are checked before the first launch, so an error
 * status means nothing was enqueued.  The workspace is shared by the layers
 * (stream order); size it, and zero it once, as for one layer's attention.  sm_scale 0 selects
 * 1/sqrt(score dim).  Other shapes, limits and outputs as for the per-layer
 * calls above.  In a model the layers' q and new rows come from the layer
 * below; here they are given up front (the projections between layers are
 * not this library's). */
#define KVFP8_STEP_FUSED_CHECK 1u

typedef struct kvfp8_layer_stack {
  int32_t num_layers;
  void* k_pools;
  void* v_pools;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* k_scales; /* host */
  const float* v_scales; /* host */
  uint16_t* out;
  uint32_t options;      /* 0, or KVFP8_STEP_FUSED_CHECK */
} kvfp8_layer_stack;

int kv_decode_step_fp8(const kvfp8_pool_desc* desc, const kvfp8_layer_stack* layers, int32_t num_q_heads,
                       const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                       int32_t max_ctx_len, const uint32_t* page_tags, const uint32_t* expected_tags,
                       uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);
int kv_decode_step_bf16(const kvfp8_pool_desc* desc, const kvfp8_layer_stack* layers, int32_t num_q_heads,
                        const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens, int32_t batch,
                        int32_t max_ctx_len, const uint32_t* page_tags, const uint32_t* expected_tags,
                        uint32_t* abort_flags, float sm_scale, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- page allocator  [T]
 * Host-side free list over the P pages of a pool, holding the page tags of the
 * integrity check (agentlenshq summary of the Cloudflare post, section "KV Cache
 * 完整性检查"; xujun.org note, section "一个不能出错的共享缓存": a page's tag
 * changes when the page gets a new owner, so a request still holding the old
 * (page, tag) pair fails the next kv_tag_check and is aborted).
 *   - Each allocation of a page adds 1 (mod 2^32) to its tag; freeing leaves the
 *     tag as it is.  Pages come off a stack: last freed, first handed out; a
 *     fresh allocator hands out 0, 1, 2, ... in order.
 *   - The state is a caller-owned host buffer of kv_page_alloc_state_bytes(P)
 *     bytes, 4-byte aligned, set up by kv_page_alloc_init (initial_tags: host
 *     [P] or NULL for zeros).  Host memory only: no HIP call, no allocation,
 *     not thread-safe.  Copy kv_page_alloc_tags to the device page_tags array
 *     before the next kv_tag_check.
 *   - kv_page_alloc: n pages into pages[n] with their new tags in tags[n]
 *     (tags may be NULL); KVFP8_ERR_NOSPACE (nothing taken) if fewer than n are
 *     free.  kv_page_free: KVFP8_ERR_VALUE (nothing freed) if any page is out of
 *     range, not allocated, or listed twice.  kv_page_alloc_free_count returns
 *     the number of free pages, or -1 for an uninitialised state. */
size_t kv_page_alloc_state_bytes(int32_t num_pages);
int kv_page_alloc_init(void* state, size_t state_bytes, int32_t num_pages, const uint32_t* initial_tags);
int32_t kv_page_alloc_free_count(const void* state);
int kv_page_alloc(void* state, int32_t n, int32_t* pages, uint32_t* tags);
int kv_page_free(void* state, const int32_t* pages, int32_t n);
int kv_page_alloc_tags(const void* state, uint32_t* tags);

/* ---------------------------------------------------------------- read-rate calibration
 * Read-only kernels that measure the HBM read rate attainable on the device,
 * against which the attention kernels' KV-read rates are also reported (no
 * page describes them; they compute nothing of the method).  Both read every
 * byte once with 16-byte non-temporal loads and fold the 32-bit words read
 * into XOR checksums: every thread block of the launch XORs its fold into one
 * of the KVFP8_READ_SINK_WORDS uint32 words of sink (device, 4-byte aligned),
 * so that, with the words zeroed by the caller beforehand, the XOR of them all
 * equals the XOR of every 32-bit word read.
 *   kv_read_stream: bytes consecutive bytes at src (16-byte aligned; bytes a
 *     multiple of 4).
 *   kv_read_blocks: for k < n_ids, the block_bytes bytes at
 *     base + ids[k] * block_bytes (ids int32 on the device; an id outside
 *     [0, num_blocks) is skipped); block_bytes a multiple of 16, base 16-byte
 *     aligned.  With ids listing the (page, kv head) blocks a decode step
 *     reads, in the order of its page table, this is the attention's access
 *     pattern without its arithmetic.
 * Sizes beyond 2^44 bytes (kv_read_stream) or 2^35 KiB-pieces of blocks
 * (kv_read_blocks) return KVFP8_ERR_SHAPE. */
#define KVFP8_READ_SINK_WORDS 2048
int kv_read_stream(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
int kv_read_blocks(const void* base, int64_t num_blocks, int64_t block_bytes, const int32_t* ids, int64_t n_ids,
                   uint32_t* sink, hipStream_t stream);

/* ---------------------------------------------------------------- test export
 * Read back tokens through the page table: k_out [N][Hkv][D], v_out
 * [N][Hkv][Dv] (v_out NULL for the latent cache) receive the stored
 * elements of token (tok_req[n], tok_pos[n]); a token whose request,
 * position or page is out of range gets zero elements.  v_pool NULL reads
 * k_pool as a latent pool. */
int kv_gather_fp8(const kvfp8_pool_desc* desc, const uint8_t* k_pool, const uint8_t* v_pool,
                  const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens,
                  const int32_t* page_table, int32_t batch, int32_t pt_stride, uint8_t* k_out,
                  uint8_t* v_out, hipStream_t stream);
int kv_gather_bf16(const kvfp8_pool_desc* desc, const uint16_t* k_pool, const uint16_t* v_pool,
                   const int32_t* tok_req, const int32_t* tok_pos, int32_t n_tokens,
                   const int32_t* page_table, int32_t batch, int32_t pt_stride, uint16_t* k_out,
                   uint16_t* v_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVFP8_H */
