// Kernel argument blocks and launchers shared between the kernels and the
// host-side C ABI (api.hip).  Not part of the public interface.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

struct AttnArgs {
  const uint16_t* q;          // bf16 [B][Hq][D]
  const void* k_pool;         // [P][Hkv][S][D]
  const void* v_pool;         // [P][Hkv][Dv][S]
  const int32_t* page_table;  // [B][pt_stride]
  const int32_t* ctx_lens;    // [B]
  const uint32_t* flags;      // [B] or null
  float* o_part;              // [B][Hq][num_splits][Dv] (num_splits > 1)
  float* lse_part;            // [B][Hq][num_splits]
  uint32_t* count;            // [B][Hkv] finished split blocks (merge_here): zero before and after a launch
  int32_t merge_here;         // several splits merged by the launch itself (else by a merge launch after it)
  uint16_t* out;              // bf16 [B][Hq][Dv]
  int32_t num_pages, page_size, num_kv_heads, group, num_q_heads, pt_stride;
  int32_t chunk_tiles;        // 64-token tiles per split
  int32_t num_splits;
  int32_t max_ctx;
  float qk_scale_log2;        // sm_scale * k_scale * log2(e)
  float v_scale;
  // Optional: this step's new token of every request (bf16 rows [B][Hkv][D] / [B][Hkv][Dv]), written
  // at position ctx_lens[r] - 1 by the block whose chunk holds it and folded into that block's softmax
  // from registers (null: the token is already in the pool).  k_inv, v_inv: fl32(1/scale) (FP8).
  const uint16_t* k_new;
  const uint16_t* v_new;
  float k_inv, v_inv;
  // Optional: the pages' tag check in the same launch (page_tags non-null; flags then null).  Every
  // block checks all pages of its request before it reads any; block (split 0, head 0) stores the
  // request's flag in flags_out, which the merge launch reads.
  const uint32_t* page_tags;  // [P]
  const uint32_t* expected;   // [B][pt_stride]
  uint32_t* flags_out;        // [B]
};

struct MergeArgs {
  const float* o_part;
  const float* lse_part;
  uint16_t* out;
  const int32_t* ctx_lens;
  const uint32_t* flags;
  int32_t num_q_heads, v_dim, num_splits, chunk_tokens, max_ctx, pt_stride, page_size;
  // part_f16: the partials are fp16 (in o_part's first half, same indices) and the merged row is multiplied
  // by out_scale (the FP8 latent cache: its partials are convex combinations of e4m3 values, |x| <= 448,
  // stored before the tensor scale); otherwise fp32 partials and out_scale 1
  int32_t part_f16;
  float out_scale;
  int64_t rows;  // batch * num_q_heads (set by launch_merge)
};

struct AppendArgs {
  void* k_pool;
  void* v_pool;               // null for the latent cache
  const uint16_t* k_new;      // bf16 [N][Hkv][D]
  const uint16_t* v_new;      // bf16 [N][Hkv][Dv]
  const int32_t* tok_req;
  const int32_t* tok_pos;
  const int32_t* page_table;
  const uint32_t* flags;
  int32_t n_tokens, batch, pt_stride;
  int32_t num_pages, page_size, num_kv_heads, head_dim, v_dim;
  float k_inv, v_inv;         // fl32(1/scale)
};

struct GatherArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* tok_req;
  const int32_t* tok_pos;
  const int32_t* page_table;
  void* k_out;
  void* v_out;
  int32_t n_tokens, batch, pt_stride;
  int32_t num_pages, page_size, num_kv_heads, head_dim, v_dim;
};

struct TagArgs {
  const uint32_t* page_tags;
  const int32_t* page_table;
  const uint32_t* expected;
  const int32_t* ctx_lens;
  uint32_t* flags;
  int32_t num_pages, pt_stride, batch, page_size;
  // check + write launch only: a request longer than this (the attention grid's bound) keeps its flag
  // but its token is not written, as the attention launches of a decode step treat it (0: no bound)
  int32_t max_ctx;
};

struct LatentArgs {
  const uint16_t* q;          // bf16 [B][Hq][576]
  const void* pool;           // row-major pool [P][S][576]
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const uint32_t* flags;
  float* o_part;              // [B][Hq][num_splits][512]
  float* lse_part;            // [B][Hq][num_splits]
  uint16_t* out;              // bf16 [B][Hq][512]
  int32_t num_pages, page_size, num_q_heads, pt_stride;
  int32_t chunk_tiles;        // 32-token tiles per split
  int32_t num_splits, max_ctx, batch, n_hg;
  float qk_scale_log2;        // sm_scale * scale * log2(e)
  float v_scale;
  // Optional (later layers of a decode step): this step's new latent row of every request (bf16
  // [B][576]), written at position ctx_lens[r] - 1 by the block(s) whose chunk holds it before they
  // copy any tile, so their copies read it back (null: the token is already in the pool).  c_inv:
  // fl32(1/scale) for the FP8 cache, as the append computes it.
  const uint16_t* c_new;
  float c_inv;
  // Optional: the pages' tag check in the same launch (page_tags non-null; flags then null).  Every
  // block checks all pages of its request before it reads or writes any; block (split 0, head group
  // 0) stores the request's flag in flags_out, which the merge launch reads.
  const uint32_t* page_tags;  // [P]
  const uint32_t* expected;   // [B][pt_stride]
  uint32_t* flags_out;        // [B]
};

constexpr int kAttnTileTokens = 64;
constexpr int kLatentTileTokens = 32;
constexpr int kLatentDim = 576;
constexpr int kLatentVDim = 512;
constexpr int kLatentHeadsPerBlock = 128;

hipError_t launch_attn_gqa(const AttnArgs& a, bool fp8, int batch, hipStream_t stream);
// pairs (FP8 only): the wave-pair kernel on 64-head groups (a.n_hg counts them) instead of the 128-head one
hipError_t launch_attn_latent(const LatentArgs& a, bool fp8, bool pairs, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& m, int batch, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_tag_check(const TagArgs& a, hipStream_t stream);
hipError_t launch_check_append(const TagArgs& c, const AppendArgs& a, bool fp8, hipStream_t stream);
constexpr int kCheckAppendMaxPairs = 8 * 256;  // (Hkv*D)/2 and (Hkv*Dv)/2 limit of the fused kernel
hipError_t launch_absmax(const uint16_t* x, int64_t n, uint32_t* out, hipStream_t stream);
constexpr int kReadSinkWords = 2048;  // checksum words of the read-rate kernels
hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_read_blocks(const void* base, int64_t num_blocks, const int32_t* ids, int64_t n_ids,
                              int64_t block_bytes, uint32_t* sink, hipStream_t stream);

}  // namespace kvfp8
