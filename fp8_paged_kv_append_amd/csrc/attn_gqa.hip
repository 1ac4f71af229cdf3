// Split-K paged decode attention over an FP8 (e4m3) or BF16 KV cache, GQA,
// head_dim 128, for gfx950.
//
// What it computes (Cloudflare blog "Smaller, faster, safer: running Kimi and
// GLM at scale", section "Quantized KV cache"): for every request and query
// head, softmax attention of the one decode query over the cached K/V of the
// request's context, with the FP8 cache converted to floating point as it is
// read from the pages.  Split-K with an online softmax and a log-sum-exp
// merge is an exact rewrite of that softmax up to rounding.
//
// Work decomposition.  Block = (split c, KV head g, request r), 4 waves.  The
// block's token range [c0, c1) is cut into 64-token tiles; wave w takes tiles
// w, w+4, ...  A tile is four 16-token sub-pages (a page of 16, or a quarter
// of a page of 64).  The G <= 16 query heads of group g are the 16 columns of
// every MFMA (G = 8 fills half of them).
//
// Per tile, with lane = 16*q + n (q = lane group 0..3, n = 0..15):
//  * QK^T: four v_mfma_f32_16x16x32_bf16 chains S_s (s = 0..3), A = K rows,
//    B = q^T.  Row m of chain s is token (sub-page m/4, position 4s + m%4);
//    the contraction index of lane group q, k-step kk, slot j is dimension
//    32q + 8kk + j (any permutation of the head dimension is valid as long as
//    both operands use it).  Lane (q, n) loads 32 bytes (64 for bf16) of
//    each of its 4 K rows; the K pool keeps those bytes as 16-byte chunks
//    256 bytes apart, so that each load instruction of the wave reads four
//    runs of 256 contiguous bytes (one per page) instead of 64 half lines.
//  * C layout of a 16x16 MFMA: lane (q, n) holds rows 4q..4q+3 of column n,
//    so it ends up with head n's scores for sub-page q, positions 4s+i: the
//    sixteen tokens of sub-page q.
//  * PV: O^T[d][head] += V^T[d][tok] P^T[tok][head] with eight d-blocks j and
//    two k-blocks kb; lane group q supplies sub-page q, positions 8kb..8kb+7,
//    which is exactly the P it already holds (no shuffle) and 8 consecutive
//    bytes of a V^T row.  That is why V pages are stored transposed
//    ([d][slot] per page and head): the load is one 16-byte read per d row.
//  * Online softmax per head n in the log2 domain; only the tile max needs
//    cross-lane traffic (two xor shuffles).  The accumulator layout (column =
//    head n) keeps the rescale lane-local, and it is lazy: it runs only when
//    a head's running max grows by more than 2^8.
// The four waves merge their (m, l, O) through LDS; with one split the block
// writes bf16 output, otherwise normalised fp32 partials and lse for the merge
// kernel.
//
// The same launch can be the whole decode step of a layer (Cloudflare blog,
// section "Quantized KV cache", for the conversion on read; the tag check of
// the agentlenshq summary, section "KV Cache 完整性检查"): with page tags given,
// every block first checks all pages of its request (the flag bits of the
// batched check) before it reads any of them, and block (split 0, head 0)
// stores the flag; with the step's new rows given, the block whose chunk holds
// position L - 1 quantises the token as the append does (staged in LDS at the
// start), stores it in its page in the epilogue, and adds its score and value
// to the merged softmax -- its tiles stop before L - 1, so nothing reads the
// token back.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kTile = 64;
constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLazy = 8.f;  // log2-domain slack before the accumulators are rescaled

// --- per-dtype loads and operand conversions -------------------------------------------------

template <bool FP8>
struct KRow;  // one lane's slice of one K row
// Streaming loads: every KV byte is read once per step, so they bypass cache retention.
__device__ __forceinline__ u32x4_t ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// K rows live in chunk-reordered sub-page blocks: a lane's k-th 16-byte chunk of its row is
// 256*k bytes after its first one (see k_elem_offset).
template <>
struct KRow<true> {
  u32x4_t w[2];  // 32 bytes: dims 32q .. 32q+31
  __device__ __forceinline__ void load(const uint8_t* p) {
    w[0] = ld_stream(p);
    w[1] = ld_stream(p + 256);
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ bf16x8_t op(int kk) const {
    const u32x4_t& x = w[kk >> 1];
    uint32_t a = x[(kk & 1) * 2], b = x[(kk & 1) * 2 + 1];
    u32x2_t lo = e4m3x4_to_bf16x4(a), hi = e4m3x4_to_bf16x4(b);
    u32x4_t r = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8_t, r);
  }
};
template <>
struct KRow<false> {
  u32x4_t w[4];  // 64 bytes: dims 32q .. 32q+31 as bf16
  __device__ __forceinline__ void load(const uint8_t* p) {
    w[0] = ld_stream(p);
    w[1] = ld_stream(p + 256);
    w[2] = ld_stream(p + 512);
    w[3] = ld_stream(p + 768);
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = w[2] = w[3] = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ bf16x8_t op(int kk) const { return __builtin_bit_cast(bf16x8_t, w[kk]); }
};

template <bool FP8>
struct VRow;  // one lane's slice of one V^T row: 16 consecutive slots
template <>
struct VRow<true> {
  u32x4_t w;  // 16 e4m3 codes
  __device__ __forceinline__ void load(const uint8_t* p) { w = ld_stream(p); }
  __device__ __forceinline__ void zero() { w = u32x4_t{0, 0, 0, 0}; }
  // keep slots < nv, zero the rest (nv in [0, 16])
  __device__ __forceinline__ void mask(int nv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int k = nv - 4 * i;
      uint32_t m = k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : ((1u << (8 * k)) - 1u));
      w[i] &= m;
    }
  }
  __device__ __forceinline__ f16x8_t op(int kb) const {
    u32x2_t lo = e4m3x4_to_f16x4(w[2 * kb]), hi = e4m3x4_to_f16x4(w[2 * kb + 1]);
    u32x4_t r = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(f16x8_t, r);
  }
};
template <>
struct VRow<false> {
  u32x4_t w[2];  // 16 bf16
  __device__ __forceinline__ void load(const uint8_t* p) {
    w[0] = ld_stream(p);
    w[1] = ld_stream(p + 16);
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ void mask(int nv) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int k = nv - 2 * i;
      uint32_t m = k >= 2 ? 0xFFFFFFFFu : (k <= 0 ? 0u : 0xFFFFu);
      w[i >> 2][i & 3] &= m;
    }
  }
  __device__ __forceinline__ bf16x8_t op(int kb) const { return __builtin_bit_cast(bf16x8_t, w[kb]); }
};

template <bool FP8>
__device__ __forceinline__ uint32_t pack_p(float a, float b) {
  return FP8 ? pack_f16x2(a, b) : pack_bf16x2(a, b);
}

template <bool FP8>
__device__ __forceinline__ f32x4_t mfma_pv(const VRow<FP8>& v, int kb, u32x4_t p, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma_pv<true>(const VRow<true>& v, int kb, u32x4_t p, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(v.op(kb), __builtin_bit_cast(f16x8_t, p), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma_pv<false>(const VRow<false>& v, int kb, u32x4_t p, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(v.op(kb), __builtin_bit_cast(bf16x8_t, p), c, 0, 0, 0);
}

// --- the split kernel ---------------------------------------------------------------------------

// Page ids of the block's token range are staged in LDS, at most kPidWin entries at a time.
constexpr int kPidWin = 2048;
// Page-table entries per thread whose loads are issued together (the first batch with the context
// length itself).
constexpr int kPtBatch = 4;

// One tile's loads for one lane, plus what the softmax needs to mask it.
template <bool FP8>
struct TileRegs {
  KRow<FP8> k[4];
  VRow<FP8> v[8];
  int nv;  // valid slots of this lane's V sub-page (0 when the tile or page is absent)
};

template <bool FP8>
__device__ __forceinline__ void issue_tile(TileRegs<FP8>& T, int tb, int w1, int e0, int ne, const int* s_pid,
                                           const uint8_t* kpool, const uint8_t* vpool, int64_t blk, int S,
                                           int lgS, int Hkv, int g, int q4, int n) {
  constexpr int ELT = FP8 ? 1 : 2;
  const int tok_k = tb + 16 * (n >> 2);
  const int tok_v = tb + 16 * q4;
  // LDS index clamped into the staged range, the result discarded past w1: no branch
  // (S a power of two: page and slot by shift and mask)
  const int ik = min((tok_k >> lgS) - e0, ne - 1), iv = min((tok_v >> lgS) - e0, ne - 1);
  const int sk = s_pid[ik], sv = s_pid[iv];
  const int pid_k = tok_k < w1 ? sk : -1;
  const int pid_v = tok_v < w1 ? sv : -1;
  // Absent or invalid pages read the pool's first bytes (one cached line per wave) and are
  // masked afterwards, so every tile issues the same loads with no branch around them.
  // offsets computed for max(pid, 0) and zeroed by a mask: arithmetic, not a branch
  // K: sub-page block base + lane (q4, i = n&3)'s first chunk of token 4s+i (byte offsets)
  const int64_t ko = ((((int64_t)max(pid_k, 0) * Hkv + g) * blk + (int64_t)(tok_k & (S - 1)) * kD) * ELT + 64 * q4 +
                      16 * (n & 3)) & -(int64_t)(pid_k >= 0);
  const int64_t vo = ((((int64_t)max(pid_v, 0) * Hkv + g) * blk + (int64_t)n * S + (tok_v & (S - 1))) * ELT) &
                     -(int64_t)(pid_v >= 0);
  const uint8_t* kb = kpool + ko;
  const uint8_t* vb = vpool + vo;
#pragma unroll
  for (int s = 0; s < 4; ++s) T.k[s].load(kb + 4 * s * kD * ELT);
#pragma unroll
  for (int j = 0; j < 8; ++j) T.v[j].load(vb + (int64_t)(16 * j) * S * ELT);
  T.nv = pid_v >= 0 ? max(0, min(16, w1 - tok_v)) : 0;
}

struct SoftmaxState {
  float m, l;
  f32x4_t acc[8];
};

template <bool FP8>
__device__ __forceinline__ void compute_tile(TileRegs<FP8>& T, const u32x4_t (&qv)[4], float c_log2,
                                             SoftmaxState& st) {
#pragma unroll
  for (int j = 0; j < 8; ++j) T.v[j].mask(T.nv);
  // S^T = K q^T, four chains of 16 tokens
  f32x4_t sc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    sc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[s].op(kk), __builtin_bit_cast(bf16x8_t, qv[kk]), sc[s],
                                                      0, 0, 0);
  }
  // online softmax for head n over the 16 tokens of sub-page q4 this lane holds
  float x[16];
  float tmax = -INFINITY;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = 4 * s + i;
      const float v = pos < T.nv ? sc[s][i] * c_log2 : -INFINITY;
      x[pos] = v;
      tmax = fmaxf(tmax, v);
    }
  tmax = max_x32(max_x16(tmax));
  // The accumulators stay referenced to st.m until a tile's max exceeds it by more than kLazy
  // (log2 units): p <= 2^kLazy meanwhile (exact up to rounding) and the rescale of the
  // AGPR-resident accumulators runs only when some head's max really grows.
  const bool grow = tmax > st.m + kLazy;  // st.m = -inf: any finite tile max grows it
  if (__any(grow)) {
    const float m_new = grow ? tmax : st.m;
    const float alpha = grow ? exp2f(st.m - m_new) : 1.f;  // st.m = -inf -> 0
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] *= alpha;
    st.m = m_new;
  }
  const float m_use = st.m == -INFINITY ? 0.f : st.m;
  float psum = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    x[k] = __builtin_amdgcn_exp2f(x[k] - m_use);  // v_exp_f32: weights below 2^-126 flush to 0
    psum += x[k];
  }
  st.l += psum;
  u32x4_t pp[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) pp[kb][e] = pack_p<FP8>(x[8 * kb + 2 * e], x[8 * kb + 2 * e + 1]);
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) st.acc[j] = mfma_pv<FP8>(T.v[j], kb, pp[kb], st.acc[j]);
}

// ---- split-K: the merge inside the attention launch -------------------------------------------
//
// With several splits every block stores its G rows' partials (o / l and lse) with device-coherent stores
// (sc1: they reach the point every XCD reads from, with no L2 writeback), waits for them and counts itself
// finished for its (request, KV head); the block that finishes last merges all splits' partials into the
// bf16 output, reading them with device-coherent loads, and sets the count back to zero.  The counts sit
// at the head of the workspace, one per 128-byte line (kCountStride words apart): zero before a launch,
// zero after it.  Counts that shared a line made the blocks of different KV heads queue on it (one
// request, 61 layers: 16 splits 12.84 -> 12.68 us per layer; 24 / 32 splits merged here 14.5 / 15.7 ->
// 13.7 / 14.2 us).  FP8 partials are fp16 in units of the e4m3 codes: o / l is a convex combination of
// decoded codes (|x| <= 448, no overflow, rounding at most 2^-11 relative) and the merge applies v_scale; half
// the bytes of fp32 partials to store and to merge (12.74 -> 12.64 us per layer).  BF16 partials are fp32.
constexpr int kCohAux = 16;       // cache-policy operand of a buffer access: sc1
constexpr int kMergeGroup = 16;   // splits whose lse and partials are loaded together
constexpr int kCountStride = 32;  // words between two split counts
constexpr uint32_t kOffOOB = 0x80000000u;  // a buffer offset past the buffer: the load returns 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// The LSE merge of rows row0 .. row0 + G - 1 over the splits, as the separate merge kernel computes it:
// splits in groups of kMergeGroup, all of a group's loads issued before any is used, later groups
// rescaling the running sums to the new maximum; a split that saw a bad page (lse NaN) zeroes the row.
template <bool F16>
__device__ __forceinline__ void merge_rows_in_launch(const AttnArgs& a, int r, int g, int L, bool zero_rows) {
  const int G = a.group, S = a.num_splits;
  const int64_t row0 = (int64_t)r * a.num_q_heads + (int64_t)g * G;
  constexpr int kEB = F16 ? 2 : 4;  // bytes per partial element
  const __amdgpu_buffer_rsrc_t orc = coh_rsrc(reinterpret_cast<const uint8_t*>(a.o_part) + row0 * S * kD * kEB,
                                              (int64_t)G * S * kD * kEB);
  const __amdgpu_buffer_rsrc_t lrc = coh_rsrc(a.lse_part + row0 * S, (int64_t)G * S * 4);
  const int chunk = a.chunk_tiles * kTile;
  const int nvalid = zero_rows ? 0 : min(S, (L + chunk - 1) / chunk);
  for (int t = threadIdx.x; t < G * (kD / 4); t += kThreads) {
    const int hn = t / (kD / 4), d = 4 * (t % (kD / 4));
    float M = -INFINITY, s = 0.f;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    bool nan = false;
    for (int c0 = 0; c0 < nvalid; c0 += kMergeGroup) {
      float x[kMergeGroup];
      f32x4_t pv[kMergeGroup];
      u32x2_t ph[kMergeGroup];
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        const int c = c0 + j;
        const bool in = c < nvalid;
        const uint32_t lo = in ? (uint32_t)(hn * S + c) * 4u : kOffOOB;
        const uint32_t po = in ? (uint32_t)(((int64_t)(hn * S + c) * kD + d) * kEB) : kOffOOB;
        const uint32_t xl = __builtin_amdgcn_raw_buffer_load_b32(lrc, lo, 0, kCohAux);
        if constexpr (F16)
          ph[j] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(orc, po, 0, kCohAux));
        else
          pv[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(orc, po, 0, kCohAux));
        x[j] = in ? __uint_as_float(xl) : -INFINITY;
      }
      float gm = M;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        nan |= x[j] != x[j];
        gm = fmaxf(gm, x[j]);
      }
      if (gm == -INFINITY) continue;  // nothing but empty splits so far
      const float rs = exp2f(M - gm);  // 0 while M is still -inf
      s *= rs;
      o *= rs;
#pragma unroll
      for (int j = 0; j < kMergeGroup; ++j) {
        const float f = exp2f(x[j] - gm);
        s += f;
        if constexpr (F16) {
          const uint32_t w0 = ph[j][0], w1 = ph[j][1];
          const f32x4_t v = {(float)__builtin_bit_cast(_Float16, (uint16_t)(w0 & 0xFFFFu)),
                             (float)__builtin_bit_cast(_Float16, (uint16_t)(w0 >> 16)),
                             (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 & 0xFFFFu)),
                             (float)__builtin_bit_cast(_Float16, (uint16_t)(w1 >> 16))};
          o += f * v;
        } else {
          o += f * pv[j];
        }
      }
      M = gm;
    }
    if (nan || zero_rows) {
      s = 0.f;
      o = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float inv = s > 0.f ? (F16 ? a.v_scale : 1.f) / s : 0.f;
    *reinterpret_cast<u32x2_t*>(a.out + (row0 + hn) * kD + d) =
        u32x2_t{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
  }
}

template <bool FP8>
// At least two waves per SIMD (eight per CU, two blocks): the register budget the tile pipeline is
// written for.
__global__ __launch_bounds__(kThreads, 2) void attn_gqa_split_kernel(AttnArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  // wave index in an SGPR: the tile loop is then a scalar loop, not an exec-masked one
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int q4 = lane >> 4, n = lane & 15;
  const int G = a.group;
  const int S = a.page_size;
  const int lgS = __builtin_ctz(S);   // S is a power of two (checked on the host)

  __shared__ int s_pid[kPidWin];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_acc[kWaves][16][kD];
  __shared__ int s_bad;
  __shared__ float s_knew[kD], s_vnew[kD], s_snew[16];
  __shared__ uint16_t s_kcode[kD], s_vcode[kD];
  __shared__ int s_newpage;
  __shared__ uint32_t s_flag[kWaves];
  __shared__ uint32_t s_last;

  const int chunk = a.chunk_tiles * kTile;
  const int c0 = split * chunk;
  const bool check = a.page_tags != nullptr;
  const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
  const uint32_t* ex = check ? a.expected + (int64_t)r * a.pt_stride : nullptr;
  // Page-table words the block reads whatever the context length turns out to be are loaded
  // together with that length, not after it: with the check, the row's first kPtBatch * kThreads
  // entries (all checked); without it, the first entries of this split's chunk (its first
  // page-id window).  Every row holds pt_stride entries, so these loads stay inside the table;
  // no KV page is read before its tag has been checked.
  const int64_t sbase = check ? 0 : c0 / S;
  int32_t sp[kPtBatch];
  uint32_t se[kPtBatch];
#pragma unroll
  for (int j = 0; j < kPtBatch; ++j) {
    const int64_t i = sbase + threadIdx.x + j * kThreads;
    const bool in = i < a.pt_stride;
    sp[j] = in ? pt[i] : -1;
    se[j] = (check && in) ? ex[i] : 0u;
  }
  const int L = a.ctx_lens[r];
  // q^T operand: lane (q4, n) holds head g*G+n, dims 32*q4 .. 32*q4+31 (zero for padding heads);
  // issued first, so that its latency overlaps the tag check
  u32x4_t qv[4];
  if (n < G) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(
        a.q + ((int64_t)r * a.num_q_heads + g * G + n) * kD + 32 * q4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qv[kk] = qp[kk];
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qv[kk] = u32x4_t{0, 0, 0, 0};
  }

  // The step's token, when passed in, belongs to position L - 1: the block whose chunk holds it
  // writes it into its page and adds it to its softmax from LDS (its tiles stop before it, so
  // nothing reads it back).  Its rows and its page id are loaded now, staged after the check.
  const bool fold = a.k_new != nullptr;
  const bool owner = fold && L > 0 && c0 <= L - 1 && L - 1 < c0 + chunk;
  uint32_t kb = 0, vb = 0;
  int newpage = -1;
  if (owner) {
    const int64_t row = ((int64_t)r * a.num_kv_heads + g) * kD;
    if (threadIdx.x < kD) {
      kb = a.k_new[row + threadIdx.x];
      vb = a.v_new[row + threadIdx.x];
    }
    if ((L - 1) / S < a.pt_stride) newpage = a.page_table[(int64_t)r * a.pt_stride + (L - 1) / S];
  }

  // this block's token range and its first page-id window ([c0, c1) is empty past the context)
  const int c1 = min(fold ? L - 1 : L, c0 + chunk);
  // tokens per page-id window: a multiple of the tile, at most kPidWin - 1 pages long, so that even
  // a window that does not start on a page boundary touches at most kPidWin pages
  const int win = ((kPidWin - 1) * S / kTile) * kTile;
  const int fe0 = c0 / S;
  const int fne = c0 < c1 ? (min(c1, c0 + win) - 1) / S - fe0 + 1 : 0;

  uint32_t checked = 0;
  if (check) {
    // the tag check of every page request r's context spans, before any of them is read: bit 0 a
    // page whose tag differs from the one the request recorded, bit 1 a page id out of the pool or
    // a context longer than the page table.  Entries go in batches of kPtBatch per thread whose
    // loads, then tag gathers, are all issued before any is used; the entries of this block's
    // first window are staged in LDS on the way (for a request that passes they lie inside the
    // `need` entries checked here).
    uint32_t f = 0;
    if (L > 0) {
      const int64_t need = ((int64_t)L + S - 1) / S;
      const int64_t np = min(need, (int64_t)a.pt_stride);
      if (need > a.pt_stride) f |= 2u;
      for (int64_t base = 0; base < np; base += kPtBatch * kThreads) {
        int32_t pg[kPtBatch];
        uint32_t ev[kPtBatch], tv[kPtBatch];
#pragma unroll
        for (int jj = 0; jj < kPtBatch; ++jj) {
          const int64_t i = base + threadIdx.x + jj * kThreads;
          if (base == 0) {
            pg[jj] = sp[jj];
            ev[jj] = se[jj];
          } else {
            pg[jj] = i < np ? pt[i] : -1;
            ev[jj] = i < np ? ex[i] : 0u;
          }
        }
#pragma unroll
        for (int jj = 0; jj < kPtBatch; ++jj) {
          const int64_t i = base + threadIdx.x + jj * kThreads;
          const bool ok = pg[jj] >= 0 && pg[jj] < a.num_pages;
          tv[jj] = (i < np && ok) ? a.page_tags[pg[jj]] : 0u;
        }
#pragma unroll
        for (int jj = 0; jj < kPtBatch; ++jj) {
          const int64_t i = base + threadIdx.x + jj * kThreads;
          if (i < np) {
            const bool ok = pg[jj] >= 0 && pg[jj] < a.num_pages;
            if (!ok)
              f |= 2u;
            else if (tv[jj] != ev[jj])
              f |= 1u;
            const int64_t k = i - fe0;
            if (k >= 0 && k < fne) s_pid[k] = ok ? pg[jj] : -1;
          }
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) f |= shfl_xor(f, m);
    if (lane == 0) s_flag[wave] = f;
    __syncthreads();
    checked = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
    if (split == 0 && g == 0 && threadIdx.x == 0) a.flags_out[r] = checked;
  }
  if (owner) {  // quantised as the append does; the decoded values are what the pool will hold
    if (threadIdx.x < kD) {
      const int d = threadIdx.x;
      if (FP8) {
        const uint32_t kc = encode_e4m3x2(bf16_bits_to_f32(kb) * a.k_inv, 0.f) & 0xFFu;
        const uint32_t vc = encode_e4m3x2(bf16_bits_to_f32(vb) * a.v_inv, 0.f) & 0xFFu;
        s_kcode[d] = (uint16_t)kc;
        s_vcode[d] = (uint16_t)vc;
        s_knew[d] = e4m3_to_f32(kc);
        s_vnew[d] = e4m3_to_f32(vc);
      } else {
        s_kcode[d] = (uint16_t)kb;
        s_vcode[d] = (uint16_t)vb;
        s_knew[d] = bf16_bits_to_f32(kb);
        s_vnew[d] = bf16_bits_to_f32(vb);
      }
    }
    if (threadIdx.x == 0) s_newpage = newpage;
  }
  const bool aborted = checked != 0u || (a.flags != nullptr && a.flags[r] != 0u);
  const bool bad_len = L <= 0 || L > a.max_ctx || L > a.pt_stride * S;
  // several splits: count this block finished (its partials, if any, stored); the last one merges
  auto finish = [&](bool zero_rows) {
    __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores are complete before the block counts
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t* cnt = a.count + ((int64_t)r * a.num_kv_heads + g) * kCountStride;
      const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = done == (uint32_t)(a.num_splits - 1);
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last ? 1u : 0u;
    }
    __syncthreads();
    if (s_last != 0u) merge_rows_in_launch<FP8>(a, r, g, L, zero_rows);
  };
  if (aborted || bad_len) {
    if (a.num_splits == 1) {  // rows of this group are zero
      for (int e = threadIdx.x; e < G * kD; e += kThreads)
        a.out[((int64_t)r * a.num_q_heads + g * G + e / kD) * kD + e % kD] = 0;
    } else if (a.merge_here) {
      finish(true);  // the last split block zeroes the rows
    }
    return;  // (else the merge launch zeroes them)
  }
  if (c0 >= L) {  // past this request's context: no partials, and the merge does not read this split
    if (a.merge_here) finish(false);
    return;
  }

  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v_pool);
  const int64_t blk = (int64_t)S * kD;  // elements per (page, head) block
  const float c_log2 = a.qk_scale_log2;

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  for (int w0 = c0; w0 < c1; w0 += win) {
    const int w1 = min(c1, w0 + win);
    const int e0 = w0 / S;
    const int ne = (w1 - 1) / S - e0 + 1;  // entries of the pages holding [w0, w1)
    __syncthreads();                       // the previous window's ids are no longer read
    if (!(check && w0 == c0)) {            // with the check, the first window's ids are staged;
      const bool first = w0 == c0;         // without it, its first batch was loaded with L
      for (int base = 0; base < ne; base += kPtBatch * kThreads) {
#pragma unroll
        for (int jj = 0; jj < kPtBatch; ++jj) {
          const int i = base + threadIdx.x + jj * kThreads;
          if (i < ne) {
            int p = (first && base == 0) ? sp[jj] : pt[e0 + i];
            if (p < 0 || p >= a.num_pages) {
              bad = true;
              p = -1;
            }
            s_pid[i] = p;
          }
        }
      }
    }
    __syncthreads();
    const int ntile = (w1 - w0 + kTile - 1) / kTile;
    int t = wave;
#define KVFP8_ISSUE(T_, t_) \
  issue_tile<FP8>(T_, w0 + (t_) * kTile, w1, e0, ne, s_pid, kpool, vpool, blk, S, lgS, a.num_kv_heads, g, q4, n)
    if (FP8) {
      // Two tiles in flight per wave (A older than B).  The first two are issued whatever the wave's
      // count (a tile past the end reads masked copies of the pool's first line); after them no refill
      // goes past the wave's last tile -- such loads still cost their issue and return, and the block's
      // final wait waits for them.  The loop runs while both refills lie inside; the last two or three
      // tiles form a tail after it, the third issued only if it exists (a branch after the loop, so the
      // loop's load counts stay exact).
      const int nt = wave < ntile ? (ntile - wave + kWaves - 1) / kWaves : 0;  // this wave's tiles
      TileRegs<FP8> A, B;
      KVFP8_ISSUE(A, t);
      __builtin_amdgcn_sched_barrier(0);
      KVFP8_ISSUE(B, t + kWaves);
      __builtin_amdgcn_sched_barrier(0);
      int i = 0;
      for (; i + 4 <= nt; i += 2) {
        compute_tile<FP8>(A, qv, c_log2, st);
        KVFP8_ISSUE(A, t + (i + 2) * kWaves);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile<FP8>(B, qv, c_log2, st);
        KVFP8_ISSUE(B, t + (i + 3) * kWaves);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i + 2 <= nt) {
        compute_tile<FP8>(A, qv, c_log2, st);
        if (i + 3 == nt) KVFP8_ISSUE(A, t + (i + 2) * kWaves);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile<FP8>(B, qv, c_log2, st);
        i += 2;
      }
      if (i < nt) compute_tile<FP8>(A, qv, c_log2, st);
    } else {
      // bf16 tiles are twice as large: one tile in flight per wave
      for (; t < ntile; t += kWaves) {
        TileRegs<FP8> A;
        KVFP8_ISSUE(A, t);
        compute_tile<FP8>(A, qv, c_log2, st);
      }
    }
#undef KVFP8_ISSUE
  }

  // ---- merge the four waves
  float l_run = st.l;
  l_run = sum_x32(sum_x16(l_run));
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (owner) {
    // the token into its page (a bad page id only marks the rows, as a bad page of the tiles does)
    const int page = s_newpage;
    const bool ok = page >= 0 && page < a.num_pages;
    if (!ok) bad = true;
    if (ok && threadIdx.x < kD) {
      const int d = threadIdx.x, slot = (L - 1) % S, H = a.num_kv_heads;
      const int64_t ko = k_elem_offset<FP8 ? 1 : 2>(page, g, slot, d, H, S, kD);
      const int64_t vo = ((int64_t)page * H + g) * kD * S + (int64_t)d * S + slot;
      if (FP8) {
        const_cast<uint8_t*>(kpool)[ko] = (uint8_t)s_kcode[d];
        const_cast<uint8_t*>(vpool)[vo] = (uint8_t)s_vcode[d];
      } else {
        reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(kpool))[ko] = s_kcode[d];
        reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(vpool))[vo] = s_vcode[d];
      }
    }
    // its score per head, log2 domain like the tiles', from the q operand lane (q4, n) holds:
    // head n, dims 32 q4 + 8 kk + j
    float dot = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = qv[kk][e];
        const int d = 32 * q4 + 8 * kk + 2 * e;
        dot += __uint_as_float(w << 16) * s_knew[d] + __uint_as_float(w & 0xFFFF0000u) * s_knew[d + 1];
      }
    dot = sum_x32(sum_x16(dot));
    if (q4 == 0 && n < G) s_snew[n] = dot * c_log2;
  }
  if (q4 == 0) {
    s_m[wave][n] = st.m;
    s_l[wave][n] = l_run;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<f32x4_t*>(&s_acc[wave][n][16 * j + 4 * q4]) = st.acc[j];
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;

  const int Hq = a.num_q_heads;
  const int64_t row0 = (int64_t)r * Hq + (int64_t)g * G;
  constexpr int kEB = FP8 ? 2 : 4;  // bytes per partial element: fp16 (FP8 cache) or fp32
  const __amdgpu_buffer_rsrc_t orc = coh_rsrc(reinterpret_cast<const uint8_t*>(a.o_part) + row0 * a.num_splits * kD * kEB,
                                              (int64_t)G * a.num_splits * kD * kEB);
  const __amdgpu_buffer_rsrc_t lrc = coh_rsrc(a.lse_part + row0 * a.num_splits, (int64_t)G * a.num_splits * 4);
  for (int e = threadIdx.x; e < G * kD; e += kThreads) {
    const int hn = e / kD, d = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hn]);
    if (owner) M = fmaxf(M, s_snew[hn]);
    float lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(s_m[w][hn] - M);
        lsum += s_l[w][hn] * f;
        o += s_acc[w][hn][d] * f;
      }
      if (owner) {
        const float f = exp2f(s_snew[hn] - M);
        lsum += f;
        o += s_vnew[d] * f;
      }
    }
    const int64_t row = (int64_t)r * Hq + g * G + hn;
    if (a.num_splits == 1) {
      const float val = (any_bad || lsum == 0.f) ? 0.f : o * (a.v_scale / lsum);
      a.out[row * kD + d] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
    } else {
      const uint32_t slot = (uint32_t)(hn * a.num_splits + split);   // inside the block's rows
      if constexpr (FP8) {
        const float ov = lsum == 0.f ? 0.f : o / lsum;
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_f16x2(ov, 0.f) & 0xFFFFu), orc,
                                              (slot * kD + d) * 2u, 0, kCohAux);
      } else {
        const float ov = lsum == 0.f ? 0.f : o * (a.v_scale / lsum);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), orc, (slot * kD + d) * 4u, 0, kCohAux);
      }
      if (d == 0) {
        const float lv = any_bad ? NAN : (lsum == 0.f ? -INFINITY : M + __log2f(lsum));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), lrc, slot * 4u, 0, kCohAux);
      }
    }
  }
  if (a.merge_here) finish(false);
}

// --- merge of the split partials ----------------------------------------------------------------

// One thread per VEC consecutive value dims of a (request, head) row (4 for fp32 partials, 8 for fp16
// partials: one 16-byte load of each split's partial either way); the rows of one block are consecutive,
// so a block reads contiguous partials.
constexpr int kMergeThreads = 128;

template <int kGroup, bool F16>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(MergeArgs a) {
  constexpr int VEC = F16 ? 8 : 4;
  const int tpr = a.v_dim / VEC;  // threads per row
  const int64_t row = (int64_t)blockIdx.x * (kMergeThreads / tpr) + threadIdx.x / tpr;  // r * Hq + h
  if (row >= a.rows) return;
  const int d = VEC * (threadIdx.x % tpr);
  const int r = (int)(row / a.num_q_heads);
  const int L = a.ctx_lens[r];
  const bool aborted = a.flags != nullptr && a.flags[r] != 0u;
  uint16_t* out = a.out + row * a.v_dim + d;
  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;
  auto store_out = [&](float scale) {
    uint32_t w[VEC / 2];
#pragma unroll
    for (int e = 0; e < VEC / 2; ++e) w[e] = pack_bf16x2(o[2 * e] * scale, o[2 * e + 1] * scale);
    if constexpr (F16)
      *reinterpret_cast<u32x4_t*>(out) = u32x4_t{w[0], w[1], w[2], w[3]};
    else
      *reinterpret_cast<u32x2_t*>(out) = u32x2_t{w[0], w[1]};
  };
  if (aborted || L <= 0 || L > a.max_ctx || L > a.pt_stride * a.page_size) {
    store_out(0.f);
    return;
  }
  const int nvalid = min(a.num_splits, (L + a.chunk_tokens - 1) / a.chunk_tokens);
  const float* lse = a.lse_part + row * a.num_splits;
  // split c's 16 bytes: at element (row * num_splits + c) * v_dim + d of the fp32 or fp16 partials
  const int64_t e0 = row * a.num_splits * a.v_dim + d;
  const u32x4_t* part = F16 ? reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.o_part) + e0)
                            : reinterpret_cast<const u32x4_t*>(a.o_part + e0);
  const int stride = a.v_dim / VEC;  // 16-byte vectors per split row
  // Splits in groups of kGroup (4, 8, 16 or 32: the split count rounded up, at most 32) whose lse values
  // and partials are all loaded before any is used: one memory round trip per group (with few rows,
  // one request and many splits, the loads each thread has in flight are all the memory-level
  // parallelism there is; with few splits a small group keeps registers and ALU work down).  Groups
  // after the first rescale the running sums to the new maximum, as the online softmax does.
  float M = -INFINITY, s = 0.f;
  bool nan = false;
  for (int c0 = 0; c0 < nvalid; c0 += kGroup) {
    float x[kGroup];
    u32x4_t p[kGroup];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (c0 + j < nvalid) {
        x[j] = lse[c0 + j];
        p[j] = part[(int64_t)(c0 + j) * stride];
      } else {
        x[j] = -INFINITY;
        p[j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    float gm = M;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      nan |= x[j] != x[j];
      gm = fmaxf(gm, x[j]);
    }
    if (gm == -INFINITY) continue;  // nothing but empty splits so far
    const float rs = exp2f(M - gm);  // 0 while M is still -inf
    s *= rs;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] *= rs;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float f = exp2f(x[j] - gm);
      s += f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        // the element is copied out first: a bit cast of a vector element expression read element 0 here
        const uint32_t u = p[j][F16 ? e >> 1 : e];
        float v;
        if constexpr (F16)
          v = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> (16 * (e & 1))));
        else
          v = __builtin_bit_cast(float, u);
        o[e] += f * v;
      }
    }
    M = gm;
  }
  if (nan) {  // a bad page seen by some split: the row is zero
    s = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = 0.f;
  }
  store_out(s > 0.f ? a.out_scale / s : 0.f);
}

hipError_t launch_attn_gqa(const AttnArgs& a, bool fp8, int batch, hipStream_t stream) {
  dim3 grid(a.num_splits, a.num_kv_heads, batch);
  if (fp8)
    hipLaunchKernelGGL(attn_gqa_split_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_gqa_split_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1 || a.merge_here) return e;
  MergeArgs m;
  m.o_part = a.o_part;
  m.lse_part = a.lse_part;
  m.out = a.out;
  m.ctx_lens = a.ctx_lens;
  m.flags = a.page_tags != nullptr ? a.flags_out : a.flags;
  m.num_q_heads = a.num_q_heads;
  m.v_dim = kD;
  m.num_splits = a.num_splits;
  m.chunk_tokens = a.chunk_tiles * kTile;
  m.max_ctx = a.max_ctx;
  m.pt_stride = a.pt_stride;
  m.page_size = a.page_size;
  m.part_f16 = fp8 ? 1 : 0;
  m.out_scale = fp8 ? a.v_scale : 1.f;
  return launch_merge(m, batch, stream);
}

hipError_t launch_merge(const MergeArgs& m_in, int batch, hipStream_t stream) {
  MergeArgs m = m_in;
  m.rows = (int64_t)batch * m.num_q_heads;
  const int tpr = m.v_dim / (m.part_f16 ? 8 : 4);  // v_dim 128 or 512: tpr a power of two dividing kMergeThreads
  const int64_t rows_per_block = kMergeThreads / tpr;
  const int64_t blocks = (m.rows + rows_per_block - 1) / rows_per_block;
  const dim3 g((uint32_t)blocks), t(kMergeThreads);
  if (m.part_f16) {
    if (m.num_splits <= 4) hipLaunchKernelGGL((attn_merge_kernel<4, true>), g, t, 0, stream, m);
    else if (m.num_splits <= 8) hipLaunchKernelGGL((attn_merge_kernel<8, true>), g, t, 0, stream, m);
    else if (m.num_splits <= 16) hipLaunchKernelGGL((attn_merge_kernel<16, true>), g, t, 0, stream, m);
    else hipLaunchKernelGGL((attn_merge_kernel<32, true>), g, t, 0, stream, m);
  } else {
    if (m.num_splits <= 4) hipLaunchKernelGGL((attn_merge_kernel<4, false>), g, t, 0, stream, m);
    else if (m.num_splits <= 8) hipLaunchKernelGGL((attn_merge_kernel<8, false>), g, t, 0, stream, m);
    else if (m.num_splits <= 16) hipLaunchKernelGGL((attn_merge_kernel<16, false>), g, t, 0, stream, m);
    else hipLaunchKernelGGL((attn_merge_kernel<32, false>), g, t, 0, stream, m);
  }
  return hipGetLastError();
}

}  // namespace kvfp8
