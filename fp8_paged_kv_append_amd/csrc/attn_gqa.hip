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
//    both operands use it).  Lane (q, n) loads 32 contiguous bytes (64 for
//    bf16) of each of its 4 K rows.
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
//    head n) keeps the rescale lane-local.
// The four waves merge their (m, l, O) through LDS; with one split the block
// writes bf16 output, otherwise normalised fp32 partials and lse for the merge
// kernel.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kTile = 64;
constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// --- per-dtype loads and operand conversions -------------------------------------------------

template <bool FP8>
struct KRow;  // one lane's slice of one K row
template <>
struct KRow<true> {
  u32x4_t w[2];  // 32 bytes: dims 32q .. 32q+31
  __device__ __forceinline__ void load(const uint8_t* p) {
    const u32x4_t* v = reinterpret_cast<const u32x4_t*>(p);
    w[0] = v[0];
    w[1] = v[1];
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
    const u32x4_t* v = reinterpret_cast<const u32x4_t*>(p);
    w[0] = v[0];
    w[1] = v[1];
    w[2] = v[2];
    w[3] = v[3];
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = w[2] = w[3] = u32x4_t{0, 0, 0, 0}; }
  __device__ __forceinline__ bf16x8_t op(int kk) const { return __builtin_bit_cast(bf16x8_t, w[kk]); }
};

template <bool FP8>
struct VRow;  // one lane's slice of one V^T row: 16 consecutive slots
template <>
struct VRow<true> {
  u32x4_t w;  // 16 e4m3 codes
  __device__ __forceinline__ void load(const uint8_t* p) { w = *reinterpret_cast<const u32x4_t*>(p); }
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
    const u32x4_t* v = reinterpret_cast<const u32x4_t*>(p);
    w[0] = v[0];
    w[1] = v[1];
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

template <bool FP8>
__global__ __launch_bounds__(kThreads) void attn_gqa_split_kernel(AttnArgs a) {
  constexpr int ELT = FP8 ? 1 : 2;
  const int split = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int q4 = lane >> 4, n = lane & 15;
  const int G = a.group;
  const int S = a.page_size;

  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_acc[kWaves][16][kD];
  __shared__ int s_bad;

  const int L = a.ctx_lens[r];
  const bool aborted = a.flags != nullptr && a.flags[r] != 0u;
  const bool bad_len = L <= 0 || L > a.max_ctx || L > a.pt_stride * S;
  const int chunk = a.chunk_tiles * kTile;
  const int c0 = split * chunk;
  if (aborted || bad_len) {
    if (a.num_splits == 1) {  // rows of this group are zero
      for (int e = threadIdx.x; e < G * kD; e += kThreads)
        a.out[((int64_t)r * a.num_q_heads + g * G + e / kD) * kD + e % kD] = 0;
    }
    return;  // the merge kernel zeroes the rows itself
  }
  if (c0 >= L) return;  // past this request's context: the merge does not read this split
  const int c1 = min(L, c0 + chunk);
  const int ntile = (c1 - c0 + kTile - 1) / kTile;

  if (threadIdx.x == 0) s_bad = 0;

  // q^T operand: lane (q4, n) holds head g*G+n, dims 32*q4 .. 32*q4+31 (zero for padding heads)
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

  const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
  const uint8_t* kpool = reinterpret_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vpool = reinterpret_cast<const uint8_t*>(a.v_pool);
  const int64_t head_blk_k = (int64_t)S * kD;  // elements per (page, head) block
  const float c_log2 = a.qk_scale_log2;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  for (int t = wave; t < ntile; t += kWaves) {
    const int tb = c0 + t * kTile;
    // page of the sub-page this lane reads K rows from (n/4) and V^T rows from (q4)
    const int tok_k = tb + 16 * (n >> 2);
    const int tok_v = tb + 16 * q4;
    int pid_k = -1, pid_v = -1;
    if (tok_k < c1) {
      pid_k = pt[tok_k / S];
      if (pid_k < 0 || pid_k >= a.num_pages) pid_k = -1;
    }
    if (tok_v < c1) {
      pid_v = pt[tok_v / S];
      if (pid_v < 0 || pid_v >= a.num_pages) {
        pid_v = -1;
        bad = true;
      }
    }
    const int off_k = tok_k % S, off_v = tok_v % S;

    KRow<FP8> kr[4];
    if (pid_k >= 0) {
      const uint8_t* kb = kpool + (((int64_t)pid_k * a.num_kv_heads + g) * head_blk_k +
                                   (int64_t)(off_k + (n & 3)) * kD + 32 * q4) * ELT;
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[s].load(kb + (int64_t)(4 * s) * kD * ELT);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[s].zero();
    }
    VRow<FP8> vr[8];
    const int nv = max(0, min(16, c1 - tok_v));
    if (pid_v >= 0) {
      const uint8_t* vb = vpool + (((int64_t)pid_v * a.num_kv_heads + g) * kD * S +
                                   (int64_t)n * S + off_v) * ELT;
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j].load(vb + (int64_t)(16 * j) * S * ELT);
      if (nv < 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j].mask(nv);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[j].zero();
    }

    // S^T = K q^T, four chains of 16 tokens
    f32x4_t sc[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[s].op(kk), __builtin_bit_cast(bf16x8_t, qv[kk]),
                                                        sc[s], 0, 0, 0);
    }
    // online softmax for head n over the 16 tokens of sub-page q4 this lane holds
    float x[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 4 * s + i;
        const bool valid = pid_v >= 0 && pos < nv;
        const float v = valid ? sc[s][i] * c_log2 : -INFINITY;
        x[pos] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);  // m_run = -inf -> 0
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      x[k] = exp2f(x[k] - m_use);
      psum += x[k];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4_t pp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) pp[kb][e] = pack_p<FP8>(x[8 * kb + 2 * e], x[8 * kb + 2 * e + 1]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc[j] = mfma_pv<FP8>(vr[j], kb, pp[kb], acc[j]);
    }
  }

  // ---- merge the four waves
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (q4 == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_run;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<f32x4_t*>(&s_acc[wave][n][16 * j + 4 * q4]) = acc[j];
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;

  const int Hq = a.num_q_heads;
  for (int e = threadIdx.x; e < G * kD; e += kThreads) {
    const int hn = e / kD, d = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hn]);
    float lsum = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(s_m[w][hn] - M);
        lsum += s_l[w][hn] * f;
        o += s_acc[w][hn][d] * f;
      }
    }
    const int64_t row = (int64_t)r * Hq + g * G + hn;
    if (a.num_splits == 1) {
      const float val = (any_bad || lsum == 0.f) ? 0.f : o * (a.v_scale / lsum);
      a.out[row * kD + d] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xFFFFu);
    } else {
      const int64_t slot = row * a.num_splits + split;
      a.o_part[slot * kD + d] = lsum == 0.f ? 0.f : o * (a.v_scale / lsum);
      if (d == 0) a.lse_part[slot] = any_bad ? NAN : (lsum == 0.f ? -INFINITY : M + __log2f(lsum));
    }
  }
}

// --- merge of the split partials ----------------------------------------------------------------

__global__ __launch_bounds__(kD) void attn_merge_kernel(MergeArgs a) {
  const int row = blockIdx.x;  // r * Hq + h
  const int r = row / a.num_q_heads;
  const int d = threadIdx.x;
  const int L = a.ctx_lens[r];
  const bool aborted = a.flags != nullptr && a.flags[r] != 0u;
  uint16_t* out = a.out + (int64_t)row * a.v_dim;
  if (aborted || L <= 0 || L > a.max_ctx || L > a.pt_stride * a.page_size) {
    for (int e = d; e < a.v_dim; e += blockDim.x) out[e] = 0;
    return;
  }
  const int nvalid = min(a.num_splits, (L + a.chunk_tokens - 1) / a.chunk_tokens);
  const float* lse = a.lse_part + (int64_t)row * a.num_splits;
  float M = -INFINITY;
  bool nan = false;
  for (int c = 0; c < nvalid; ++c) {
    const float x = lse[c];
    nan |= x != x;
    M = fmaxf(M, x);
  }
  for (int e = d; e < a.v_dim; e += blockDim.x) {
    float o = 0.f, s = 0.f;
    if (!nan && M != -INFINITY) {
      for (int c = 0; c < nvalid; ++c) {
        const float f = exp2f(lse[c] - M);
        s += f;
        o += f * a.o_part[((int64_t)row * a.num_splits + c) * a.v_dim + e];
      }
    }
    out[e] = (uint16_t)(pack_bf16x2(s > 0.f ? o / s : 0.f, 0.f) & 0xFFFFu);
  }
}

hipError_t launch_attn_gqa(const AttnArgs& a, bool fp8, int batch, hipStream_t stream) {
  dim3 grid(a.num_splits, a.num_kv_heads, batch);
  if (fp8)
    hipLaunchKernelGGL(attn_gqa_split_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_gqa_split_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  MergeArgs m;
  m.o_part = a.o_part;
  m.lse_part = a.lse_part;
  m.out = a.out;
  m.ctx_lens = a.ctx_lens;
  m.flags = a.flags;
  m.num_q_heads = a.num_q_heads;
  m.v_dim = kD;
  m.num_splits = a.num_splits;
  m.chunk_tokens = a.chunk_tiles * kTile;
  m.max_ctx = a.max_ctx;
  m.pt_stride = a.pt_stride;
  m.page_size = a.page_size;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(batch * a.num_q_heads), dim3(kD), 0, stream, m);
  return hipGetLastError();
}

}  // namespace kvfp8
