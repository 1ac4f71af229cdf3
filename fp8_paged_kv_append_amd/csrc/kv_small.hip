// The small kernels of the decode path on gfx950: the batched page-tag check,
// the write path (quantise + scatter into pages), the read-back gather used by
// tests, and the max-abs reduction behind per-tensor scale calibration.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

// ------------------------------------------------------------------ integrity check
// agentlenshq summary of the Cloudflare post, section "KV Cache 完整性检查"; xujun.org
// note, section "一个不能出错的共享缓存": each physical page's tag is compared with the
// tag the request recorded; a mismatch aborts the request.  One block per request,
// a plain OR over its used entries, one writer per flag: no atomics, no cross-block
// communication, so the check cannot race with anything launched after it.
__global__ __launch_bounds__(256) void tag_check_kernel(TagArgs a) {
  __shared__ uint32_t s_or[4];
  const int r = blockIdx.x;
  const int64_t L = a.ctx_lens[r];
  uint32_t f = 0;
  if (L > 0) {
    const int64_t need = (L + a.page_size - 1) / a.page_size;
    int64_t n = need;
    if (need > a.pt_stride) {
      f |= 2u;
      n = a.pt_stride;
    }
    const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
    const uint32_t* ex = a.expected + (int64_t)r * a.pt_stride;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
      const int32_t p = pt[i];
      if (p < 0 || p >= a.num_pages)
        f |= 2u;
      else if (a.page_tags[p] != ex[i])
        f |= 1u;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) f |= shfl_xor(f, m);
  if ((threadIdx.x & 63) == 0) s_or[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) a.flags[r] = s_or[0] | s_or[1] | s_or[2] | s_or[3];
}

hipError_t launch_tag_check(const TagArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tag_check_kernel, dim3(a.batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ write path
// Cloudflare post, section "Quantized KV cache": the cache holds e4m3 instead of bf16.
// One wave per (token, KV head).  K rows go to the chunk-reordered sub-page block (a latent
// pool, written with no V pool, is plain row-major); V goes to the transposed page block, one
// element per d row.
struct AppendTarget {
  int page, slot;
};

__device__ __forceinline__ bool append_target(const AppendArgs& a, int tok, AppendTarget& t) {
  const int r = a.tok_req[tok], pos = a.tok_pos[tok];
  if (r < 0 || r >= a.batch || pos < 0 || (int64_t)pos >= (int64_t)a.pt_stride * a.page_size) return false;
  if (a.flags != nullptr && a.flags[r] != 0u) return false;
  const int page = a.page_table[(int64_t)r * a.pt_stride + pos / a.page_size];
  if (page < 0 || page >= a.num_pages) return false;
  t.page = page;
  t.slot = pos % a.page_size;
  return true;
}

template <bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= (int64_t)a.n_tokens * a.num_kv_heads) return;
  const int tok = (int)(item / a.num_kv_heads), h = (int)(item % a.num_kv_heads);
  AppendTarget t;
  if (!append_target(a, tok, t)) return;
  const int H = a.num_kv_heads, S = a.page_size, D = a.head_dim, Dv = a.v_dim;

  const uint32_t* ksrc = reinterpret_cast<const uint32_t*>(a.k_new + ((int64_t)tok * H + h) * D);
  for (int d2 = lane; d2 < D / 2; d2 += kWave) {
    const uint32_t w = ksrc[d2];
    // elements 2*d2 and 2*d2+1 share a 16-byte chunk: one 2-element store
    const int64_t o = a.v_pool ? k_elem_offset<FP8 ? 1 : 2>(t.page, h, t.slot, 2 * d2, H, S, D)
                               : c_elem_offset(t.page, h, t.slot, 2 * d2, H, S, D);
    if (FP8) {
      const float x0 = bf16_bits_to_f32(w & 0xFFFFu) * a.k_inv;
      const float x1 = bf16_bits_to_f32(w >> 16) * a.k_inv;
      reinterpret_cast<uint16_t*>(a.k_pool)[o >> 1] = (uint16_t)encode_e4m3x2(x0, x1);
    } else {
      reinterpret_cast<uint32_t*>(a.k_pool)[o >> 1] = w;
    }
  }
  if (a.v_pool == nullptr) return;
  const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(a.v_new + ((int64_t)tok * H + h) * Dv);
  const int64_t vbase = ((int64_t)t.page * H + h) * Dv * S + t.slot;
  for (int d2 = lane; d2 < Dv / 2; d2 += kWave) {
    const uint32_t w = vsrc[d2];
    const int64_t o = vbase + (int64_t)(2 * d2) * S;
    if (FP8) {
      const float x0 = bf16_bits_to_f32(w & 0xFFFFu) * a.v_inv;
      const float x1 = bf16_bits_to_f32(w >> 16) * a.v_inv;
      const uint32_t c = encode_e4m3x2(x0, x1);
      uint8_t* vp = reinterpret_cast<uint8_t*>(a.v_pool);
      vp[o] = (uint8_t)(c & 0xFFu);
      vp[o + S] = (uint8_t)(c >> 8);
    } else {
      uint16_t* vp = reinterpret_cast<uint16_t*>(a.v_pool);
      vp[o] = (uint16_t)(w & 0xFFFFu);
      vp[o + S] = (uint16_t)(w >> 16);
    }
  }
}

hipError_t launch_append(const AppendArgs& a, bool fp8, hipStream_t stream) {
  const int64_t items = (int64_t)a.n_tokens * a.num_kv_heads;
  const int64_t blocks = (items + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL(append_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ check + write in one launch
// The decode step's first two passes fused per request: block r ORs the flags of request r's used
// pages exactly as tag_check_kernel does, and only when they are clear writes r's new token
// (position ctx_lens[r] - 1) exactly as append_kernel would.  The new rows and the first
// kCaBatch * 256 page-table and expected-tag words of the row are loaded together with the context
// length (every row holds pt_stride words, so these loads stay inside the tables whatever the
// length turns out to be), so the check's first tag gathers follow one memory round trip after the
// launch.  Check before write is preserved inside the block.
// With c.page_tags null there is no check: the flags (when given) were set by an earlier launch and
// are only read -- the later layers of a step that shares one check -- and the page id of the
// written slot is validated here instead.
constexpr int kCaBatch = 2;  // page-table words per thread loaded with the length (512 cover 8192 tokens at S = 16)

template <bool FP8>
__global__ __launch_bounds__(256) void check_append_kernel(TagArgs c, AppendArgs a) {
  __shared__ uint32_t s_or[4];
  const int r = blockIdx.x;
  const int H = a.num_kv_heads, S = a.page_size, D = a.head_dim, Dv = a.v_dim;
  constexpr int kMaxPairs = 8;  // new-row element pairs per thread held across the check
  const int nk = H * D / 2, nv = a.v_pool ? H * Dv / 2 : 0;
  uint32_t kw[kMaxPairs], vw[kMaxPairs];
  const uint32_t* ksrc = reinterpret_cast<const uint32_t*>(a.k_new + (int64_t)r * H * D);
  const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(a.v_new + (int64_t)r * H * Dv);
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int e = threadIdx.x + 256 * i;
    kw[i] = e < nk ? ksrc[e] : 0u;
    vw[i] = e < nv ? vsrc[e] : 0u;
  }
  const bool check = c.page_tags != nullptr;
  const int32_t* pt = c.page_table + (int64_t)r * c.pt_stride;
  const uint32_t* ex = check ? c.expected + (int64_t)r * c.pt_stride : nullptr;
  int32_t sp[kCaBatch];
  uint32_t se[kCaBatch];
#pragma unroll
  for (int j = 0; j < kCaBatch; ++j) {
    const int64_t i = threadIdx.x + 256 * j;
    const bool in = check && i < c.pt_stride;
    sp[j] = in ? pt[i] : -1;
    se[j] = in ? ex[i] : 0u;
  }
  const int64_t L = c.ctx_lens[r];
  if (!check) {
    // ---- no check: honour the flags an earlier launch wrote
    if (L <= 0 || (c.flags != nullptr && c.flags[r] != 0u)) return;
    if ((L - 1) / a.page_size >= a.pt_stride) return;
  } else {
    // ---- the check
    uint32_t f = 0;
    if (L > 0) {
      const int64_t need = (L + c.page_size - 1) / c.page_size;
      int64_t n = need;
      if (need > c.pt_stride) {
        f |= 2u;
        n = c.pt_stride;
      }
      uint32_t tv[kCaBatch];
#pragma unroll
      for (int j = 0; j < kCaBatch; ++j) {
        const int64_t i = threadIdx.x + 256 * j;
        const bool ok = sp[j] >= 0 && sp[j] < c.num_pages;
        tv[j] = (i < n && ok) ? c.page_tags[sp[j]] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kCaBatch; ++j) {
        const int64_t i = threadIdx.x + 256 * j;
        if (i < n) {
          if (sp[j] < 0 || sp[j] >= c.num_pages)
            f |= 2u;
          else if (tv[j] != se[j])
            f |= 1u;
        }
      }
      for (int64_t i = threadIdx.x + 256 * kCaBatch; i < n; i += 256) {
        const int32_t p = pt[i];
        if (p < 0 || p >= c.num_pages)
          f |= 2u;
        else if (c.page_tags[p] != ex[i])
          f |= 1u;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) f |= shfl_xor(f, m);
    if ((threadIdx.x & 63) == 0) s_or[threadIdx.x >> 6] = f;
    __syncthreads();
    const uint32_t flag = s_or[0] | s_or[1] | s_or[2] | s_or[3];
    if (threadIdx.x == 0) c.flags[r] = flag;
    if (flag != 0u || L <= 0) return;
  }
  if (c.max_ctx > 0 && L > c.max_ctx) return;  // beyond the step's grid: flagged as usual, not written
  // ---- the write, for a request whose pages all check out
  const int pos = (int)(L - 1);
  const int page = a.page_table[(int64_t)r * a.pt_stride + pos / S];  // in range: checked above
  if (page < 0 || page >= a.num_pages) return;                         // (the no-check mode's guard)
  const int slot = pos % S;
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int e = threadIdx.x + 256 * i;
    if (e < nk) {
      const int h = e / (D / 2), d2 = e % (D / 2);
      const int64_t o = a.v_pool ? k_elem_offset<FP8 ? 1 : 2>(page, h, slot, 2 * d2, H, S, D)
                                 : c_elem_offset(page, h, slot, 2 * d2, H, S, D);
      if (FP8) {
        const float x0 = bf16_bits_to_f32(kw[i] & 0xFFFFu) * a.k_inv;
        const float x1 = bf16_bits_to_f32(kw[i] >> 16) * a.k_inv;
        reinterpret_cast<uint16_t*>(a.k_pool)[o >> 1] = (uint16_t)encode_e4m3x2(x0, x1);
      } else {
        reinterpret_cast<uint32_t*>(a.k_pool)[o >> 1] = kw[i];
      }
    }
    if (e < nv) {
      const int h = e / (Dv / 2), d2 = e % (Dv / 2);
      const int64_t o = ((int64_t)page * H + h) * Dv * S + (int64_t)(2 * d2) * S + slot;
      if (FP8) {
        const float x0 = bf16_bits_to_f32(vw[i] & 0xFFFFu) * a.v_inv;
        const float x1 = bf16_bits_to_f32(vw[i] >> 16) * a.v_inv;
        const uint32_t cc = encode_e4m3x2(x0, x1);
        uint8_t* vp = reinterpret_cast<uint8_t*>(a.v_pool);
        vp[o] = (uint8_t)(cc & 0xFFu);
        vp[o + S] = (uint8_t)(cc >> 8);
      } else {
        uint16_t* vp = reinterpret_cast<uint16_t*>(a.v_pool);
        vp[o] = (uint16_t)(vw[i] & 0xFFFFu);
        vp[o + S] = (uint16_t)(vw[i] >> 16);
      }
    }
  }
}

hipError_t launch_check_append(const TagArgs& c, const AppendArgs& a, bool fp8, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL(check_append_kernel<true>, dim3(c.batch), dim3(256), 0, stream, c, a);
  else
    hipLaunchKernelGGL(check_append_kernel<false>, dim3(c.batch), dim3(256), 0, stream, c, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ gather (read back)
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= (int64_t)a.n_tokens * a.num_kv_heads) return;
  const int tok = (int)(item / a.num_kv_heads), h = (int)(item % a.num_kv_heads);
  const int H = a.num_kv_heads, S = a.page_size, D = a.head_dim, Dv = a.v_dim;
  const int r = a.tok_req[tok], pos = a.tok_pos[tok];
  int page = -1;
  if (r >= 0 && r < a.batch && pos >= 0 && (int64_t)pos < (int64_t)a.pt_stride * S) {
    page = a.page_table[(int64_t)r * a.pt_stride + pos / S];
    if (page >= a.num_pages) page = -1;
  }
  const int slot = pos % S;
  T* ko = reinterpret_cast<T*>(a.k_out) + ((int64_t)tok * H + h) * D;
  const T* kp = reinterpret_cast<const T*>(a.k_pool);
  for (int d = lane; d < D; d += kWave)
    ko[d] = page < 0 ? T(0)
                     : kp[a.v_pool ? k_elem_offset<sizeof(T)>(page, h, slot, d, H, S, D)
                                   : c_elem_offset(page, h, slot, d, H, S, D)];
  if (a.v_out == nullptr) return;
  T* vo = reinterpret_cast<T*>(a.v_out) + ((int64_t)tok * H + h) * Dv;
  const T* vp = reinterpret_cast<const T*>(a.v_pool);
  for (int d = lane; d < Dv; d += kWave)
    vo[d] = page < 0 ? T(0) : vp[(((int64_t)page * H + h) * Dv + d) * S + slot];
}

hipError_t launch_gather(const GatherArgs& a, bool fp8, hipStream_t stream) {
  const int64_t blocks = ((int64_t)a.n_tokens * a.num_kv_heads + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL(gather_kernel<uint8_t>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ max |x| for the scale
// bf16 magnitudes order like their bit patterns (sign cleared), so the maximum is an
// exact integer max; NaN patterns (magnitude bits above 0x7F80) are skipped.
__device__ __forceinline__ uint32_t mag_max(uint32_t m, uint32_t b) {
  const uint32_t v = b & 0x7FFFu;
  return v <= 0x7F80u ? max(m, v) : m;
}

__global__ __launch_bounds__(256) void absmax_kernel(const uint16_t* x, int64_t n, uint32_t* out) {
  __shared__ uint32_t s_max[4];
  uint32_t m = 0;
  const int64_t n8 = n / 8;
  const u32x4_t* x8 = reinterpret_cast<const u32x4_t*>(x);
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    const u32x4_t v = x8[i];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = mag_max(m, v[k]);
      m = mag_max(m, v[k] >> 16);
    }
  }
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) m = mag_max(m, x[i]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = max(m, shfl_xor(m, k));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    atomicMax(out, b << 16);
  }
}

hipError_t launch_absmax(const uint16_t* x, int64_t n, uint32_t* out, hipStream_t stream) {
  int64_t blocks = (n / 8 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(absmax_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, x, n, out);
  return hipGetLastError();
}

}  // namespace kvfp8
