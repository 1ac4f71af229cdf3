// Device-side helpers shared by the gfx950 kernels: vector types, e4m3 and
// bf16 conversions, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfp8 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// e4m3 encode of two fp32 values into the low 16 bits (byte 0 = a, byte 1 = b).
// OCP E4M3, round to nearest even; magnitudes above 448 saturate (the
// conversion is fed values clamped to +-448, which under round-to-nearest
// gives the same code as saturating after rounding); NaN -> 0x7F | sign.
__device__ __forceinline__ uint32_t e4m3_clamp_nan_fix(float x, uint32_t code) {
  // code: the hardware code for the clamped value; NaN gets the input's sign.
  uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
  return (x != x) ? (0x7Fu | s) : code;
}

__device__ __forceinline__ float clamp448(float x) {
  // NaN passes through unchanged (both compares are false).
  return fabsf(x) > kE4M3Max ? copysignf(kE4M3Max, x) : x;
}

__device__ __forceinline__ uint32_t encode_e4m3x2(float a, float b) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  uint32_t c0 = e4m3_clamp_nan_fix(a, w & 0xFFu);
  uint32_t c1 = e4m3_clamp_nan_fix(b, (w >> 8) & 0xFFu);
  return c0 | (c1 << 8);
}

// Four e4m3 codes (one dword, byte 0 first) -> four exact bf16 / f16 values.
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(uint32_t w) {
  bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  u32x2_t r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

__device__ __forceinline__ u32x2_t e4m3x4_to_f16x4(uint32_t w) {
  f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  u32x2_t r;
  r[0] = __builtin_bit_cast(uint32_t, lo);
  r[1] = __builtin_bit_cast(uint32_t, hi);
  return r;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  // element 0 of the packed conversion of byte 0
  return __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFFu, false)[0];
}

// Element offset of K element (page, head, slot, d) in a K-layout pool of ELT-byte elements.
// Each (page, head) block is [S/16] sub-page blocks of 16 tokens x D; inside a sub-page block
// the rows are cut into 16-byte chunks c = q*NI + k (NI = D*ELT/64, q = 0..3) and token
// t = 4s + i of the sub-page keeps chunk c at chunk position ((s*NI + k)*4 + q)*4 + i.  A wave
// that reads lane (q, i)'s k-th chunk of four tokens from four pages then touches four runs of
// 256 contiguous bytes per instruction.
template <int ELT>
__device__ __forceinline__ int64_t k_elem_offset(int page, int head, int slot, int d, int H, int S, int D) {
  constexpr int E = 16 / ELT;
  const int NI = D * ELT / 64;
  const int u = slot >> 4, t = slot & 15, s = t >> 2, i = t & 3;
  const int c = d / E, q = c / NI, k = c - q * NI;
  const int chunk = ((s * NI + k) * 4 + q) * 4 + i;
  return ((int64_t)page * H + head) * S * D + (int64_t)u * 16 * D + (int64_t)chunk * E + (d % E);
}

// Element offset of element (page, head, slot, d) of a latent pool (written with no V pool):
// plain row-major [P][Hkv][S][D], so a tile of consecutive tokens of one page is contiguous.
__device__ __forceinline__ int64_t c_elem_offset(int page, int head, int slot, int d, int H, int S, int D) {
  return (((int64_t)page * H + head) * S + slot) * D + d;
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// xor-16 / xor-32 lane reductions on the VALU (gfx950 lane swaps: a row of 16 lanes with its neighbour,
// or the wave's two halves), with no LDS round trip.  Each lane ends with the same pair of operands as
// its partner, so both compute the same result.
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The step's new row of request r (DIM elements, bf16 bits at a.c_new + r * DIM) quantised as the
// append does and stored at position L - 1 of a row-major latent pool [page][slot][DIM].  Only the
// stores are issued here: the caller waits for them (vmcnt, which counts stores on this GPU family)
// and crosses a barrier before anything reads the row back.  Returns false, writing nothing, for a
// page id outside the pool or past the page table.
template <bool FP8, int DIM, class Args>
__device__ __forceinline__ bool store_latent_row(const Args& a, int r, int L, int nthreads) {
  const int S = a.page_size;
  const int e = (L - 1) / S;
  const int page = e < a.pt_stride ? a.page_table[(int64_t)r * a.pt_stride + e] : -1;
  if (page < 0 || page >= a.num_pages) return false;
  const int64_t row = ((int64_t)page * S + (L - 1) % S) * DIM;
  const uint16_t* src = a.c_new + (int64_t)r * DIM;
  for (int d = threadIdx.x; d < DIM; d += nthreads) {
    const uint32_t x = src[d];
    if (FP8)
      reinterpret_cast<uint8_t*>(const_cast<void*>(a.pool))[row + d] =
          (uint8_t)(encode_e4m3x2(__uint_as_float(x << 16) * a.c_inv, 0.f) & 0xFFu);
    else
      reinterpret_cast<uint16_t*>(const_cast<void*>(a.pool))[row + d] = (uint16_t)x;
  }
  return true;
}

// The tag check of every page request r's context spans, by a whole block (NW waves), before any
// of them is read or written: bit 0 a page whose tag differs from the one the request recorded,
// bit 1 a page id outside the pool or a context longer than the page table.  Returns the request's
// flag to every thread (s_flag: NW words of LDS).
template <int NW, class Args>
__device__ __forceinline__ uint32_t block_tag_check(const Args& a, int r, int L, uint32_t* s_flag) {
  uint32_t f = 0;
  if (L > 0) {
    const int64_t need = ((int64_t)L + a.page_size - 1) / a.page_size;
    const int64_t np = need < a.pt_stride ? need : (int64_t)a.pt_stride;
    if (need > a.pt_stride) f |= 2u;
    const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
    const uint32_t* ex = a.expected + (int64_t)r * a.pt_stride;
    for (int64_t i = threadIdx.x; i < np; i += NW * kWave) {
      const int32_t p = pt[i];
      if (p < 0 || p >= a.num_pages)
        f |= 2u;
      else if (a.page_tags[p] != ex[i])
        f |= 1u;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) f |= shfl_xor(f, m);
  if ((threadIdx.x & (kWave - 1)) == 0) s_flag[threadIdx.x / kWave] = f;
  __syncthreads();
  uint32_t all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) all |= s_flag[w];
  return all;
}


}  // namespace kvfp8
