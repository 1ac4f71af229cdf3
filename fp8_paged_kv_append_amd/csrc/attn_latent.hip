// Split-K paged decode attention over a latent (MLA-style) cache: one vector of
// width 576 per token, shared by every query head; scores use all 576 dims, the
// values are its first 512.  FP8 (e4m3) or BF16 cache, gfx950.
//
// What it computes is the same softmax attention as the GQA kernel (Cloudflare
// blog "Smaller, faster, safer: running Kimi and GLM at scale", section
// "Quantized KV cache": the FP8 cache is converted as it is read), with one
// cached vector serving as both key and value.  Unlike GQA this shape is bound
// by the matrix units, not by HBM: 128 heads x (576 + 512) MACs per cached byte.
//
// Block = (request r, 64-head group hg, split c), 8 waves: wave (hb, kh) works
// on heads 16hb..16hb+15 of the group, half kh of the contraction and half kh
// of the value dims.  The head groups of one (r, c) are 8 block ids apart, so
// round-robin dispatch puts them on the same XCD and later reads of a tile hit
// L2.  Each 32-token tile is copied once into LDS as stored (e4m3 bytes or
// bf16), one padded row per token, into one of two buffers: the copy of tile
// t+1 (whose global loads were issued during tile t-1) and the math of tile t
// share one barrier.  With lane = 16*q + n:
//  * S^T = C q^T: two 16-token blocks; wave (hb, kh) contracts dims
//    288kh + 72q + 8kk + j (kk = 0..8) with A = C rows (lane (q, m) reads 8
//    elements of token m, e4m3 converted to bf16 in registers) and B = q^T
//    (lane (q, n) holds head n).  The two partial sums of a pair meet in LDS;
//    fp32 addition commutes, so both waves hold the same scores and the same
//    softmax state, bit for bit.
//  * C layout: lane (q, n) holds head n's scores for tokens 16mb + 4q + i;
//    the PV contraction slot (q, j) is token 16(j/4) + 4q + j%4, so the P it
//    holds is already the B operand.
//  * O^T += V^T P^T over value dims 256kh .. 256kh+255: the A operand (8 tokens
//    at one value dim per lane) is read straight from the token rows with the
//    gfx950 LDS transpose loads: ds_read_b64_tr_b8 gives lane 8h+e byte e of
//    the 8-byte blocks named by lanes h, h+2, .., h+14 of its 16-lane group,
//    ds_read_b64_tr_b16 gives lane 4a+e element e of the blocks named by
//    lanes a, a+4, a+8, a+12.
//  * 16 accumulator blocks per lane, column = head n: the online-softmax
//    rescale is lane-local, and lazy (see below).
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kLD = 576;            // latent width (score dim)
constexpr int kLV = 512;            // value dim
constexpr int kLT = 32;             // tokens per tile
constexpr int kLWaves = 8;
constexpr int kLThreads = kLWaves * kWave;
constexpr int kLHeadsPerBlock = 64;
constexpr int kLPidWin = 1024;
constexpr float kLazy = 8.f;        // log2-domain slack before the accumulators are rescaled

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
#define KVFP8_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

template <bool FP8>
__global__ __launch_bounds__(kLThreads) void attn_latent_split_kernel(LatentArgs a) {
  constexpr int ELT = FP8 ? 1 : 2;
  constexpr int NI = kLD * ELT / 64;           // chunks per 64-byte slice of a row
  constexpr int SUBCH = 16 * kLD * ELT / 16;   // 16-byte chunks per 16-token sub-page block
  constexpr int NCH = 2 * SUBCH;               // chunks per 32-token tile
  constexpr int NLD = (NCH + kLThreads - 1) / kLThreads;
  constexpr int RS = kLD * ELT + 16;           // LDS bytes per token row (16 bytes of padding)
  constexpr int BUF = kLT * RS;                // LDS bytes per tile buffer

  __shared__ __align__(16) uint8_t s_tile[2 * BUF];
  __shared__ __align__(16) f32x4_t s_part[kLWaves][2][kWave];  // partial scores of each wave
  __shared__ int s_pid[kLPidWin];

  // XCD-aware block decode: head groups of one (request, split) unit are 8 ids apart
  const int b = blockIdx.x;
  const int grp = b / (8 * a.n_hg), rem = b % (8 * a.n_hg);
  const int hg = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= a.batch * a.num_splits) return;
  const int r = unit / a.num_splits, split = unit % a.num_splits;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hb = wave >> 1, kh = wave & 1;
  const int q4 = lane >> 4, n = lane & 15;
  const int S = a.page_size;
  const int Hq = a.num_q_heads;
  const int h0 = hg * kLHeadsPerBlock + hb * 16;       // this wave's first head
  const bool active = h0 < Hq;                          // wave-uniform, equal within a pair
  const int hb0 = hg * kLHeadsPerBlock, hb1 = min(Hq, hb0 + kLHeadsPerBlock);

  const int L = a.ctx_lens[r];
  const bool aborted = a.flags != nullptr && a.flags[r] != 0u;
  const bool bad_len = L <= 0 || L > a.max_ctx || L > a.pt_stride * S;
  const int chunk = a.chunk_tiles * kLT;
  const int c0 = split * chunk;
  if (aborted || bad_len) {
    if (a.num_splits == 1) {
      for (int e = threadIdx.x; e < (hb1 - hb0) * kLV; e += kLThreads)
        a.out[((int64_t)r * Hq + hb0) * kLV + e] = 0;
    }
    return;
  }
  if (c0 >= L) return;
  const int c1 = min(L, c0 + chunk);

  // q^T operand: lane (q4, n) holds head h0+n, dims 288*kh + 72*q4 + 8*kk .. +8 for kk = 0..8
  const int dim0 = 288 * kh + 72 * q4;
  u32x4_t qv[9];
  if (active) {
    const uint16_t* qp = a.q + ((int64_t)r * Hq + h0 + n) * kLD + dim0;
#pragma unroll
    for (int kk = 0; kk < 9; ++kk) qv[kk] = *reinterpret_cast<const u32x4_t*>(qp + 8 * kk);
  }

  // LDS byte offsets this lane reads, relative to a tile buffer
  const int qk_off = n * RS + dim0 * ELT;  // + 16*RS per token block, + 8*ELT bytes per k-step
  int pv_off0, pv_off1 = 0;               // PV source addresses for this wave's first d-block
  if (FP8) {
    const int j = (lane & 15) >> 1, h = lane & 1;
    pv_off0 = (16 * (j >> 2) + 4 * q4 + (j & 3)) * RS + 8 * h + 256 * kh;
  } else {
    const int jj = (lane & 15) >> 2, aa = lane & 3;
    pv_off0 = (4 * q4 + jj) * RS + 8 * aa + 512 * kh;
    pv_off1 = (16 + 4 * q4 + jj) * RS + 8 * aa + 512 * kh;
  }

  const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
  const uint8_t* pool = reinterpret_cast<const uint8_t*>(a.pool);
  const float c_log2 = a.qk_scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  // at most kLPidWin - 1 pages of tokens per window: a window starting mid-page still fits kLPidWin ids
  const int win = ((kLPidWin - 1) * S / kLT) * kLT;
  for (int w0 = c0; w0 < c1; w0 += win) {
    const int w1 = min(c1, w0 + win);
    const int e0 = w0 / S;
    const int ne = (w1 - 1) / S - e0 + 1;
    __syncthreads();
    for (int i = threadIdx.x; i < ne; i += kLThreads) {
      int p = pt[e0 + i];
      if (p < 0 || p >= a.num_pages) {
        bad = true;
        p = -1;
      }
      s_pid[i] = p;
    }
    __syncthreads();
    const int ntile = (w1 - w0 + kLT - 1) / kLT;

    // This thread's chunks of one tile, in storage order; each goes to LDS row tok, bytes 16c.
    u32x4_t raw[NLD];
    int dst[NLD];
    auto issue = [&](int t) {
      const int tb = w0 + t * kLT;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int pa = threadIdx.x + kLThreads * j;
        const int sub = pa / SUBCH, p = pa % SUBCH;
        const int i = p & 3, qq = (p >> 2) & 3, rest = p >> 4;
        const int kq = rest % NI, s = rest / NI;
        const int tok = 16 * sub + 4 * s + i;
        dst[j] = pa < NCH ? tok * RS + 16 * (qq * NI + kq) : -1;
        const int tok_sub = tb + 16 * sub;
        int pid = -1;
        if (t < ntile && pa < NCH && tok_sub < w1) pid = s_pid[min(tok_sub / S - e0, ne - 1)];
        if (pid >= 0 && tb + tok < w1) {
          const uint8_t* src = pool + ((int64_t)pid * S * kLD + (int64_t)(tok_sub % S) * kLD) * ELT + 16 * (int64_t)p;
          raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src));
        } else {
          raw[j] = u32x4_t{0, 0, 0, 0};     // absent token: zeros (masked below)
        }
      }
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        if (dst[j] >= 0) *reinterpret_cast<u32x4_t*>(&s_tile[buf * BUF + dst[j]]) = raw[j];
    };

    issue(0);
    __syncthreads();  // the previous window's last tile is no longer read
    stage(0);
    issue(1);
    for (int t = 0; t < ntile; ++t) {
      const int tb = w0 + t * kLT;
      const int cur = t & 1;
      __syncthreads();  // tile t is in LDS; buffer cur^1 and the score exchange are free
      if (t + 1 < ntile) {
        stage(cur ^ 1);
        issue(t + 2);
      }
      const uint8_t* tile = &s_tile[cur * BUF];

      // ---- partial S^T = C q^T over this wave's half of the dims, two 16-token blocks
      f32x4_t sc[2];
      if (active) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          f32x4_t ch[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
          const uint8_t* row = tile + qk_off + 16 * mb * RS;
#pragma unroll
          for (int kk = 0; kk < 9; ++kk) {
            u32x4_t av;
            if (FP8) {
              const u32x2_t c8 = *reinterpret_cast<const u32x2_t*>(row + 8 * kk);
              const u32x2_t lo = e4m3x4_to_bf16x4(c8[0]), hi = e4m3x4_to_bf16x4(c8[1]);
              av = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
            } else {
              av = *reinterpret_cast<const u32x4_t*>(row + 16 * kk);
            }
            ch[kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                                 __builtin_bit_cast(bf16x8_t, qv[kk]), ch[kk & 1], 0,
                                                                 0, 0);
          }
          sc[mb] = ch[0] + ch[1];
          s_part[wave][mb][lane] = sc[mb];
        }
      }
      __syncthreads();  // both halves of every pair's scores are in LDS
      if (!active) continue;
      {
        const f32x4_t o0 = s_part[wave ^ 1][0][lane], o1 = s_part[wave ^ 1][1][lane];
        // same operands in the same order in both waves of the pair
        sc[0] = kh == 0 ? sc[0] + o0 : o0 + sc[0];
        sc[1] = kh == 0 ? sc[1] + o1 : o1 + sc[1];
      }
      // ---- online softmax for head n over tokens 16mb + 4q4 + i.  The accumulators stay
      // referenced to m_run until a tile's max exceeds it by more than kLazy (log2 units):
      // p <= 2^kLazy meanwhile, exact up to rounding, and the rescale is rare.
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool valid = tb + 16 * mb + 4 * q4 + i < w1;
          const float v = valid ? sc[mb][i] * c_log2 : -INFINITY;
          x[4 * mb + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const bool grow = tmax > m_run + kLazy;  // m_run = -inf: any finite tile max grows it
      if (__any(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? exp2f(m_run - m_new) : 1.f;  // m_run = -inf -> 0
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 16; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        x[k] = exp2f(x[k] - m_use);
        psum += x[k];
      }
      l_run += psum;
      const u32x4_t pp = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                          pack_bf16x2(x[6], x[7])};
      // ---- O^T += V^T P^T, 16 blocks of 16 value dims, A operand by LDS transpose reads
      __attribute__((address_space(3))) uint8_t* lt = (__attribute__((address_space(3))) uint8_t*)(tile);
#pragma unroll
      for (int db = 0; db < 16; ++db) {
        u32x4_t vv;
        if (FP8) {
          const i32x2_t t8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(KVFP8_LDS(i32x2_t, lt + pv_off0 + 16 * db));
          const u32x2_t lo = e4m3x4_to_bf16x4((uint32_t)t8[0]), hi = e4m3x4_to_bf16x4((uint32_t)t8[1]);
          vv = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        } else {
          const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(KVFP8_LDS(i16x4_t, lt + pv_off0 + 32 * db));
          const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(KVFP8_LDS(i16x4_t, lt + pv_off1 + 32 * db));
          const u32x2_t a0 = __builtin_bit_cast(u32x2_t, t0), a1 = __builtin_bit_cast(u32x2_t, t1);
          vv = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv),
                                                          __builtin_bit_cast(bf16x8_t, pp), acc[db], 0, 0, 0);
      }
    }
  }

  // ---- write this wave's heads and value half (a page id outside the pool zeroes the request)
  __syncthreads();
  if (threadIdx.x == 0) s_pid[0] = 0;
  __syncthreads();
  if (bad) s_pid[0] = 1;
  __syncthreads();
  const bool any_bad = s_pid[0] != 0;
  if (!active) return;
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  const int h = h0 + n;
  const int64_t row = (int64_t)r * Hq + h;
  const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
  const int dv0 = 256 * kh + 4 * q4;
  if (a.num_splits == 1) {
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const float o0 = any_bad ? 0.f : acc[db][0] * inv, o1 = any_bad ? 0.f : acc[db][1] * inv;
      const float o2 = any_bad ? 0.f : acc[db][2] * inv, o3 = any_bad ? 0.f : acc[db][3] * inv;
      const u32x2_t v2 = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
      *reinterpret_cast<u32x2_t*>(&a.out[row * kLV + dv0 + 16 * db]) = v2;
    }
  } else {
    const int64_t slot = row * a.num_splits + split;
#pragma unroll
    for (int db = 0; db < 16; ++db)
      *reinterpret_cast<f32x4_t*>(&a.o_part[slot * kLV + dv0 + 16 * db]) = acc[db] * inv;
    if (q4 == 0 && kh == 0) a.lse_part[slot] = any_bad ? NAN : (l_run == 0.f ? -INFINITY : m_run + __log2f(l_run));
  }
}

hipError_t launch_attn_latent(const LatentArgs& a, bool fp8, hipStream_t stream) {
  const int units = a.batch * a.num_splits;
  const int blocks = ((units + 7) / 8) * 8 * a.n_hg;
  if (fp8)
    hipLaunchKernelGGL(attn_latent_split_kernel<true>, dim3(blocks), dim3(kLThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_latent_split_kernel<false>, dim3(blocks), dim3(kLThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  MergeArgs m;
  m.o_part = a.o_part;
  m.lse_part = a.lse_part;
  m.out = a.out;
  m.ctx_lens = a.ctx_lens;
  m.flags = a.flags;
  m.num_q_heads = a.num_q_heads;
  m.v_dim = kLV;
  m.num_splits = a.num_splits;
  m.chunk_tokens = a.chunk_tiles * kLT;
  m.max_ctx = a.max_ctx;
  m.pt_stride = a.pt_stride;
  m.page_size = a.page_size;
  return launch_merge(m, a.batch, stream);
}

}  // namespace kvfp8
