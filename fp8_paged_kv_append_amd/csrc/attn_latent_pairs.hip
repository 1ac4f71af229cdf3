// Split-K paged decode attention over an FP8 (e4m3) latent cache, gfx950: the
// same softmax attention as attn_latent_split_kernel<true> (Cloudflare blog
// "Smaller, faster, safer: running Kimi and GLM at scale", section "Quantized
// KV cache": the cache is converted as it is read), with a work split that
// lets two waves share each SIMD.
//
// Block = (request r, split c, group of 64 query heads), 8 waves.  Waves w and
// w ^ 4 form a pair over the 16 heads 16 (w & 3) .. +15 of the group; wave
// half x = w >> 2 contracts the score over its 288 of the 576 dims and
// accumulates its 256 of the 512 value dims.  Per wave: O is 64 AGPRs, q's two
// e4m3 terms 36 VGPRs.  The pair's partial scores meet in LDS: each wave parks
// its partial for the next tile, and after the per-tile barrier both add the
// two in the same order, so their softmax states stay identical.
// With lane l = 16 q4 + n:
//  * S^T partial = C q^T on v_mfma_scale_f32_16x16x128_f8f6f4 (A row = lane
//    mod 16 = token, B column = lane mod 16 = head, both over bytes
//    32 q4 .. 32 q4 + 31 of the 128-wide k-step) for dims 256 x + 128 j, and
//    one v_mfma_f32_16x16x32_fp8_fp8 step (8 bytes 8 q4 .. 8 q4 + 7) for dims
//    512 + 32 x.  Two token blocks of 16 (mb); the C layout gives lane
//    (q4, n) head n's scores for tokens 16 mb + 4 q4 + i.
//  * O^T += V^T P^T per 16-dim block on v_mfma_f32_16x16x32_bf16: slot 8 q4 + j
//    is token 4 q4 + j (j < 4) or 16 + 4 q4 + j - 4, i.e. register j of the
//    lane's scores, so B = P needs no shuffle; A = V^T comes from one
//    ds_read_b64_tr_b8 per block, whose lane 2 i + h names token slot i at
//    dim offset 8 h: lane 8 h + e then receives dim 8 h + e of the 8 tokens.
//  * Online softmax in the log2 domain with the lazy rescale (only when a
//    head's running max grows by more than 2^8).
// In a decode step the same launch may also check the request's page tags
// (every block, before it reads or writes any page) and store the step's token
// (both head-group blocks of the split holding position L - 1, the same bytes,
// before their first tile copy), as attn_latent_split_kernel does.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

namespace {

constexpr int kPD = kLatentDim;            // 576
constexpr int kPV = kLatentVDim;           // 512
constexpr int kPT = kLatentTileTokens;     // 32 tokens per tile
constexpr int kPW = 8;                     // waves per block
constexpr int kPThreads = kPW * kWave;
constexpr int kPHB = 64;                   // heads per block
constexpr int kPPidWin = 1024;
constexpr float kPLazy = 8.f;

constexpr int kRowB = kPD;                 // bytes per token row (e4m3)
constexpr int kRS = kRowB + 16;            // LDS row stride
constexpr int kCH = kRowB / 16;            // 16-byte chunks per row
constexpr int kSlots = kRS / 16;           // chunk slots per LDS row
constexpr int kNInst = (kPT * kSlots + 63) / 64;      // 1 KiB copies per tile
constexpr int kNPW = (kNInst + kPW - 1) / kPW;        // copies per wave per tile
constexpr int kBuf = kNPW * kPW * 1024;               // bytes per tile buffer
constexpr int kNBuf = 5;                              // tile buffers (with the rest, just under 160 KB)

typedef float f32x16p_t __attribute__((ext_vector_type(16)));
typedef int i32x2p_t __attribute__((ext_vector_type(2)));
typedef int v8ip_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_b;

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16*lane (lds_addr
// wave-uniform, in M0); asm so that LDS reads of other buffers do not wait for it, waited for
// explicitly before the barrier that publishes a tile.  M0 is restored.
__device__ __forceinline__ void pair_copy16(const void* src, uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

template <int N>
__device__ __forceinline__ void pair_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most the copies of n tiles (NPW loads each; n clamped to 0 .. MAXT) are outstanding
template <int NPW, int MAXT>
__device__ __forceinline__ void pair_vm_wait_tiles(int n) {
  if constexpr (MAXT > 0) {
    if (n >= MAXT) {
      pair_vm_wait<NPW * MAXT>();
      return;
    }
    pair_vm_wait_tiles<NPW, MAXT - 1>(n);
  } else {
    pair_vm_wait<0>();
  }
}

// token of PV slot 8 q4 + j
__device__ __forceinline__ int pv_token(int q4, int j) { return j < 4 ? 4 * q4 + j : 16 + 4 * q4 + (j - 4); }

// LDS row of tile token t: the second 16 tokens rotated by 8 rows.  Rows 16 apart share banks (the
// 592-byte stride repeats every 16 rows); a PV transpose read takes tokens 4 q4 .. +3 and
// 16 + 4 q4 .. +3 together, which then sit in 8 distinct rows mod 16 (conflict-free), and the 16
// rows one QK read touches stay distinct mod 16.
__device__ __forceinline__ int lrow(int t) { return t < 16 ? t : 16 + ((t - 8) & 15); }
__device__ __forceinline__ int ltok(int row) { return row < 16 ? row : 16 + ((row - 8) & 15); }

// four floats as two e4m3 terms: {hi, lo} with lo = e4m3(f - hi)
__device__ __forceinline__ i32x2p_t to_hilo(float f0, float f1, float f2, float f3) {
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, hi, true);
  const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0 - b0[0], f1 - b0[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(f2 - b1[0], f3 - b1[1], lo, true);
  return i32x2p_t{hi, lo};
}

}  // namespace

__global__ __launch_bounds__(kPThreads, 1) void attn_latent_pair_kernel(LatentArgs a) {
  __shared__ __align__(1024) uint8_t s_tile[kNBuf * kBuf];
  __shared__ int s_pid[kPPidWin];
  __shared__ f32x4_t s_sc[2][kPW][2][kWave];   // [tile parity][wave][token block][lane]: partial scores
  __shared__ int s_bad;
  __shared__ uint32_t s_flag[kPW];

  // XCD-aware block decode: head groups of one (request, split) unit are 8 ids apart
  const int n_hg = (a.num_q_heads + kPHB - 1) / kPHB;
  const int b = blockIdx.x;
  const int grp = b / (8 * n_hg), rem = b % (8 * n_hg);
  const int hg = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= a.batch * a.num_splits) return;
  const int r = unit / a.num_splits, split = unit % a.num_splits;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, q4 = lane >> 4;
  const int x = wave >> 2;                       // half of the dims
  const int S = a.page_size;
  const int lgS = __builtin_ctz(S);   // S is a power of two (checked on the host)
  const int Hq = a.num_q_heads;
  const int hb0 = hg * kPHB, hb1 = min(Hq, hb0 + kPHB);
  const int h0 = hb0 + 16 * (wave & 3);          // this pair's first head
  const bool active = h0 < Hq;                   // wave-uniform (Hq is a multiple of 16)

  const int L = a.ctx_lens[r];
  uint32_t checked = 0;
  if (a.page_tags != nullptr) {  // the check in this launch: before any page of r is read or written
    checked = block_tag_check<kPW>(a, r, L, s_flag);
    if (split == 0 && hg == 0 && threadIdx.x == 0) a.flags_out[r] = checked;
  }
  const bool aborted = checked != 0u || (a.flags != nullptr && a.flags[r] != 0u);
  const bool bad_len = L <= 0 || L > a.max_ctx || L > a.pt_stride * S;
  const int chunk = a.chunk_tiles * kPT;
  const int c0 = split * chunk;
  if (aborted || bad_len) {
    if (a.num_splits == 1) {
      for (int e = threadIdx.x; e < (hb1 - hb0) * kPV; e += kPThreads)
        a.out[((int64_t)r * Hq + hb0) * kPV + e] = 0;
    }
    return;
  }
  if (c0 >= L) return;
  const int c1 = min(L, c0 + chunk);

  // ---- q: lane (q4, n) holds head h0 + n as two e4m3 terms hi + lo of q * s, s a power of two per head
  // with max|q s| in [128, 256) over all 576 dims (both waves of the pair find the same s).  Big k-step
  // j: dims 256 x + 128 j + 32 q4 + b (b < 32) as byte b of qh[j] / ql[j]; small step: dims
  // 512 + 32 x + 8 q4 + b (b < 8) of qsh / qsl.
  v8ip_t qh[2], ql[2];
  i32x2p_t qsh, qsl;
  float q_unscale = 1.f;
  {
    const bool live = active && h0 + n < Hq;
    const uint16_t* qrow = a.q + ((int64_t)r * Hq + h0 + n) * kPD;
    float amax = 0.f;
    if (live) {
#pragma unroll
      for (int i = 0; i < 18; ++i) {  // dims 144 q4 + 8 i .. +8
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(qrow + 144 * q4 + 8 * i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w[e] & 0xFFFFu)), fabsf(bf16_bits_to_f32(w[e] >> 16))));
      }
    }
    amax = fmaxf(amax, shfl_xor(amax, 16));
    amax = fmaxf(amax, shfl_xor(amax, 32));
    int ex;
    frexpf(amax, &ex);
    const float qs = ldexpf(1.f, 8 - ex);
    q_unscale = ldexpf(1.f, ex - 8);
    auto load8 = [&](int d0, float (&f)[8]) {
      const u32x4_t w = live ? *reinterpret_cast<const u32x4_t*>(qrow + d0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu) * qs;
        f[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16) * qs;
      }
    };
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float f[8];
        load8(256 * x + 128 * j + 32 * q4 + 8 * i, f);
        const i32x2p_t t0 = to_hilo(f[0], f[1], f[2], f[3]), t1 = to_hilo(f[4], f[5], f[6], f[7]);
        qh[j][2 * i] = t0[0];
        ql[j][2 * i] = t0[1];
        qh[j][2 * i + 1] = t1[0];
        ql[j][2 * i + 1] = t1[1];
      }
    float f[8];
    load8(512 + 32 * x + 8 * q4, f);
    const i32x2p_t t0 = to_hilo(f[0], f[1], f[2], f[3]), t1 = to_hilo(f[4], f[5], f[6], f[7]);
    qsh = i32x2p_t{t0[0], t1[0]};
    qsl = i32x2p_t{t0[1], t1[1]};
  }
  // The step's token (later layers of a decode step), stored before any tile copy by both head-group
  // blocks whose chunk holds position L - 1 (the same bytes); the wait below also retires these
  // stores, and the barrier that opens the window loop orders them before every wave's copies.
  const bool tok_bad = a.c_new != nullptr && c0 <= L - 1 && L - 1 < c0 + chunk &&
                       !store_latent_row<true, kPD>(a, r, L, kPThreads);
  pair_vm_wait<0>();  // q has landed (and the token's stores are done) before any tile copy is in flight

  // LDS offsets this lane reads inside a tile buffer (token block mb: token 16 mb + n at lrow)
  const int qk_off0 = lrow(n) * kRS + 256 * x + 32 * q4, qk_off1 = lrow(16 + n) * kRS + 256 * x + 32 * q4;  // + 128 j
  const int qs_off0 = lrow(n) * kRS + 512 + 32 * x + 8 * q4, qs_off1 = lrow(16 + n) * kRS + 512 + 32 * x + 8 * q4;
  const int pv_off = lrow(pv_token(q4, n >> 1)) * kRS + 256 * x + 8 * (n & 1);   // + 16 db
  // this lane's share of each tile copy: slot 64 j + lane (j = wave NPW + k) is chunk c of row rho
  uint32_t cp_tc[kNPW];
#pragma unroll
  for (int k = 0; k < kNPW; ++k) {
    const int slot = 64 * (wave * kNPW + k) + lane;
    const int rho = slot / kSlots, c = slot % kSlots;
    const int tok = ltok(rho);
    cp_tc[k] = (rho < kPT && c < kCH) ? (uint32_t)((tok << 16) | ((tok & 15) * kRowB + 16 * c)) : 0u;
  }

  const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
  const uint8_t* pool = reinterpret_cast<const uint8_t*>(a.pool);
  const float c_qk = a.qk_scale_log2 * q_unscale;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t own[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};  // this wave's partial, next tile
  bool bad = tok_bad;

  const int win = ((kPPidWin - 1) * S / kPT) * kPT;
  for (int w0 = c0; w0 < c1; w0 += win) {
    const int w1 = min(c1, w0 + win);
    const int e0 = w0 / S;
    const int ne = (w1 - 1) / S - e0 + 1;
    __syncthreads();  // the previous window's ids and tiles are no longer read
    for (int i = threadIdx.x; i < ne; i += kPThreads) {
      int p = pt[e0 + i];
      if (p < 0 || p >= a.num_pages) {
        bad = true;
        p = -1;
      }
      s_pid[i] = p;
    }
    __syncthreads();
    const int ntile = (w1 - w0 + kPT - 1) / kPT;

    // Copy tile t into buffer bi; a tile past the window is not copied (such loads would still cost
    // their issue and return).  Every load stays inside the pool (tokens past the end and padding
    // slots re-read the tile's first row; a bad page id reads page 0).
    auto copy_tile = [&](int t, int bi) {
      if (t >= ntile) return;
      const int tb_c = w0 + t * kPT;  // t < ntile
      const int nv = w1 - tb_c;
      // (S a power of two: page and slot by shift and mask; both page ids read from LDS together)
      const int s0 = __builtin_amdgcn_readfirstlane(s_pid[(tb_c >> lgS) - e0]);
      const int s1 = __builtin_amdgcn_readfirstlane(s_pid[min(((tb_c + 16) >> lgS) - e0, ne - 1)]);
      const int pid0 = s0;
      const int pid1 = nv > 16 ? s1 : pid0;
      const uint8_t* base0 = pool + (pid0 >= 0 ? (((int64_t)pid0 << lgS) + (tb_c & (S - 1))) * kRowB : 0);
      const uint8_t* base1 =
          nv > 16 ? pool + (pid1 >= 0 ? (((int64_t)pid1 << lgS) + ((tb_c + 16) & (S - 1))) * kRowB : 0) : base0;
      const uint32_t dst = (uint32_t)(uintptr_t)((lds_b*)(s_tile + bi * kBuf) + 1024 * wave * kNPW);
#pragma unroll
      for (int k = 0; k < kNPW; ++k) {
        const uint32_t tc = cp_tc[k];
        const int tok = (int)(tc >> 16);
        const uint32_t off = tok < nv ? (tc & 0xFFFFu) : 0u;
        pair_copy16((tok < nv && tok >= 16 ? base1 : base0) + off, dst + 1024 * k);
      }
    };

#pragma unroll
    for (int t = 0; t < kNBuf - 2; ++t) copy_tile(t, t);
    for (int t = -1; t < ntile; ++t) {
      // this wave's copies of tile t+1 have landed: those issued after them are the copies of the next
      // kNBuf-3 tiles that exist
      pair_vm_wait_tiles<kNPW, kNBuf - 3>(ntile - (t + 2));
      __syncthreads();                     // everyone's have; everyone is done with tile t-1
      copy_tile(t + kNBuf - 1, (t + kNBuf - 1) % kNBuf);
      if (!active) continue;
      const bool has_cur = t >= 0;
      uint32_t off_n = (uint32_t)(((t + 1) % kNBuf) * kBuf), off_c = (uint32_t)(((t + kNBuf) % kNBuf) * kBuf);
      asm volatile("" : "+s"(off_n), "+s"(off_c));
      const uint8_t* tile_n = s_tile + off_n;
      const lds_b* lt_c = (const lds_b*)(s_tile + off_c);
      const int nv = w1 - (w0 + t * kPT);

      // ---- softmax of tile t: the pair's partial scores added (own from registers, the partner's from
      // LDS; a + b == b + a, so both waves get the same sums)
      float xs[8];
      if (has_cur) {
        const int pa = t & 1;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const f32x4_t v = s_sc[pa][wave ^ 4][mb][lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool valid = 16 * mb + 4 * q4 + i < nv;
            xs[4 * mb + i] = valid ? (own[mb][i] + v[i]) * c_qk : -INFINITY;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[j] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) tmax = fmaxf(tmax, xs[j]);
      tmax = max_x16(tmax);
      tmax = max_x32(tmax);
      const bool grow = tmax > m_run + kPLazy;
      if (__any(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 16; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;

      // ---- partial S^T of tile t+1 over this wave's dims (past the last tile the reads hit stale data);
      // the two token blocks' MFMA chains alternate
      f32x4_t sn[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v8ip_t av[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const uint8_t* src = tile_n + (mb ? qk_off1 : qk_off0) + 128 * j;
          const u32x4_t k0 = *reinterpret_cast<const u32x4_t*>(src), k1 = *reinterpret_cast<const u32x4_t*>(src + 16);
          av[mb] = v8ip_t{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3], (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
        }
        sn[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[0], qh[j], sn[0], 0, 0, 0, 0, 0, 0);
        sn[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[1], qh[j], sn[1], 0, 0, 0, 0, 0, 0);
        sn[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[0], ql[j], sn[0], 0, 0, 0, 0, 0, 0);
        sn[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[1], ql[j], sn[1], 0, 0, 0, 0, 0, 0);
      }
      {
        const long qa = (long)(((uint64_t)(uint32_t)qsh[1] << 32) | (uint32_t)qsh[0]);
        const long qb = (long)(((uint64_t)(uint32_t)qsl[1] << 32) | (uint32_t)qsl[0]);
        const u32x2_t k0 = *reinterpret_cast<const u32x2_t*>(tile_n + qs_off0);
        const u32x2_t k1 = *reinterpret_cast<const u32x2_t*>(tile_n + qs_off1);
        const long ka0 = (long)(((uint64_t)k0[1] << 32) | k0[0]), ka1 = (long)(((uint64_t)k1[1] << 32) | k1[0]);
        sn[0] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka0, qa, sn[0], 0, 0, 0);
        sn[1] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka1, qa, sn[1], 0, 0, 0);
        sn[0] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka0, qb, sn[0], 0, 0, 0);
        sn[1] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(ka1, qb, sn[1], 0, 0, 0);
      }
      // exponentials of tile t while the MFMAs run
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        xs[j] = __builtin_amdgcn_exp2f(xs[j] - m_use);
        psum += xs[j];
      }
      const int pn = (t + 1) & 1;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s_sc[pn][wave][mb][lane] = sn[mb];
        own[mb] = sn[mb];
      }

      if (has_cur) {
        // ---- O^T += V^T P^T of tile t over this wave's 256 value dims: 16 blocks of 16 dims
        l_run += psum;
        u32x4_t pp;
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[e] = pack_bf16x2(xs[2 * e], xs[2 * e + 1]);
        constexpr int PD = 4;  // transpose reads ahead
        i32x2p_t vb[PD + 1];
#pragma unroll
        for (int i = 0; i < PD; ++i)
          vb[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2p_t*)(lt_c + pv_off + 16 * i));
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          if (db + PD < 16)
            vb[(db + PD) % (PD + 1)] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2p_t*)(lt_c + pv_off + 16 * (db + PD)));
          const i32x2p_t raw = vb[db % (PD + 1)];
          const u32x2_t lo = e4m3x4_to_bf16x4((uint32_t)raw[0]), hi = e4m3x4_to_bf16x4((uint32_t)raw[1]);
          const u32x4_t va = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                            __builtin_bit_cast(bf16x8_t, pp), acc[db], 0, 0, 0);
        }
      }
    }
    pair_vm_wait<0>();  // copies issued past the window's last tile have landed before the buffers are reused
  }

  // ---- write this wave's heads and value dims (a page id outside the pool zeroes the request)
  __syncthreads();
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;
  if (!active) return;
  l_run = sum_x16(l_run);
  l_run = sum_x32(l_run);
  const int h = h0 + n;
  if (h >= Hq) return;
  const int64_t row = (int64_t)r * Hq + h;
  const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
  if (a.num_splits == 1) {
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const int d0 = 256 * x + 16 * db + 4 * q4;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = any_bad ? 0.f : acc[db][i] * inv;
      *reinterpret_cast<u32x2_t*>(&a.out[row * kPV + d0]) = u32x2_t{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  } else {
    // fp16 partials of acc / l (convex combinations of e4m3 values, |x| <= 448: no overflow, an 11-bit
    // significand); the merge applies the tensor scale
    const int64_t slot = row * a.num_splits + split;
    const float il = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* oh = reinterpret_cast<uint16_t*>(a.o_part);
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const int d0 = 256 * x + 16 * db + 4 * q4;
      const f32x4_t v = acc[db] * il;
      *reinterpret_cast<u32x2_t*>(&oh[slot * kPV + d0]) = u32x2_t{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    }
    if (x == 0 && q4 == 0)
      a.lse_part[slot] = any_bad ? NAN : (l_run == 0.f ? -INFINITY : m_run + __log2f(l_run));
  }
}

// Grid: 8-aligned groups of (request, split) units times head groups of 64.
hipError_t launch_attn_latent_pairs(const LatentArgs& a, hipStream_t stream) {
  const int n_hg = (a.num_q_heads + kPHB - 1) / kPHB;
  const int units = a.batch * a.num_splits;
  const int blocks = ((units + 7) / 8) * 8 * n_hg;
  hipLaunchKernelGGL(attn_latent_pair_kernel, dim3(blocks), dim3(kPThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvfp8
