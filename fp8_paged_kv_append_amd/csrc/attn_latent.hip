// Split-K paged decode attention over a latent (MLA-style) cache: one vector of
// width 576 per token, shared by every query head; scores use all 576 dims, the
// values are its first 512.  FP8 (e4m3) or BF16 cache, gfx950.
//
// What it computes is the same softmax attention as the GQA kernel (Cloudflare
// blog "Smaller, faster, safer: running Kimi and GLM at scale", section
// "Quantized KV cache": the FP8 cache is converted as it is read), with one
// cached vector serving as both key and value.  Unlike GQA this shape is bound
// by the matrix units, not by HBM: 128 heads x (576 + 512) MACs per cached element.
//
// Block = (request r, split c, group of 128 query heads), 4 waves, one wave per
// SIMD.  Wave w owns 32 heads over the whole contraction and all 512 value dims:
// its q (144 VGPRs) and its O accumulators (256 registers, AGPRs) stay resident,
// so every element a wave converts feeds a 32-head MFMA, and no partial sums
// cross waves.  The latent pool is row-major ([page][slot][576]); each 32-token
// tile is copied as stored into LDS by direct global->LDS loads (no VGPRs), into
// a ring of NBUF buffers, NBUF-1 tiles ahead of the math; one barrier per tile.
// A token row sits at LDS row sigma(t) with a 16-byte pad: both the row reads
// of QK and the transpose reads of PV then touch every bank once per phase.
// With lane l = 32*hh + n (n = head within the wave):
//  * S^T = C q^T: v_mfma_f32_32x32x16_bf16, A = 32 token rows x 16 dims (lane
//    reads 8 dims of row l%32), B = q^T (lane holds head n).  Contraction slot
//    (k-step 2p+x, half hh, element e) is dim 32p + 16hh + 8x + e, so a lane
//    reads 16 contiguous bytes of its row per pair of k-steps.
//  * C layout: lane (hh, n) holds head n's scores for tokens 8(j/4) + 4hh + j%4
//    (j = 0..15); the softmax is lane-local apart from one xor-32 shuffle.
//  * O^T += V^T P^T per 32-dim block: B = P^T, slot (hh, e) of k-step ks is
//    token 8(2ks + e/4) + 4hh + e%4 -- register 8ks + e of the scores, so the
//    lane already holds its P.  A = V^T comes from the gfx950 LDS transpose
//    loads: ds_read_b64_tr_b8 gives lane 8h+e of a 16-lane group byte e of the
//    8-byte blocks named by lanes h, h+2, .., h+14; ds_read_b64_tr_b16 gives
//    lane 4a+e element e of the blocks named by lanes a, a+4, a+8, a+12.
//  * Online softmax in the log2 domain, lazy: the accumulators are rescaled
//    only when a head's running max grows by more than 2^8.
// In a decode step the same launch may also store the step's token (the
// block(s) whose split holds position L - 1 quantise it and store it into its
// page before their first tile copy, then read it back like any other row) and,
// for the FP8 cache, check the request's page tags first (every block, before
// it reads or writes any page; a variant of its own, CHECK).
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kLD = kLatentDim;           // 576: latent width (score dim)
constexpr int kLV = kLatentVDim;          // 512: value dim
constexpr int kLT = kLatentTileTokens;    // 32 tokens per tile
constexpr int kLWaves = 4;
constexpr int kLThreads = kLWaves * kWave;
constexpr int kLHW = 32;                  // heads per wave
constexpr int kLPidWin = 1024;
constexpr float kLazy = 8.f;              // log2-domain slack before the accumulators are rescaled
static_assert(kLPidWin % kLThreads == 0, "a window's page ids are loaded as kLPidWin / kLThreads per thread");

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

template <bool FP8>
struct LCfg {
  static constexpr int ELT = FP8 ? 1 : 2;
  static constexpr int ROWB = kLD * ELT;                          // bytes per token row
  static constexpr int RS = ROWB + 16;                            // LDS row stride
  static constexpr int CH = ROWB / 16;                            // 16-byte chunks per row
  static constexpr int SLOTS = RS / 16;                           // chunk slots per LDS row
  static constexpr int NINST = (kLT * SLOTS + 63) / 64;           // 1 KiB copies per tile
  static constexpr int NPW = (NINST + kLWaves - 1) / kLWaves;     // copies per wave per tile
  static constexpr int BUF = NPW * kLWaves * 1024;                // bytes per tile buffer
  static constexpr int NBUF = FP8 ? 4 : 3;                        // tile buffers
};

// LDS row of tile token t.  FP8: the 8 tokens a PV transpose read of one half-wave
// gathers land on rows 2 apart (mod 16); BF16: its 4 tokens land on rows 4 apart.
template <bool FP8>
__device__ __forceinline__ int lat_row(int t) {
  return FP8 ? 16 * (t >> 4) + 8 * ((t >> 3) & 1) + 2 * (t & 3) + ((t >> 2) & 1)
             : 16 * (t >> 4) + 4 * (t & 3) + 2 * ((t >> 2) & 1) + ((t >> 3) & 1);
}
template <bool FP8>
__device__ __forceinline__ int lat_tok(int row) {  // inverse of lat_row
  const int u = row >> 4, x = row & 15;
  return FP8 ? 16 * u + 8 * (x >> 3) + 4 * (x & 1) + ((x >> 1) & 3)
             : 16 * u + 8 * (x & 1) + 4 * ((x >> 1) & 1) + (x >> 2);
}
// tile token of PV contraction slot k (0..15) of k-step ks
__device__ __forceinline__ int pv_tok(int ks, int k) { return 8 * (2 * ks + ((k & 7) >> 2)) + 4 * (k >> 3) + (k & 3); }

// 16 bytes per lane from global memory straight into LDS at lds_addr + 16*lane (lds_addr
// wave-uniform, in M0).  Issued through asm so that the compiler does not treat every later LDS
// read as possibly aliasing an in-flight copy (it would wait for all copies before each tile);
// the copies are waited for explicitly with vm_wait before the barrier that publishes a tile.
// M0 is reserved by the compiler, so the asm restores it.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds_addr) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "v"(src), "s"(lds_addr)
      : "memory");
}

// wait until at most N vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most the copies of n tiles (NPW loads each; n clamped to 0 .. MAXT) are outstanding
template <int NPW, int MAXT>
__device__ __forceinline__ void vm_wait_tiles(int n) {
  if constexpr (MAXT > 0) {
    if (n >= MAXT) {
      vm_wait<NPW * MAXT>();
      return;
    }
    vm_wait_tiles<NPW, MAXT - 1>(n);
  } else {
    vm_wait<0>();
  }
}

// CHECK: the launch also runs the tag check (a.page_tags non-null).  A variant of its own, so that the
// launches without it keep the register allocation of the kernel without the check code (the
// 128-head kernel uses the whole register file).
template <bool FP8, bool CHECK>
__global__ __launch_bounds__(kLThreads) void attn_latent_split_kernel(LatentArgs a) {
  using C = LCfg<FP8>;
  constexpr int ELT = C::ELT;
  __shared__ __align__(1024) uint8_t s_tile[C::NBUF * C::BUF];
  __shared__ int s_pid[kLPidWin];
  __shared__ f32x4_t s_sc[FP8 ? 1 : kLWaves][4][kWave];  // BF16: each wave's next-tile scores, parked across PV
  __shared__ int s_bad;
  __shared__ uint32_t s_flag[kLWaves];

  // XCD-aware block decode: head groups of one (request, split) unit are 8 ids apart
  const int b = blockIdx.x;
  const int grp = b / (8 * a.n_hg), rem = b % (8 * a.n_hg);
  const int hg = rem / 8;
  const int unit = grp * 8 + rem % 8;
  if (unit >= a.batch * a.num_splits) return;
  const int r = unit / a.num_splits, split = unit % a.num_splits;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int S = a.page_size;
  const int lgS = __builtin_ctz(S);   // S is a power of two (checked on the host)
  const int Hq = a.num_q_heads;
  const int hb0 = hg * kLatentHeadsPerBlock, hb1 = min(Hq, hb0 + kLatentHeadsPerBlock);
  const int h0 = hb0 + wave * kLHW;     // this wave's first head
  const bool active = h0 < Hq;          // wave-uniform

  const int L = a.ctx_lens[r];
  uint32_t checked = 0;
  if constexpr (CHECK) {  // the check in this launch: before any page of r is read or written
    checked = block_tag_check<kLWaves>(a, r, L, s_flag);
    if (split == 0 && hg == 0 && threadIdx.x == 0) a.flags_out[r] = checked;
  }
  const bool aborted = checked != 0u || (a.flags != nullptr && a.flags[r] != 0u);
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

  // q operand.  BF16 cache (bf16 MFMA): lane (hh, n) holds head h0+n, dims 32p + 16hh + 8x .. +8 as
  // qv[2p + x].  FP8 cache: QK runs on FP8 MFMAs (v_mfma_f32_32x32x64_f8f6f4) over the cached e4m3 bytes
  // as stored; q*s, with s a power of two per head that puts max|q*s| in [128, 256), is held as two e4m3
  // terms hi + lo, lo = e4m3(q*s - hi) (exact for every element within 2^9 of the head's max |q|), and
  // 1/s joins the score scale.  Lane (hh, n) holds dims 64ks + 32hh + b (b = 0..31) of k-step ks as byte b
  // of qhi[ks] / qlo[ks].
  u32x4_t qv[36];
  v8i_t qhi[9], qlo[9];
  const bool q_live = h0 + n < Hq;
  if constexpr (FP8) {
    // the raw bf16 q (dims 64ks + 32hh .. +32 of this lane's head: 16 words per k-step, the first 8 in
    // qhi[ks], the rest in qlo[ks]) is loaded here and turned into its two e4m3 terms in place once the
    // first tiles' copies are in flight (below), so that its load overlaps the page-id loads and its
    // conversion the copies
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q + ((int64_t)r * Hq + h0 + n) * kLD + 32 * hh);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t w = q_live ? qp[8 * ks + i] : u32x4_t{0, 0, 0, 0};  // dims 64ks + 32hh + 8i .. +8
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (i < 2)
            qhi[ks][4 * i + e] = (int)w[e];
          else
            qlo[ks][4 * (i - 2) + e] = (int)w[e];
        }
      }
  } else {
    if (q_live) {
      const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(a.q + ((int64_t)r * Hq + h0 + n) * kLD + 16 * hh);
#pragma unroll
      for (int p = 0; p < 18; ++p) {
        qv[2 * p] = qp[4 * p];
        qv[2 * p + 1] = qp[4 * p + 1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 36; ++k) qv[k] = u32x4_t{0, 0, 0, 0};
    }
  }
  // FP8: q*s, with s a power of two per head that puts max|q*s| in [128, 256), as two e4m3 terms hi + lo,
  // lo = e4m3(q*s - hi) (exact for every element within 2^9 of the head's max |q|); 1/s joins the score
  // scale.  Lane (hh, n) then holds dims 64ks + 32hh + b (b = 0..31) of k-step ks as byte b of qhi[ks] /
  // qlo[ks].
  float q_unscale = 1.f;
  auto q_to_fp8 = [&]() {
    float amax = 0.f;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w0 = (uint32_t)qhi[ks][j], w1 = (uint32_t)qlo[ks][j];
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w0 & 0xFFFFu)), fabsf(bf16_bits_to_f32(w0 >> 16))));
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(w1 & 0xFFFFu)), fabsf(bf16_bits_to_f32(w1 >> 16))));
      }
    amax = fmaxf(amax, shfl_xor(amax, 32));
    int ex;
    frexpf(amax, &ex);  // amax < 2^ex
    const float qs = ldexpf(1.f, 8 - ex);
    q_unscale = ldexpf(1.f, ex - 8);
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) {
      // one k-step at a time, its words taken as new values: otherwise the compiler keeps the max pass's
      // unpacked floats of all of q live for this pass and runs out of registers
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" : "+v"(qhi[ks]), "+v"(qlo[ks]));
      uint32_t w[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w[j] = (uint32_t)qhi[ks][j];
        w[8 + j] = (uint32_t)qlo[ks][j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const uint32_t wa = w[4 * i + 2 * h2], wb = w[4 * i + 2 * h2 + 1];
          const float f0 = bf16_bits_to_f32(wa & 0xFFFFu) * qs, f1 = bf16_bits_to_f32(wa >> 16) * qs;
          const float f2 = bf16_bits_to_f32(wb & 0xFFFFu) * qs, f3 = bf16_bits_to_f32(wb >> 16) * qs;
          int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f0, f1, 0, false);
          hi = __builtin_amdgcn_cvt_pk_fp8_f32(f2, f3, hi, true);
          const auto b0 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false), b1 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
          int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0 - b0[0], f1 - b0[1], 0, false);
          lo = __builtin_amdgcn_cvt_pk_fp8_f32(f2 - b1[0], f3 - b1[1], lo, true);
          qhi[ks][2 * i + h2] = hi;
          qlo[ks][2 * i + h2] = lo;
        }
    }
  };

  // The step's token (later layers of a decode step), stored before any tile copy by the block(s)
  // whose chunk holds position L - 1 (all head groups of that chunk store the same bytes); the wait
  // below also retires these stores, and the barrier that opens the window loop orders them before
  // every wave's copies, which then read the token back like any other row.
  const bool tok_bad = a.c_new != nullptr && c0 <= L - 1 && L - 1 < c0 + chunk &&
                       !store_latent_row<FP8, kLD>(a, r, L, kLThreads);

  // LDS byte offsets this lane reads, relative to a tile buffer
  // QK row reads: FP8 32 bytes at lat_row(n)*RS + 32hh + 64*ks; BF16 32 bytes at lat_row(n)*RS + 32hh + 64*p
  const int qk_off = lat_row<FP8>(n) * C::RS + 32 * hh;
  // PV source of k-step ks, read rd: pv_off + ks*16*RS + rd*RS (+ 32*db*ELT per d-block) -- the
  // tokens of k-step 1 are those of k-step 0 plus 16 (LDS rows + 16), and the second BF16 read's
  // tokens are the first's plus 8 (LDS row + 1), under lat_row
  int pv_off;
  {
    const int g = lane >> 4;
    if (FP8) {
      const int h = lane & 1, i = (lane & 15) >> 1;
      pv_off = lat_row<FP8>(pv_tok(0, 8 * (g >> 1) + i)) * C::RS + 16 * (g & 1) + 8 * h;
    } else {
      const int aa = lane & 3, i = (lane & 15) >> 2;
      pv_off = lat_row<FP8>(pv_tok(0, 8 * (g >> 1) + i)) * C::RS + 2 * (16 * (g & 1) + 4 * aa);
    }
  }
  // this lane's share of each tile copy: copy k of the wave fills LDS slots [64j, 64j+64),
  // j = wave*NPW + k; slot 64j+lane is chunk c of LDS row rho = token lat_tok(rho), or padding
  // each entry: (token << 16) | byte offset of the chunk inside its 16-token half (token & 15
  // rows in), or 0 for a padding slot (token 0, chunk 0: a harmless re-read)
  uint32_t cp_tc[C::NPW];
#pragma unroll
  for (int k = 0; k < C::NPW; ++k) {
    const int slot = 64 * (wave * C::NPW + k) + lane;
    const int rho = slot / C::SLOTS, c = slot % C::SLOTS;
    const int tok = lat_tok<FP8>(rho);
    cp_tc[k] = (rho < kLT && c < C::CH) ? (uint32_t)((tok << 16) | ((tok & 15) * C::ROWB + 16 * c)) : 0u;
  }

  const int32_t* pt = a.page_table + (int64_t)r * a.pt_stride;
  const uint8_t* pool = reinterpret_cast<const uint8_t*>(a.pool);
  float c_qk = a.qk_scale_log2;  // log2-domain score scale (FP8: times 1/s, once q is converted)
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) acc[db] = f32x16_t{};
  bool bad = tok_bad;

  // Tokens [c0, c1) in windows of at most kLPidWin - 1 pages (a window starting mid-page still fits
  // kLPidWin ids), whose page ids are staged in LDS.
  const int win = ((kLPidWin - 1) * S / kLT) * kLT;
  int w0 = c0, w1 = 0, e0 = 0, ne = 0, ntile = 0;
  auto window_setup = [&]() {
    w1 = min(c1, w0 + win);
    e0 = w0 / S;
    ne = (w1 - 1) / S - e0 + 1;
    // the window's page ids (at most kLPidWin: kLPidWin / kLThreads per thread), loaded before the
    // barrier; in the first window they are in flight with q's loads and the token's stores, all of
    // which have landed before any tile copy is issued (the tile loop then carries no waits for them)
    int pre[kLPidWin / kLThreads];
#pragma unroll
    for (int k = 0; k < kLPidWin / kLThreads; ++k) {
      const int i = threadIdx.x + k * kLThreads;
      pre[k] = i < ne ? pt[e0 + i] : 0;
    }
    vm_wait<0>();
    __syncthreads();  // the previous window's ids and tiles are no longer read
#pragma unroll
    for (int k = 0; k < kLPidWin / kLThreads; ++k) {
      const int i = threadIdx.x + k * kLThreads;
      if (i < ne) {
        int p = pre[k];
        if (p < 0 || p >= a.num_pages) {
          bad = true;
          p = -1;
        }
        s_pid[i] = p;
      }
    }
    __syncthreads();
    ntile = (w1 - w0 + kLT - 1) / kLT;
  };

  // Copy tile t of the window into buffer bi: NPW 16-byte global->LDS loads per lane.  FP8 copies no
  // tile past the window's end (such loads would still cost their issue and return); BF16 does, since
  // the branch costs it a spill.  Every lane of every copy loads from inside the pool: tokens past the
  // window end re-read the tile's first row (finite data, weight 0), padding slots and tiles past the
  // end read the first row too, and a page id outside the pool reads the pool's first page (the
  // request is zeroed).
  struct CopyTile {
    const uint8_t* base0;
    const uint8_t* base1;
    uint32_t dst;
    int nv;
  };
  auto copy_prep = [&](int t, int bi) {
    CopyTile ct;
    const int tb = w0 + t * kLT;
    const bool live = t < ntile;
    ct.nv = live ? w1 - tb : 0;
    const int tb_c = live ? tb : w0;
    // the two 16-token halves of a tile each lie inside one page (tile starts are 32-aligned, S % 16 == 0)
    // wave-uniform: kept in SGPRs, so the copy state costs no VGPRs across QK and PV
    // (S a power of two: page and slot by shift and mask; both page ids read from LDS together, the
    // second clamped into the window's staged entries when the tile has no second half)
    const int s0 = __builtin_amdgcn_readfirstlane(s_pid[(tb_c >> lgS) - e0]);
    const int s1 = __builtin_amdgcn_readfirstlane(s_pid[min(((tb_c + 16) >> lgS) - e0, ne - 1)]);
    const int pid0 = s0;
    const int pid1 = ct.nv > 16 ? s1 : pid0;
    ct.base0 = pool + (pid0 >= 0 ? (((int64_t)pid0 << lgS) + (tb_c & (S - 1))) * C::ROWB : 0);
    ct.base1 = ct.nv > 16 ? pool + (pid1 >= 0 ? (((int64_t)pid1 << lgS) + ((tb_c + 16) & (S - 1))) * C::ROWB : 0)
                          : ct.base0;
    ct.dst = (uint32_t)(uintptr_t)((lds_u8*)(s_tile + bi * C::BUF) + 1024 * wave * C::NPW);
    return ct;
  };
  auto copy_one = [&](const CopyTile& ct, int k) {
    const uint32_t tc = cp_tc[k];
    const int tok = (int)(tc >> 16);
    const uint32_t off = tok < ct.nv ? (tc & 0xFFFFu) : 0u;  // past the end: the tile's first row
    const uint8_t* src = (tok < ct.nv && tok >= 16 ? ct.base1 : ct.base0) + off;
    lds_copy16(src, ct.dst + 1024 * k);
  };
  auto copy_tile = [&](int t, int bi) {
    if constexpr (FP8) {
      if (t >= ntile) return;
    }
    const CopyTile ct = copy_prep(t, bi);
#pragma unroll
    for (int k = 0; k < C::NPW; ++k) copy_one(ct, k);
  };

  // Tiles are software-pipelined by one: iteration t publishes tile t+1 and computes its scores
  // (QK MFMAs) while tile t's exponentials run between them, then accumulates tile t (PV).  The
  // ring holds tile t (PV), tile t+1 (QK) and NBUF-2 tiles whose copies are in flight.
  constexpr int QD = FP8 ? 1 : 1, PD = FP8 ? 4 : 2;  // operand reads ahead of the math
  auto qk_read = [&](const uint8_t* tile, int p, u32x4_t(&dst)[2]) {  // 32 bytes of this lane's row
    dst[0] = *reinterpret_cast<const u32x4_t*>(tile + qk_off + 64 * p);
    dst[1] = *reinterpret_cast<const u32x4_t*>(tile + qk_off + 64 * p + 16);
  };
  auto pv_read = [&](const lds_u8* lt, int i, u32x4_t& dst) {  // PV step i = 16*ks + db
    const int db = i & 15, ks = i >> 4;
    const lds_u8* src = lt + pv_off + ks * 16 * C::RS + 32 * ELT * db;
    if (FP8) {
      const i32x2_t t8 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)src);
      dst[0] = (uint32_t)t8[0];
      dst[1] = (uint32_t)t8[1];
    } else {
      const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)src);
      const i16x4_t t1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(src + C::RS));
      const u32x2_t u0 = __builtin_bit_cast(u32x2_t, t0), u1 = __builtin_bit_cast(u32x2_t, t1);
      dst = u32x4_t{u0[0], u0[1], u1[0], u1[1]};
    }
  };
  auto pv_cvt = [&](const u32x4_t& raw) {
    if (FP8) {
      const u32x2_t lo = e4m3x4_to_bf16x4(raw[0]), hi = e4m3x4_to_bf16x4(raw[1]);
      return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
    return raw;
  };

  f32x16_t sc_next = f32x16_t{};  // scores of the next tile, from one iteration's QK to the next one's softmax
  window_setup();
#pragma unroll
  for (int t = 0; t < C::NBUF - 2; ++t) copy_tile(t, t);
  if constexpr (FP8) {  // q's e4m3 terms, while the first tiles land
    q_to_fp8();
    c_qk = a.qk_scale_log2 * q_unscale;
  }
  while (true) {
    for (int t = -1; t < ntile; ++t) {
      // this wave's copies of tile t+1 have landed: those issued after them are the copies of the next
      // NBUF-3 tiles (FP8: of those that exist)
      vm_wait_tiles<C::NPW, C::NBUF - 3>(FP8 ? ntile - (t + 2) : C::NBUF - 3);
      __syncthreads();                    // everyone's have; everyone is done with tile t-1
      copy_tile(t + C::NBUF - 1, (t + C::NBUF - 1) % C::NBUF);
      if (!active) continue;
      const bool has_cur = t >= 0;
      // buffer offsets as opaque scalars: every LDS read is then base + lane offset + immediate,
      // rather than one precomputed address per ring slot and step
      uint32_t off_n = (uint32_t)(((t + 1) % C::NBUF) * C::BUF), off_c = (uint32_t)(((t + C::NBUF) % C::NBUF) * C::BUF);
      asm volatile("" : "+s"(off_n), "+s"(off_c));
      const uint8_t* tile_n = s_tile + off_n;
      const lds_u8* lt_c = (const lds_u8*)(s_tile + off_c);
      const int nv = w1 - (w0 + t * kLT);  // valid tokens of tile t (may exceed 32)

      // ---- softmax of tile t, first part: masked scores (log2 domain), tile max, lazy rescale;
      // the scores of head n are those of tokens 8(j/4) + 4hh + j%4 (computed in iteration t-1)
      // the scores of tile t (unused, every token masked, while there is no tile t)
      f32x16_t sc = sc_next;
      if constexpr (!FP8) {
        if (has_cur) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const f32x4_t v = s_sc[wave][k][lane];
            sc[4 * k] = v[0];
            sc[4 * k + 1] = v[1];
            sc[4 * k + 2] = v[2];
            sc[4 * k + 3] = v[3];
          }
        }
      }
      float x[16];
      if (has_cur && nv >= kLT) {  // a full tile: no token to mask
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = sc[j] * c_qk;
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bool valid = has_cur && 8 * (j >> 2) + 4 * hh + (j & 3) < nv;
          x[j] = valid ? sc[j] * c_qk : -INFINITY;
        }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, x[j]);
      tmax = max_x32(tmax);
      const bool grow = tmax > m_run + kLazy;  // m_run = -inf: any finite tile max grows it
      if (__any(grow)) {
        const float m_new = grow ? tmax : m_run;
        const float alpha = grow ? exp2f(m_run - m_new) : 1.f;  // m_run = -inf -> 0
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 16; ++db) {
          // the accumulators live in AGPRs; the empty asm statements pin that register class around
          // the multiply, which would otherwise move all 256 of them into VGPRs
          f32x16_t tv = acc[db];
          asm volatile("" : "+a"(tv));
          f32x16_t u = tv * alpha;
          asm volatile("" : "+v"(u));
          tv = u;
          asm volatile("" : "+a"(tv));
          acc[db] = tv;
        }
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;

      // ---- S^T of tile t+1 = C q^T over all 576 dims (past the last tile the reads hit a buffer whose
      // contents are stale and the result is unused).  Step p issues the read QD steps ahead and one or two
      // of tile t's exponentials while the MFMAs of step p-1 run, then issues step p's MFMAs.
      float psum = 0.f;
      u32x4_t qb[QD + 1][2];
#pragma unroll
      for (int p = 0; p < QD; ++p) qk_read(tile_n, p, qb[p]);
      f32x16_t sn = f32x16_t{};  // the first MFMA starts from an inline zero
      if constexpr (FP8) {
        // 9 k-steps of 64 dims, each two FP8 MFMAs (q hi and lo terms) over the raw cached bytes
#pragma unroll
        for (int p = 0; p < 9; ++p) {
          if (p + QD < 9) qk_read(tile_n, p + QD, qb[(p + QD) % (QD + 1)]);
          if (p < 8) {
            x[2 * p] = __builtin_amdgcn_exp2f(x[2 * p] - m_use);  // v_exp_f32: weights below 2^-126 flush to 0
            x[2 * p + 1] = __builtin_amdgcn_exp2f(x[2 * p + 1] - m_use);
            psum += x[2 * p] + x[2 * p + 1];
            // kept here, between the QK MFMAs: otherwise the compiler moves the exponentials into the PV
            // section, where their only uses are
            asm volatile("" : "+v"(x[2 * p]), "+v"(x[2 * p + 1]), "+v"(psum));
          }
          __builtin_amdgcn_sched_barrier(0);
          const u32x4_t(&kr)[2] = qb[p % (QD + 1)];
          const v8i_t av = {(int)kr[0][0], (int)kr[0][1], (int)kr[0][2], (int)kr[0][3],
                            (int)kr[1][0], (int)kr[1][1], (int)kr[1][2], (int)kr[1][3]};
          sn = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qhi[p], sn, 0, 0, 0, 0, 0, 0);
          sn = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, qlo[p], sn, 0, 0, 0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        // 18 pairs of 16-dim k-steps on bf16 MFMAs
#pragma unroll
        for (int p = 0; p < 18; ++p) {
          if (p + QD < 18) qk_read(tile_n, p + QD, qb[(p + QD) % (QD + 1)]);
          if (p < 16) {
            x[p] = __builtin_amdgcn_exp2f(x[p] - m_use);  // v_exp_f32: weights below 2^-126 flush to 0
            psum += x[p];
            asm volatile("" : "+v"(x[p]), "+v"(psum));
          }
          __builtin_amdgcn_sched_barrier(0);
          const u32x4_t(&raw)[2] = qb[p % (QD + 1)];
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, raw[0]),
                                                       __builtin_bit_cast(bf16x8_t, qv[2 * p]), sn, 0, 0, 0);
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, raw[1]),
                                                       __builtin_bit_cast(bf16x8_t, qv[2 * p + 1]), sn, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the scores are read by VALU: VGPRs (the AGPRs hold the 256 accumulators).  FP8: kept in registers
      // until the next iteration (in those tile t's exponentials leave free once PV has packed them);
      // BF16, whose PV holds more registers, parks them in LDS
      asm volatile("" : "+v"(sn));
      if constexpr (FP8) {
        sc_next = sn;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) s_sc[wave][k][lane] = f32x4_t{sn[4 * k], sn[4 * k + 1], sn[4 * k + 2], sn[4 * k + 3]};
      }

      if (has_cur) {
        // ---- O^T += V^T P^T of tile t: 2 k-steps of 16 tokens x 16 blocks of 32 value dims (the
        // two MFMAs of one accumulator 16 steps apart); step i reads step i+PD and converts step
        // i+1 while the MFMA of step i-1 runs
        u32x4_t vb[PD + 1];
#pragma unroll
        for (int i = 0; i < PD; ++i) pv_read(lt_c, i, vb[i]);
        l_run += psum;
        u32x4_t pp[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 4; ++e) pp[ks][e] = pack_bf16x2(x[8 * ks + 2 * e], x[8 * ks + 2 * e + 1]);
        u32x4_t vop[2];
        vop[0] = pv_cvt(vb[0]);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i + PD < 32) pv_read(lt_c, i + PD, vb[(i + PD) % (PD + 1)]);
          if (i + 1 < 32) vop[(i + 1) & 1] = pv_cvt(vb[(i + 1) % (PD + 1)]);
          __builtin_amdgcn_sched_barrier(0);
          acc[i & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vop[i & 1]),
                                                                __builtin_bit_cast(bf16x8_t, pp[i >> 4]),
                                                                acc[i & 15], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    vm_wait<0>();  // copies issued past the window's last tile have landed before the buffers are reused
    w0 += win;
    if (w0 >= c1) break;
    window_setup();
#pragma unroll
    for (int t = 0; t < C::NBUF - 2; ++t) copy_tile(t, t);
  }

  // ---- write this wave's heads (a page id outside the pool zeroes the request)
  __syncthreads();
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  if (bad) s_bad = 1;
  __syncthreads();
  const bool any_bad = s_bad != 0;
  if (!active) return;
  l_run = sum_x32(l_run);
  const int h = h0 + n;
  if (h >= Hq) return;
  const int64_t row = (int64_t)r * Hq + h;
  const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
  if (a.num_splits == 1) {
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hh;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = any_bad ? 0.f : acc[db][4 * jg + i] * inv;
        const u32x2_t v2 = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        *reinterpret_cast<u32x2_t*>(&a.out[row * kLV + d0]) = v2;
      }
  } else if constexpr (FP8) {
    // fp16 partials of acc / l: convex combinations of e4m3 values (|x| <= 448, so no overflow and an
    // 11-bit significand); the merge applies the tensor scale.  Half the bytes of fp32 partials, written
    // here and read by the merge.
    const int64_t slot = row * a.num_splits + split;
    const float il = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* oh = reinterpret_cast<uint16_t*>(a.o_part);
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hh;
        const u32x2_t v2 = {pack_f16x2(acc[db][4 * jg] * il, acc[db][4 * jg + 1] * il),
                            pack_f16x2(acc[db][4 * jg + 2] * il, acc[db][4 * jg + 3] * il)};
        *reinterpret_cast<u32x2_t*>(&oh[slot * kLV + d0]) = v2;
      }
    if (hh == 0) a.lse_part[slot] = any_bad ? NAN : (l_run == 0.f ? -INFINITY : m_run + __log2f(l_run));
  } else {
    const int64_t slot = row * a.num_splits + split;
#pragma unroll
    for (int db = 0; db < 16; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = 32 * db + 8 * jg + 4 * hh;
        const f32x4_t v4 = {acc[db][4 * jg] * inv, acc[db][4 * jg + 1] * inv, acc[db][4 * jg + 2] * inv,
                            acc[db][4 * jg + 3] * inv};
        *reinterpret_cast<f32x4_t*>(&a.o_part[slot * kLV + d0]) = v4;
      }
    if (hh == 0) a.lse_part[slot] = any_bad ? NAN : (l_run == 0.f ? -INFINITY : m_run + __log2f(l_run));
  }
}

hipError_t launch_attn_latent_pairs(const LatentArgs& a, hipStream_t stream);  // attn_latent_pairs.hip

hipError_t launch_attn_latent(const LatentArgs& a, bool fp8, bool pairs, hipStream_t stream) {
  const int units = a.batch * a.num_splits;
  const int blocks = ((units + 7) / 8) * 8 * a.n_hg;
  // FP8 at small grids: the wave-pair kernel (two waves per SIMD, 64 heads per block)
  if (fp8 && pairs) {
    hipError_t e0 = launch_attn_latent_pairs(a, stream);
    if (e0 != hipSuccess) return e0;
  } else if (fp8) {
    if (a.page_tags != nullptr)
      hipLaunchKernelGGL((attn_latent_split_kernel<true, true>), dim3(blocks), dim3(kLThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_latent_split_kernel<true, false>), dim3(blocks), dim3(kLThreads), 0, stream, a);
  } else {  // BF16: the check runs in a launch of its own (the host never asks for it here)
    hipLaunchKernelGGL((attn_latent_split_kernel<false, false>), dim3(blocks), dim3(kLThreads), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  MergeArgs m;
  m.o_part = a.o_part;
  m.lse_part = a.lse_part;
  m.out = a.out;
  m.ctx_lens = a.ctx_lens;
  m.flags = a.page_tags != nullptr ? a.flags_out : a.flags;
  m.num_q_heads = a.num_q_heads;
  m.v_dim = kLV;
  // both FP8 kernels store fp16 partials of acc / l; the merge applies the tensor scale
  m.part_f16 = fp8 ? 1 : 0;
  m.out_scale = fp8 ? a.v_scale : 1.f;
  m.num_splits = a.num_splits;
  m.chunk_tokens = a.chunk_tiles * kLT;
  m.max_ctx = a.max_ctx;
  m.pt_stride = a.pt_stride;
  m.page_size = a.page_size;
  return launch_merge(m, a.batch, stream);
}

}  // namespace kvfp8
