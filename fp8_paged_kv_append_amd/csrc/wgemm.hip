// Weight-quantised decode GEMM on gfx950: y[M][N] = x[M][K] W^T with bf16 activations (M <= 64
// requests) and weights stored as INT4 (W4A16) or FP8 e4m3 (W8A16) codes with one bf16 scale per
// group of 128 input channels of an output channel.
//
// What it computes follows the pages' weight compression (Cloudflare post, section "Compressed model
// weights"; agentlenshq summary, section "模型权重压缩以降低延迟"): decode streams every weight once per
// token, so fewer weight bytes mean a faster step, and the 4-bit codes are expanded to a wider type
// before the multiply.  Here the expansion happens in registers, right before bf16 matrix-core
// instructions, and nothing expanded is ever written back.
//
// Storage (tile = 16 output channels x 128 input channels, tiles ordered [N/16][K/128]; inside a
// tile lane l = 16*qq + nn owns channel 16t + nn and inputs 128g + 32j + 8qq + e, j 0..3, e 0..7,
// which is exactly the B operand of v_mfma_f32_16x16x32_bf16 for k-step j):
//  * INT4: 16 bytes per lane; dword j holds nibbles q + 8 with e = 2*(s%4) + s/4 in slot s, so
//    (dword >> 4i) & 0x000F000F | 0x43004300 is the bf16 pair (128 + n_e, 128 + n_e+1) for e = 2i:
//    two ALU operations expand two codes.  The values are q + 136; the bias is removed after the
//    MFMAs of a group as 136 * (sum of the group's activations), computed once per block.
//  * FP8: 32 bytes per lane, bytes 8j + e; expanded exactly to bf16 by the hardware conversion.
// The group's partial sum (fp32, exact products) is scaled by the group's scale and accumulated in
// fp32; the result is rounded to bf16.
//
// Work decomposition.  Block = 4 waves = 64 output channels x one split of the K range; wave w owns
// output tile 4*blockIdx.x + w.  For M <= 16 the split's activation rows stay resident in LDS; above,
// 256-wide K chunks are staged in LDS (double buffered, the next chunk's global loads issued a chunk
// ahead).  Either way the four waves share them; each wave streams its own weight tiles with a register
// ring of 8 groups (8 KB of INT4 / 16 KB of FP8 in flight per wave; 4 INT4 / 8 FP8 groups when the waves
// split one tile's K range; M > 16: 8 groups up to 32 rows, 4 above), whose last pass issues no refills.
// With several splits, fp32 partials go to the workspace and the last block of each column group to
// finish adds them in split order, inside the same launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvfp8.h"
#include "../../include/wgemm.h"
#include "kvfp8_device.h"

namespace kvfp8 {
namespace wq {

constexpr int kGroup = 128;          // input channels per scale group
constexpr int kChunk = 256;          // input channels staged in LDS per step (two groups)
constexpr int kRing = 8;             // weight groups in flight per wave
constexpr int kRowBytes = kChunk * 2 + 16;  // LDS row stride of the staged activations (padded)
constexpr float kW4Bias = 136.0f;    // the expansion yields q + 136
constexpr int kMaxGroupsChunked = 64;  // groups per split of the M > 16 kernel (its scales sit in LDS)
// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima)
constexpr int vm_wait_enc(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct WgemmArgs {
  const uint16_t* x;        // bf16 [M][K]
  const uint8_t* w;         // packed codes
  const uint16_t* s;        // bf16 scales [N/16][K/128][16]
  float* part;              // fp32 [splits][M][N] (splits > 1)
  uint32_t* count;          // finished splits per column group (splits > 1): zero before a launch and after it
  uint16_t* y;              // bf16 [M][N]
  int32_t M, N, K, splits, groups_per_split;
};

constexpr uint32_t kOOB = 0x80000000u;    // a buffer offset past every buffer (all < 2^31 bytes): loads give 0
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)
constexpr int kNT = 2;                    // cache policy of a load: non-temporal (weights are read once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kRsrcWord3);
}

// Sum over the 16 lanes of each DPP row (lanes 16h..16h+15), every lane of the row receiving it: quad
// permutations [1,0,3,2] and [2,3,0,1] give the quad sum, rotations by 4 and 8 inside the row add the
// other quads.  All VALU (a __shfl_xor compiles to an LDS permute: a round trip per step).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x128>(v);   // row_ror:8
  return v;
}

// Sum of the eight bf16 values of a 16-byte load (a bf16 widens to fp32 by a shift or a mask).
__device__ __forceinline__ float sum8_bf16(const u32x4_t& v) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s += __uint_as_float(v[e] << 16) + __uint_as_float(v[e] & 0xFFFF0000u);
  return s;
}

// bf16 pair of two INT4 codes (plus the bias 136) from the nibbles at bits 4i and 16 + 4i: a shift and one
// v_and_or_b32.  The bias passes through an empty asm so that the compiler sees a register, not a
// constant: with two 32-bit constants it splits the AND-OR into two instructions (a three-operand ALU
// instruction of this ISA takes no literal).  The AND-OR itself stays compiler-generated, so the wait
// states the compiler inserts between an ALU write and a matrix-core read of the same register apply to it.
__device__ __forceinline__ uint32_t w4_pair(uint32_t w, int i, uint32_t bias) {
  return ((w >> (4 * i)) & 0x000F000Fu) | bias;
}
__device__ __forceinline__ uint32_t w4_bias() {
  uint32_t b = 0x43004300u;
  asm("" : "+v"(b));
  return b;
}

// One wave's stream of weight groups: the codes of output tile `tile`, groups g0 + g.  Every load is
// issued unconditionally; a group past the split (or a tile past N) reads zeros through an out-of-range
// buffer offset, so the loop is straight-line code.  Only these loads are counted by vmcnt inside the
// loop (scales and activations come from LDS), which keeps the compiler's waits exact: a conditional
// load, or a second load kind issued in another order before the loop, makes it wait for the whole ring.
// POL: the loads' cache policy (non-temporal by default; see the M <= 16 kernel for the exception).
// rot: the stream starts at group rot (mod ng) and wraps around, so that waves whose ranges start a
// multiple of 16 KB apart do not read the same offset of them at the same time.
template <bool W4, int POL = kNT>
struct WStream {
  static constexpr int kB = W4 ? 16 : 32;   // code bytes per lane per group
  __amdgpu_buffer_rsrc_t codes;
  uint32_t cbase;
  int ng, rot;
  bool active;
  __device__ WStream(const WgemmArgs& a, int tile, int g0, int ng_, int lane, int rot_ = 0) {
    const int KG = a.K / kGroup;
    active = tile * 16 < a.N;
    ng = ng_;
    rot = ng_ > 0 ? rot_ % ng_ : 0;
    codes = make_rsrc(a.w, (uint32_t)((int64_t)a.N * a.K / (W4 ? 2 : 1)));
    cbase = (uint32_t)((((int64_t)tile * KG + g0) * 64 + lane) * kB);
  }
  __device__ __forceinline__ int idx(int g) const {   // the group read in place g of the stream
    const int gg = g + rot;
    return gg >= ng ? gg - ng : gg;
  }
  __device__ __forceinline__ void load(u32x4_t (&w)[kB / 16], int g) const {
    const uint32_t co = (active && g < ng) ? cbase + (uint32_t)idx(g) * 64 * kB : kOOB;
#pragma unroll
    for (int d = 0; d < kB / 16; ++d) w[d] = __builtin_amdgcn_raw_buffer_load_b128(codes, co + 16 * d, 0, POL);
  }
};

// The block's group scales -> LDS s_sc[tile of the block][group][16] (bf16), zeros past N or the split.
__device__ __forceinline__ void load_scales(const WgemmArgs& a, int tile0, int ntiles, int g0, int ng, int gcap,
                                            uint16_t* s_sc, int nthreads = 256) {
  const int KG = a.K / kGroup;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, (uint32_t)((int64_t)a.N * KG * 2));
  // ntiles x gcap groups x 32 bytes, 16 bytes per thread and pass
  for (int i = threadIdx.x; i < ntiles * gcap * 2; i += nthreads) {
    const int t = i / (gcap * 2), g = (i / 2) % gcap, h = i & 1;
    const int tile = tile0 + t;
    const bool ok = tile * 16 < a.N && g < ng;
    const uint32_t off = ok ? (uint32_t)(((int64_t)tile * KG + g0 + g) * 32 + 16 * h) : kOOB;
    *reinterpret_cast<u32x4_t*>(s_sc + (t * gcap + g) * 16 + 8 * h) = __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, 0);
  }
}

// The same scales in two steps, so that their load latency overlaps the weight ring's instead of coming
// before it: passes before the last (only when the block's scales exceed one pass of its threads) are
// staged at once; the last pass is loaded into `last` and the LDS element offset it belongs at returned
// (-1: none), for the caller to store after the wait that retires it.
__device__ __forceinline__ int load_scales_split(const WgemmArgs& a, int tile0, int ntiles, int g0, int ng, int gcap,
                                                 uint16_t* s_sc, int nthreads, u32x4_t& last) {
  const int KG = a.K / kGroup;
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.s, (uint32_t)((int64_t)a.N * KG * 2));
  const int total = ntiles * gcap * 2;
  const int last0 = (total - 1) / nthreads * nthreads;
  auto off = [&](int i) {
    const int t = i / (gcap * 2), g = (i / 2) % gcap;
    const bool ok = i < total && (tile0 + t) * 16 < a.N && g < ng;
    return ok ? (uint32_t)(((int64_t)(tile0 + t) * KG + g0 + g) * 32 + 16 * (i & 1)) : kOOB;
  };
  auto slot = [&](int i) { return ((i / (gcap * 2)) * gcap + (i / 2) % gcap) * 16 + 8 * (i & 1); };
  for (int i = threadIdx.x; i < last0; i += nthreads)
    *reinterpret_cast<u32x4_t*>(s_sc + slot(i)) = __builtin_amdgcn_raw_buffer_load_b128(sr, off(i), 0, 0);
  const int i = last0 + threadIdx.x;
  last = __builtin_amdgcn_raw_buffer_load_b128(sr, off(i), 0, 0);
  return i < total ? slot(i) : -1;
}

// The B operand of k-step j (eight bf16 values e = 0..7) from one group's codes.
template <bool W4>
__device__ __forceinline__ u32x4_t expand(const u32x4_t (&w)[W4 ? 1 : 2], int j) {
  u32x4_t b;
  if constexpr (W4) {
    const uint32_t wd = w[0][j], bias = w4_bias();
    b[0] = w4_pair(wd, 0, bias);
    b[1] = w4_pair(wd, 1, bias);
    b[2] = w4_pair(wd, 2, bias);
    b[3] = w4_pair(wd, 3, bias);
  } else {
    const u32x2_t lo = e4m3x4_to_bf16x4(w[j >> 1][2 * (j & 1)]);
    const u32x2_t hi = e4m3x4_to_bf16x4(w[j >> 1][2 * (j & 1) + 1]);
    b[0] = lo[0];
    b[1] = lo[1];
    b[2] = hi[0];
    b[3] = hi[1];
  }
  return b;
}

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// acc += s * group sum.  For INT4 the group's MFMAs start from -136 * (sum of the group's activations)
// instead of zero, which removes the expansion's bias from the sum they accumulate.
__device__ __forceinline__ void add_group(f32x4_t& acc, const f32x4_t& accg, float sc) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = fmaf(sc, accg[r], acc[r]);
}

template <int MT>
__device__ __forceinline__ void store_y(const WgemmArgs& a, const f32x4_t (&acc)[MT], int tile, int nn, int qq) {
  if (tile * 16 >= a.N) return;
  const int n = tile * 16 + nn;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * qq + r;
      if (m < a.M) a.y[(int64_t)m * a.N + n] = (uint16_t)(pack_bf16x2(acc[mt][r], 0.f) & 0xFFFFu);
    }
  }
}

// The block's results, called by every thread of the block.  One split: y directly.  Several: each block
// stores its fp32 partials, 16 bytes per lane and row tile, with device-coherent stores (sc1: they reach
// the point every XCD reads from, and no L2 writeback is needed), waits for them, and counts itself
// finished for its column group; the block that finishes last reads the other splits' partials with
// device-coherent loads, all issued before any is used, adds them in split order (the order a separate
// reduction would take), writes y and sets the count back to zero.  Partials sit at
// [split][column group][wave][row tile][lane] in 16-byte units.
constexpr int kCohAux = 16;   // cache-policy operand of a buffer access: sc1
constexpr int kCountStride = 32;  // words between two split counts
constexpr int kFinishBatch = 4;

template <int MT>
__device__ __forceinline__ void store_out(const WgemmArgs& a, const f32x4_t (&acc)[MT], int tile, int nn, int qq) {
  if (a.splits == 1) {
    store_y<MT>(a, acc, tile, nn, qq);
    return;
  }
  __shared__ uint32_t s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const __amdgpu_buffer_rsrc_t pr =
      make_rsrc(a.part, (uint32_t)((int64_t)a.splits * gridDim.x * nw * MT * 64 * 16));
  auto off = [&](int sp, int mt) {
    return (uint32_t)(((((int64_t)sp * gridDim.x + blockIdx.x) * nw + wave) * MT + mt) * 64 + lane) * 16;
  };
  const bool live = tile * 16 < a.N;
  if (live) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[mt]), pr, off(blockIdx.y, mt), 0, kCohAux);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partials are stored before the block counts itself done
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t done = __hip_atomic_fetch_add(a.count + blockIdx.x * kCountStride, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    const bool last = done == (uint32_t)(a.splits - 1);
    if (last) __hip_atomic_store(a.count + blockIdx.x * kCountStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  if (s_last == 0u || !live) return;
  f32x4_t sum[MT];
  for (int sp0 = 0; sp0 < a.splits; sp0 += kFinishBatch) {
    u32x4_t v[kFinishBatch][MT];
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int sp = sp0 + b;
        v[b][mt] = (sp < a.splits && sp != (int)blockIdx.y)
                       ? __builtin_amdgcn_raw_buffer_load_b128(pr, off(sp, mt), 0, kCohAux)
                       : __builtin_bit_cast(u32x4_t, acc[mt]);
      }
#pragma unroll
    for (int b = 0; b < kFinishBatch; ++b)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4_t x = __builtin_bit_cast(f32x4_t, v[b][mt]);
        if (sp0 + b == 0) sum[mt] = x;
        else if (sp0 + b < a.splits) sum[mt] += x;
      }
  }
  store_y<MT>(a, sum, tile, nn, qq);
}

// ---- M <= 16: the block's whole K range of the activations stays in LDS (rows 0..M-1, then the
// group sums [group][16]); after one load the waves only stream weights, with no barrier.
// WK = false: the block covers WB output tiles, one per wave, each over the whole split (the staging is
// shared by WB tiles).
// WK = true: the block is one output tile and its WB (kWkWaves = 4) waves split its K range (wave w takes
// the w-th part of the groups); they add their results through LDS in wave order -- a K split with
// neither a workspace nor a second launch.  Eight or sixteen waves per tile measured slower at M=1
// (INT4 11.0 / 11.8 against 9.1 us on 8192 x 8192).
// XB: activation loads per thread and batch (0: 4096 / threads); the launch sizes it to the split's rows so
// that no pass of the last batch lies wholly past them in the split form.
template <bool W4, bool WK, int WB, int XB = 0>
__global__ __launch_bounds__(64 * WB) void wgemm_small_kernel(WgemmArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int kTiles = WK ? 1 : WB;
  constexpr int kThr = 64 * WB;
  // groups in flight per wave, measured on 8192 x 8192: with the K range cut among the waves (M <= 4),
  // INT4 4 (M=1 9.1 us; 6 / 8 / 16: 9.5 / 9.8 / 11.9), FP8 8 (M=1 14.5 against 14.9 with 4); split over
  // blocks, 4 and 8 are alike and 12 and 16 slower
  constexpr int kRingS = WK ? (W4 ? 4 : 8) : kRing;
  // Activation passes wholly past the data are skipped (a load past the buffer still costs an issue slot and a
  // return: at M=1 the 12 of 16 that are empty cost ~2 us per launch) -- in the K-split form only: the branches
  // raise the eight-wave kernel from 87 to 239 VGPRs (one block per CU instead of two, INT4 M=16 13.7 -> 16.1 us)
  constexpr bool kXLim = WK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 15, qq = lane >> 4;
  const int KG = a.K / kGroup;
  const int g0 = blockIdx.y * a.groups_per_split;
  const int ng = min(a.groups_per_split, KG - g0);
  const int gcap = a.groups_per_split;
  const int row_bytes = ng * kGroup * 2 + 16;
  float* xs = reinterpret_cast<float*>(smem + a.M * row_bytes);                        // [gcap][16]
  uint16_t* s_sc = reinterpret_cast<uint16_t*>(smem + a.M * row_bytes + gcap * 64);      // [kTiles][gcap][16]
  f32x4_t* s_red = reinterpret_cast<f32x4_t*>(smem + a.M * row_bytes + gcap * 64 + kTiles * gcap * 32);

  // the wave's tile and groups
  const int tile = WK ? blockIdx.x : blockIdx.x * WB + wave;
  const int gq = WK ? (ng + WB - 1) / WB : ng;
  const int gw0 = WK ? wave * gq : 0;                    // first group of the wave inside the split
  const int ngw = WK ? max(0, min(gq, ng - gw0)) : ng;
  const int st = WK ? 0 : wave;                          // the wave's tile inside s_sc

  // FP8 codes over split blocks stream faster with the default cache policy than non-temporal (M = 8 / 16:
  // 18.35 -> 17.6 / 19.4 -> 18.3 us on 8192 x 8192); every other form measured level or slower with it.
  // Over split blocks each wave also starts its groups at a rotation of its own (tiles are 64 KB apart in
  // memory): M = 8 INT4 12.5 -> 12.0, FP8 17.6 -> 16.8 us; the K-split form measured slower with it.
  const WStream<W4, (!W4 && !WK) ? 0 : kNT> ws(a, tile, g0 + gw0, ngw, lane, WK ? 0 : tile * 7 + wave * 5);
  constexpr int kB = WStream<W4>::kB;
  u32x4_t sc_last;
  const int sc_slot = load_scales_split(a, WK ? blockIdx.x : blockIdx.x * WB, kTiles, g0, ng, gcap, s_sc, kThr, sc_last);

  // Activations, then the weight ring, then one wait that leaves exactly the ring outstanding: the
  // loads retire in issue order, so the activations go first (their latency overlaps the ring's), and
  // the wait -- the builtin, which the compiler's load counting sees -- also retires the out-of-range
  // activation loads whose data is never read (left outstanding, they would make the compiler wait for
  // the whole ring inside the loop).  Batches before the last (only when M * groups > 256) are plain.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.K * 2));
  const int per_row = ng * (kGroup / 8), total = a.M * per_row;
  auto x_off = [&](int i) {
    const int r = i / per_row, c = i % per_row;
    return i < total ? (uint32_t)(((int64_t)r * a.K + g0 * kGroup + 8 * c) * 2) : kOOB;
  };
  auto x_put = [&](int i, const u32x4_t& v) {
    if (i < total) *reinterpret_cast<u32x4_t*>(smem + (i / per_row) * row_bytes + 16 * (i % per_row)) = v;
    // INT4: -136 * group sum on the way, the starting value of the group's MFMAs (it removes the code
    // bias; FP8 codes carry none): a group of a row is 16 consecutive columns, i.e. 16 aligned lanes
    // (per_row and the thread count are multiples of 16); out-of-range lanes loaded zeros
    if constexpr (W4) {
      const float sum = row_sum16(sum8_bf16(v));
      if (i < total && (threadIdx.x & 15) == 0) xs[((i % per_row) >> 4) * 16 + i / per_row] = -kW4Bias * sum;
    }
  };
  constexpr int kXB = XB ? XB : 4096 / kThr;             // activation loads per thread and batch
  int xbase = 0;
  for (; xbase + kThr * kXB < total; xbase += kThr * kXB) {
    u32x4_t v[kXB];
#pragma unroll
    for (int t = 0; t < kXB; ++t) v[t] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off(xbase + kThr * t + tid), 0, 0);
#pragma unroll
    for (int t = 0; t < kXB; ++t) x_put(xbase + kThr * t + tid, v[t]);
  }
  u32x4_t v[kXB];
#pragma unroll
  for (int t = 0; t < kXB; ++t) {
    if (!kXLim || xbase + kThr * t < total) v[t] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off(xbase + kThr * t + tid), 0, 0);
    else v[t] = u32x4_t{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_sched_barrier(0);
  u32x4_t wr[kRingS][kB / 16];
#pragma unroll
  for (int u = 0; u < kRingS; ++u) {
    ws.load(wr[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(vm_wait_enc(kRingS * (kB / 16)));
#pragma unroll
  for (int t = 0; t < kXB; ++t)
    if (!kXLim || xbase + kThr * t < total) x_put(xbase + kThr * t + tid, v[t]);
  if (sc_slot >= 0) *reinterpret_cast<u32x4_t*>(s_sc + sc_slot) = sc_last;
  __syncthreads();

  // rows >= M read row M-1: their results are never stored
  const uint8_t* xa = smem + min(nn, a.M - 1) * row_bytes + 16 * qq;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto group = [&](int base, int u, bool refill) {
    const int gc = gw0 + ws.idx(min(base + u, ngw - 1));   // past the wave's range: zero codes and scale
    u32x4_t av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const u32x4_t*>(xa + (gc * kGroup + 32 * j) * 2);
    const float sc = bf16_bits_to_f32(s_sc[(st * gcap + gc) * 16 + nn]);
    // rows >= M start from whatever their unused entries hold: their results are never stored
    f32x4_t accg = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (W4) accg = *reinterpret_cast<const f32x4_t*>(&xs[gc * 16 + 4 * qq]);
#pragma unroll
    for (int j = 0; j < 4; ++j) accg = mfma_bf16(av[j], expand<W4>(wr[u], j), accg);
    add_group(acc, accg, base + u < ngw ? sc : 0.f);
    // refill this slot now: without the fence the scheduler sinks all refills of the unrolled loop
    // to its end, and every pass then waits a full memory latency for loads it has just issued
    if (refill) ws.load(wr[u], base + u + kRingS);
    __builtin_amdgcn_sched_barrier(0);
  };
  // the last pass refills nothing (refills past the wave's groups would be out-of-range loads)
  int base = 0;
  for (; base + kRingS < ngw; base += kRingS) {
#pragma unroll
    for (int u = 0; u < kRingS; ++u) group(base, u, true);
  }
  if (base < ngw) {
#pragma unroll
    for (int u = 0; u < kRingS; ++u) group(base, u, false);
  }
  if constexpr (WK) {
    s_red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = s_red[lane];
#pragma unroll
    for (int w = 1; w < WB; ++w) acc += s_red[w * 64 + lane];
  }
  f32x4_t out[1] = {acc};
  store_out<1>(a, out, tile, nn, qq);
}

// ---- M > 16: activations staged per 256-wide chunk (two groups) through double-buffered LDS, the next
// chunk's loads issued at the start of the current one; rows >= M and chunks past the split load zeros.
// WB waves per block, one 16-channel tile each; the block stages each activation chunk (and, for
// INT4, its group sums) once for all of them, so more waves per block stage less per output channel.
template <int MT, bool W4, int WB>
__global__ __launch_bounds__(64 * WB, 8 / WB) void wgemm_kernel(WgemmArgs a) {
  constexpr int kRows = 16 * MT;
  constexpr int kR = MT <= 2 ? kRing : kRing / 2;   // groups in flight (more rows: more work per byte)
  constexpr int kThr = 64 * WB;
  constexpr int kXP = kRows / (kThr / 32);          // staging passes: kThr / 32 rows of 32 x 16 bytes each
  __shared__ __align__(16) uint8_t s_x[2][kRows * kRowBytes];
  __shared__ __align__(16) float s_xs[2][2][kRows];   // [buffer][group of the chunk][row]
  __shared__ __align__(16) uint16_t s_sc[WB * kMaxGroupsChunked * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nn = lane & 15, qq = lane >> 4;
  const int KG = a.K / kGroup;
  const int g0 = blockIdx.y * a.groups_per_split;
  const int ng = min(a.groups_per_split, KG - g0);    // even
  const int nch = ng / 2;

  // ---- activation staging: thread -> (row (kThr/32) p + tid/32, 16-byte column tid%32) of a chunk
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, (uint32_t)((int64_t)a.M * a.K * 2));
  // Two register sets: chunk c's rows are loaded at the start of chunk c - 2 and stored to LDS at the
  // end of chunk c - 1.  Loads retire in issue order, so the store's wait also retires every weight
  // load issued before them; loading two chunks ahead keeps the weight loads of the last two chunks in
  // flight through that wait (one chunk ahead left only the newest two groups in flight).
  const int xr_row = tid >> 5, xr_col = tid & 31;
  u32x4_t xr[2][kXP];
  auto x_load = [&](int set, int ch) {   // chunk ch of the split into register set `set`
#pragma unroll
    for (int p = 0; p < kXP; ++p) {
      const int row = (kThr / 32) * p + xr_row;
      const uint32_t off = (row < a.M && ch < nch)
                               ? (uint32_t)(((int64_t)row * a.K + (int64_t)(g0 / 2 + ch) * kChunk + 8 * xr_col) * 2)
                               : kOOB;
      xr[set][p] = __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0);
    }
  };
  auto x_store = [&](int set, int buf) {
#pragma unroll
    for (int p = 0; p < kXP; ++p) {
      const int row = (kThr / 32) * p + xr_row;
      *reinterpret_cast<u32x4_t*>(s_x[buf] + row * kRowBytes + 16 * xr_col) = xr[set][p];
      // INT4 only: the 16 lanes of one (row, group) are lanes 16h..16h+15 of this wave
      if constexpr (W4) {
        const float sum = row_sum16(sum8_bf16(xr[set][p]));
        if ((xr_col & 15) == 0) s_xs[buf][xr_col >> 4][row] = -kW4Bias * sum;
      }
    }
  };

  const int tile = blockIdx.x * WB + wave;
  const WStream<W4> ws(a, tile, g0, ng, lane);
  constexpr int kB = WStream<W4>::kB;
  u32x4_t wr[kR][kB / 16];
#pragma unroll
  for (int u = 0; u < kR; ++u) {
    ws.load(wr[u], u);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_scales(a, blockIdx.x * WB, WB, g0, ng, kMaxGroupsChunked, s_sc, kThr);
  x_load(0, 0);
  x_load(1, 1);
  x_store(0, 0);
  __syncthreads();

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the last pass refills nothing (refills past the split would be out-of-range loads)
  auto pass = [&](int base, bool refill) {
#pragma unroll
    for (int u = 0; u < kR; ++u) {
      const int buf = (u >> 1) & 1;           // chunk parity (base is a multiple of 4 groups)
      const int gl = u & 1;                   // group inside the chunk
      if (gl == 0) x_load(buf, (base + u) / 2 + 2);
      f32x4_t accg[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        accg[mt] = W4 ? *reinterpret_cast<const f32x4_t*>(&s_xs[buf][gl][16 * mt + 4 * qq]) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t b = expand<W4>(wr[u], j);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          accg[mt] = mfma_bf16(*reinterpret_cast<const u32x4_t*>(s_x[buf] + (16 * mt + nn) * kRowBytes +
                                                                 (gl * kGroup + 32 * j + 8 * qq) * 2),
                               b, accg[mt]);
      }
      const float sc = bf16_bits_to_f32(s_sc[(wave * kMaxGroupsChunked + min(base + u, kMaxGroupsChunked - 1)) * 16 + nn]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) add_group(acc[mt], accg[mt], base + u < ng ? sc : 0.f);
      if (refill) ws.load(wr[u], base + u + kR);
      __builtin_amdgcn_sched_barrier(0);
      if (gl == 1) {
        x_store(buf ^ 1, buf ^ 1);
        __syncthreads();
      }
    }
  };
  int base = 0;
  for (; base + kR < ng; base += kR) pass(base, true);
  pass(base, false);
  store_out<MT>(a, acc, tile, nn, qq);
}

// ---- quantise + pack: block = one 16 x 128 tile; thread (row nn = tid/16, 8-channel column c = tid%16)
template <bool W4>
__global__ __launch_bounds__(256) void wquant_kernel(const uint16_t* w, int32_t K, uint8_t* packed,
                                                     uint16_t* scales) {
  const int t = blockIdx.x, g = blockIdx.y, KG = K / kGroup;
  const int tid = threadIdx.x, nn = tid >> 4, c = tid & 15;
  const u32x4_t v = *reinterpret_cast<const u32x4_t*>(w + (int64_t)(16 * t + nn) * K + g * kGroup + 8 * c);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(v[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(v[i] >> 16);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, dpp<0xB1>(amax));    // max over the 16 lanes of the DPP row (one output channel)
  amax = fmaxf(amax, dpp<0x4E>(amax));
  amax = fmaxf(amax, dpp<0x124>(amax));
  amax = fmaxf(amax, dpp<0x128>(amax));
  const uint32_t sb = pack_bf16x2(__fdiv_rn(amax, W4 ? 7.0f : kE4M3Max), 0.f) & 0xFFFFu;
  const float s = bf16_bits_to_f32(sb);
  const float inv = s > 0.f ? __fdiv_rn(1.0f, s) : 0.f;
  // this thread holds inputs 8c..8c+7 of the group: k-step j = c/4, lane group qq = c%4
  const int j = c >> 2, lane = 16 * (c & 3) + nn;
  const int64_t tile = (int64_t)t * KG + g;
  if (W4) {
    uint32_t d = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = fminf(fmaxf(rintf(x[e] * inv), -8.f), 7.f);
      const uint32_t nib = (uint32_t)((int)q + 8) & 0xFu;
      const int slot = (e & 1) * 4 + (e >> 1);
      d |= nib << (4 * slot);
    }
    reinterpret_cast<uint32_t*>(packed)[(tile * 64 + lane) * 4 + j] = d;
  } else {
    u32x2_t d;
    d[0] = encode_e4m3x2(x[0] * inv, x[1] * inv) | (encode_e4m3x2(x[2] * inv, x[3] * inv) << 16);
    d[1] = encode_e4m3x2(x[4] * inv, x[5] * inv) | (encode_e4m3x2(x[6] * inv, x[7] * inv) << 16);
    reinterpret_cast<u32x2_t*>(packed)[(tile * 64 + lane) * 4 + j] = d;
  }
  if (c == 0) scales[tile * 16 + nn] = (uint16_t)sb;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The split-K workspace opens with one uint32 count per possible column group (one per 16 output
// channels, whatever the launch's group width), each in a 128-byte line of its own (kCountStride words),
// padded to 256 bytes; the fp32 partials follow.  Counts that shared a line made the split blocks of
// neighbouring column groups queue on it: 8192 x 8192, INT4 M = 8..64 0.3-0.5 us slower per GEMM, FP8
// 0.1-0.2.
inline size_t count_bytes(int32_t n) { return (((size_t)(n + 15) / 16) * kCountStride * 4 + 255) / 256 * 256; }

int check_shape(int32_t n, int32_t k) {
  if (n < 16 || k < kChunk || n % 16 != 0 || k % kChunk != 0) return KVFP8_ERR_SHAPE;
  return KVFP8_OK;
}

int quantize_common(const uint16_t* w, int32_t n, int32_t k, uint8_t* packed, uint16_t* scales, bool w4,
                    hipStream_t stream) {
  if (!w || !packed || !scales) return KVFP8_ERR_NULL;
  int st = check_shape(n, k);
  if (st) return st;
  if (!aligned16(w) || !aligned16(packed) || (reinterpret_cast<uintptr_t>(scales) & 1u)) return KVFP8_ERR_ALIGN;
  const dim3 grid(n / 16, k / kGroup);
  if (w4)
    hipLaunchKernelGGL(wquant_kernel<true>, grid, dim3(256), 0, stream, w, k, packed, scales);
  else
    hipLaunchKernelGGL(wquant_kernel<false>, grid, dim3(256), 0, stream, w, k, packed, scales);
  return hipGetLastError() == hipSuccess ? KVFP8_OK : KVFP8_ERR_HIP;
}

constexpr int64_t kTargetBlocks = 512;      // two blocks of four waves per CU

constexpr size_t kSmallLdsMax = 80 * 1024;  // dynamic LDS of the M <= 16 kernel (two 4-wave blocks fit a CU)

// activations [M][gps*128 + 8] bf16, group sums [gps][16] fp32, scales [tiles][gps][16] bf16, and for
// the in-block K split the waves' results [kWkWaves][64] f32x4
// Tiles (waves) per block of the split M <= 16 kernel: INT4 gains from sharing the staging and group
// sums among eight (M=16 17.7 -> 15.2 us on 8192 x 8192), FP8, streaming twice the bytes, keeps two
// blocks of four per CU (19.7 us against 22.6 with eight).  The LDS size allows for eight either way.
constexpr int kSmallWaves = 8;
constexpr int kWkWaves = 4;
constexpr int small_waves(bool w4) { return w4 ? 8 : 4; }

size_t small_lds_bytes(int32_t m, int32_t gps, bool wk = false) {
  return (size_t)m * (gps * kGroup * 2 + 16) + (size_t)gps * 16 * 4 + (size_t)(wk ? 1 : kSmallWaves) * gps * 16 * 2 +
         (wk ? kWkWaves * 64 * 16 : 0);
}

// M <= 16 with enough output tiles to fill the chip: one split, K cut among a block's waves
bool use_wk(int32_t m, int32_t n, int32_t k) {
  return m <= 16 && n / 16 >= 256 && small_lds_bytes(m, k / kGroup, true) <= kSmallLdsMax;
}

int32_t auto_splits(int32_t m, int32_t n, int32_t k) {
  if (m < 1 || n < 16 || k < kChunk) return 1;
  if (use_wk(m, n, k)) return 1;
  const int64_t cols = (n / 16 + 3) / 4;
  const int64_t chunks = k / kChunk;
  int64_t s = (kTargetBlocks + cols - 1) / cols;
  // at least four chunks (eight groups, one ring) per split
  int64_t cap = chunks / 4;
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  if (s < 1) s = 1;
  // M <= 16: the split's activations must fit the resident kernel's LDS; M > 16: at most
  // kMaxGroupsChunked groups per split (the chunked kernel keeps its split's scales in LDS)
  while (s < chunks && (m <= 16 ? small_lds_bytes(m, 2 * (int32_t)((chunks + s - 1) / s)) > kSmallLdsMax
                                : 2 * ((chunks + s - 1) / s) > kMaxGroupsChunked))
    ++s;
  return (int32_t)s;
}

// Waves (16-channel tiles) per block of the M > 16 kernel: eight halve the activation staging per
// channel, which INT4 (group sums included) always gains from; FP8 from three row tiles up (measured
// on 8192 x 8192: INT4 M=64 28.9 -> 26.2 us, FP8 M=64 27.9 -> 25.4 us, FP8 M=32 24.2 -> 25.5 us).
template <int MT, bool W4>
void launch_mt(const WgemmArgs& a, int32_t n, int32_t splits, hipStream_t stream) {
  constexpr int WB = (W4 || MT >= 3) ? 8 : 4;
  const dim3 grid((n / 16 + WB - 1) / WB, splits);
  hipLaunchKernelGGL((wgemm_kernel<MT, W4, WB>), grid, dim3(64 * WB), 0, stream, a);
}

int gemm_common(const uint16_t* x, int32_t m, const uint8_t* w, const uint16_t* scales, int32_t n, int32_t k,
                int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* y, bool w4,
                hipStream_t stream) {
  if (!x || !w || !scales || !y) return KVFP8_ERR_NULL;
  if (m < 1 || m > 64 || num_splits < 0) return KVFP8_ERR_SHAPE;
  int st = check_shape(n, k);
  if (st) return st;
  // buffer offsets are 32-bit with the top bit reserved for out-of-range loads
  if ((int64_t)n * k >= (int64_t)1 << 31 || (int64_t)m * k * 2 >= (int64_t)1 << 31) return KVFP8_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (reinterpret_cast<uintptr_t>(scales) & 1u))
    return KVFP8_ERR_ALIGN;
  const int32_t chunks = k / kChunk;
  int32_t splits = num_splits == 0 ? auto_splits(m, n, k) : num_splits;
  if (splits > chunks) return KVFP8_ERR_SHAPE;
  const int32_t cps = (chunks + splits - 1) / splits;   // chunks per split
  splits = (chunks + cps - 1) / cps;                    // drop empty splits
  WgemmArgs a;
  a.x = x;
  a.w = w;
  a.s = scales;
  a.y = y;
  a.part = nullptr;
  a.count = nullptr;
  a.M = m;
  a.N = n;
  a.K = k;
  a.splits = splits;
  a.groups_per_split = 2 * cps;
  if (splits > 1) {
    const size_t need = wgemm_workspace_bytes(m, n, k, splits);
    if (!workspace) return KVFP8_ERR_NULL;
    if (workspace_bytes < need) return KVFP8_ERR_WORKSPACE;
    if (!aligned16(workspace)) return KVFP8_ERR_ALIGN;
    a.count = reinterpret_cast<uint32_t*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + count_bytes(n));
  }
  const size_t lds = small_lds_bytes(m, a.groups_per_split);
  const bool wk = splits == 1 && m <= 16 && small_lds_bytes(m, a.groups_per_split, true) <= kSmallLdsMax;
  const bool small = m <= 16 && lds <= kSmallLdsMax;
  if (!wk && !small && a.groups_per_split > kMaxGroupsChunked) return KVFP8_ERR_UNSUPPORTED;
  if (wk) {
    const size_t lw = small_lds_bytes(m, a.groups_per_split, true);
    if (w4)
      hipLaunchKernelGGL((wgemm_small_kernel<true, true, kWkWaves>), dim3(n / 16, 1), dim3(64 * kWkWaves), lw, stream, a);
    else
      hipLaunchKernelGGL((wgemm_small_kernel<false, true, kWkWaves>), dim3(n / 16, 1), dim3(64 * kWkWaves), lw, stream, a);
  } else if (small) {
    constexpr int W8 = small_waves(true), W4 = small_waves(false);
    // loads per thread that cover a full split's rows: half the default where that suffices
    const int64_t rows16 = (int64_t)m * a.groups_per_split * (kGroup / 8);   // 16-byte activation loads
    const dim3 g8((n / 16 + W8 - 1) / W8, splits), g4((n / 16 + W4 - 1) / W4, splits);
    if (w4) {
      if (rows16 <= 64 * W8 * (2048 / (64 * W8)))
        hipLaunchKernelGGL((wgemm_small_kernel<true, false, W8, 2048 / (64 * W8)>), g8, dim3(64 * W8), lds, stream, a);
      else
        hipLaunchKernelGGL((wgemm_small_kernel<true, false, W8>), g8, dim3(64 * W8), lds, stream, a);
    } else {
      if (rows16 <= 64 * W4 * (2048 / (64 * W4)))
        hipLaunchKernelGGL((wgemm_small_kernel<false, false, W4, 2048 / (64 * W4)>), g4, dim3(64 * W4), lds, stream, a);
      else
        hipLaunchKernelGGL((wgemm_small_kernel<false, false, W4>), g4, dim3(64 * W4), lds, stream, a);
    }
  } else {
    const int mt = (m + 15) / 16;
    if (w4) {
      if (mt == 1) launch_mt<1, true>(a, n, splits, stream);
      else if (mt == 2) launch_mt<2, true>(a, n, splits, stream);
      else if (mt == 3) launch_mt<3, true>(a, n, splits, stream);
      else launch_mt<4, true>(a, n, splits, stream);
    } else {
      if (mt == 1) launch_mt<1, false>(a, n, splits, stream);
      else if (mt == 2) launch_mt<2, false>(a, n, splits, stream);
      else if (mt == 3) launch_mt<3, false>(a, n, splits, stream);
      else launch_mt<4, false>(a, n, splits, stream);
    }
  }
  if (hipGetLastError() != hipSuccess) return KVFP8_ERR_HIP;
  return KVFP8_OK;
}

}  // namespace wq
}  // namespace kvfp8

using namespace kvfp8::wq;

extern "C" {

size_t w4_packed_bytes(int32_t n, int32_t k) {
  return check_shape(n, k) ? 0 : (size_t)n * k / 2;
}

size_t w8_packed_bytes(int32_t n, int32_t k) {
  return check_shape(n, k) ? 0 : (size_t)n * k;
}

size_t wq_scales_count(int32_t n, int32_t k) {
  return check_shape(n, k) ? 0 : (size_t)n * (k / kGroup);
}

int w4_quantize_bf16(const uint16_t* w, int32_t n, int32_t k, uint8_t* packed, uint16_t* scales,
                     hipStream_t stream) {
  return quantize_common(w, n, k, packed, scales, true, stream);
}

int w8_quantize_bf16(const uint16_t* w, int32_t n, int32_t k, uint8_t* packed, uint16_t* scales,
                     hipStream_t stream) {
  return quantize_common(w, n, k, packed, scales, false, stream);
}

int32_t wgemm_auto_splits(int32_t m, int32_t n, int32_t k) { return auto_splits(m, n, k); }

size_t wgemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t num_splits) {
  if (m < 1 || n < 1 || k < 1 || num_splits <= 1) return 0;
  // partials: 16 bytes per lane, row tile and 16-channel wave tile, over the column groups' whole tiles
  // (the widest group, eight tiles, rounds N up the most)
  const size_t tiles = ((size_t)(n + 127) / 128) * 8, row_tiles = ((size_t)m + 15) / 16;
  return count_bytes(n) + (size_t)num_splits * tiles * row_tiles * 64 * 16;
}

int w4a16_gemm(const uint16_t* x, int32_t m, const uint8_t* w_packed, const uint16_t* scales, int32_t n, int32_t k,
               int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* y, hipStream_t stream) {
  return gemm_common(x, m, w_packed, scales, n, k, num_splits, workspace, workspace_bytes, y, true, stream);
}

int w8a16_gemm(const uint16_t* x, int32_t m, const uint8_t* w_packed, const uint16_t* scales, int32_t n, int32_t k,
               int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* y, hipStream_t stream) {
  return gemm_common(x, m, w_packed, scales, n, k, num_splits, workspace, workspace_bytes, y, false, stream);
}

}  // extern "C"
