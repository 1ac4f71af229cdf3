// Read-only streaming kernels that measure the HBM read rate a kernel can attain on this GPU, next to
// which the attention kernels' rates are reported: a plain sequential stream, and a gather of
// fixed-size blocks named by an id list (the attention's pattern: one 2 KiB (page, head) block of K
// or V per id, the ids in random order), with no arithmetic on the bytes beyond folding them into a
// checksum so the loads cannot be dropped.
//
// Each thread XORs every 32-bit word it reads into one accumulator; a block folds its threads'
// accumulators with wave shuffles and LDS and stores one word, sink[blockIdx.x].  Every word of the
// input is read by exactly one thread, so the XOR of all sink words equals the XOR of all words read.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per thread

__device__ __forceinline__ u32x4_t ld_nt(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ void block_fold_store(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t s_w[kStreamThreads / kWave];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= shfl_xor(acc, m);
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) x ^= s_w[w];
    sink[blockIdx.x] = x;
  }
}

// n16 16-byte vectors, then tail_words trailing 32-bit words (bytes a multiple of 4).
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const u32x4_t* src, int64_t n16,
                                                                     const uint32_t* tail, int tail_words,
                                                                     uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4_t v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = ld_nt(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = ld_nt(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < tail_words) acc ^= tail[threadIdx.x];
  block_fold_store(acc, sink);
}

// Block ids[k] of block_bytes bytes at base + ids[k] * block_bytes, for k < n_ids; an id outside
// [0, num_blocks) is skipped (never dereferenced).  A wave reads one block at a time, 16 bytes per
// lane and load; each thread keeps kStreamUnroll loads (of up to kStreamUnroll blocks) in flight.
__global__ __launch_bounds__(kStreamThreads) void read_blocks_kernel(const uint8_t* base, int64_t num_blocks,
                                                                     const int32_t* ids, int64_t n_ids,
                                                                     int64_t block_bytes, uint32_t* sink) {
  uint32_t acc = 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kStreamThreads + threadIdx.x) / kWave;
  const int64_t waves = (int64_t)gridDim.x * (kStreamThreads / kWave);
  const int64_t per_block = block_bytes / 16;  // 16-byte vectors per block
  // work item j = (id index k, vector v of that block, in steps of 64 lanes)
  const int64_t steps = (per_block + kWave - 1) / kWave;
  const int64_t items = n_ids * steps;
  int64_t j = wave;
  for (; j + (kStreamUnroll - 1) * waves < items; j += kStreamUnroll * waves) {
    u32x4_t v[kStreamUnroll];
    bool ok[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t jj = j + u * waves;
      const int64_t k = jj / steps, vec = (jj - k * steps) * kWave + lane;
      const int32_t id = ids[k];
      const bool in = id >= 0 && id < num_blocks;
      ok[u] = in && vec < per_block;
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + (int64_t)(in ? id : 0) * block_bytes) +
                         (ok[u] ? vec : 0);
      v[u] = ld_nt(p);
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u)
      if (ok[u]) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; j < items; j += waves) {
    const int64_t k = j / steps, vec = (j - k * steps) * kWave + lane;
    const int32_t id = ids[k];
    if (id >= 0 && id < num_blocks && vec < per_block) {
      const u32x4_t v = ld_nt(reinterpret_cast<const u32x4_t*>(base + (int64_t)id * block_bytes) + vec);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  block_fold_store(acc, sink);
}

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int tail_words = (int)((bytes % 16) / 4);
  const uint32_t* tail = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(src) + n16 * 16);
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), n16, tail, tail_words, sink);
  return hipGetLastError();
}

hipError_t launch_read_blocks(const void* base, int64_t num_blocks, const int32_t* ids, int64_t n_ids,
                              int64_t block_bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(read_blocks_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint8_t*>(base), num_blocks, ids, n_ids, block_bytes, sink);
  return hipGetLastError();
}

}  // namespace kvfp8
