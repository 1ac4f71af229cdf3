// Read-only streaming kernels that measure the HBM read rate a kernel can attain on this GPU, next to
// which the attention kernels' rates are reported: a plain sequential stream, and a gather of
// fixed-size blocks named by an id list (the attention's pattern: one 2 KiB (page, head) block of K
// or V per id, the ids in random order), with no arithmetic on the bytes beyond folding them into a
// checksum so the loads cannot be dropped.
//
// Both are one pass with no loop: every thread issues a fixed number of 16-byte non-temporal loads
// (all in flight together) and the grid covers the input, so the hardware's dispatcher keeps every CU
// full.  Measured on MI355X over the 1.06 GB of a 64 x 8192 decode step, eight loads per thread stream at
// 6.9 TB/s and read the step's 2 KiB page blocks at 6.35 TB/s (four loads: 6.7 and 6.0; sixteen: 6.8 and
// 5.9), where a grid-stride loop over a fixed 2048 blocks reached ~5.5 TB/s.  Each thread XORs the
// 32-bit words it reads into one accumulator; a block folds its threads' accumulators with wave
// shuffles and LDS and XORs the result into sink[blockIdx.x % kSinkWords] (one atomic per block).  Every word of the input is read by
// exactly one thread, so the XOR of all sink words equals the XOR of all words read.
#include "kvfp8_device.h"
#include "kvfp8_internal.h"

namespace kvfp8 {

constexpr int kStreamThreads = 256;
constexpr int kStreamVecs = 8;  // 16-byte loads per thread

__device__ __forceinline__ u32x4_t ld_nt(const u32x4_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ void block_fold_xor(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t s_w[kStreamThreads / kWave];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= shfl_xor(acc, m);
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / kWave; ++w) x ^= s_w[w];
    atomicXor(sink + blockIdx.x % kReadSinkWords, x);
  }
}

// Vectors [b * 2048, (b + 1) * 2048) of the n16 16-byte vectors for block b, thread t reading
// b * 2048 + u * 256 + t; block 0 also reads the tail_words trailing 32-bit words.
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const u32x4_t* src, int64_t n16,
                                                                     const uint32_t* tail, int tail_words,
                                                                     uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * (kStreamThreads * kStreamVecs) + threadIdx.x;
  u32x4_t v[kStreamVecs];
#pragma unroll
  for (int u = 0; u < kStreamVecs; ++u) {
    const int64_t i = base + u * kStreamThreads;
    v[u] = i < n16 ? ld_nt(src + i) : u32x4_t{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kStreamVecs; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (blockIdx.x == 0 && (int)threadIdx.x < tail_words) acc ^= tail[threadIdx.x];
  block_fold_xor(acc, sink);
}

// Block ids[k] of block_bytes bytes at base + ids[k] * block_bytes, for k < n_ids, cut into 1 KiB
// pieces (64 lanes x 16 bytes; the last piece of a block may be short).  Wave w of the grid reads
// pieces w * kStreamVecs .. w * kStreamVecs + kStreamVecs - 1, consecutive pieces of one block lying
// next to each other.  An id outside [0, num_blocks) is skipped (never dereferenced).
__global__ __launch_bounds__(kStreamThreads) void read_blocks_kernel(const uint8_t* base, int64_t num_blocks,
                                                                     const int32_t* ids, int64_t n_ids,
                                                                     int64_t block_bytes, uint32_t* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * kStreamThreads + threadIdx.x) / kWave;
  const int64_t per_block = block_bytes / 16;               // 16-byte vectors per block
  const int64_t steps = (per_block + kWave - 1) / kWave;    // 1 KiB pieces per block
  const int64_t items = n_ids * steps;
  u32x4_t v[kStreamVecs];
  bool ok[kStreamVecs];
#pragma unroll
  for (int u = 0; u < kStreamVecs; ++u) {
    const int64_t j = wave * kStreamVecs + u;
    const int64_t k = j < items ? j / steps : 0;
    const int64_t vec = (j - k * steps) * kWave + lane;
    const int32_t id = j < items ? ids[k] : -1;
    const bool in = id >= 0 && id < num_blocks;
    ok[u] = in && vec < per_block;
    v[u] = ok[u] ? ld_nt(reinterpret_cast<const u32x4_t*>(base + (int64_t)id * block_bytes) + vec)
                 : u32x4_t{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kStreamVecs; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  block_fold_xor(acc, sink);
}

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int tail_words = (int)((bytes % 16) / 4);
  const uint32_t* tail = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(src) + n16 * 16);
  const int64_t per = kStreamThreads * kStreamVecs;
  const int64_t blocks = n16 > 0 ? (n16 + per - 1) / per : 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3((uint32_t)blocks), dim3(kStreamThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), n16, tail, tail_words, sink);
  return hipGetLastError();
}

hipError_t launch_read_blocks(const void* base, int64_t num_blocks, const int32_t* ids, int64_t n_ids,
                              int64_t block_bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t steps = (block_bytes / 16 + kWave - 1) / kWave;
  const int64_t per = (kStreamThreads / kWave) * kStreamVecs;  // pieces per thread block
  const int64_t blocks = (n_ids * steps + per - 1) / per;
  hipLaunchKernelGGL(read_blocks_kernel, dim3((uint32_t)blocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const uint8_t*>(base), num_blocks, ids, n_ids, block_bytes, sink);
  return hipGetLastError();
}

}  // namespace kvfp8
