// copy_blocks.hip - copy-on-write at block granularity: whole blocks of
// both pools are copied, source to destination, on the device.  A shared
// block about to be written is first copied into the writer's private block
// ("Why vLLM Uses PagedAttention", section "The bonus"); only that block is
// copied ("PagedAttention: how vLLM manages the KV cache", section
// "Copy-on-write makes shared prefixes practical").
#include "pkv_device.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;                                     // 16-byte loads in flight per thread
constexpr int64_t kCopyChunk = kCopyThreads * kCopyUnroll * 16;    // bytes per workgroup pass

// grid: x = pair, y = pool (0: K, 1: V), z = chunk of the block.  Every
// block is one contiguous run of block_bytes in each pool, whatever the
// layout inside it, so the copy is a plain 16-byte streaming copy.  Either
// side may be pinned host memory mapped into the device's address space
// (swapping): the same loads and stores then cross the host link.
__global__ void __launch_bounds__(kCopyThreads) copy_blocks_kernel(CopyBlocksArgs a) {
  const int64_t src = a.block_mapping[2 * (int64_t)blockIdx.x];
  const int64_t dst = a.block_mapping[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= a.src_num_blocks || dst < 0 || dst >= a.dst_num_blocks) return;
  const char *s = static_cast<const char *>(blockIdx.y ? a.src_v : a.src_k) + src * a.block_bytes;
  char *d = static_cast<char *>(blockIdx.y ? a.dst_v : a.dst_k) + dst * a.block_bytes;
  for (int64_t off = (int64_t)blockIdx.z * kCopyChunk; off < a.block_bytes;
       off += (int64_t)gridDim.z * kCopyChunk) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t o = off + (int64_t)(u * kCopyThreads + threadIdx.x) * 16;
      if (o < a.block_bytes) x[u] = load_stream16(s + o);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t o = off + (int64_t)(u * kCopyThreads + threadIdx.x) * 16;
      if (o < a.block_bytes) __builtin_nontemporal_store(x[u], reinterpret_cast<u32x4 *>(d + o));
    }
  }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, int num_pairs, hipStream_t st) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t chunks = (a.block_bytes + kCopyChunk - 1) / kCopyChunk;
  const dim3 grid((unsigned)num_pairs, 2, (unsigned)(chunks < 64 ? chunks : 64));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
