// read_probe.hip - measurement helper of bench.py (not part of the library):
// the read bandwidth HBM delivers to a trivial kernel that reads tiles of a
// large buffer in a given order, the access pattern of the paged decode
// (independent 4 KiB tiles at random places), without any arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // tiles per thread in flight

// Workgroup b reads tiles b, b + grid, ... of `order`; each thread one
// 16-byte chunk per tile (tile_bytes = 256 * 16), XORs them, and writes
// its result so nothing is optimised away.
__global__ void __launch_bounds__(kThreads)
read_tiles_kernel(const char *buf, const int64_t *order, int64_t n_tiles, int64_t tile_bytes,
                  uint32_t *sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t t = (int64_t)blockIdx.x * kInFlight; t < n_tiles;
       t += (int64_t)gridDim.x * kInFlight) {
    u32x4 x[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t k = t + u;
      x[u] = k < n_tiles ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                               buf + order[k] * tile_bytes + threadIdx.x * 16))
                         : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= x[u];
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// Reads n_tiles tiles of 4096 bytes of `buf` (device), tile order[i]
// (device int64, each < the buffer's tile count) in turn; `sink` (device,
// grid * 256 uint32) receives junk.  Asynchronous; returns a hipError_t.
int pkv_probe_read_tiles(const void *buf, const int64_t *order, int64_t n_tiles, int grid,
                         uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(read_tiles_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     static_cast<const char *>(buf), order, n_tiles, (int64_t)4096, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
