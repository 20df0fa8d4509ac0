// Read-bandwidth probe: a gather of 16 KiB chunks with nothing else to do,
// the ceiling against which the attention's own gather rate is judged.  The
// attention reads each selected (page, KV head) block of K and of V as one
// 16 KiB chunk at a random page; this kernel reads a given list of such
// chunks with 16-byte loads and as much parallelism as the list allows.
//
// One 256-thread workgroup per `per` consecutive chunks of the list; thread
// t reads bytes 16t, 16t + 4 KiB, 16t + 8 KiB, 16t + 12 KiB of each, with
// non-temporal loads (the data is used once).  The XOR of every 16-byte
// word a workgroup read goes to sink[workgroup] (so nothing can be skipped,
// and a test can check what was read).
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

typedef const __attribute__((address_space(1))) u32x4 *GlobalWords;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint64_t *addr, int32_t n, int32_t per, u32x4 *sink) {
  __shared__ u32x4 part[4];
  const int t = threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int c0 = blockIdx.x * per;
  const int c1 = min(n, c0 + per);
#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    // an address read from memory, cast to the global address space so that
    // the loads are global loads (waits count only the loads before them)
    const GlobalWords p = (GlobalWords)(uintptr_t)addr[c];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= __builtin_nontemporal_load(p + 256 * k + t);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    acc.x ^= (uint32_t)__shfl_xor((int)acc.x, m, 64);
    acc.y ^= (uint32_t)__shfl_xor((int)acc.y, m, 64);
    acc.z ^= (uint32_t)__shfl_xor((int)acc.z, m, 64);
    acc.w ^= (uint32_t)__shfl_xor((int)acc.w, m, 64);
  }
  if ((t & 63) == 0) part[t >> 6] = acc;
  __syncthreads();
  if (t == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_read_probe(const uint64_t *addr, int32_t n, int32_t per, void *sink, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + per - 1) / per);
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, st, addr, n, per, reinterpret_cast<u32x4 *>(sink));
  return hipGetLastError();
}

}  // namespace sas
