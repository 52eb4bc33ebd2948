// Memory-system probes for the benchmark (not part of the eviction path).
//
// kvp_read: a plain streaming read of a device buffer (16-byte loads, one
//   per lane per iteration, 2048 workgroups of 256 lanes), the read ceiling
//   of the HBM on this device.  The benchmark also uses it to evict the
//   caches with clean lines before a cold-cache step.
// kvp_read_ring: the same bytes streamed the way the scorer streams K and V:
//   one workgroup of 4 waves per (KV head, key chunk), a 2-stage LDS ring of
//   64-key tiles filled by direct global->LDS loads, one workgroup barrier
//   per tile, two workgroups per CU; each wave then reads 16 bytes of the
//   tile.  Its rate is the ceiling of that streaming structure.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kveprobe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadGrid = 2048;

__global__ __launch_bounds__(256) void kvp_read_kernel(const u32x4* __restrict__ p, long n16, uint32_t* sink) {
  uint32_t acc = 0;
  for (long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += static_cast<long>(gridDim.x) * 256) {
    const u32x4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;   // keeps the loads; practically never taken
}

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(gptr), "s"(lds_base) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

constexpr int KT = 64;              // keys per tile
constexpr int TILE = KT * 256;      // bytes of one K (or V) tile, 128 bf16 per row
constexpr int NBW = TILE / 1024 / 4;

__global__ __launch_bounds__(256, 2) void kvp_ring_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                          int n, int CH, int P, uint32_t* sink) {
  __shared__ __align__(1024) char ring[2 * 2 * TILE];
  const int h = blockIdx.x / P, c = blockIdx.x % P;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t base = (static_cast<size_t>(h) * n + static_cast<size_t>(c) * CH) * 256;
  const uint32_t r0 = lds_addr(ring);
  const int ntile = CH / KT;
  auto issue = [&](int t) {
    const int st = t & 1;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int blk = wave * NBW + i;
      const size_t off = base + static_cast<size_t>(t) * TILE + blk * 1024 + lane * 16;
      const uint32_t l = __builtin_amdgcn_readfirstlane(r0 + st * 2 * TILE + blk * 1024);
      dma16(k + off, l);
      dma16(v + off, l + TILE);
    }
  };
  issue(0);
  uint32_t acc = 0;
  for (int t = 0; t < ntile; ++t) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 1 < ntile) issue(t + 1);
    acc ^= *reinterpret_cast<const uint32_t*>(ring + (t & 1) * 2 * TILE + threadIdx.x * 16);
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

int kvp_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t st) {
  if (!p || !sink || bytes % 16) return -1;
  hipLaunchKernelGGL(kvp_read_kernel, dim3(kReadGrid), dim3(256), 0, st, static_cast<const u32x4*>(p),
                     static_cast<long>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int kvp_read_sink_words(void) { return kReadGrid; }

int kvp_read_ring(const void* k, const void* v, int Hkv, int n, int chunk, uint32_t* sink, hipStream_t st) {
  if (!k || !v || !sink || Hkv < 1 || chunk < KT || chunk % KT || n % chunk) return -1;
  const int P = n / chunk;
  if (static_cast<long>(Hkv) * P > kReadGrid) return -1;
  hipLaunchKernelGGL(kvp_ring_kernel, dim3(Hkv * P), dim3(256), 0, st, static_cast<const char*>(k),
                     static_cast<const char*>(v), n, chunk, P, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
