// w4a16_probe.hip - the practical HBM read ceiling of the device, for reporting beside the
// published peak: a plain streaming read with the same 16-byte non-temporal loads the GEMM
// kernels use for the packed codes, and no arithmetic beyond folding what was read.
#include "w4a16_device.hpp"
#include "w4a16_launch.hpp"

namespace w4a16 {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // independent 16-byte loads in flight per lane

// Each wave streams one contiguous run of the buffer, 1 KiB per load instruction (lane l reads
// chunk l of each 64-chunk step), four instructions in flight, the access pattern of a GEMM
// wave streaming its k-blocks. Every chunk is read exactly once; the words are XOR-folded per
// wave and one lane per wave XORs the fold into one of kProbeSinkWords sink words (so no load
// can be dropped as dead code, and no single address takes every wave's atomic).
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u4_t* __restrict__ buf,
                                                                   size_t chunks,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave = (size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  const size_t waves = (size_t)gridDim.x * (kProbeThreads / 64);
  const size_t per = (chunks + waves - 1) / waves;
  const size_t c0 = wave * per;
  const size_t c1 = c0 + per < chunks ? c0 + per : chunks;
  uint32_t acc = 0;
  size_t c = c0 + lane;
  for (; c + 64 * (kProbeUnroll - 1) < c1; c += 64 * kProbeUnroll) {
    u4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + c + 64 * u);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; c < c1; c += 64) {
    const u4_t v = __builtin_nontemporal_load(buf + c);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= __shfl_xor(acc, m);
  if (lane == 0) atomicXor(sink + (wave % kProbeSinkWords), acc);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (cus <= 0) cus = 256;
  const size_t chunks = bytes / 16;
  const size_t need = (chunks + kProbeThreads - 1) / kProbeThreads;
  const unsigned grid = (unsigned)(need < (size_t)cus * 8 ? need : (size_t)cus * 8);  // 8 per CU
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, s,
                     static_cast<const u4_t*>(buf), chunks, sink);
  return hipGetLastError();
}

}  // namespace w4a16
