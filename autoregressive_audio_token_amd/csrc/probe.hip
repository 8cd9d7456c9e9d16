// Calibration kernels for the measurements: a plain streaming read, which gives the HBM read
// bandwidth this part reaches for a given byte count in one launch (the ceiling the attention
// launch is compared against, beside the 8 TB/s specification), an empty kernel, which gives
// the fixed cost of one node of a captured graph, and a clock reading, which marks points
// inside a captured graph.
//
// The read is shaped as the fastest of the layouts measured for a single ~100 MB launch: every
// wave reads its own 8 KiB (eight 1 KiB loads, all in flight, 16 bytes per lane), and the grid has
// one workgroup of four waves per 32 KiB, so the hardware dispatcher balances the CUs.  The loads
// are XOR-folded per lane and compared with a constant, which keeps them live without writing
// per-lane results; a buffer descriptor spans each wave's own range, so a ragged last wave reads
// zeros past the end instead of memory outside the buffer.
#include "probe.h"

namespace dec {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWord3 = 0x00020000;   // raw buffer resource word 3 (gfx950)
constexpr int kNonTemporal = 2;
constexpr int kWavesPerGroup = 4;

__global__ __launch_bounds__(kWavesPerGroup * 64) void probe_read_kernel(const uint8_t* buf,
                                                                          size_t bytes,
                                                                          uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const size_t wave =
      (size_t)blockIdx.x * kWavesPerGroup + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t off = wave * kProbeWaveBytes;
  if (off >= bytes) return;
  const size_t left = bytes - off;
  const int n = left < (size_t)kProbeWaveBytes ? (int)left : kProbeWaveBytes;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf + off), 0, n, kWord3);
  u32x4 v[kProbeWaveBytes / 1024];
#pragma unroll
  for (int u = 0; u < kProbeWaveBytes / 1024; ++u)
    v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, u * 1024 + lane * 16, 0, kNonTemporal);
  u32x4 acc = v[0];
#pragma unroll
  for (int u = 1; u < kProbeWaveBytes / 1024; ++u) acc ^= v[u];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == kProbeMagic) sink[0] = (uint32_t)(wave * 64 + lane);
}

__global__ __launch_bounds__(64) void probe_empty_kernel() {}

// The dispatcher deals workgroups to the XCDs in turn, so kProbeClockSlots workgroups reach
// every XCD; each writes that XCD's 100 MHz clock (XCDs keep separate clocks, so a reading
// is compared only with readings of the same XCD).  Workgroups on one XCD write the same
// slot within nanoseconds of each other.
__global__ __launch_bounds__(64) void probe_clock_kernel(uint64_t* clocks) {
  if (threadIdx.x != 0) return;
  const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20) & (kProbeClockSlots - 1);
  clocks[xcc] = __builtin_amdgcn_s_memrealtime();
}

}  // namespace

hipError_t probe_read_launch(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const size_t per_group = (size_t)kWavesPerGroup * kProbeWaveBytes;
  const size_t blocks = (bytes + per_group - 1) / per_group;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kWavesPerGroup * 64), 0,
                     stream, static_cast<const uint8_t*>(buf), bytes, sink);
  return hipGetLastError();
}

hipError_t probe_empty_launch(hipStream_t stream) {
  hipLaunchKernelGGL(probe_empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError();
}

hipError_t probe_clock_launch(uint64_t* clocks, hipStream_t stream) {
  hipLaunchKernelGGL(probe_clock_kernel, dim3(kProbeClockSlots), dim3(64), 0, stream, clocks);
  return hipGetLastError();
}

}  // namespace dec
