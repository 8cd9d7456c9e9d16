// Calibration kernels for the measurements (not steps of a decode step).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dec {

constexpr int kProbeWaveBytes = 8192;            // bytes one wave reads: 8 loads of 1 KiB in flight
constexpr uint32_t kProbeMagic = 0x9E3779B9u;    // a lane whose words XOR to this writes the sink

// Streams [buf, buf + bytes) once with 16-byte non-temporal loads.  A lane whose 32 words XOR
// to kProbeMagic stores its global lane index (wave * 64 + lane) to sink[0]; nothing else is
// written.
hipError_t probe_read_launch(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// One workgroup of one wave that does nothing.
hipError_t probe_empty_launch(hipStream_t stream);

constexpr int kProbeClockSlots = 16;   // clock slots, indexed by XCD id (4 bits)

// kProbeClockSlots workgroups of one wave: each writes its XCD's constant-rate clock to
// clocks[XCD id].
hipError_t probe_clock_launch(uint64_t* clocks, hipStream_t stream);

}  // namespace dec
