// Throughput probes for the block FMHA's roofline (libsparge_probe.so).
//
// Not part of the attention path: the benchmark launches them beside the
// FMHA to report what the matrix pipes sustain on this part with realistic
// fp16 operands (kind SPARGE_PROBE_MFMA) and with the FMHA loop's
// per-wavefront instruction volume but none of its dependences (kind
// SPARGE_PROBE_LOOP_VOLUME).  The kernels' header comment in
// csrc/ceiling_probe.hip lists the volume per iteration.
#pragma once

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPARGE_PROBE_MFMA = 0,
  SPARGE_PROBE_LOOP_VOLUME = 1,
};

#define SPARGE_PROBE_MAX_WORKGROUPS 65536
#define SPARGE_PROBE_MAX_ITERS 1000000

// Launch one probe on `stream` (a hipStream_t; null = the default stream).
// workgroups: 1 .. SPARGE_PROBE_MAX_WORKGROUPS, 256 threads each (4
//   wavefronts).
// iters: 1 .. SPARGE_PROBE_MAX_ITERS loop iterations per wavefront.
// out: device buffer of workgroups * 256 floats, owned by the caller; each
//   lane writes one value (a checksum that keeps the work alive).
// Returns 0 (hipSuccess) or a hipError_t code: hipErrorInvalidValue for an
// argument out of range, else the launch error.  Asynchronous: time it with
// events on the same stream.
int sparge_probe_launch(int kind, int workgroups, int iters, float* out, void* stream);

// MFMA flops one launch performs: workgroups * 4 wavefronts * iters * 16
// v_mfma_f32_32x32x16_f16 * 32768.
double sparge_probe_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif
