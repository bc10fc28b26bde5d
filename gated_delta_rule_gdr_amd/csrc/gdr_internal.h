// Internal declarations and device helpers shared by the HIP sources of
// libgdr. Not part of the public ABI (include/gdr.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {

// ---------------------------------------------------------------------------
// scalar conversions (bf16 carried as its 16-bit pattern)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN. (One hardware
// conversion, v_cvt_pk_bf16_f32, with the other half unused.)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// hi = bf16(x), lo = bf16(x - hi): hi + lo carries 16 significant bits of x.
__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Internal flag (never accepted from callers): the prefill walks each
// sequence's rows backwards, its last row first, and writes each output row
// to the row it was read from. Taken by the warp-specialised kernel (bf16
// inputs, no channel gate, one transition per token) only.
constexpr uint32_t kFlagReverse = 1u << 31;

// Transitions per token (Gated DeltaProduct's n_h; 0 in the arguments means 1).
constexpr int kMaxProducts = 8;
inline int products_of(const gdr_args &a) { return a.products > 1 ? a.products : 1; }

// ---------------------------------------------------------------------------
// launchers (defined next to their kernels)
// ---------------------------------------------------------------------------

hipError_t launch_recurrent_step(const gdr_args &a, hipStream_t stream);
// (ring != nullptr: the verify of a speculative window, recording into ring)
hipError_t launch_recurrent_fwd(const gdr_args &a, hipStream_t stream, float *ring = nullptr);
// Elements of one verify record: e (DV), k (DK), the gate (1, DK or none);
// records lie ring_record_stride apart (rounded up to a multiple of 4).
int ring_record_elements(const gdr_args &a);
int ring_record_stride(const gdr_args &a);
hipError_t launch_state_fold(const gdr_args &a, const float *ring, const int32_t *accepted, hipStream_t stream);
hipError_t launch_chunk_fwd(const gdr_args &a, hipStream_t stream);
// Linear-attention backward: three chunkwise forward passes with exchanged
// roles (linear_bwd.hip); its workspace in bytes.
size_t linear_bwd_workspace(const gdr_args &a);
hipError_t launch_linear_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dg,
                             void *ws, hipStream_t stream);
// The backward's forward walk: the general prefill kernel storing S^T at the
// start of every chunk to ckpt ([flat chunk][HV][DK][DV] fp32, flat chunk
// floor(cu[n] / 64) + n + c), writing neither outputs nor the pool
// (chunk_fwd.hip; delta rule, gate NONE or SCALAR, chunks of 64).
hipError_t launch_chunk_states(const gdr_args &a, float *ckpt, hipStream_t stream);
// The same walk on the warp-specialised kernel (bf16 inputs), which also
// writes the outputs to a.o and the final states to a.state_pool: the caller
// points both at scratch.
hipError_t launch_chunk_states_ws(const gdr_args &a, float *ckpt, hipStream_t stream);
// Chunkwise backward of the gated delta rule (chunk_bwd.hip): its workspace
// in bytes, and the launch.
size_t chunk_bwd_workspace(const gdr_args &a);
hipError_t launch_chunk_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                            float *dg, float *dstate0, void *ws, hipStream_t stream);
// True when GDR_PREFILL_KERNEL=generic asks for the general prefill kernel in
// every case (used to compare kernels).
bool prefill_force_generic();
// Compute units of the current device (cached per device).
int cu_count();

// Channel-gate prefill (bf16 inputs, delta rule): two kernels per slice of
// chunks, sharing per-chunk records through the caller's workspace.
bool chunk_fwd_kda_applies(const gdr_args &a);
size_t chunk_fwd_kda_workspace(const gdr_args &a);       // preferred bytes
size_t chunk_fwd_kda_min_workspace(const gdr_args &a);   // fewest bytes that work
hipError_t launch_chunk_fwd_kda(const gdr_args &a, void *ws, size_t ws_bytes, hipStream_t stream);
// The wait-timeout word of the warp-specialised prefill (also run by the
// linear-attention backward) and of the channel-gate pair: cleared
// (clear = true) or copied to the host int *out, enqueued on `stream`.
hipError_t ws_wait_flag(int *out, bool clear, hipStream_t stream);
hipError_t kda_wait_flag(int *out, bool clear, hipStream_t stream);

}  // namespace gdr
