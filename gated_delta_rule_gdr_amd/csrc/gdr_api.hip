// Host side of libgdr: argument validation, dispatch, status strings.
//
// Validation reads only host-visible fields of gdr_args (never device memory)
// and runs before anything is enqueued, so a rejected call has no side
// effects. Device-side index arrays are checked only under
// GDR_FLAG_DEBUG_CHECKS, by a small kernel whose result (a static device
// word, no allocation) is copied back; the same flag reports bounded waits
// inside the prefill kernels that ran out.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "gdr_internal.h"
#include "recurrent_bwd.h"

#define GDR_EXPORT extern "C" __attribute__((visibility("default")))

namespace gdr {
namespace {

thread_local char g_last_error[512] = "";

gdr_status fail(gdr_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

size_t dtype_bytes(gdr_dtype d) { return d == GDR_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == GDR_F32 || d == GDR_BF16; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void *p, int64_t rows, int64_t row_stride, int64_t row_len, size_t elem) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0) return {lo, lo};
  return {lo, lo + static_cast<uintptr_t>(((rows - 1) * row_stride + row_len) * (int64_t)elem)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// Which entry point is validating: the chunk prefill, the one-token step or
// the tokenwise recurrence over a ragged batch.
enum class Call { Chunk, Step, Recur };

// Checks shared by the entry points.
gdr_status validate(const gdr_args *a, Call call) {
  const bool prefill = call != Call::Step;   // a ragged batch described by cu_seqlens
  g_last_error[0] = '\0';
  if (!a) return fail(GDR_E_INVALID, "args is NULL");
  if (a->N < 0) return fail(GDR_E_INVALID, "N = %d < 0", a->N);
  if (a->T_total < 0) return fail(GDR_E_INVALID, "T_total = %lld < 0", (long long)a->T_total);
  if (a->HK <= 0 || a->HV <= 0) return fail(GDR_E_INVALID, "HK = %d, HV = %d must be positive", a->HK, a->HV);
  if (a->HV % a->HK != 0) return fail(GDR_E_INVALID, "HV = %d is not a multiple of HK = %d", a->HV, a->HK);
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->out_dtype) || !dtype_ok(a->state_dtype))
    return fail(GDR_E_INVALID, "unknown dtype code");
  if (a->rule != GDR_RULE_DELTA && a->rule != GDR_RULE_LINEAR) return fail(GDR_E_INVALID, "unknown rule %d", (int)a->rule);
  if (a->gate != GDR_GATE_NONE && a->gate != GDR_GATE_SCALAR && a->gate != GDR_GATE_CHANNEL)
    return fail(GDR_E_INVALID, "unknown gate %d", (int)a->gate);
  if (a->flags & ~(uint32_t)(GDR_FLAG_ZERO_INIT | GDR_FLAG_DEBUG_CHECKS | GDR_FLAG_QK_L2NORM))
    return fail(GDR_E_INVALID, "unknown flag bits 0x%x", a->flags);
  if ((a->flags & GDR_FLAG_QK_L2NORM) && call != Call::Recur)
    return fail(GDR_E_UNSUPPORTED, "GDR_FLAG_QK_L2NORM is taken by gdr_recurrent_fwd only");
  if (!std::isfinite(a->scale)) return fail(GDR_E_INVALID, "scale is not finite");
  if (a->products < 0 || a->products > kMaxProducts)
    return fail(GDR_E_INVALID, "products = %d: 0 .. %d transitions per token", a->products, kMaxProducts);
  if (!((a->DK == 64 || a->DK == 128) && a->DV == a->DK))
    return fail(GDR_E_UNSUPPORTED, "head dims DK = %d, DV = %d: built for DK = DV in {64, 128}", a->DK, a->DV);
  if (!prefill && a->T_total != a->N)
    return fail(GDR_E_INVALID, "recurrent step needs one token per sequence (T_total = %lld, N = %d)",
                (long long)a->T_total, a->N);
  if (call == Call::Chunk && a->chunk_size != 16 && a->chunk_size != 32 && a->chunk_size != 64)
    return fail(GDR_E_UNSUPPORTED, "chunk_size = %d: 16, 32 or 64 tokens", a->chunk_size);
  if (a->N == 0) return GDR_OK;  // nothing to do; pointers may be NULL

  if (!a->state_pool || !a->slot_idx) return fail(GDR_E_INVALID, "state_pool / slot_idx is NULL");
  if (prefill && !a->cu_seqlens) return fail(GDR_E_INVALID, "cu_seqlens is NULL");
  if (a->num_slots < a->N) return fail(GDR_E_INVALID, "num_slots = %lld < N = %d (slots must be distinct)",
                                       (long long)a->num_slots, a->N);
  if (a->T_total > 0) {
    if (!a->q || !a->k || !a->v || !a->o) return fail(GDR_E_INVALID, "q / k / v / o is NULL");
    if (a->rule == GDR_RULE_DELTA && !a->beta) return fail(GDR_E_INVALID, "beta is NULL for the delta rule");
    if (a->gate != GDR_GATE_NONE && !a->g) return fail(GDR_E_INVALID, "g is NULL for a gated call");
    const int64_t kd = (int64_t)a->HK * a->DK, vd = (int64_t)a->HV * a->DV;
    if (a->q_stride_t < kd || a->k_stride_t < kd || a->v_stride_t < vd)
      return fail(GDR_E_INVALID, "token strides (%lld, %lld, %lld) shorter than a token (%lld, %lld)",
                  (long long)a->q_stride_t, (long long)a->k_stride_t, (long long)a->v_stride_t,
                  (long long)kd, (long long)vd);
    const size_t ie = dtype_bytes(a->in_dtype);
    const int64_t TP = a->T_total * products_of(*a);   // key / value / beta rows
    const Range ro = span(a->o, a->T_total, vd, vd, dtype_bytes(a->out_dtype));
    const Range ins[] = {
        span(a->q, a->T_total, a->q_stride_t, kd, ie),
        span(a->k, TP, a->k_stride_t, kd, ie),
        span(a->v, TP, a->v_stride_t, vd, ie),
        span(a->g, a->gate == GDR_GATE_NONE ? 0 : a->T_total, 1, 1,
             4 * (size_t)a->HV * (a->gate == GDR_GATE_CHANNEL ? a->DK : 1)),
        span(a->beta, a->rule == GDR_RULE_DELTA ? TP : 0, 1, 1, 4 * (size_t)a->HV),
        span(a->state_pool, 1, 0, a->num_slots * a->HV * (int64_t)a->DK * a->DV, dtype_bytes(a->state_dtype)),
    };
    for (const Range &r : ins)
      if (overlap(ro, r)) return fail(GDR_E_INVALID, "o overlaps an input or the state pool");
    // the kernels move q, k, v, g and o rows in 16-byte units
    const void *ptrs[] = {a->q, a->k, a->v, a->g, a->o, a->state_pool};
    for (const void *ptr : ptrs)
      if (reinterpret_cast<uintptr_t>(ptr) % 16)
        return fail(GDR_E_INVALID, "q, k, v, g, o and state_pool must be 16-byte aligned");
    if ((a->q_stride_t * (int64_t)ie) % 16 || (a->k_stride_t * (int64_t)ie) % 16 ||
        (a->v_stride_t * (int64_t)ie) % 16)
      return fail(GDR_E_INVALID, "token strides of q, k, v must be multiples of 16 bytes");
  }
  return GDR_OK;
}

// Result of the device-side index check (0: valid, else the code of the
// first defect found), written by index_check_kernel on each device. Calls
// that overlap on one device with GDR_FLAG_DEBUG_CHECKS share it and race.
__device__ int g_index_check;

__global__ void index_check_kernel(const int32_t *cu, const int32_t *slots, int32_t N,
                                   int64_t T_total, int64_t num_slots, int prefill) {
  __shared__ int code;
  if (threadIdx.x == 0) code = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    if (prefill) {
      if ((i == 0 && cu[0] != 0) || (i == N - 1 && cu[N] != T_total)) atomicMax(&code, 1);
      if (cu[i + 1] < cu[i]) atomicMax(&code, 2);
    }
    const int32_t s = slots[i];
    if (s < 0 || s >= num_slots) {
      atomicMax(&code, 3);
    } else {
      for (int j = i + 1; j < N; ++j)
        if (slots[j] == s) atomicMax(&code, 4);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) g_index_check = code;
}

// GDR_FLAG_DEBUG_CHECKS, before the call's kernels: verify cu_seqlens and
// slot_idx on the device (synchronising the stream) and clear the bounded
// waits' timeout words. Allocates nothing.
gdr_status run_debug_checks(const gdr_args *a, bool prefill, hipStream_t stream) {
  hipLaunchKernelGGL(index_check_kernel, dim3(1), dim3(256), 0, stream, a->cu_seqlens, a->slot_idx, a->N,
                     (int64_t)a->T_total, (int64_t)a->num_slots, prefill ? 1 : 0);
  hipError_t e = hipGetLastError();
  int h = -1;
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(&h, HIP_SYMBOL(g_index_check), sizeof(int), 0, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = ws_wait_flag(nullptr, true, stream);
  if (e == hipSuccess) e = kda_wait_flag(nullptr, true, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "debug checks: %s", hipGetErrorString(e));
  switch (h) {
    case 0: return GDR_OK;
    case 1: return fail(GDR_E_DEVICE_CHECK, "cu_seqlens[0] != 0 or cu_seqlens[N] != T_total");
    case 2: return fail(GDR_E_DEVICE_CHECK, "cu_seqlens is not non-decreasing");
    case 3: return fail(GDR_E_DEVICE_CHECK, "slot_idx out of [0, num_slots)");
    case 4: return fail(GDR_E_DEVICE_CHECK, "slot_idx has duplicates");
    default: return fail(GDR_E_DEVICE_CHECK, "device check code %d", h);
  }
}

// GDR_FLAG_DEBUG_CHECKS, after the call's kernels: wait for them and report a
// bounded wait on an LDS counter that ran out (a producer that never
// signalled, so the results are not to be trusted).
gdr_status finish_debug_checks(hipStream_t stream) {
  int ws = 0, kda = 0;
  hipError_t e = ws_wait_flag(&ws, false, stream);
  if (e == hipSuccess) e = kda_wait_flag(&kda, false, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "debug checks: %s", hipGetErrorString(e));
  if (ws || kda)
    return fail(GDR_E_DEVICE_CHECK, "a bounded wait inside the %s prefill kernel ran out; results are invalid",
                ws ? "warp-specialised" : "channel-gate");
  return GDR_OK;
}

}  // namespace
}  // namespace gdr

using namespace gdr;

GDR_EXPORT int gdr_abi_version(void) { return GDR_ABI_VERSION; }

namespace {
// The channel-gate prefill for bf16 inputs runs as two kernels that pass
// per-chunk records through the workspace; every other prefill is one fused
// kernel and needs none.
// What the linear-attention backward covers (the linear rule of the page
// that derives it, plain or with a scalar gate, with grouped key heads), on
// top of the forward's checks of the arguments. `gated` says whether the
// caller takes the gate's gradient.
gdr_status validate_bwd_shape(const gdr_args *a, bool gated) {
  if (a->rule != GDR_RULE_LINEAR) return fail(GDR_E_UNSUPPORTED, "the backward covers the linear rule");
  if (a->gate == GDR_GATE_CHANNEL) return fail(GDR_E_UNSUPPORTED, "the backward takes no channel gate");
  if (gated && a->gate != GDR_GATE_SCALAR)
    return fail(GDR_E_UNSUPPORTED, "gdr_gated_linear_chunk_bwd takes the scalar gate");
  if (!gated && a->gate != GDR_GATE_NONE)
    return fail(GDR_E_UNSUPPORTED, "a gated backward is gdr_gated_linear_chunk_bwd (it forms the gate's gradient)");
  if (products_of(*a) > 1) return fail(GDR_E_UNSUPPORTED, "the backward takes one transition per token");
  return GDR_OK;
}

gdr_status validate_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv, float *dg, bool gated) {
  if (!a) return fail(GDR_E_INVALID, "args is NULL");
  gdr_args b = *a;
  b.o = dv;   // the forward's checks then cover dv as its output
  if (a->T_total > 0 && a->N > 0 && !dv) return fail(GDR_E_INVALID, "dv is NULL");
  gdr_status st = validate(&b, Call::Chunk);
  if (st != GDR_OK) return st;
  if ((st = validate_bwd_shape(a, gated)) != GDR_OK) return st;
  if (a->N == 0 || a->T_total == 0) return GDR_OK;
  if (!dout || !dq || !dk) return fail(GDR_E_INVALID, "dout / dq / dk is NULL");
  if (gated && !dg) return fail(GDR_E_INVALID, "dg is NULL");
  const void *ptrs[] = {dout, dq, dk};
  for (const void *ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return fail(GDR_E_INVALID, "dout, dq and dk must be 16-byte aligned");
  if (gated && reinterpret_cast<uintptr_t>(dg) % 4) return fail(GDR_E_INVALID, "dg must be 4-byte aligned");
  const int64_t vrow = (int64_t)a->HV * a->DV, krow = (int64_t)a->HK * a->DK;
  const size_t ie = dtype_bytes(a->in_dtype), oe = dtype_bytes(a->out_dtype);
  const Range outs[] = {span(dq, a->T_total, krow, krow, oe), span(dk, a->T_total, krow, krow, oe),
                        span(dv, a->T_total, vrow, vrow, oe),
                        gated ? span(dg, a->T_total, a->HV, a->HV, 4) : Range{}};
  const Range ins[] = {span(a->q, a->T_total, a->q_stride_t, krow, ie),
                       span(a->k, a->T_total, a->k_stride_t, krow, ie),
                       span(a->v, a->T_total, a->v_stride_t, vrow, ie), span(dout, a->T_total, vrow, vrow, ie),
                       gated ? span(a->g, a->T_total, a->HV, a->HV, 4) : Range{},
                       span(a->state_pool, 1, 0, a->num_slots * a->HV * (int64_t)a->DK * a->DV,
                            dtype_bytes(a->state_dtype))};
  const int nout = gated ? 4 : 3;
  for (int i = 0; i < nout; ++i) {
    for (const Range &r : ins)
      if (overlap(outs[i], r)) return fail(GDR_E_INVALID, "a gradient overlaps an input or the state pool");
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDR_E_INVALID, "the gradients overlap each other");
  }
  return GDR_OK;
}

// What the tokenwise backward takes, on top of the forward's checks (with
// dv standing in for the output): one transition per token, no in-kernel
// L2 normalisation, and the gradients' buffers.
gdr_status validate_rbwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                         float *dg, float *dstate0) {
  if (!a) return fail(GDR_E_INVALID, "args is NULL");
  gdr_args b = *a;
  b.o = dv;   // dv [T_total, HV, DV] in out_dtype has the output's layout
  if (a->T_total > 0 && a->N > 0 && !dv) return fail(GDR_E_INVALID, "dv is NULL");
  gdr_status st = validate(&b, Call::Recur);
  if (st != GDR_OK) return st;
  if (a->flags & GDR_FLAG_QK_L2NORM)
    return fail(GDR_E_UNSUPPORTED, "the backward does not differentiate the in-kernel L2 normalisation");
  if (products_of(*a) > 1) return fail(GDR_E_UNSUPPORTED, "the backward takes one transition per token");
  if (a->N == 0) return GDR_OK;
  if (a->T_total > 0) {
    if (!dout || !dq || !dk) return fail(GDR_E_INVALID, "dout / dq / dk is NULL");
    if (a->rule == GDR_RULE_DELTA && !dbeta) return fail(GDR_E_INVALID, "dbeta is NULL for the delta rule");
    if (a->gate != GDR_GATE_NONE && !dg) return fail(GDR_E_INVALID, "dg is NULL for a gated call");
  }
  const void *al[] = {dout, dq, dk};
  for (const void *ptr : al)
    if (reinterpret_cast<uintptr_t>(ptr) % 16) return fail(GDR_E_INVALID, "dout, dq and dk must be 16-byte aligned");
  const void *al4[] = {dbeta, dg, dstate0};
  for (const void *ptr : al4)
    if (reinterpret_cast<uintptr_t>(ptr) % 4) return fail(GDR_E_INVALID, "dbeta, dg and dstate0 must be 4-byte aligned");
  const int64_t kd = (int64_t)a->HK * a->DK, vd = (int64_t)a->HV * a->DV, T = a->T_total;
  const size_t ie = dtype_bytes(a->in_dtype), oe = dtype_bytes(a->out_dtype);
  const int64_t gw = a->gate == GDR_GATE_CHANNEL ? (int64_t)a->HV * a->DK : a->HV;
  const Range outs[] = {span(dv, T, vd, vd, oe),
                        span(dq, T, kd, kd, oe),
                        span(dk, T, kd, kd, oe),
                        span(dbeta, a->rule == GDR_RULE_DELTA ? T : 0, a->HV, a->HV, 4),
                        span(dg, a->gate != GDR_GATE_NONE ? T : 0, gw, gw, 4),
                        span(dstate0, 1, 0, (int64_t)a->N * a->HV * a->DK * a->DV, 4)};
  const Range ins[] = {span(a->q, T, a->q_stride_t, kd, ie), span(a->k, T, a->k_stride_t, kd, ie),
                       span(a->v, T, a->v_stride_t, vd, ie), span(dout, T, vd, vd, ie),
                       span(a->g, a->gate == GDR_GATE_NONE ? 0 : T, gw, gw, 4),
                       span(a->beta, a->rule == GDR_RULE_DELTA ? T : 0, a->HV, a->HV, 4),
                       span(a->state_pool, 1, 0, a->num_slots * a->HV * (int64_t)a->DK * a->DV,
                            dtype_bytes(a->state_dtype))};
  for (int i = 0; i < 6; ++i) {
    for (const Range &r : ins)
      if (overlap(outs[i], r)) return fail(GDR_E_INVALID, "a gradient buffer overlaps an input or the state pool");
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return fail(GDR_E_INVALID, "gradient buffers overlap each other");
  }
  return GDR_OK;
}

bool uses_workspace(const gdr_args *a) {
  return a->N > 0 && a->T_total > 0 && chunk_fwd_kda_applies(*a) && !prefill_force_generic();
}
}  // namespace

GDR_EXPORT size_t gdr_chunk_fwd_workspace_bytes(const gdr_args *a) {
  if (validate(a, Call::Chunk) != GDR_OK || !uses_workspace(a)) return 0;
  return chunk_fwd_kda_workspace(*a);
}

GDR_EXPORT gdr_status gdr_chunk_fwd(const gdr_args *a, void *workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  gdr_status s = validate(a, Call::Chunk);
  if (s != GDR_OK) return s;
  const bool ws_path = uses_workspace(a);
  if (ws_path) {
    const size_t need = chunk_fwd_kda_min_workspace(*a);
    if (!workspace || ws_bytes < need)
      return fail(GDR_E_WORKSPACE, "workspace of %zu bytes at %p: this call needs at least %zu "
                  "(gdr_chunk_fwd_workspace_bytes gives the preferred size)", ws_bytes, workspace, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(GDR_E_INVALID, "workspace is not 256-byte aligned");
  }
  if (a->N == 0) return GDR_OK;
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = ws_path ? launch_chunk_fwd_kda(*a, workspace, ws_bytes, stream)
                         : launch_chunk_fwd(*a, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "chunk_fwd launch: %s", hipGetErrorString(e));
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) return finish_debug_checks(stream);
  return GDR_OK;
}

// ---------------------------------------------------------------------------
// gdr_chunk_fwd_noalloc: the prefill with the library's own device scratch
// ---------------------------------------------------------------------------

namespace {

// Scratch of the allocation-free prefill: one array per device, held until
// the process ends. In host code `scratch` names a host-side stand-in, never
// the device memory; its device address comes from hipGetSymbolAddress, once
// per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {nullptr};

// Device address of `scratch` on device `dev` (made current for the lookup,
// the previous current device restored afterwards).
hipError_t scratch_address(int dev, void **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

GDR_EXPORT gdr_status gdr_chunk_fwd_noalloc(const gdr_args *a, hipStream_t stream) {
  gdr_status s = validate(a, Call::Chunk);
  if (s != GDR_OK) return s;
  if (!uses_workspace(a)) return gdr_chunk_fwd(a, nullptr, 0, stream);
  const size_t need = chunk_fwd_kda_min_workspace(*a);
  if (need > (size_t)GDR_NOALLOC_SCRATCH_BYTES)
    return fail(GDR_E_WORKSPACE, "this call needs at least %zu bytes of scratch, more than the %zu of "
                "gdr_chunk_fwd_noalloc (N * HV * DK * DV * 4 bytes of state carry plus one chunk's "
                "records for every value head); pass a workspace to gdr_chunk_fwd instead",
                need, (size_t)GDR_NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  void *ptr = nullptr;
  if (e == hipSuccess) e = scratch_address(dev, &ptr);
  if (e != hipSuccess) return fail(GDR_E_HIP, "scratch of gdr_chunk_fwd_noalloc: %s", hipGetErrorString(e));
  return gdr_chunk_fwd(a, ptr, (size_t)GDR_NOALLOC_SCRATCH_BYTES, stream);
}

GDR_EXPORT gdr_status gdr_recurrent_step(const gdr_args *a, hipStream_t stream) {
  gdr_status s = validate(a, Call::Step);
  if (s != GDR_OK) return s;
  if (a->N == 0) return GDR_OK;
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, false, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_recurrent_step(*a, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "recurrent_step launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

GDR_EXPORT size_t gdr_linear_chunk_bwd_workspace_bytes(const gdr_args *a) {
  if (!a) return 0;
  g_last_error[0] = '\0';
  if (validate_bwd_shape(a, a->gate == GDR_GATE_SCALAR) != GDR_OK || a->N <= 0 || a->T_total <= 0) return 0;
  if (!((a->DK == 64 || a->DK == 128) && a->DV == a->DK) || a->HK <= 0 || a->HV % a->HK) return 0;
  return linear_bwd_workspace(*a);
}

namespace {
gdr_status linear_bwd_call(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv, float *dg, bool gated,
                           void *workspace, size_t ws_bytes, hipStream_t stream) {
  gdr_status s = validate_bwd(a, dout, dq, dk, dv, dg, gated);
  if (s != GDR_OK) return s;
  if (a->N == 0 || a->T_total == 0) return GDR_OK;
  const size_t need = linear_bwd_workspace(*a);
  if (!workspace || ws_bytes < need)
    return fail(GDR_E_WORKSPACE, "workspace of %zu bytes at %p: the backward needs %zu", ws_bytes, workspace, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_E_INVALID, "workspace is not 256-byte aligned");
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_linear_bwd(*a, dout, dq, dk, dv, dg, workspace, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "linear_chunk_bwd launch: %s", hipGetErrorString(e));
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) return finish_debug_checks(stream);
  return GDR_OK;
}
}  // namespace

GDR_EXPORT gdr_status gdr_linear_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                           void *workspace, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_call(a, dout, dq, dk, dv, nullptr, false, workspace, ws_bytes, stream);
}

GDR_EXPORT gdr_status gdr_gated_linear_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                                 float *dg, void *workspace, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_call(a, dout, dq, dk, dv, dg, true, workspace, ws_bytes, stream);
}

GDR_EXPORT int gdr_ring_record_elements(const gdr_args *a) { return a ? ring_record_elements(*a) : 0; }

GDR_EXPORT int gdr_ring_record_stride(const gdr_args *a) { return a ? ring_record_stride(*a) : 0; }

GDR_EXPORT gdr_status gdr_verify_ring(const gdr_args *a, float *ring, hipStream_t stream) {
  gdr_status s = validate(a, Call::Recur);
  if (s != GDR_OK) return s;
  if (products_of(*a) > 1) return fail(GDR_E_UNSUPPORTED, "the verify takes one transition per token");
  if (a->N == 0 || a->T_total == 0) return GDR_OK;
  if (!ring) return fail(GDR_E_INVALID, "ring is NULL");
  if (reinterpret_cast<uintptr_t>(ring) % 16) return fail(GDR_E_INVALID, "ring must be 16-byte aligned");
  const Range rr = span(ring, a->T_total * a->HV, ring_record_stride(*a), ring_record_stride(*a), 4);
  const Range others[] = {span(a->o, a->T_total, (int64_t)a->HV * a->DV, (int64_t)a->HV * a->DV, dtype_bytes(a->out_dtype)),
                          span(a->state_pool, 1, 0, a->num_slots * a->HV * (int64_t)a->DK * a->DV, dtype_bytes(a->state_dtype)),
                          span(a->q, a->T_total, a->q_stride_t, (int64_t)a->HK * a->DK, dtype_bytes(a->in_dtype)),
                          span(a->k, a->T_total, a->k_stride_t, (int64_t)a->HK * a->DK, dtype_bytes(a->in_dtype)),
                          span(a->v, a->T_total, a->v_stride_t, (int64_t)a->HV * a->DV, dtype_bytes(a->in_dtype))};
  for (const Range &r : others)
    if (overlap(rr, r)) return fail(GDR_E_INVALID, "ring overlaps o, an input or the state pool");
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_recurrent_fwd(*a, stream, ring);
  if (e != hipSuccess) return fail(GDR_E_HIP, "verify_ring launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

GDR_EXPORT gdr_status gdr_state_fold(const gdr_args *a, const float *ring, const int32_t *accepted,
                                     hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!a) return fail(GDR_E_INVALID, "args is NULL");
  if (a->N < 0 || a->HK <= 0 || a->HV <= 0 || a->HV % a->HK)
    return fail(GDR_E_INVALID, "N = %d, HK = %d, HV = %d", a->N, a->HK, a->HV);
  if (!((a->DK == 64 || a->DK == 128) && a->DV == a->DK))
    return fail(GDR_E_UNSUPPORTED, "head dims DK = %d, DV = %d: built for DK = DV in {64, 128}", a->DK, a->DV);
  if (!dtype_ok(a->state_dtype)) return fail(GDR_E_INVALID, "unknown state dtype");
  if (a->gate != GDR_GATE_NONE && a->gate != GDR_GATE_SCALAR && a->gate != GDR_GATE_CHANNEL)
    return fail(GDR_E_INVALID, "unknown gate %d", (int)a->gate);
  if (a->N == 0) return GDR_OK;
  if (!a->state_pool || !a->slot_idx || !a->cu_seqlens || !ring || !accepted)
    return fail(GDR_E_INVALID, "state_pool / slot_idx / cu_seqlens / ring / accepted is NULL");
  if (a->num_slots < a->N) return fail(GDR_E_INVALID, "num_slots = %lld < N = %d", (long long)a->num_slots, a->N);
  if (reinterpret_cast<uintptr_t>(ring) % 16 || reinterpret_cast<uintptr_t>(a->state_pool) % 16)
    return fail(GDR_E_INVALID, "ring and state_pool must be 16-byte aligned");
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    gdr_status s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_state_fold(*a, ring, accepted, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "state_fold launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

GDR_EXPORT gdr_status gdr_recurrent_fwd(const gdr_args *a, hipStream_t stream) {
  gdr_status s = validate(a, Call::Recur);
  if (s != GDR_OK) return s;
  if (a->N == 0) return GDR_OK;
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_recurrent_fwd(*a, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "recurrent_fwd launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

GDR_EXPORT const char *gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_E_INVALID: return "invalid argument";
    case GDR_E_UNSUPPORTED: return "unsupported configuration";
    case GDR_E_WORKSPACE: return "workspace too small";
    case GDR_E_HIP: return "HIP runtime error";
    case GDR_E_DEVICE_CHECK: return "device-side index check failed";
    default: return "unknown status";
  }
}

GDR_EXPORT const char *gdr_last_error(void) { return g_last_error; }

// What the chunkwise backward covers, on top of the tokenwise backward's
// checks: the delta rule, gate NONE or SCALAR.
gdr_status chunk_bwd_covers(const gdr_args *a) {
  if (a->rule != GDR_RULE_DELTA)
    return fail(GDR_E_UNSUPPORTED, "the chunkwise backward covers the delta rule (the linear rule: "
                "gdr_linear_chunk_bwd / gdr_gated_linear_chunk_bwd)");
  if (a->gate == GDR_GATE_CHANNEL)
    return fail(GDR_E_UNSUPPORTED, "the chunkwise backward takes gate NONE or SCALAR");
  return GDR_OK;
}

GDR_EXPORT size_t gdr_chunk_bwd_workspace_bytes(const gdr_args *a) {
  if (validate(a, Call::Recur) != GDR_OK || a->N == 0) return 0;
  if (chunk_bwd_covers(a) != GDR_OK) return 0;
  return chunk_bwd_workspace(*a);
}

GDR_EXPORT gdr_status gdr_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                    float *dbeta, float *dg, float *dstate0, void *workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  gdr_status s = validate_rbwd(a, dout, dq, dk, dv, dbeta, dg, dstate0);
  if (s != GDR_OK) return s;
  if ((s = chunk_bwd_covers(a)) != GDR_OK) return s;
  if (a->N == 0) return GDR_OK;
  const size_t need = chunk_bwd_workspace(*a);
  if (!workspace || ws_bytes < need)
    return fail(GDR_E_WORKSPACE, "workspace of %zu bytes at %p: this call needs %zu "
                "(gdr_chunk_bwd_workspace_bytes)", ws_bytes, workspace, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_E_INVALID, "workspace is not 256-byte aligned");
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_chunk_bwd(*a, dout, dq, dk, dv, dbeta, dg, dstate0, workspace, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "chunk_bwd launch: %s", hipGetErrorString(e));
  return GDR_OK;
}

GDR_EXPORT size_t gdr_recurrent_bwd_workspace_bytes(const gdr_args *a) {
  if (validate(a, Call::Recur) != GDR_OK || a->N == 0) return 0;
  return recurrent_bwd_workspace(*a);
}

GDR_EXPORT gdr_status gdr_recurrent_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                        float *dbeta, float *dg, float *dstate0, void *workspace, size_t ws_bytes,
                                        hipStream_t stream) {
  gdr_status s = validate_rbwd(a, dout, dq, dk, dv, dbeta, dg, dstate0);
  if (s != GDR_OK) return s;
  if (a->N == 0) return GDR_OK;
  const size_t need = recurrent_bwd_workspace(*a);
  if (!workspace || ws_bytes < need)
    return fail(GDR_E_WORKSPACE, "workspace of %zu bytes at %p: this call needs %zu "
                "(gdr_recurrent_bwd_workspace_bytes)", ws_bytes, workspace, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(GDR_E_INVALID, "workspace is not 256-byte aligned");
  if (a->flags & GDR_FLAG_DEBUG_CHECKS) {
    s = run_debug_checks(a, true, stream);
    if (s != GDR_OK) return s;
  }
  hipError_t e = launch_recurrent_bwd(*a, dout, dq, dk, dv, dbeta, dg, dstate0, workspace, stream);
  if (e != hipSuccess) return fail(GDR_E_HIP, "recurrent_bwd launch: %s", hipGetErrorString(e));
  return GDR_OK;
}
