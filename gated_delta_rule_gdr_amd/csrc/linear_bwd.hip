// Gradients of causal linear attention (the plain linear rule: no gate, no
// delta), for a ragged batch.
//
// "From Attention to Learned Memory", section "Backward: reverse the boundary
// scan, then differentiate each chunk": with o_t = s S_t q_t and
// S_t = S_0 + sum_{tau <= t} v_tau k_tau^T, the gradients of a loss with
// upstream dO are
//
//   dq_t   = s ( S_0^T do_t + sum_{tau <= t} (v_tau . do_t) k_tau )
//   dk_tau = s sum_{t >= tau} (do_t . v_tau) q_t
//   dv_tau = s sum_{t >= tau} (q_t . k_tau) do_t
//
// Each is itself a causal linear-attention forward pass with the roles of
// q, k, v and dO exchanged: dq runs forward in time with queries dO, keys v,
// values k and the initial state S_0^T; dk and dv run backward in time (each
// sequence's tokens reversed) with (queries v, keys dO, values q) and
// (queries k, keys q, values dO) from a zero state. The state those reversed
// passes carry from chunk to chunk is the page's boundary-state gradient G,
// scanned from the last chunk back. So the backward runs on the chunkwise
// forward kernels, MFMA and all. With bf16 inputs the warp-specialised kernel
// walks the sequences backwards itself (reading and writing the original
// rows); otherwise this file copies the inputs with each sequence's rows
// reversed and reverses the two outputs back. It also forms the transposed
// initial states and the slot indices of the scratch pool the passes write
// their (unused) final states to.
//
// Readings where the page is silent: the final state's gradient is zero (the
// loss reads the outputs only) and the initial state's gradient is not formed.
#include <cstdint>

#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int RTPB = 64;   // threads per reversed row

// dst row (bos + eos - 1 - t) = src row t, for t in sequence n = [bos, eos):
// `units` 16-byte units per row, rows src_stride / dst_stride bytes apart.
__global__ __launch_bounds__(RTPB) void reverse_rows_kernel(const char *src, int64_t src_stride, char *dst,
                                                            int64_t dst_stride, int units,
                                                            const int32_t *cu, int N) {
  const int64_t t = blockIdx.x;
  // the sequence holding row t: the last n with cu[n] <= t (zero-length
  // sequences before it share its cu value and are skipped)
  int lo = 0, hi = N;   // cu[lo] <= t < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int64_t r = (int64_t)cu[lo] + cu[lo + 1] - 1 - t;
  const uint4 *s = reinterpret_cast<const uint4 *>(src + t * src_stride);
  uint4 *d = reinterpret_cast<uint4 *>(dst + r * dst_stride);
  for (int u = threadIdx.x; u < units; u += RTPB) d[u] = s[u];
}

// aux[n][h] = (pool[slot_idx[n]][h])^T in fp32: the pool holds S_0^T
// [DK, DV]; the dq pass (keys v, values k) starts from S_0^T, whose transpose
// S_0 [DV, DK] is what its pool slot holds. 32 x 32 tiles through LDS.
template <bool ST_BF16>
__global__ __launch_bounds__(256) void transpose_state_kernel(const void *pool, const int32_t *slot_idx,
                                                              float *aux, int HV, int D) {
  __shared__ float tile[32][33];
  const int nh = blockIdx.x;                 // n * HV + h
  const int n = nh / HV, h = nh - n * HV;
  const int64_t src = ((int64_t)slot_idx[n] * HV + h) * (int64_t)D * D;
  const int64_t dst = (int64_t)nh * D * D;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int bi = 0; bi < D; bi += 32)
    for (int bj = 0; bj < D; bj += 32) {
      for (int y = ty; y < 32; y += 8) {
        const int64_t e = src + (int64_t)(bi + y) * D + bj + tx;
        tile[y][tx] = ST_BF16 ? bf16_to_f32(static_cast<const uint16_t *>(pool)[e])
                              : static_cast<const float *>(pool)[e];
      }
      __syncthreads();
      for (int y = ty; y < 32; y += 8) aux[dst + (int64_t)(bj + y) * D + bi + tx] = tile[tx][y];
      __syncthreads();
    }
}

__global__ void iota_kernel(int32_t *x, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = i;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t rq, rk, rv, rdo, rout, pool, slots, total;
};

// Whether the passes run on reversed copies (the general kernel) or walk the
// sequences backwards themselves (the warp-specialised kernel, bf16 inputs).
bool walks_backwards(const gdr_args &a) { return a.in_dtype == GDR_BF16 && !prefill_force_generic(); }

BwdLayout layout(const gdr_args &a) {
  const size_t ie = a.in_dtype == GDR_BF16 ? 2 : 4, oe = a.out_dtype == GDR_BF16 ? 2 : 4;
  // one [T, H, D] array (HK = HV, DK = DV), when copies are needed
  const size_t rows = walks_backwards(a) ? 0 : (size_t)a.T_total * a.HV * a.DK;
  BwdLayout l;
  l.rq = 0;
  l.rk = l.rq + align256(rows * ie);
  l.rv = l.rk + align256(rows * ie);
  l.rdo = l.rv + align256(rows * ie);
  l.rout = l.rdo + align256(rows * ie);
  l.pool = l.rout + align256(rows * oe);
  l.slots = l.pool + align256((size_t)a.N * a.HV * a.DK * a.DV * 4);
  l.total = l.slots + align256((size_t)a.N * 4);
  return l;
}

}  // namespace

size_t linear_bwd_workspace(const gdr_args &a) { return layout(a).total; }

hipError_t launch_linear_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, void *ws,
                             hipStream_t stream) {
  const BwdLayout l = layout(a);
  char *w = static_cast<char *>(ws);
  const size_t ie = a.in_dtype == GDR_BF16 ? 2 : 4, oe = a.out_dtype == GDR_BF16 ? 2 : 4;
  const int64_t HD = (int64_t)a.HV * a.DK;        // elements of one token's row (every array)
  const int units_in = (int)(HD * ie / 16), units_out = (int)(HD * oe / 16);
  int32_t *slots = reinterpret_cast<int32_t *>(w + l.slots);
  float *aux = reinterpret_cast<float *>(w + l.pool);
  const unsigned T = (unsigned)a.T_total;

  hipLaunchKernelGGL(iota_kernel, dim3((a.N + 255) / 256), dim3(256), 0, stream, slots, a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // one forward pass of the linear rule from the given state (or zero)
  auto pass = [&](const void *q, int64_t qs, const void *k, int64_t ks, const void *v, int64_t vs, void *o,
                  bool zero, bool rev) {
    gdr_args b = a;
    b.q = q; b.k = k; b.v = v;
    b.q_stride_t = qs; b.k_stride_t = ks; b.v_stride_t = vs;
    b.g = nullptr; b.beta = nullptr;
    b.o = o;
    b.state_pool = aux; b.state_dtype = GDR_F32; b.num_slots = a.N; b.slot_idx = slots;
    b.rule = GDR_RULE_LINEAR; b.gate = GDR_GATE_NONE; b.products = 1;
    b.chunk_size = 64;
    b.flags = (zero ? GDR_FLAG_ZERO_INIT : 0u) | (rev ? kFlagReverse : 0u);
    return launch_chunk_fwd(b, stream);
  };
  const bool zero = (a.flags & GDR_FLAG_ZERO_INIT) != 0;
  auto dq_pass = [&]() {
    // dq: forward time, queries dO, keys v, values k, from S_0^T
    if (!zero) {
      if (a.state_dtype == GDR_BF16)
        hipLaunchKernelGGL(transpose_state_kernel<true>, dim3(a.N * a.HV), dim3(256), 0, stream, a.state_pool,
                           a.slot_idx, aux, a.HV, a.DK);
      else
        hipLaunchKernelGGL(transpose_state_kernel<false>, dim3(a.N * a.HV), dim3(256), 0, stream, a.state_pool,
                           a.slot_idx, aux, a.HV, a.DK);
      const hipError_t te = hipGetLastError();
      if (te != hipSuccess) return te;
    }
    return pass(dout, HD, a.v, a.v_stride_t, a.k, a.k_stride_t, dq, zero, false);
  };

  if (walks_backwards(a)) {
    // the warp-specialised kernel walks the sequences backwards itself
    if ((e = pass(a.k, a.k_stride_t, a.q, a.q_stride_t, dout, HD, dv, true, true)) != hipSuccess) return e;
    if ((e = pass(a.v, a.v_stride_t, dout, HD, a.q, a.q_stride_t, dk, true, true)) != hipSuccess) return e;
    return dq_pass();
  }

  // reversed copies of q, k, v (token strides as given) and dO (contiguous)
  auto rev_in = [&](const void *src, int64_t stride_elems, size_t off) {
    hipLaunchKernelGGL(reverse_rows_kernel, dim3(T), dim3(RTPB), 0, stream, static_cast<const char *>(src),
                       (int64_t)(stride_elems * ie), w + off, (int64_t)(HD * ie), units_in, a.cu_seqlens, a.N);
  };
  rev_in(a.q, a.q_stride_t, l.rq);
  rev_in(a.k, a.k_stride_t, l.rk);
  rev_in(a.v, a.v_stride_t, l.rv);
  rev_in(dout, HD, l.rdo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  auto rev_out = [&](void *dst) {
    hipLaunchKernelGGL(reverse_rows_kernel, dim3(T), dim3(RTPB), 0, stream, (const char *)(w + l.rout),
                       (int64_t)(HD * oe), static_cast<char *>(dst), (int64_t)(HD * oe), units_out, a.cu_seqlens,
                       a.N);
    return hipGetLastError();
  };
  // dv: reversed time, queries k, keys q, values dO
  if ((e = pass(w + l.rk, HD, w + l.rq, HD, w + l.rdo, HD, w + l.rout, true, false)) != hipSuccess) return e;
  if ((e = rev_out(dv)) != hipSuccess) return e;
  // dk: reversed time, queries v, keys dO, values q
  if ((e = pass(w + l.rv, HD, w + l.rdo, HD, w + l.rq, HD, w + l.rout, true, false)) != hipSuccess) return e;
  if ((e = rev_out(dk)) != hipSuccess) return e;
  return dq_pass();
}

}  // namespace gdr
