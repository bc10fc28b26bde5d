// Gradients of causal linear attention, plain or with a scalar gate (the
// linear rule: no delta), for a ragged batch with grouped key heads.
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
// reversed and reverses the outputs back. It also forms the transposed
// initial states and the slot indices of the scratch pool the passes write
// their (unused) final states to.
//
// With a scalar gate (S_t = alpha_t S_{t-1} + v_t k_t^T, G_t the cumulative
// log-decay over the sequence) every term above carries e^{G_t - G_tau}
// (e^{G_t} on S_0), the decay over the tokens tau+1 .. t. The dq pass takes
// the gates as they are; the reversed passes take them shifted by one token
// (the decay from tau to t is that of tau+1 .. t), the first reversed token
// taking none. The log-decays' gradient is dg_t = sum_{i >= t} dG_i over the
// sequence's tokens with dG_i = q_i . dq_i - k_i . dk_i per value head (the
// query side of every term minus its key side, the same identity as for the
// exponent of each pair).
//
// Grouped key heads (HV a multiple of HK): the dv pass keeps the forward's
// layout (queries k and keys q per key head, values dO per value head); the
// dq and dk passes, whose values are k and q, run with one key head per value
// head on copies of k and q repeated over each group, into fp32 per value
// head, and a last kernel sums each group (and forms dG) into dq and dk.
//
// Readings where the page is silent: the final state's gradient is zero (the
// loss reads the outputs only) and the initial state's is not formed.
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

// The sequence holding row t: the last n with cu[n] <= t (zero-length
// sequences before it share its cu value and are skipped).
__device__ __forceinline__ int seq_of(const int32_t *cu, int N, int64_t t) {
  int lo = 0, hi = N;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Gates of the reversed passes, [T, HV] fp32. REVERSED false: gs[t] =
// g[t + 1] within t's sequence and 0 on its last token (a pass that walks
// the sequence backwards itself reads row bos + eos - 1 - p at its step p);
// REVERSED true: gs[bos + p] = g[eos - p] for p >= 1 and 0 for p = 0 (the
// reversed copy's own order).
template <bool REVERSED>
__global__ __launch_bounds__(256) void shift_gate_kernel(const float *g, float *gs, const int32_t *cu, int N,
                                                          int HV, int64_t T) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * HV) return;
  const int64_t t = i / HV;
  const int h = (int)(i - t * HV);
  const int n = seq_of(cu, N, t);
  const int64_t bos = cu[n], eos = cu[n + 1];
  float x = 0.f;
  if constexpr (REVERSED) {
    const int64_t pp = t - bos;
    if (pp > 0) x = g[(eos - pp) * HV + h];
  } else {
    if (t + 1 < eos) x = g[(t + 1) * HV + h];
  }
  gs[i] = x;
}

// dst[t][h][:] = src[t][h / R][:] (D elements of `eb` bytes; src rows
// src_stride bytes apart, dst contiguous [T, HV, D]).
__global__ __launch_bounds__(256) void expand_heads_kernel(const char *src, int64_t src_stride, char *dst, int HV,
                                                           int R, int row_bytes) {
  const int64_t t = blockIdx.x;
  const int units = row_bytes / 16;
  for (int u = threadIdx.x; u < HV * units; u += 256) {
    const int h = u / units, c = u - h * units;
    const uint4 x = reinterpret_cast<const uint4 *>(src + t * src_stride + (int64_t)(h / R) * row_bytes)[c];
    reinterpret_cast<uint4 *>(dst + (t * HV + h) * (int64_t)row_bytes)[c] = x;
  }
}

template <bool BF16>
__device__ __forceinline__ float ld_x(const void *p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

// One token per workgroup: dq[t][hk] = sum of dqh[t][h] over the group of hk
// (dk likewise), in the output dtype; with GATED also
// dG[t][h] = q[t][hk] . dqh[t][h] - k[t][hk] . dkh[t][h] (a wave per head).
template <bool IN_BF16, bool OUT_BF16, bool GATED>
__global__ __launch_bounds__(256) void group_sum_kernel(const float *dqh, const float *dkh, void *dq, void *dk,
                                                        const void *q, int64_t q_stride, const void *k,
                                                        int64_t k_stride, float *dG, int HK, int HV, int D) {
  const int64_t t = blockIdx.x;
  const int R = HV / HK;
  const float *qh = dqh + t * HV * D, *kh = dkh + t * HV * D;
  for (int e = threadIdx.x; e < HK * D; e += 256) {
    const int hk = e / D, d = e - hk * D;
    float sq = 0.f, sk = 0.f;
    for (int r = 0; r < R; ++r) {
      sq += qh[(hk * R + r) * D + d];
      sk += kh[(hk * R + r) * D + d];
    }
    const int64_t o = t * HK * D + e;
    if constexpr (OUT_BF16) {
      static_cast<uint16_t *>(dq)[o] = f32_to_bf16(sq);
      static_cast<uint16_t *>(dk)[o] = f32_to_bf16(sk);
    } else {
      static_cast<float *>(dq)[o] = sq;
      static_cast<float *>(dk)[o] = sk;
    }
  }
  if constexpr (GATED) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int h = w; h < HV; h += 4) {
      const int hk = h / R;
      float x = 0.f;
      for (int d = lane; d < D; d += 64)
        x += ld_x<IN_BF16>(q, t * q_stride + (int64_t)hk * D + d) * qh[h * D + d] -
             ld_x<IN_BF16>(k, t * k_stride + (int64_t)hk * D + d) * kh[h * D + d];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
      if (lane == 0) dG[t * HV + h] = x;
    }
  }
}

// dg[t][h] = sum over the tokens i >= t of t's sequence of dG[i][h]: one
// workgroup per (sequence, head), each thread a contiguous run of tokens.
__global__ __launch_bounds__(256) void reverse_cumsum_kernel(const float *dG, float *dg, const int32_t *cu, int HV) {
  __shared__ float part[256];
  const int n = blockIdx.x / HV, h = blockIdx.x - n * HV;
  const int64_t bos = cu[n], L = (int64_t)cu[n + 1] - bos;
  const int tid = threadIdx.x;
  const int64_t seg = (L + 255) / 256;
  const int64_t a = min(L, tid * seg), b = min(L, a + seg);
  float s = 0.f;
  for (int64_t i = a; i < b; ++i) s += dG[(bos + i) * HV + h];
  part[tid] = s;
  __syncthreads();
  float after = 0.f;   // the runs of the later threads
  for (int j = tid + 1; j < 256; ++j) after += part[j];
  for (int64_t i = b - 1; i >= a; --i) {
    after += dG[(bos + i) * HV + h];
    dg[(bos + i) * HV + h] = after;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t rq, rk, rv, rdo, rout, qe, ke, dqh, dkh, gs, dG, pool, slots, total;
};

// Whether the passes run on reversed copies (the general kernel) or walk the
// sequences backwards themselves (the warp-specialised kernel, bf16 inputs).
bool walks_backwards(const gdr_args &a) { return a.in_dtype == GDR_BF16 && !prefill_force_generic(); }

// Whether dq and dk go through fp32 per-value-head buffers and the group sum
// (a gate, whose dG reads them in fp32, or grouped key heads).
bool via_group_sum(const gdr_args &a) { return a.gate == GDR_GATE_SCALAR || a.HV != a.HK; }

BwdLayout layout(const gdr_args &a) {
  const size_t ie = a.in_dtype == GDR_BF16 ? 2 : 4;
  const size_t T = (size_t)a.T_total, D = (size_t)a.DK;
  const bool copies = !walks_backwards(a), group = via_group_sum(a), grouped = a.HV != a.HK;
  const bool gated = a.gate == GDR_GATE_SCALAR;
  BwdLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  l.rq = take(copies ? T * a.HK * D * ie : 0);
  l.rk = take(copies ? T * a.HK * D * ie : 0);
  l.rv = take(copies ? T * a.HV * D * ie : 0);
  l.rdo = take(copies ? T * a.HV * D * ie : 0);
  l.rout = take(copies ? T * a.HV * D * 4 : 0);   // a reversed output (fp32 room for any dtype)
  l.qe = take(grouped ? T * a.HV * D * ie : 0);
  l.ke = take(grouped ? T * a.HV * D * ie : 0);
  l.dqh = take(group ? T * a.HV * D * 4 : 0);
  l.dkh = take(group ? T * a.HV * D * 4 : 0);
  l.gs = take(gated ? T * a.HV * 4 : 0);
  l.dG = take(gated ? T * a.HV * 4 : 0);
  l.pool = take((size_t)a.N * a.HV * D * D * 4);
  l.slots = take((size_t)a.N * 4);
  l.total = o;
  return l;
}

}  // namespace

size_t linear_bwd_workspace(const gdr_args &a) { return layout(a).total; }

hipError_t launch_linear_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dg, void *ws,
                             hipStream_t stream) {
  const BwdLayout l = layout(a);
  char *w = static_cast<char *>(ws);
  const size_t ie = a.in_dtype == GDR_BF16 ? 2 : 4, oe = a.out_dtype == GDR_BF16 ? 2 : 4;
  const int D = a.DK, HV = a.HV, HK = a.HK, R = HV / HK;
  const int64_t HVD = (int64_t)HV * D, HKD = (int64_t)HK * D;   // elements of one token's rows
  const bool gated = a.gate == GDR_GATE_SCALAR, group = via_group_sum(a), grouped = HV != HK;
  int32_t *slots = reinterpret_cast<int32_t *>(w + l.slots);
  float *aux = reinterpret_cast<float *>(w + l.pool);
  float *dqh = reinterpret_cast<float *>(w + l.dqh), *dkh = reinterpret_cast<float *>(w + l.dkh);
  float *gs = reinterpret_cast<float *>(w + l.gs), *dG = reinterpret_cast<float *>(w + l.dG);
  const unsigned T = (unsigned)a.T_total;
  const bool backwards = walks_backwards(a);

  hipLaunchKernelGGL(iota_kernel, dim3((a.N + 255) / 256), dim3(256), 0, stream, slots, a.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // one forward pass of the linear rule from the given state (or zero), with
  // `hk` key heads (the values' heads are HV) and the given gate (or none)
  auto pass = [&](const void *q, int64_t qs, const void *k, int64_t ks, const void *v, int64_t vs, void *o,
                  gdr_dtype odt, int hk, const float *gate, bool zero, bool rev) {
    gdr_args b = a;
    b.q = q; b.k = k; b.v = v;
    b.q_stride_t = qs; b.k_stride_t = ks; b.v_stride_t = vs;
    b.HK = hk;
    b.g = gate; b.beta = nullptr;
    b.o = o; b.out_dtype = odt;
    b.state_pool = aux; b.state_dtype = GDR_F32; b.num_slots = a.N; b.slot_idx = slots;
    b.rule = GDR_RULE_LINEAR; b.gate = gate ? GDR_GATE_SCALAR : GDR_GATE_NONE; b.products = 1;
    b.chunk_size = 64;
    b.flags = (zero ? GDR_FLAG_ZERO_INIT : 0u) | (rev ? kFlagReverse : 0u);
    return launch_chunk_fwd(b, stream);
  };
  const bool zero = (a.flags & GDR_FLAG_ZERO_INIT) != 0;
  // where dq and dk go: the outputs, or the per-value-head fp32 buffers
  void *dq_to = group ? (void *)dqh : dq;
  const gdr_dtype dqk_dt = group ? GDR_F32 : a.out_dtype;
  const int hk_qk = grouped ? HV : HK;   // key heads of the dq and dk passes
  // the key-head operands repeated over each group (dq and dk passes' values)
  auto expand = [&](const void *src, int64_t stride_elems, size_t off) {
    hipLaunchKernelGGL(expand_heads_kernel, dim3(T), dim3(256), 0, stream, static_cast<const char *>(src),
                       (int64_t)(stride_elems * ie), w + off, HV, R, (int)(D * ie));
    return hipGetLastError();
  };
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
    const void *kv = a.k;
    int64_t kvs = a.k_stride_t;
    if (grouped) {
      const hipError_t xe = expand(a.k, a.k_stride_t, l.ke);
      if (xe != hipSuccess) return xe;
      kv = w + l.ke;
      kvs = HVD;
    }
    return pass(dout, HVD, a.v, a.v_stride_t, kv, kvs, dq_to, dqk_dt, hk_qk, gated ? a.g : nullptr, zero, false);
  };
  // the group sums into dq and dk, dG and its reverse cumulative sum into dg
  auto finish = [&]() {
    if (!group) return hipSuccess;
#define GDR_GSUM(IB, OB, GT)                                                                                 \
  hipLaunchKernelGGL((group_sum_kernel<IB, OB, GT>), dim3(T), dim3(256), 0, stream, dqh, dkh, dq, dk, a.q,    \
                     a.q_stride_t, a.k, a.k_stride_t, dG, HK, HV, D)
    const bool ib = a.in_dtype == GDR_BF16, ob = a.out_dtype == GDR_BF16;
    if (gated) {
      if (ib && ob) GDR_GSUM(true, true, true);
      else if (ib) GDR_GSUM(true, false, true);
      else if (ob) GDR_GSUM(false, true, true);
      else GDR_GSUM(false, false, true);
    } else {
      if (ib && ob) GDR_GSUM(true, true, false);
      else if (ib) GDR_GSUM(true, false, false);
      else if (ob) GDR_GSUM(false, true, false);
      else GDR_GSUM(false, false, false);
    }
#undef GDR_GSUM
    hipError_t fe = hipGetLastError();
    if (fe != hipSuccess || !gated) return fe;
    hipLaunchKernelGGL(reverse_cumsum_kernel, dim3(a.N * HV), dim3(256), 0, stream, dG, dg, a.cu_seqlens, HV);
    return hipGetLastError();
  };
  const unsigned gblocks = (unsigned)((a.T_total * HV + 255) / 256);

  if (backwards) {
    // the warp-specialised kernel walks the sequences backwards itself
    if (gated) {
      hipLaunchKernelGGL(shift_gate_kernel<false>, dim3(gblocks), dim3(256), 0, stream, a.g, gs, a.cu_seqlens,
                         a.N, HV, a.T_total);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const float *rg = gated ? gs : nullptr;
    if ((e = pass(a.k, a.k_stride_t, a.q, a.q_stride_t, dout, HVD, dv, a.out_dtype, HK, rg, true, true)) !=
        hipSuccess)
      return e;
    const void *qv = a.q;
    int64_t qvs = a.q_stride_t;
    if (grouped) {
      if ((e = expand(a.q, a.q_stride_t, l.qe)) != hipSuccess) return e;
      qv = w + l.qe;
      qvs = HVD;
    }
    void *dk_to = group ? (void *)dkh : dk;
    if ((e = pass(a.v, a.v_stride_t, dout, HVD, qv, qvs, dk_to, dqk_dt, hk_qk, rg, true, true)) != hipSuccess)
      return e;
    if ((e = dq_pass()) != hipSuccess) return e;
    return finish();
  }

  // reversed copies of q, k, v (token strides as given) and dO (contiguous)
  auto rev_in = [&](const void *src, int64_t stride_elems, int64_t row_elems, size_t off) {
    hipLaunchKernelGGL(reverse_rows_kernel, dim3(T), dim3(RTPB), 0, stream, static_cast<const char *>(src),
                       (int64_t)(stride_elems * ie), w + off, (int64_t)(row_elems * ie), (int)(row_elems * ie / 16),
                       a.cu_seqlens, a.N);
  };
  rev_in(a.q, a.q_stride_t, HKD, l.rq);
  rev_in(a.k, a.k_stride_t, HKD, l.rk);
  rev_in(a.v, a.v_stride_t, HVD, l.rv);
  rev_in(dout, HVD, HVD, l.rdo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (gated) {
    hipLaunchKernelGGL(shift_gate_kernel<true>, dim3(gblocks), dim3(256), 0, stream, a.g, gs, a.cu_seqlens, a.N,
                       HV, a.T_total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const float *rg = gated ? gs : nullptr;
  auto rev_out = [&](void *dst, size_t esz) {
    hipLaunchKernelGGL(reverse_rows_kernel, dim3(T), dim3(RTPB), 0, stream, (const char *)(w + l.rout),
                       (int64_t)(HVD * esz), static_cast<char *>(dst), (int64_t)(HVD * esz), (int)(HVD * esz / 16),
                       a.cu_seqlens, a.N);
    return hipGetLastError();
  };
  // dv: reversed time, queries k, keys q, values dO
  if ((e = pass(w + l.rk, HKD, w + l.rq, HKD, w + l.rdo, HVD, w + l.rout, a.out_dtype, HK, rg, true, false)) !=
      hipSuccess)
    return e;
  if ((e = rev_out(dv, oe)) != hipSuccess) return e;
  // dk: reversed time, queries v, keys dO, values q (repeated over each group)
  const void *qv = w + l.rq;
  int64_t qvs = HKD;
  if (grouped) {
    if ((e = expand(w + l.rq, HKD, l.qe)) != hipSuccess) return e;
    qv = w + l.qe;
    qvs = HVD;
  }
  if ((e = pass(w + l.rv, HVD, w + l.rdo, HVD, qv, qvs, w + l.rout, dqk_dt, hk_qk, rg, true, false)) != hipSuccess)
    return e;
  if (group) {
    if ((e = rev_out(dkh, 4)) != hipSuccess) return e;
  } else {
    if ((e = rev_out(dk, oe)) != hipSuccess) return e;
  }
  if ((e = dq_pass()) != hipSuccess) return e;
  return finish();
}

}  // namespace gdr
