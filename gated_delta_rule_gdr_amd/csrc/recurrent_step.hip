// Tokenwise recurrent step of the gated delta rule over a slot-indexed pool.
//
// One workgroup owns one (sequence n, value head h). It reads the state S^T
// [DK, DV] of slot slot_idx[n] once, applies the five steps of the rule for
// the sequence's single new token (decay, predict, correct, write, read; the
// "gated_delta" Mojo page lists them, the KDA page boxes them in sections 3
// and 4) and writes the state back in place. The step is a pure HBM
// read-modify-write of the state: 2 * DK * DV * sizeof(state) bytes per
// (sequence, head) against ~6 DK DV flops. With n_h > 1 transitions per token
// (Gated DeltaProduct, "Linear attention visualized") the decay is applied
// once and steps 2-4 repeat for each substep's key, value and beta before the
// read.
//
// Thread layout (TPB threads): thread t owns value elements 4*jq .. 4*jq+3
// (jq = t % (DV/4)) for key rows kg*KP .. kg*KP+KP-1 (kg = t / (DV/4)). A
// warp-quad of lanes therefore reads 4 consecutive fp32 (16 bytes) and the
// DV/4 lanes of one key row read one contiguous row of S^T: fully coalesced
// 16-byte accesses. Reductions over the key dimension (S k and S q) are
// lane-local over KP rows, then across the lanes of a wave that share jq, then
// across the waves through LDS.
#include "gdr_internal.h"

namespace gdr {
namespace {

struct StepParams {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  void *o;
  void *pool;
  const int32_t *slot_idx;
  int32_t HV, ratio;  // ratio = HV / HK
  float scale;
  int zero_init;
  int32_t products;   // transitions per token (rows of k, v, beta per token)
};

template <bool BF16>
__device__ __forceinline__ float ld_in(const void *p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming state access: each state element is read and written once per
// step, so the loads and stores carry the nontemporal hint (measured on
// MI355X: an in-place 537 MB read-modify-write stream runs ~10% faster).
__device__ __forceinline__ f32x4 ld_nt(const float *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
}
__device__ __forceinline__ void st_nt(float *p, f32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ u32x2 ld_nt(const uint16_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ void st_nt(uint16_t *p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

// Reduce 4 partial sums over the lanes/waves that share jq. `buf` is one
// [NW waves][QUADS][4] slice of LDS; every thread receives the total.
template <int QUADS, int NW>
__device__ __forceinline__ void reduce_over_k(float (&x)[4], float *buf) {
#pragma unroll
  for (int off = QUADS; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] += __shfl_xor(x[j], off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < QUADS) {
    float4 v = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(buf)[wave * QUADS + lane] = v;
  }
  __syncthreads();
  const int jq = threadIdx.x % QUADS;
  float4 s = reinterpret_cast<const float4 *>(buf)[jq];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    float4 t = reinterpret_cast<const float4 *>(buf)[w * QUADS + jq];
    s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
  }
  x[0] = s.x; x[1] = s.y; x[2] = s.z; x[3] = s.w;
}

// PROD: more than one transition per token (Gated DeltaProduct's substeps).
template <bool IN_BF16, bool ST_BF16, bool OUT_BF16, int GATE, int RULE, bool PROD, int DK, int DV, int TPB>
__global__ __launch_bounds__(TPB) void recurrent_step_kernel(StepParams p) {
  constexpr int QUADS = DV / 4;       // lanes across one key row
  constexpr int KG = TPB / QUADS;     // key-row groups
  constexpr int KP = DK / KG;         // key rows per thread
  constexpr int NW = TPB / 64;        // waves
  static_assert(KP >= 1 && DK % KG == 0 && QUADS <= 64, "head dims");
  // reductions of the substeps' predictions alternate between red[0] and
  // red[1] (a buffer is rewritten only after every thread has passed the
  // barrier that follows its last read); the last buffer takes the output's
  constexpr int NRED = PROD ? 3 : 2;
  __shared__ float4 red[NRED][NW * QUADS];

  const int n = blockIdx.x / p.HV;
  const int h = blockIdx.x - n * p.HV;
  const int hk = h / p.ratio;
  const int t = threadIdx.x;
  const int jq = t % QUADS;
  const int kg = t / QUADS;
  const int k0 = kg * KP;

  const int64_t slot = p.slot_idx[n];
  const int64_t sbase = (slot * p.HV + h) * (int64_t)(DK * DV) + 4 * jq;

  // ---- load the state rows this thread owns (in flight first) ----
  float s[KP][4];
  if (p.zero_init) {
#pragma unroll
    for (int r = 0; r < KP; ++r) s[r][0] = s[r][1] = s[r][2] = s[r][3] = 0.f;
  } else if constexpr (ST_BF16) {
    const uint16_t *sp = static_cast<const uint16_t *>(p.pool) + sbase;
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      const u32x2 w = ld_nt(sp + (int64_t)(k0 + r) * DV);
      s[r][0] = __uint_as_float(w[0] << 16);
      s[r][1] = __uint_as_float(w[0] & 0xffff0000u);
      s[r][2] = __uint_as_float(w[1] << 16);
      s[r][3] = __uint_as_float(w[1] & 0xffff0000u);
    }
  } else {
    const float *sp = static_cast<const float *>(p.pool) + sbase;
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      const f32x4 w = ld_nt(sp + (int64_t)(k0 + r) * DV);
      s[r][0] = w[0]; s[r][1] = w[1]; s[r][2] = w[2]; s[r][3] = w[3];
    }
  }

  // ---- token inputs (substep 0's key, value and beta) ----
  const int P = PROD ? p.products : 1;
  float kv[KP], qv[KP];
  const int64_t qoff = n * p.q_stride + (int64_t)hk * DK + k0;
  const int64_t koff = (int64_t)n * P * p.k_stride + (int64_t)hk * DK + k0;
#pragma unroll
  for (int r = 0; r < KP; ++r) {
    kv[r] = ld_in<IN_BF16>(p.k, koff + r);
    qv[r] = ld_in<IN_BF16>(p.q, qoff + r);
  }
  float vv[4];
  const int64_t voff = (int64_t)n * P * p.v_stride + (int64_t)h * DV + 4 * jq;
#pragma unroll
  for (int j = 0; j < 4; ++j) vv[j] = ld_in<IN_BF16>(p.v, voff + j);
  const int64_t th = (int64_t)n * p.HV + h;
  float bv = RULE == GDR_RULE_DELTA ? p.beta[(int64_t)n * P * p.HV + h] : 0.f;

  // ---- 1. decay ----
  if constexpr (GATE == GDR_GATE_SCALAR) {
    const float a = __expf(p.g[th]);
#pragma unroll
    for (int r = 0; r < KP; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) s[r][j] *= a;
  } else if constexpr (GATE == GDR_GATE_CHANNEL) {
    const float *gp = p.g + th * DK + k0;
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      const float a = __expf(gp[r]);
#pragma unroll
      for (int j = 0; j < 4; ++j) s[r][j] *= a;
    }
  }

  // ---- 2-4. predict, correct, write: once per substep, in order (with
  // more than one, Gated DeltaProduct's transitions of one token) ----
  for (int sub = 0;;) {
    if constexpr (RULE == GDR_RULE_DELTA) {
      float vh[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < KP; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) vh[j] += s[r][j] * kv[r];
      reduce_over_k<QUADS, NW>(vh, reinterpret_cast<float *>(red[sub & 1]));
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = bv * (vv[j] - vh[j]);
#pragma unroll
      for (int r = 0; r < KP; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[r][j] += kv[r] * e[j];
    } else {
#pragma unroll
      for (int r = 0; r < KP; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) s[r][j] += kv[r] * vv[j];
    }
    if (!PROD || ++sub == P) break;
    // the next substep's key, value and beta (row n * P + sub)
    const int64_t m = (int64_t)n * P + sub;
#pragma unroll
    for (int r = 0; r < KP; ++r) kv[r] = ld_in<IN_BF16>(p.k, m * p.k_stride + (int64_t)hk * DK + k0 + r);
#pragma unroll
    for (int j = 0; j < 4; ++j) vv[j] = ld_in<IN_BF16>(p.v, m * p.v_stride + (int64_t)h * DV + 4 * jq + j);
    if constexpr (RULE == GDR_RULE_DELTA) bv = p.beta[m * p.HV + h];
  }

  // ---- write the state back (in place) ----
  if constexpr (ST_BF16) {
    uint16_t *sp = static_cast<uint16_t *>(p.pool) + sbase;
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      u32x2 w;
      w[0] = (uint32_t)f32_to_bf16(s[r][0]) | ((uint32_t)f32_to_bf16(s[r][1]) << 16);
      w[1] = (uint32_t)f32_to_bf16(s[r][2]) | ((uint32_t)f32_to_bf16(s[r][3]) << 16);
      st_nt(sp + (int64_t)(k0 + r) * DV, w);
    }
  } else {
    float *sp = static_cast<float *>(p.pool) + sbase;
#pragma unroll
    for (int r = 0; r < KP; ++r)
      st_nt(sp + (int64_t)(k0 + r) * DV, f32x4{s[r][0], s[r][1], s[r][2], s[r][3]});
  }

  // ---- 5. read with the updated state ----
  float ov[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < KP; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] += s[r][j] * qv[r];
  reduce_over_k<QUADS, NW>(ov, reinterpret_cast<float *>(red[NRED - 1]));
  if (kg == 0) {
    const int64_t ooff = th * DV + 4 * jq;
    if constexpr (OUT_BF16) {
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(p.scale * ov[0]) | ((uint32_t)f32_to_bf16(p.scale * ov[1]) << 16);
      w.y = (uint32_t)f32_to_bf16(p.scale * ov[2]) | ((uint32_t)f32_to_bf16(p.scale * ov[3]) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.o) + ooff) = w;
    } else {
      *reinterpret_cast<float4 *>(static_cast<float *>(p.o) + ooff) =
          make_float4(p.scale * ov[0], p.scale * ov[1], p.scale * ov[2], p.scale * ov[3]);
    }
  }
}

// 1024 threads (4 key rows per thread at DK = 128): of 256, 512 and 1024 it
// gave the highest HBM throughput for the 537 MB decode pool on MI355X.
constexpr int STEP_TPB = 1024;

template <bool IN_BF16, bool ST_BF16, bool OUT_BF16, int GATE, int RULE, int D>
hipError_t launch_t(const StepParams &p, int blocks, hipStream_t stream) {
  if (p.products > 1)
    hipLaunchKernelGGL((recurrent_step_kernel<IN_BF16, ST_BF16, OUT_BF16, GATE, RULE, true, D, D, STEP_TPB>),
                       dim3(blocks), dim3(STEP_TPB), 0, stream, p);
  else
    hipLaunchKernelGGL((recurrent_step_kernel<IN_BF16, ST_BF16, OUT_BF16, GATE, RULE, false, D, D, STEP_TPB>),
                       dim3(blocks), dim3(STEP_TPB), 0, stream, p);
  return hipGetLastError();
}

template <bool IN_BF16, bool ST_BF16, bool OUT_BF16, int GATE, int RULE>
hipError_t by_dim(const gdr_args &a, const StepParams &p, int blocks, hipStream_t s) {
  if (a.DK == 128) return launch_t<IN_BF16, ST_BF16, OUT_BF16, GATE, RULE, 128>(p, blocks, s);
  return launch_t<IN_BF16, ST_BF16, OUT_BF16, GATE, RULE, 64>(p, blocks, s);
}

template <bool IN_BF16, bool ST_BF16, bool OUT_BF16, int GATE>
hipError_t by_rule(const gdr_args &a, const StepParams &p, int blocks, hipStream_t s) {
  if (a.rule == GDR_RULE_DELTA) return by_dim<IN_BF16, ST_BF16, OUT_BF16, GATE, GDR_RULE_DELTA>(a, p, blocks, s);
  return by_dim<IN_BF16, ST_BF16, OUT_BF16, GATE, GDR_RULE_LINEAR>(a, p, blocks, s);
}

template <bool IN_BF16, bool ST_BF16, bool OUT_BF16>
hipError_t by_gate(const gdr_args &a, const StepParams &p, int blocks, hipStream_t s) {
  switch (a.gate) {
    case GDR_GATE_SCALAR: return by_rule<IN_BF16, ST_BF16, OUT_BF16, GDR_GATE_SCALAR>(a, p, blocks, s);
    case GDR_GATE_CHANNEL: return by_rule<IN_BF16, ST_BF16, OUT_BF16, GDR_GATE_CHANNEL>(a, p, blocks, s);
    default: return by_rule<IN_BF16, ST_BF16, OUT_BF16, GDR_GATE_NONE>(a, p, blocks, s);
  }
}

template <bool IN_BF16, bool ST_BF16>
hipError_t by_out(const gdr_args &a, const StepParams &p, int blocks, hipStream_t s) {
  if (a.out_dtype == GDR_BF16) return by_gate<IN_BF16, ST_BF16, true>(a, p, blocks, s);
  return by_gate<IN_BF16, ST_BF16, false>(a, p, blocks, s);
}

template <bool IN_BF16>
hipError_t by_state(const gdr_args &a, const StepParams &p, int blocks, hipStream_t s) {
  if (a.state_dtype == GDR_BF16) return by_out<IN_BF16, true>(a, p, blocks, s);
  return by_out<IN_BF16, false>(a, p, blocks, s);
}

}  // namespace

hipError_t launch_recurrent_step(const gdr_args &a, hipStream_t stream) {
  StepParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx;
  p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.products = products_of(a);
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  const int blocks = a.N * a.HV;
  if (a.in_dtype == GDR_BF16) return by_state<true>(a, p, blocks, stream);
  return by_state<false>(a, p, blocks, stream);
}

}  // namespace gdr
