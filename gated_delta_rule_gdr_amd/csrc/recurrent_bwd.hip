// Gradients of the gated delta rule and of the gated linear rule, tokenwise,
// for a ragged batch.
//
// The forward is the recurrence of recurrent_fwd.hip ("You Could Have Come Up
// With Kimi Delta Attention", the recurrent form; "gated_delta" Mojo page, the
// state update; "Linear attention visualized", the gated variants). With S
// value-by-key [DV, DK] and a_t = exp(g_t) (a scalar, or a scale per key
// column for the channel gate):
//
//   St~ = S_{t-1} a_t,  u_t = St~ k_t,  e_t = beta_t (v_t - u_t)  (e_t = v_t
//   for the linear rule),  S_t = St~ + e_t k_t^T,  o_t = scale S_t q_t.
//
// The pages give no backward for the delta rule. This file differentiates
// that recurrence in reverse mode, one operation at a time. Walking t
// backwards with D = dL/dS_t (zero after the last token):
//
//   D += scale do_t q_t^T;  dq_t = scale S_t^T do_t;  de = D k_t;  dk_t = D^T e_t
//   delta rule: dv_t = beta_t de, dbeta_t = de . (v_t - u_t),
//               dk_t -= beta_t St~^T de, D -= beta_t de k_t^T
//   linear rule: dv_t = de
//   dg_t = <D, St~> (per key column for the channel gate);  D *= a_t
//
// After the first token D is the gradient of the initial state.
//
// Schedule. Each row j of S and of D evolves on its own in both directions,
// so one workgroup takes RW = 32 value rows of one (sequence, value head) and
// walks the whole sequence without talking to other workgroups. Only dq, dk,
// dg and dbeta sum over rows: each workgroup writes its partial sums to the
// workspace and a second kernel adds them up, over the row groups and over
// the value heads that share a key head.
//   Phase 1 runs the forward over the sequence and stores the state at the
//   start of every block of B tokens (a checkpoint) in the workspace.
//   Phase 2 takes the blocks last to first: it reloads the block's
//   checkpoint, reruns the block's forward steps keeping St~, u and e of each
//   token in registers, then walks the block's tokens backwards.
// A thread holds RW/(4 NW) rows x DK/16 columns of S (and of D), NW waves per
// workgroup (8: one row per thread, two waves per SIMD); the 16 lanes of
// a DPP row share those rows, so the dots over k (u, de) are 16-lane DPP sums,
// and
// the sums over rows are lane swaps across the four 16-lane groups of a
// wave, then a sum over the waves through LDS at the end of the block.
#include <cstdint>

#include "recurrent_bwd.h"

namespace gdr {
namespace {

constexpr int BB = 8;     // tokens per block (checkpoint spacing)

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Sum over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror: the other quad of the 8
  x += dpp_mov<0x140>(x);   // row_mirror: the other 8 of the 16
  return x;
}
// Sum over the four 16-lane groups of the wave (the same lane of each), with
// gfx950's lane swaps: permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second, permlane32_swap the upper
// half of the first with the lower half of the second. With x in both, every
// lane ends up holding x in one result and its partner's x in the other, so
// their sum adds the partner lane (lane ^ 16, then lane ^ 32) in the VALU.
__device__ __forceinline__ float sum_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <bool F32>
__device__ __forceinline__ float ld(const void *p, int64_t i) {
  if constexpr (F32) return static_cast<const float *>(p)[i];
  else return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
}
__device__ __forceinline__ void st_out(void *p, int64_t i, float x, bool bf16) {
  if (bf16) static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
  else static_cast<float *>(p)[i] = x;
}

struct BwdParams {
  const void *q, *k, *v, *dout;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  const void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t N, HV, ratio;
  float scale;
  int zero_init, st_bf16, out_bf16;
  float *ckpt;     // [slots of B tokens][HV][D rows][D]
  float *part;     // [T][HV][NS][NVEC][D]: dq, dk (and dg, channel gate) partial sums
  float *partb;    // [T][HV][NS]: dbeta partial sums (delta rule)
  float *partg;    // [T][HV][NS]: dg partial sums (scalar gate)
  void *dv;        // [T][HV][D], out dtype
  float *dstate0;  // [N][HV][D][D] (S^T layout) or null
};

template <int GATE>
constexpr int nvec() { return GATE == GDR_GATE_CHANNEL ? 3 : 2; }

template <int GATE, int D, int RW, int NW>
struct BwdSmem {
  static constexpr int GP = GATE == GDR_GATE_CHANNEL ? D : 1;
  alignas(16) float kk[BB][D];
  alignas(16) float qq[BB][D];
  alignas(16) float ga[BB][GP];   // exp(g)
  float vv[BB][RW], dd[BB][RW], bb[BB];
  alignas(16) float red[BB][NW][nvec<GATE>() * D];   // per wave: the block's column sums
  float redb[BB][NW], redg[BB][NW];
  float dvs[BB][RW];
};

// Stage tokens t0 .. t0 + len - 1 of the block: keys (and queries, upstream
// gradients with `back`), this workgroup's value rows, beta and exp(g).
template <bool IN_F32, int GATE, bool DELTA, int D, int RW, int NW>
__device__ __forceinline__ void stage(BwdSmem<GATE, D, RW, NW> &sm, const BwdParams &p, int64_t t0, int len, int h,
                                      int hk, int r0, bool back, int tid) {
  for (int e = tid; e < BB * D; e += 64 * NW) {
    const int i = e / D, c = e % D;
    if (i < len) {
      const int64_t t = t0 + i;
      sm.kk[i][c] = ld<IN_F32>(p.k, t * p.k_stride + (int64_t)hk * D + c);
      if (back) sm.qq[i][c] = ld<IN_F32>(p.q, t * p.q_stride + (int64_t)hk * D + c);
      if constexpr (GATE == GDR_GATE_CHANNEL) sm.ga[i][c] = __expf(p.g[(t * p.HV + h) * D + c]);
    }
  }
  for (int e = tid; e < BB * RW; e += 64 * NW) {
    const int i = e / RW, r = e % RW;
    if (i < len) {
      const int64_t t = t0 + i;
      sm.vv[i][r] = ld<IN_F32>(p.v, t * p.v_stride + (int64_t)h * D + r0 + r);
      if (back) sm.dd[i][r] = ld<IN_F32>(p.dout, (t * p.HV + h) * D + r0 + r);
    }
  }
  if (tid < len) {
    const int64_t t = t0 + tid;
    if constexpr (DELTA) sm.bb[tid] = p.beta[t * p.HV + h];
    if constexpr (GATE == GDR_GATE_SCALAR) sm.ga[tid][0] = __expf(p.g[t * p.HV + h]);
  }
}

template <bool IN_F32, int GATE, bool DELTA, int D, int RW, int NW>
__global__ __launch_bounds__(64 * NW) void recurrent_bwd_kernel(BwdParams p) {
  constexpr int C = D / 16;          // key columns per thread
  constexpr int NS = D / RW;         // row groups per head
  constexpr int NV = nvec<GATE>();
  constexpr int R = RW / (4 * NW);   // rows per thread (each wave: four 16-lane row groups)
  static_assert(R >= 1 && R * 4 * NW == RW, "rows per workgroup must fill the waves");
  __shared__ BwdSmem<GATE, D, RW, NW> sm;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int rg = lane >> 4, cg = lane & 15;
  const int kc = cg * C;                 // first key column
  const int lr = w * (RW / NW) + rg * R;  // first of the thread's local rows
  const int split = blockIdx.x % NS;
  const int nh = blockIdx.x / NS;
  const int n = nh / p.HV, h = nh - n * p.HV, hk = h / p.ratio;
  const int r0 = split * RW;             // first value row of the workgroup
  const int64_t bos = p.cu_seqlens[n], L = (int64_t)p.cu_seqlens[n + 1] - bos;
  const int nb = (int)((L + BB - 1) / BB);
  const int64_t slot0 = bos / BB + n;    // this sequence's first checkpoint
  const int64_t HD2 = (int64_t)D * D;

  float s[R][C];
  if (p.zero_init) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int x = 0; x < C; ++x) s[r][x] = 0.f;
  } else {
    const int64_t base = ((int64_t)p.slot_idx[n] * p.HV + h) * HD2;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int x = 0; x < C; ++x) {
        const int64_t e = base + (int64_t)(kc + x) * D + r0 + lr + r;
        s[r][x] = p.st_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p.pool)[e])
                            : static_cast<const float *>(p.pool)[e];
      }
  }

  auto ck = [&](int b, int r) {
    return p.ckpt + ((slot0 + b) * p.HV + h) * HD2 + (int64_t)(r0 + lr + r) * D + kc;
  };

  // One forward step of token i of the staged block: s becomes S_t; returns
  // u and e of the two rows (st, if given, receives St~).
  auto fwd = [&](int i, float (&u)[R], float (&e)[R], float (*st)[C]) {
    float k[C];
#pragma unroll
    for (int x = 0; x < C; ++x) k[x] = sm.kk[i][kc + x];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a = 0.f;
#pragma unroll
      for (int x = 0; x < C; ++x) {
        if constexpr (GATE == GDR_GATE_SCALAR) s[r][x] *= sm.ga[i][0];
        else if constexpr (GATE == GDR_GATE_CHANNEL) s[r][x] *= sm.ga[i][kc + x];
        if (st) st[r][x] = s[r][x];
        a = fmaf(s[r][x], k[x], a);
      }
      u[r] = sum16(a);
      const float v = sm.vv[i][lr + r];
      e[r] = DELTA ? sm.bb[i] * (v - u[r]) : v;
#pragma unroll
      for (int x = 0; x < C; ++x) s[r][x] = fmaf(e[r], k[x], s[r][x]);
    }
  };

  // phase 1: forward over the sequence, a checkpoint at every block start
  for (int b = 0; b < nb; ++b) {
    const int64_t t0 = bos + (int64_t)b * BB;
    const int len = (int)min<int64_t>(BB, L - (int64_t)b * BB);
    stage<IN_F32, GATE, DELTA, D, RW, NW>(sm, p, t0, len, h, hk, r0, false, tid);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float4 *dst = reinterpret_cast<float4 *>(ck(b, r));
#pragma unroll
      for (int x = 0; x < C; x += 4) dst[x / 4] = make_float4(s[r][x], s[r][x + 1], s[r][x + 2], s[r][x + 3]);
    }
    for (int i = 0; i < len; ++i) {
      float u[R], e[R];
      fwd(i, u, e, nullptr);
    }
    __syncthreads();
  }

  // phase 2: blocks last to first
  float D_[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int x = 0; x < C; ++x) D_[r][x] = 0.f;

  for (int b = nb - 1; b >= 0; --b) {
    const int64_t t0 = bos + (int64_t)b * BB;
    const int len = (int)min<int64_t>(BB, L - (int64_t)b * BB);
    stage<IN_F32, GATE, DELTA, D, RW, NW>(sm, p, t0, len, h, hk, r0, true, tid);
    __syncthreads();
    // the block's checkpoint (written by this same thread in phase 1)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float4 *src = reinterpret_cast<const float4 *>(ck(b, r));
#pragma unroll
      for (int x = 0; x < C; x += 4) {
        const float4 f = src[x / 4];
        s[r][x] = f.x; s[r][x + 1] = f.y; s[r][x + 2] = f.z; s[r][x + 3] = f.w;
      }
    }
    float sts[BB][R][C], us[BB][R], es[BB][R];
#pragma unroll
    for (int i = 0; i < BB; ++i)
      if (i < len) fwd(i, us[i], es[i], sts[i]);

#pragma unroll
    for (int i = BB - 1; i >= 0; --i) {
      if (i >= len) continue;
      float k[C], q[C], dov[R];
#pragma unroll
      for (int x = 0; x < C; ++x) {
        k[x] = sm.kk[i][kc + x];
        q[x] = sm.qq[i][kc + x];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) dov[r] = sm.dd[i][lr + r];
      float pq[C], pk[C], pg[C];
      float de[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float sd = p.scale * dov[r];
        float a = 0.f;
#pragma unroll
        for (int x = 0; x < C; ++x) {
          D_[r][x] = fmaf(sd, q[x], D_[r][x]);
          a = fmaf(D_[r][x], k[x], a);
        }
        de[r] = sum16(a);
      }
#pragma unroll
      for (int x = 0; x < C; ++x) {
        // S_t = St~ + e k^T for dq; D^T e for dk
        pq[x] = 0.f;
        pk[x] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          pq[x] = fmaf(fmaf(es[i][r], k[x], sts[i][r][x]), dov[r], pq[x]);
          pk[x] = fmaf(D_[r][x], es[i][r], pk[x]);
        }
      }
      float db = 0.f, dvr[R];
      if constexpr (DELTA) {
        const float beta = sm.bb[i];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          dvr[r] = beta * de[r];
          db = fmaf(de[r], sm.vv[i][lr + r] - us[i][r], db);
          const float du = -beta * de[r];
#pragma unroll
          for (int x = 0; x < C; ++x) {
            pk[x] = fmaf(sts[i][r][x], du, pk[x]);
            D_[r][x] = fmaf(du, k[x], D_[r][x]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) dvr[r] = de[r];
      }
      float gs = 0.f;
      if constexpr (GATE == GDR_GATE_SCALAR) {
        const float a = sm.ga[i][0];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int x = 0; x < C; ++x) {
            gs = fmaf(D_[r][x], sts[i][r][x], gs);
            D_[r][x] *= a;
          }
        gs = sum_groups(sum16(gs));
      } else if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
        for (int x = 0; x < C; ++x) {
          const float a = sm.ga[i][kc + x];
          pg[x] = 0.f;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            pg[x] = fmaf(D_[r][x], sts[i][r][x], pg[x]);
            D_[r][x] *= a;
          }
        }
      }
#pragma unroll
      for (int x = 0; x < C; ++x) {
        pq[x] = sum_groups(pq[x]);
        pk[x] = sum_groups(pk[x]);
        if constexpr (GATE == GDR_GATE_CHANNEL) pg[x] = sum_groups(pg[x]);
      }
      if constexpr (DELTA) db = sum_groups(db);
      if (rg == 0) {
        float *rd = sm.red[i][w];
#pragma unroll
        for (int x = 0; x < C; x += 4) {
          *reinterpret_cast<float4 *>(rd + kc + x) = make_float4(pq[x], pq[x + 1], pq[x + 2], pq[x + 3]);
          *reinterpret_cast<float4 *>(rd + D + kc + x) = make_float4(pk[x], pk[x + 1], pk[x + 2], pk[x + 3]);
          if constexpr (GATE == GDR_GATE_CHANNEL)
            *reinterpret_cast<float4 *>(rd + 2 * D + kc + x) = make_float4(pg[x], pg[x + 1], pg[x + 2], pg[x + 3]);
        }
      }
      if (lane == 0) {
        sm.redb[i][w] = db;
        sm.redg[i][w] = gs;
      }
      if (cg == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) sm.dvs[i][lr + r] = dvr[r];
      }
    }
    __syncthreads();
    // the block's partial sums over this workgroup's rows, and dv
    for (int e = tid; e < len * NV * D; e += 64 * NW) {
      const int i = e / (NV * D), c = e - i * (NV * D);
      float x = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) x += sm.red[i][v][c];
      p.part[(((t0 + i) * p.HV + h) * NS + split) * (NV * D) + c] = x;
    }
    for (int e = tid; e < len * RW; e += 64 * NW) {
      const int i = e / RW, r = e % RW;
      st_out(p.dv, ((t0 + i) * p.HV + h) * D + r0 + r, sm.dvs[i][r], p.out_bf16);
    }
    if (tid < len) {
      const int64_t o = ((t0 + tid) * p.HV + h) * NS + split;
      float sb = 0.f, sg = 0.f;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        sb += sm.redb[tid][v];
        sg += sm.redg[tid][v];
      }
      if constexpr (DELTA) p.partb[o] = sb;
      if constexpr (GATE == GDR_GATE_SCALAR) p.partg[o] = sg;
    }
  }

  // the initial state's gradient, transposed like the pool
  if (p.dstate0) {
    const int64_t base = ((int64_t)n * p.HV + h) * HD2;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int x = 0; x < C; ++x) p.dstate0[base + (int64_t)(kc + x) * D + r0 + lr + r] = D_[r][x];
  }
}

// dq, dk (summed over row groups and over the value heads of a key head), dg
// and dbeta (summed over row groups). One workgroup per token.
template <int GATE, bool DELTA, int D, int RW>
__global__ __launch_bounds__(256) void recurrent_bwd_reduce_kernel(const float *part, const float *partb,
                                                                   const float *partg, void *dq, void *dk,
                                                                   float *dbeta, float *dg, int HK, int HV,
                                                                   float scale, int out_bf16) {
  constexpr int NS = D / RW, NV = nvec<GATE>();
  const int64_t t = blockIdx.x;
  const int G = HV / HK;
  for (int e = threadIdx.x; e < HK * D; e += 256) {
    const int hk = e / D, c = e - hk * D;
    float sq = 0.f, sk = 0.f;
    for (int j = 0; j < G; ++j)
      for (int s = 0; s < NS; ++s) {
        const float *pp = part + ((t * HV + hk * G + j) * NS + s) * (NV * D);
        sq += pp[c];
        sk += pp[D + c];
      }
    st_out(dq, (t * HK + hk) * D + c, scale * sq, out_bf16);
    st_out(dk, (t * HK + hk) * D + c, sk, out_bf16);
  }
  if constexpr (GATE == GDR_GATE_CHANNEL) {
    for (int e = threadIdx.x; e < HV * D; e += 256) {
      const int h = e / D, c = e - h * D;
      float sg = 0.f;
      for (int s = 0; s < NS; ++s) sg += part[((t * HV + h) * NS + s) * (NV * D) + 2 * D + c];
      dg[(t * HV + h) * D + c] = sg;
    }
  }
  for (int h = threadIdx.x; h < HV; h += 256) {
    float sb = 0.f, sg = 0.f;
    for (int s = 0; s < NS; ++s) {
      if constexpr (DELTA) sb += partb[(t * HV + h) * NS + s];
      if constexpr (GATE == GDR_GATE_SCALAR) sg += partg[(t * HV + h) * NS + s];
    }
    if constexpr (DELTA) dbeta[t * HV + h] = sb;
    if constexpr (GATE == GDR_GATE_SCALAR) dg[t * HV + h] = sg;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct RbLayout {
  size_t ckpt, part, partb, partg, total;
};

// Value rows per workgroup. 32 rows (one workgroup per compute unit on the
// headline shapes) ran faster than 16 rows (two per compute unit, twice the
// partial sums): 8.6 against 9.3 ms.
constexpr int kRows = 32;
constexpr int kWaves = 8;   // one row per thread: two waves per SIMD

RbLayout rb_layout(const gdr_args &a) {
  const int D = a.DK, NS = D / kRows, NV = a.gate == GDR_GATE_CHANNEL ? 3 : 2;
  const size_t T = (size_t)a.T_total;
  const size_t slots = T / BB + (size_t)a.N + 1;   // bounds bos/B + n + blocks over every sequence
  RbLayout l;
  l.ckpt = 0;
  l.part = align256(slots * a.HV * (size_t)D * D * 4);
  l.partb = l.part + align256(T * a.HV * NS * NV * (size_t)D * 4);
  l.partg = l.partb + align256(T * a.HV * NS * 4);
  l.total = l.partg + align256(T * a.HV * NS * 4);
  return l;
}

template <bool IN_F32, int GATE, bool DELTA, int D, int RW, int NW>
hipError_t launch_rw(const gdr_args &a, const BwdParams &p, void *dq, void *dk, float *dbeta, float *dg,
                     hipStream_t stream) {
  constexpr int NS = D / RW;
  hipLaunchKernelGGL((recurrent_bwd_kernel<IN_F32, GATE, DELTA, D, RW, NW>), dim3((unsigned)(a.N * a.HV * NS)),
                     dim3(64 * NW),
                     0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.T_total == 0) return e;
  hipLaunchKernelGGL((recurrent_bwd_reduce_kernel<GATE, DELTA, D, RW>), dim3((unsigned)a.T_total), dim3(256), 0, stream,
                     p.part, p.partb, p.partg, dq, dk, dbeta, dg, a.HK, a.HV, a.scale, p.out_bf16);
  return hipGetLastError();
}
template <bool IN_F32, int GATE, bool DELTA, int D>
hipError_t launch_typed(const gdr_args &a, const BwdParams &p, void *dq, void *dk, float *dbeta, float *dg,
                        hipStream_t stream) {
  return launch_rw<IN_F32, GATE, DELTA, D, kRows, kWaves>(a, p, dq, dk, dbeta, dg, stream);
}

template <bool IN_F32, int GATE, bool DELTA>
hipError_t by_dim(const gdr_args &a, const BwdParams &p, void *dq, void *dk, float *dbeta, float *dg,
                  hipStream_t s) {
  return a.DK == 64 ? launch_typed<IN_F32, GATE, DELTA, 64>(a, p, dq, dk, dbeta, dg, s)
                    : launch_typed<IN_F32, GATE, DELTA, 128>(a, p, dq, dk, dbeta, dg, s);
}
template <bool IN_F32, int GATE>
hipError_t by_rule(const gdr_args &a, const BwdParams &p, void *dq, void *dk, float *dbeta, float *dg,
                   hipStream_t s) {
  return a.rule == GDR_RULE_DELTA ? by_dim<IN_F32, GATE, true>(a, p, dq, dk, dbeta, dg, s)
                                  : by_dim<IN_F32, GATE, false>(a, p, dq, dk, dbeta, dg, s);
}
template <bool IN_F32>
hipError_t by_gate(const gdr_args &a, const BwdParams &p, void *dq, void *dk, float *dbeta, float *dg,
                   hipStream_t s) {
  switch (a.gate) {
    case GDR_GATE_SCALAR: return by_rule<IN_F32, GDR_GATE_SCALAR>(a, p, dq, dk, dbeta, dg, s);
    case GDR_GATE_CHANNEL: return by_rule<IN_F32, GDR_GATE_CHANNEL>(a, p, dq, dk, dbeta, dg, s);
    default: return by_rule<IN_F32, GDR_GATE_NONE>(a, p, dq, dk, dbeta, dg, s);
  }
}

}  // namespace

size_t recurrent_bwd_workspace(const gdr_args &a) { return rb_layout(a).total; }

hipError_t launch_recurrent_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                                float *dg, float *dstate0, void *ws, hipStream_t stream) {
  const RbLayout l = rb_layout(a);
  char *w = static_cast<char *>(ws);
  BwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = dout;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta;
  p.pool = a.state_pool; p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) != 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  p.ckpt = reinterpret_cast<float *>(w + l.ckpt);
  p.part = reinterpret_cast<float *>(w + l.part);
  p.partb = reinterpret_cast<float *>(w + l.partb);
  p.partg = reinterpret_cast<float *>(w + l.partg);
  p.dv = dv;
  p.dstate0 = dstate0;
  return a.in_dtype == GDR_F32 ? by_gate<true>(a, p, dq, dk, dbeta, dg, stream)
                               : by_gate<false>(a, p, dq, dk, dbeta, dg, stream);
}

}  // namespace gdr
