// Tokenwise recurrence over a ragged batch: the decode step's schedule walked
// over every token of each sequence, with the state held in registers from
// the first token to the last (the "gated_delta" Mojo page, its thread
// mapping: one block per (sequence, value head), the state column of a value
// element in registers across the whole sequence). Per token, in the order
// of that page's five steps and of the boxed KDA update:
//
//   S~ = S alpha_t | S Diag(alpha_t);  vhat = S~ k_t;  e = beta (v_t - vhat);
//   S = S~ + e k_t^T;  o_t = S (scale q_t)          (linear rule: S = S~ + v k^T)
//
// optionally with k_t and q_t L2-normalised first (x / sqrt(|x|^2 + 1e-6)),
// folded in as scalars on the reductions as the Mojo page describes, so no
// normalised array is formed. With n_h > 1 transitions per token (Gated
// DeltaProduct, "Linear attention visualized") the kernel walks the substeps
// (rows of k, v, beta) in order: a token's decay comes with its first
// substep and its output after its last.
//
// Layout on gfx950: one workgroup of 256 threads per (sequence, value head,
// 32 value columns), numbered so that all workgroups reading one key head of
// one sequence share an XCD. Lane (w, l) owns value column 8w + l / 8 of the block
// and key group l % 8 (D / 8 consecutive keys), so the state S^T[keys,
// column] sits in D / 8 registers per lane. A reduction over the keys is the
// sum over the 8 lanes of a column: three DPP steps inside an 8-lane group
// (quad swaps, then the half-row mirror), with no LDS and no barrier.
//
// Inputs arrive in blocks of 64 tokens: the workgroup copies a block's keys,
// queries, value columns, gates and beta into LDS with coalesced 16-byte
// loads, and while the 64 tokens run from LDS the next block's loads are in
// flight in registers, so the serial per-token chain never waits on HBM.
// Outputs collect in LDS and leave as whole rows after each block; the state
// tile enters and leaves through LDS as coalesced rows as well.
#include <cstdint>
#include <type_traits>

#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int VB = 32;   // value columns per workgroup
constexpr int KG = 8;    // lanes (key groups) per value column
constexpr float L2_EPS = 1e-6f;

// (Vector types, not arrays: a block's loads stay in registers.)
template <int N>
struct U32VecR {
  typedef unsigned int type __attribute__((ext_vector_type(N)));
};
template <class Vec>
__device__ __forceinline__ void putv(Vec &v, int u, const uint4 x) {
  v[4 * u] = x.x; v[4 * u + 1] = x.y; v[4 * u + 2] = x.z; v[4 * u + 3] = x.w;
}
template <class Vec>
__device__ __forceinline__ uint4 getv(const Vec &v, int u) {
  return make_uint4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
}

struct RecParams {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  void *o;
  void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t N, HV, ratio;
  float scale;
  int zero_init, st_bf16, out_bf16;
  int32_t P;   // transitions per token: key, value and beta rows per q, g, o row
  float *ring; // (verify) records [T, HV, E]: e (D), k (D), the gate (G), padding
  int32_t E;   // record stride in floats (a multiple of 4)
};

// Sum over the 8 lanes of a key-group set: every lane of the group gets it.
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_perm<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_perm<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_perm<0x141>(x);   // row_half_mirror: the other quad of the 8
  return x;
}

constexpr int TB = 32;   // tokens staged per block

// LDS of one workgroup: a block of TB tokens' inputs, widened to fp32 once
// on the way in (keys, queries, this workgroup's value columns, gates, beta),
// and the block's outputs. The state tile passes through the key and query
// arrays at the sequence's start and end.
template <int GATE, int D>
struct RecSmem {
  static constexpr int KP = D + 4;   // row pitch: the 8 key groups of a row are contiguous
  static constexpr int GP = GATE == GDR_GATE_CHANNEL ? D + 4 : 4;
  union {
    struct {
      alignas(16) float kk[TB][KP];
      alignas(16) float qq[TB][KP];
    } tk;
    alignas(16) float st[D][VB + 4];   // state tile S^T[keys][block columns]
  };
  alignas(16) float vv[TB][VB + 4];
  alignas(16) float gg[TB][GP];
  alignas(16) float oo[TB][VB + 4];
  float bb[TB];
};

// A block's inputs in flight, per thread: 16-byte units of keys and queries
// (KU each), of values (VU), of channel gates (GU), and one float of the
// scalar gate and of beta (threads below TB).
template <bool IN_F32, int GATE, int D>
struct RecPre {
  static constexpr int ES = IN_F32 ? 4 : 2;
  static constexpr int KU = TB * D * ES / 16 / 256;
  static constexpr int VU = (TB * VB * ES / 16 + 255) / 256;
  static constexpr int GU = GATE == GDR_GATE_CHANNEL ? TB * D * 4 / 16 / 256 : 0;
  typename U32VecR<4 * KU>::type k, q;
  typename U32VecR<4 * VU>::type v;
  typename U32VecR<4 * (GU > 0 ? GU : 1)>::type g;
  float gs, beta;
};

// Rows m0 .. m0 + Lv - 1 of k, v and beta (substeps; tokens when P = 1) and
// rows r0 .. r0 + Lq - 1 of q and g (tokens), each clamped to its last row.
template <bool IN_F32, int GATE, bool DELTA, int D>
__device__ __forceinline__ void block_load(RecPre<IN_F32, GATE, D> &pf, const RecParams &p, int64_t m0,
                                           int Lv, int64_t r0, int Lq, int h, int hk, int vb, int tid) {
  using PF = RecPre<IN_F32, GATE, D>;
  constexpr int ES = PF::ES;
  constexpr int KRU = D * ES / 16;       // units per key row
  const char *kb = static_cast<const char *>(p.k) + (m0 * p.k_stride + (int64_t)hk * D) * ES;
  const char *qb = static_cast<const char *>(p.q) + (r0 * p.q_stride + (int64_t)hk * D) * ES;
#pragma unroll
  for (int u = 0; u < PF::KU; ++u) {
    const int e = tid + 256 * u, c = e % KRU;
    const int kr = min(e / KRU, Lv - 1), qr = min(e / KRU, Lq - 1);
    putv(pf.k, u, *reinterpret_cast<const uint4 *>(kb + (int64_t)kr * p.k_stride * ES + 16 * c));
    putv(pf.q, u, *reinterpret_cast<const uint4 *>(qb + (int64_t)qr * p.q_stride * ES + 16 * c));
  }
  constexpr int VRU = VB * ES / 16;      // units per value row
  const char *vbp = static_cast<const char *>(p.v) + (m0 * p.v_stride + (int64_t)h * D + vb * VB) * ES;
#pragma unroll
  for (int u = 0; u < PF::VU; ++u) {
    const int e = tid + 256 * u, row = min(e / VRU, Lv - 1), c = e % VRU;
    if (e < TB * VRU) putv(pf.v, u, *reinterpret_cast<const uint4 *>(vbp + (int64_t)row * p.v_stride * ES + 16 * c));
  }
  if constexpr (GATE == GDR_GATE_CHANNEL) {
    constexpr int GRU = D * 4 / 16;
    const float *gb = p.g + (r0 * p.HV + h) * (int64_t)D;
#pragma unroll
    for (int u = 0; u < PF::GU; ++u) {
      const int e = tid + 256 * u, row = min(e / GRU, Lq - 1), c = e % GRU;
      putv(pf.g, u, *reinterpret_cast<const uint4 *>(gb + (int64_t)row * p.HV * D + 4 * c));
    }
  }
  if (tid < TB) {
    pf.gs = GATE == GDR_GATE_SCALAR ? p.g[(r0 + min(tid, Lq - 1)) * p.HV + h] : 0.f;
    pf.beta = DELTA ? p.beta[(m0 + min(tid, Lv - 1)) * p.HV + h] : 0.f;
  }
}

// A 16-byte unit of inputs into LDS as fp32: 8 bf16 values (two float4) or
// 4 fp32 values.
template <bool IN_F32>
__device__ __forceinline__ void put_unit(float *dst, const uint4 x) {
  if constexpr (IN_F32) {
    *reinterpret_cast<uint4 *>(dst) = x;
  } else {
    *reinterpret_cast<float4 *>(dst) = make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
                                                   __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    *reinterpret_cast<float4 *>(dst + 4) = make_float4(__uint_as_float(x.z << 16), __uint_as_float(x.z & 0xffff0000u),
                                                       __uint_as_float(x.w << 16), __uint_as_float(x.w & 0xffff0000u));
  }
}

template <bool IN_F32, int GATE, bool DELTA, int D>
__device__ __forceinline__ void block_store(const RecPre<IN_F32, GATE, D> &pf, RecSmem<GATE, D> &sm, int tid) {
  using PF = RecPre<IN_F32, GATE, D>;
  constexpr int ES = PF::ES;
  constexpr int UE = 16 / ES;            // elements per unit
  constexpr int KRU = D / UE;
#pragma unroll
  for (int u = 0; u < PF::KU; ++u) {
    const int e = tid + 256 * u, row = e / KRU, c = e % KRU;
    put_unit<IN_F32>(&sm.tk.kk[row][UE * c], getv(pf.k, u));
    put_unit<IN_F32>(&sm.tk.qq[row][UE * c], getv(pf.q, u));
  }
  constexpr int VRU = VB / UE;
#pragma unroll
  for (int u = 0; u < PF::VU; ++u) {
    const int e = tid + 256 * u, row = e / VRU, c = e % VRU;
    if (e < TB * VRU) put_unit<IN_F32>(&sm.vv[row][UE * c], getv(pf.v, u));
  }
  if constexpr (GATE == GDR_GATE_CHANNEL) {
    constexpr int GRU = D * 4 / 16;
#pragma unroll
    for (int u = 0; u < PF::GU; ++u) {
      const int e = tid + 256 * u, row = e / GRU, c = e % GRU;
      *reinterpret_cast<uint4 *>(&sm.gg[row][4 * c]) = getv(pf.g, u);
    }
  }
  if (tid < TB) {
    if constexpr (GATE == GDR_GATE_SCALAR) sm.gg[tid][0] = pf.gs;
    if constexpr (DELTA) sm.bb[tid] = pf.beta;
  }
}

// One token's operands for one lane, read from LDS: its NK keys and queries,
// its value, its gate (NK channel gates, or the scalar) and beta.
template <int GATE, int NK>
struct TokOps {
  float k[NK], q[NK];
  float g[GATE == GDR_GATE_CHANNEL ? NK : 1];
  float v, beta;
};

// PROD: more than one transition per token (P > 1); without it every
// substep is a token and the substep bookkeeping compiles away.
// RING: the verify of a speculative window: the pool is read, never written,
// and every token's update is recorded as e (per value column), the key it
// is written along (normalised when L2) and its gate, so that a later fold
// applies S <- S~ + e k^T for the accepted tokens.
template <bool IN_F32, int GATE, bool DELTA, bool L2, bool PROD, bool RING, int D>
__global__ __launch_bounds__(256) void recurrent_fwd_kernel(RecParams p) {
  using SM = RecSmem<GATE, D>;
  using PF = RecPre<IN_F32, GATE, D>;
  using Ops = TokOps<GATE, D / KG>;
  constexpr int NK = D / KG;             // keys per lane
  constexpr int NVB = D / VB;
  __shared__ SM sm;
  // Workgroups go round-robin over the 8 XCDs (each with its own L2). The
  // ratio * NVB workgroups that read one key head of one sequence get ids
  // equal modulo 8, so they run on one XCD and share those reads.
  const int HK = p.HV / p.ratio;
  const int GRP = p.ratio * NVB;                 // workgroups per (sequence, key head)
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7);  // (sequence, key head) group
  if (gi >= p.N * HK) return;                    // padding of the last XCD round
  const int jg = (b >> 3) % GRP;
  const int n = gi / HK;
  const int hk = gi - n * HK;
  const int h = hk * p.ratio + jg / NVB;
  const int vb = jg % NVB;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int kg = lane & (KG - 1);
  const int vl = 8 * w + (lane >> 3);    // value column within the block
  const int col = vb * VB + vl;
  const int k0 = kg * NK;                // first key of this lane

  const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  // the workgroup's state tile: row k of S^T, columns vb*VB .. +VB-1
  const int64_t tbase = ((int64_t)p.slot_idx[n] * p.HV + h) * (int64_t)(D * D) + vb * VB;
  const int sw = p.st_bf16 ? 2 : 4;
  const int RU = VB * sw / 16;           // 16-byte units per tile row
  char *pool = static_cast<char *>(p.pool);

  if (bos == eos) {
    // a zero-length sequence under ZERO_INIT writes its zero state back
    if (!RING && p.zero_init)
      for (int e = tid; e < D * RU; e += 256)
        *reinterpret_cast<uint4 *>(pool + (tbase + (int64_t)(e / RU) * D) * sw + 16 * (e % RU)) =
            make_uint4(0, 0, 0, 0);
    return;
  }

  // state in, coalesced through LDS: s[j] = S^T[k0 + j][col]
  float s[NK];
  if (p.zero_init) {
#pragma unroll
    for (int j = 0; j < NK; ++j) s[j] = 0.f;
  } else {
    for (int e = tid; e < D * RU; e += 256) {
      const uint4 x = *reinterpret_cast<const uint4 *>(pool + (tbase + (int64_t)(e / RU) * D) * sw + 16 * (e % RU));
      const int row = e / RU, c0 = (e % RU) * (16 / sw);
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
      if (p.st_bf16) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          sm.st[row][c0 + i] = __uint_as_float((i & 1) ? (xw[i >> 1] & 0xffff0000u) : (xw[i >> 1] << 16));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.st[row][c0 + i] = __uint_as_float(xw[i]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NK; ++j) s[j] = sm.st[k0 + j][vl];
  }

  // Blocks run over substeps: sequence n's token t has substeps t*P .. t*P+P-1
  // (rows of k, v, beta); q, g and o have one row per token.
  const int P = PROD ? p.P : 1;
  const int64_t HVD = (int64_t)p.HV * D;
  const int64_t bosv = bos * P, eosv = eos * P;
  const int nblk = (int)((eosv - bosv + TB - 1) / TB);
  PF pf;
  auto load_block = [&](int64_t m0) {
    const int64_t r0 = m0 / P;
    block_load<IN_F32, GATE, DELTA, D>(pf, p, m0, (int)min<int64_t>(TB, eosv - m0), r0,
                                       (int)min<int64_t>(TB, eos - r0), h, hk, vb, tid);
  };
  load_block(bosv);
  for (int blk = 0; blk < nblk; ++blk) {
    const int64_t m0 = bosv + (int64_t)blk * TB;   // first substep of the block
    const int64_t r0 = m0 / P;                      // its token: row 0 of q, g, o
    const int L = (int)min<int64_t>(TB, eosv - m0);
    __syncthreads();   // the previous block (or the state tile) is consumed
    block_store<IN_F32, GATE, DELTA, D>(pf, sm, tid);
    __syncthreads();
    if (blk + 1 < nblk) load_block(m0 + TB);

    // operands of substep i (k, v, beta row i) of token row r (q, g row r);
    // rows past the block's end hold copies of its last row
    auto read = [&](int i, int r, Ops &t) {
#pragma unroll
      for (int j = 0; j < NK; j += 4) {
        const float4 a = *reinterpret_cast<const float4 *>(&sm.tk.kk[i][k0 + j]);
        const float4 c = *reinterpret_cast<const float4 *>(&sm.tk.qq[r][k0 + j]);
        t.k[j] = a.x; t.k[j + 1] = a.y; t.k[j + 2] = a.z; t.k[j + 3] = a.w;
        t.q[j] = c.x; t.q[j + 1] = c.y; t.q[j + 2] = c.z; t.q[j + 3] = c.w;
      }
      if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
        for (int j = 0; j < NK; j += 4) {
          const float4 gv = *reinterpret_cast<const float4 *>(&sm.gg[r][k0 + j]);
          t.g[j] = gv.x; t.g[j + 1] = gv.y; t.g[j + 2] = gv.z; t.g[j + 3] = gv.w;
        }
      } else {
        t.g[0] = sm.gg[r][0];
      }
      t.v = sm.vv[i][vl];
      t.beta = DELTA ? sm.bb[i] : 0.f;
    };
    // (verify) token row r's record: e for this lane's column, and from the
    // first column of the first block the key times rk and the gate
    auto record = [&](int r, float er, float rk, const Ops &t) {
      float *rec = p.ring + ((r0 + r) * p.HV + h) * (int64_t)p.E;
      if (kg == 0) rec[col] = er;
      if (vb == 0 && vl == 0) {
#pragma unroll
        for (int j = 0; j < NK; ++j) rec[D + k0 + j] = t.k[j] * rk;
        if constexpr (GATE == GDR_GATE_SCALAR) {
          if (kg == 0) rec[2 * D] = t.g[0];
        } else if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
          for (int j = 0; j < NK; ++j) rec[2 * D + k0 + j] = t.g[j];
        }
      }
    };
    // one substep of the recurrence on the lane's NK state entries: the
    // token's decay on its first substep (js == 0), its output on its last
    auto step = [&](int js, int r, const Ops &t) {
      // L2 norms of k and q (as scalars on the reductions)
      float rk = 1.f, rq = 1.f;
      if constexpr (L2) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          a = fmaf(t.k[j], t.k[j], a);
          c = fmaf(t.q[j], t.q[j], c);
        }
        rk = rsqrtf(sum8(a) + L2_EPS);
        rq = rsqrtf(sum8(c) + L2_EPS);
      }
      // 1. decay
      if (!PROD || js == 0) {
        if constexpr (GATE == GDR_GATE_SCALAR) {
          const float al = __expf(t.g[0]);
#pragma unroll
          for (int j = 0; j < NK; ++j) s[j] *= al;
        } else if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
          for (int j = 0; j < NK; ++j) s[j] *= __expf(t.g[j]);
        }
      }
      if constexpr (DELTA) {
        // 2-4. prediction from the decayed state, error, rank-one write
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int j = 0; j < NK; j += 2) {
          a0 = fmaf(s[j], t.k[j], a0);
          a1 = fmaf(s[j + 1], t.k[j + 1], a1);
        }
        const float vhat = sum8(a0 + a1) * rk;
        const float er = t.beta * (t.v - vhat);
        const float e = er * rk;
#pragma unroll
        for (int j = 0; j < NK; ++j) s[j] = fmaf(e, t.k[j], s[j]);
        if constexpr (RING) record(r, er, rk, t);
      } else {
        const float e = t.v * rk;
#pragma unroll
        for (int j = 0; j < NK; ++j) s[j] = fmaf(e, t.k[j], s[j]);
        if constexpr (RING) record(r, t.v, rk, t);
      }
      // 5. read after the write (after the token's last substep)
      if (!PROD || js == P - 1) {
        float b0 = 0.f, b1 = 0.f;
#pragma unroll
        for (int j = 0; j < NK; j += 2) {
          b0 = fmaf(s[j], t.q[j], b0);
          b1 = fmaf(s[j + 1], t.q[j + 1], b1);
        }
        const float o = sum8(b0 + b1) * (p.scale * rq);
        if (kg == 0) sm.oo[r][vl] = o;
      }
    };
    // two operand sets in turn: substep i + 1's LDS reads are in flight while
    // substep i computes. (js, r): substep within its token, token row.
    auto next = [&](int &js, int &r) {
      if (!PROD) {
        ++r;
      } else if (++js == P) {
        js = 0;
        ++r;
      }
    };
    int js = (int)(m0 - r0 * P), r = 0;
    Ops ta, tb;
    read(0, 0, ta);
    for (int i = 0; i < L; i += 2) {
      int js1 = js, r1 = r;
      next(js1, r1);
      read(min(i + 1, TB - 1), min(r1, TB - 1), tb);
      step(js, r, ta);
      if (i + 1 == L) break;
      int js2 = js1, r2 = r1;
      next(js2, r2);
      read(min(i + 2, TB - 1), min(r2, TB - 1), ta);
      step(js1, r1, tb);
      js = js2;
      r = r2;
    }
    __syncthreads();
    // the block's outputs, coalesced: the tokens whose last substep is in
    // this block, rows r0 .. (m0 + L) / P - 1, this workgroup's VB columns
    const int ow = p.out_bf16 ? 2 : 4;
    const int ORU = VB * ow / 16;
    const int Lo = (int)((m0 + L) / P - r0);
    char *ob = static_cast<char *>(p.o) + (r0 * HVD + (int64_t)h * D + vb * VB) * ow;
    for (int e = tid; e < Lo * ORU; e += 256) {
      const int row = e / ORU, c0 = (e % ORU) * (16 / ow);
      uint4 x;
      if (p.out_bf16) {
        uint32_t xw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          xw[m] = (uint32_t)f32_to_bf16(sm.oo[row][c0 + 2 * m]) | ((uint32_t)f32_to_bf16(sm.oo[row][c0 + 2 * m + 1]) << 16);
        x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
      } else {
        x = make_uint4(__float_as_uint(sm.oo[row][c0]), __float_as_uint(sm.oo[row][c0 + 1]),
                       __float_as_uint(sm.oo[row][c0 + 2]), __float_as_uint(sm.oo[row][c0 + 3]));
      }
      *reinterpret_cast<uint4 *>(ob + (int64_t)row * HVD * ow + 16 * (e % ORU)) = x;
    }
  }

  // state out, coalesced through LDS (RNE to a bf16 pool); a verify leaves
  // the pool as it was
  if constexpr (RING) return;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NK; ++j) sm.st[k0 + j][vl] = s[j];
  __syncthreads();
  for (int e = tid; e < D * RU; e += 256) {
    const int row = e / RU, c0 = (e % RU) * (16 / sw);
    uint4 x;
    if (p.st_bf16) {
      uint32_t xw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xw[m] = (uint32_t)f32_to_bf16(sm.st[row][c0 + 2 * m]) | ((uint32_t)f32_to_bf16(sm.st[row][c0 + 2 * m + 1]) << 16);
      x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
    } else {
      x = make_uint4(__float_as_uint(sm.st[row][c0]), __float_as_uint(sm.st[row][c0 + 1]),
                     __float_as_uint(sm.st[row][c0 + 2]), __float_as_uint(sm.st[row][c0 + 3]));
    }
    *reinterpret_cast<uint4 *>(pool + (tbase + (int64_t)row * D) * sw + 16 * (e % RU)) = x;
  }
}

template <bool IN_F32, int GATE, bool DELTA, bool L2, bool PROD, bool RING>
hipError_t by_dim(const gdr_args &a, const RecParams &p, hipStream_t st) {
  // one XCD round covers 8 (sequence, key head) groups
  const int blocks = ((a.N * a.HK + 7) / 8) * 8 * (a.HV / a.HK) * (a.DK / VB);
  if (a.DK == 128) {
    hipLaunchKernelGGL((recurrent_fwd_kernel<IN_F32, GATE, DELTA, L2, PROD, RING, 128>), dim3(blocks), dim3(256), 0,
                       st, p);
  } else {
    hipLaunchKernelGGL((recurrent_fwd_kernel<IN_F32, GATE, DELTA, L2, PROD, RING, 64>), dim3(blocks), dim3(256), 0,
                       st, p);
  }
  return hipGetLastError();
}

template <bool IN_F32, int GATE, bool DELTA, bool L2>
hipError_t by_prod(const gdr_args &a, const RecParams &p, hipStream_t st) {
  if (p.ring) return by_dim<IN_F32, GATE, DELTA, L2, false, true>(a, p, st);   // (one transition)
  if (p.P > 1) return by_dim<IN_F32, GATE, DELTA, L2, true, false>(a, p, st);
  return by_dim<IN_F32, GATE, DELTA, L2, false, false>(a, p, st);
}

template <bool IN_F32, int GATE, bool DELTA>
hipError_t by_norm(const gdr_args &a, const RecParams &p, hipStream_t st) {
  if (a.flags & GDR_FLAG_QK_L2NORM) return by_prod<IN_F32, GATE, DELTA, true>(a, p, st);
  return by_prod<IN_F32, GATE, DELTA, false>(a, p, st);
}

template <bool IN_F32, int GATE>
hipError_t by_rule(const gdr_args &a, const RecParams &p, hipStream_t st) {
  if (a.rule == GDR_RULE_DELTA) return by_norm<IN_F32, GATE, true>(a, p, st);
  return by_norm<IN_F32, GATE, false>(a, p, st);
}

template <bool IN_F32>
hipError_t by_gate(const gdr_args &a, const RecParams &p, hipStream_t st) {
  switch (a.gate) {
    case GDR_GATE_SCALAR: return by_rule<IN_F32, GDR_GATE_SCALAR>(a, p, st);
    case GDR_GATE_CHANNEL: return by_rule<IN_F32, GDR_GATE_CHANNEL>(a, p, st);
    default: return by_rule<IN_F32, GDR_GATE_NONE>(a, p, st);
  }
}

// Fold of a verify's accepted records: for sequence n, S <- S~ + e k^T with
// the records of its first accepted[n] window tokens (clamped to the window),
// in order, on pool slot slot_idx[n]. One workgroup per (sequence, value
// head, 32 value columns), the lane layout of the recurrence above; the
// state tile enters and leaves through LDS as coalesced rows.
struct FoldParams {
  const float *ring;
  const int32_t *accepted;
  void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t HV, E;
  int st_bf16;
};

template <int GATE, int D>
__global__ __launch_bounds__(256) void state_fold_kernel(FoldParams p) {
  constexpr int NK = D / KG, NVB = D / VB;
  __shared__ float st[D][VB + 4];
  const int b = blockIdx.x;
  const int vb = b % NVB, nh = b / NVB;
  const int n = nh / p.HV, h = nh - n * p.HV;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int kg = lane & (KG - 1), vl = 8 * w + (lane >> 3), col = vb * VB + vl, k0 = kg * NK;
  const int64_t bos = p.cu_seqlens[n];
  const int64_t len = p.cu_seqlens[n + 1] - bos;
  const int acc = (int)max<int64_t>(0, min<int64_t>(p.accepted[n], len));
  if (acc == 0) return;   // (uniform) nothing accepted: the state stays

  const int64_t tbase = ((int64_t)p.slot_idx[n] * p.HV + h) * (int64_t)(D * D) + vb * VB;
  const int sw = p.st_bf16 ? 2 : 4, RU = VB * sw / 16;
  char *pool = static_cast<char *>(p.pool);
  for (int e = tid; e < D * RU; e += 256) {
    const uint4 x = *reinterpret_cast<const uint4 *>(pool + (tbase + (int64_t)(e / RU) * D) * sw + 16 * (e % RU));
    const int row = e / RU, c0 = (e % RU) * (16 / sw);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
    if (p.st_bf16) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        st[row][c0 + i] = __uint_as_float((i & 1) ? (xw[i >> 1] & 0xffff0000u) : (xw[i >> 1] << 16));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[row][c0 + i] = __uint_as_float(xw[i]);
    }
  }
  __syncthreads();
  float s[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) s[j] = st[k0 + j][vl];

  for (int t = 0; t < acc; ++t) {
    const float *rec = p.ring + ((bos + t) * p.HV + h) * (int64_t)p.E;
    const float e = rec[col];
    float kx[NK];
#pragma unroll
    for (int j = 0; j < NK; j += 4) {
      const float4 k4 = *reinterpret_cast<const float4 *>(rec + D + k0 + j);
      kx[j] = k4.x; kx[j + 1] = k4.y; kx[j + 2] = k4.z; kx[j + 3] = k4.w;
    }
    if constexpr (GATE == GDR_GATE_SCALAR) {
      const float al = __expf(rec[2 * D]);
#pragma unroll
      for (int j = 0; j < NK; ++j) s[j] = fmaf(e, kx[j], s[j] * al);
    } else if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
      for (int j = 0; j < NK; ++j) s[j] = fmaf(e, kx[j], s[j] * __expf(rec[2 * D + k0 + j]));
    } else {
#pragma unroll
      for (int j = 0; j < NK; ++j) s[j] = fmaf(e, kx[j], s[j]);
    }
  }

  __syncthreads();
#pragma unroll
  for (int j = 0; j < NK; ++j) st[k0 + j][vl] = s[j];
  __syncthreads();
  for (int e = tid; e < D * RU; e += 256) {
    const int row = e / RU, c0 = (e % RU) * (16 / sw);
    uint4 x;
    if (p.st_bf16) {
      uint32_t xw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        xw[m] = (uint32_t)f32_to_bf16(st[row][c0 + 2 * m]) | ((uint32_t)f32_to_bf16(st[row][c0 + 2 * m + 1]) << 16);
      x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
    } else {
      x = make_uint4(__float_as_uint(st[row][c0]), __float_as_uint(st[row][c0 + 1]),
                     __float_as_uint(st[row][c0 + 2]), __float_as_uint(st[row][c0 + 3]));
    }
    *reinterpret_cast<uint4 *>(pool + (tbase + (int64_t)row * D) * sw + 16 * (e % RU)) = x;
  }
}

template <int GATE>
hipError_t fold_by_dim(const gdr_args &a, const FoldParams &p, hipStream_t st) {
  const unsigned blocks = (unsigned)(a.N * a.HV * (a.DK / VB));
  if (a.DK == 128) hipLaunchKernelGGL((state_fold_kernel<GATE, 128>), dim3(blocks), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((state_fold_kernel<GATE, 64>), dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace

int ring_record_elements(const gdr_args &a) {
  return a.DV + a.DK + (a.gate == GDR_GATE_SCALAR ? 1 : a.gate == GDR_GATE_CHANNEL ? a.DK : 0);
}
int ring_record_stride(const gdr_args &a) { return (ring_record_elements(a) + 3) & ~3; }

hipError_t launch_state_fold(const gdr_args &a, const float *ring, const int32_t *accepted, hipStream_t stream) {
  FoldParams p;
  p.ring = ring; p.accepted = accepted;
  p.pool = a.state_pool; p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.HV = a.HV; p.E = ring_record_stride(a);
  p.st_bf16 = a.state_dtype == GDR_BF16;
  if (a.gate == GDR_GATE_SCALAR) return fold_by_dim<GDR_GATE_SCALAR>(a, p, stream);
  if (a.gate == GDR_GATE_CHANNEL) return fold_by_dim<GDR_GATE_CHANNEL>(a, p, stream);
  return fold_by_dim<GDR_GATE_NONE>(a, p, stream);
}

hipError_t launch_recurrent_fwd(const gdr_args &a, hipStream_t stream, float *ring) {
  RecParams p;
  p.ring = ring;
  p.E = ring_record_stride(a);
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.P = products_of(a);
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  if (a.in_dtype == GDR_BF16) return by_gate<false>(a, p, stream);
  return by_gate<true>(a, p, stream);
}

}  // namespace gdr
