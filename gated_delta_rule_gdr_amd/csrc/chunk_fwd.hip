// Chunkwise prefill of the gated delta rule on gfx950 MFMA.
//
// Math (one value head, chunk of C = 64 tokens, incoming state S, value-by-key;
// section 6 of "You Could Have Come Up With Kimi Delta Attention" and section
// 4 of "From Attention to Learned Memory"). With the inclusive in-chunk
// cumulative log-decay G_i (per key channel for the channel gate):
//   R   = strict-lower( beta_i k_i^T D_{j+1:i} k_j )       key-key coefficients
//   A   = lower( s q_i^T D_{j+1:i} k_j )                    query-key coefficients
//   T   = (I + R)^-1                                        unit lower triangular
//   X   = (D_{0:i} k_i)^T S^T  rows                         prediction of the incoming state
//   Vb  = T (beta (V - X))                                  solved errors e_i
//   O   = s (D_{0:i} q_i)^T S^T + A Vb                      outputs (read after write)
//   S' = S D_{0:C-1} + sum_j e_j (D_{j+1:C-1} k_j)^T       chunk-end state
// The linear rule drops R, T and X (Vb = V, no beta).
//
// Schedule. One workgroup (4 waves) owns one (sequence, value head, block of
// 64 value columns) and walks that sequence's chunks in order; wave w owns 16
// value columns. The state S^T [DK, 16] of a wave lives in the accumulators of
// the MFMA that updates it, so it never leaves the chip between chunks: HBM
// sees q, k, v, g, beta once, o once, and the state at sequence ends only.
// Per chunk: cooperative loads into LDS; gate prefix sums; the two Gram
// matrices on MFMA; the 64x64 unit-lower inverse (forward substitution on the
// 16x16 diagonal blocks, then the block merges T21 = -T22 A21 T11 of
// section 4 of "From Attention to Learned Memory", 16 -> 32 -> 64); then each
// wave's state-dependent products on MFMA.
//
// Precision. MFMA runs on bf16 operands with fp32 accumulation. Inputs that
// are bf16 are exact operands. Every computed operand (state, T, A, the
// corrected values, decayed keys/queries, fp32 inputs) is split into
// hi = bf16(x), lo = bf16(x - hi) and multiplied as hi*hi + hi*lo + lo*hi,
// which keeps ~16 significant bits per product (a single bf16 or fp16
// rounding of these operands costs ~3e-3 of the output RMS on the 4096-token
// prefill, too much for a 3e-3 max-error budget).
//
// Scalar gate: the decay factors exp(G_i - G_j) are applied to the fp32 Gram
// entries after the MFMA, and exp(G_i), exp(G_last - G_j) to rows of fp32
// results, so no range restriction applies. Channel gate: decay sits inside
// the key contraction, so the Gram operands are e^{G} (.) q, e^{G} (.) k and
// e^{-G} (.) k with the chunk start as reference; this needs the in-chunk
// decay of every channel to stay inside the fp32 exponent range
// (|G_last - G_first| < ~80 per chunk and channel).
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16, wave64, lane l,
// r = l % 16, g = l / 16): an A fragment holds A[r][k] and a B fragment
// B[k][r] for the eight k of slot set K(g) = {4g..4g+3} u {16+4g..16+4g+3}
// of a 32-wide k step; the product pairs equal slots of A and B, so any fixed
// k labelling works as long as A and B agree. The accumulator holds
// C[4g + i][r], i = 0..3. With K(g) so chosen, two stacked 16-row accumulator
// tiles are directly the B fragment of the next product that contracts over
// those rows: no data movement between chained products.
#include <type_traits>

#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;    // tokens per chunk
constexpr int BV = 64;   // value columns per workgroup (16 per wave)

struct ChunkParams {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  void *o;
  void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t HV, ratio;
  float scale;
  int zero_init, st_bf16, out_bf16;
};

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Frag {
  bf16x8 hi, lo;
};

__device__ __forceinline__ void split8(const float (&x)[8], Frag &f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = static_cast<__bf16>(x[j]);
    f.hi[j] = h;
    f.lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
  }
}

// acc += a * b with the passes the operands need (lo terms first).
template <bool A_SPLIT, bool B_SPLIT>
__device__ __forceinline__ f32x4 mm(const Frag &a, const Frag &b, f32x4 c) {
  if constexpr (A_SPLIT) c = mfma(a.lo, b.hi, c);
  if constexpr (B_SPLIT) c = mfma(a.hi, b.lo, c);
  return mfma(a.hi, b.hi, c);
}

// Fragment of row `row`, k step starting at column col0, from a row-major LDS
// array: columns col0 + 4g + 0..3 and col0 + 16 + 4g + 0..3.
__device__ __forceinline__ void ldfrag(const uint16_t *base, int pitch, int row, int col0, int g,
                                       Frag &f) {
  const uint16_t *p = base + row * pitch + col0 + 4 * g;
  const uint2 a = *reinterpret_cast<const uint2 *>(p);
  const uint2 b = *reinterpret_cast<const uint2 *>(p + 16);
  const u32x4 u = {a.x, a.y, b.x, b.y};
  f.hi = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void ldfrag(const float *base, int pitch, int row, int col0, int g,
                                       Frag &f) {
  const float *p = base + row * pitch + col0 + 4 * g;
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 16);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split8(x, f);
}

// B fragment over 32 rows built from two stacked accumulator tiles.
__device__ __forceinline__ void chainfrag(const f32x4 &t0, const f32x4 &t1, Frag &f) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  split8(x, f);
}

// ---------------------------------------------------------------------------
// LDS layout
// ---------------------------------------------------------------------------

template <bool IN_F32, int GATE, bool DELTA, int D>
struct Smem {
  // Operand element type of the key/query arrays: bf16 when they hold exact
  // bf16 inputs, fp32 (split on load) when they hold fp32 inputs or decayed
  // (computed) values.
  static constexpr bool OPF32 = IN_F32 || GATE == GDR_GATE_CHANNEL;
  using Op = std::conditional_t<OPF32, float, uint16_t>;
  using In = std::conditional_t<IN_F32, float, uint16_t>;
  static constexpr int PK = D + (OPF32 ? 4 : 8);   // token-major rows
  static constexpr int PT = C + (OPF32 ? 4 : 8);   // key-major rows (transposed keys)
  static constexpr int PV = BV + (IN_F32 ? 4 : 8);
  static constexpr int PF = C + 4;                 // fp32 C x C
  Op kk[C][PK];   // keys (channel: e^{G} k) - A operand of X, rows of R
  Op qq[C][PK];   // queries (channel: e^{G} q)
  // Transposed keys for the state update (channel: e^{-G} k). For the channel
  // gate the same storage first holds e^{-G} k token-major for the Grams.
  union {
    Op kt[D][PT];
    Op kinv[C][PK];
  };
  In vv[C][PV];   // this workgroup's value columns
  // R then T (delta rule); during the channel-gate prep also the g staging.
  union {
    struct {
      float rt[C][PF];
      float aq[C][PF];
    };
    float gstage[C][D];
  };
  float G[C], eG[C], eGl[C], beta[C];
  float eGlastc[D];
  float eGlast;
};

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

template <bool IN_F32>
__device__ __forceinline__ void load8(const void *base, int64_t off, bool valid, float (&x)[8]) {
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
    return;
  }
  if constexpr (IN_F32) {
    const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  }
}

// Copy 8 consecutive input elements of one row into LDS unchanged.
template <bool IN_F32, class Dst>
__device__ __forceinline__ void copy8(const void *base, int64_t off, bool valid, Dst *dst) {
  if constexpr (IN_F32) {
    static_assert(std::is_same<Dst, float>::value, "fp32 input into fp32 LDS");
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (valid) {
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(base) + off);
      a = p[0];
      b = p[1];
    }
    reinterpret_cast<float4 *>(dst)[0] = a;
    reinterpret_cast<float4 *>(dst)[1] = b;
  } else {
    static_assert(std::is_same<Dst, uint16_t>::value, "bf16 input into bf16 LDS");
    uint4 u = make_uint4(0, 0, 0, 0);
    if (valid) u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
    *reinterpret_cast<uint4 *>(dst) = u;
  }
}

template <bool IN_F32, int GATE, bool DELTA, int D>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkParams p) {
  using SM = Smem<IN_F32, GATE, DELTA, D>;
  using Op = typename SM::Op;
  constexpr bool OPF32 = SM::OPF32;
  constexpr int NB = D / BV;
  constexpr int NT = D / 16;   // 16-row tiles over the key dim
  constexpr int NS = D / 32;   // 32-wide k steps over the key dim
  __shared__ SM sm;

  int b = blockIdx.x;
  const int vb = b % NB;
  b /= NB;
  const int h = b % p.HV;
  const int n = b / p.HV;
  const int hk = h / p.ratio;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int col = vb * BV + 16 * w + r;   // value column this lane owns in C tiles

  const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  const int64_t slot = p.slot_idx[n];
  const int64_t sbase = (slot * p.HV + h) * (int64_t)(D * D);

  // ---- initial state: st[m][i] = S^T[16m + 4g + i][col] ----
  f32x4 st[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e = sbase + (int64_t)(16 * m + 4 * g + i) * D + col;
      float x = 0.f;
      if (!p.zero_init)
        x = p.st_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p.pool)[e])
                      : static_cast<const float *>(p.pool)[e];
      st[m][i] = x;
    }
  }

  const int64_t HVD = (int64_t)p.HV * D;
  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int L = (int)((eos - t0) < C ? (eos - t0) : C);

    // ================= phase 0: loads =================
    // values of this workgroup's column block
    for (int it = tid; it < C * (BV / 8); it += 256) {
      const int row = it / (BV / 8), c8 = 8 * (it % (BV / 8));
      copy8<IN_F32>(p.v, (t0 + row) * p.v_stride + (int64_t)h * D + vb * BV + c8, row < L,
                    &sm.vv[row][c8]);
    }
    if constexpr (GATE != GDR_GATE_CHANNEL) {
      // keys and queries, plus transposed keys for the state update
      for (int it = tid; it < C * (D / 8); it += 256) {
        const int row = it / (D / 8), c8 = 8 * (it % (D / 8));
        const bool ok = row < L;
        copy8<IN_F32>(p.k, (t0 + row) * p.k_stride + (int64_t)hk * D + c8, ok, &sm.kk[row][c8]);
        copy8<IN_F32>(p.q, (t0 + row) * p.q_stride + (int64_t)hk * D + c8, ok, &sm.qq[row][c8]);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.kt[c8 + j][row] = sm.kk[row][c8 + j];
      }
      if (w == 0) {
        const bool ok = lane < L;
        const int64_t th = (t0 + lane) * p.HV + h;
        float gi = 0.f;
        if constexpr (GATE == GDR_GATE_SCALAR) gi = ok ? p.g[th] : 0.f;
        const float Gi = wave_scan(gi);
        const float Gl = __shfl(Gi, 63, 64);
        sm.G[lane] = Gi;
        sm.eG[lane] = __expf(Gi);
        sm.eGl[lane] = __expf(Gl - Gi);
        if (lane == 0) sm.eGlast = __expf(Gl);
        if constexpr (DELTA) sm.beta[lane] = ok ? p.beta[th] : 0.f;
      }
    } else {
      // channel gate: stage g, prefix-sum each key channel over the chunk,
      // then form e^{G} k, e^{G} q and e^{-G} k.
      for (int it = tid; it < C * (D / 4); it += 256) {
        const int row = it / (D / 4), c4 = 4 * (it % (D / 4));
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < L)
          x = *reinterpret_cast<const float4 *>(p.g + ((t0 + row) * p.HV + h) * (int64_t)D + c4);
        *reinterpret_cast<float4 *>(&sm.gstage[row][c4]) = x;
      }
      if constexpr (DELTA) {
        if (w == 0) sm.beta[lane] = lane < L ? p.beta[(t0 + lane) * p.HV + h] : 0.f;
      }
      __syncthreads();
      if (tid < D) {
        float acc = 0.f;
        for (int i = 0; i < C; ++i) {
          acc += sm.gstage[i][tid];
          sm.gstage[i][tid] = acc;
        }
        sm.eGlastc[tid] = __expf(acc);
      }
      __syncthreads();
      for (int it = tid; it < C * (D / 8); it += 256) {
        const int row = it / (D / 8), c8 = 8 * (it % (D / 8));
        const bool ok = row < L;
        float kx[8], qx[8];
        load8<IN_F32>(p.k, (t0 + row) * p.k_stride + (int64_t)hk * D + c8, ok, kx);
        load8<IN_F32>(p.q, (t0 + row) * p.q_stride + (int64_t)hk * D + c8, ok, qx);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float Gv = sm.gstage[row][c8 + j];
          const float e = __expf(Gv), ei = __expf(-Gv);
          sm.kk[row][c8 + j] = kx[j] * e;
          sm.qq[row][c8 + j] = qx[j] * e;
          if constexpr (DELTA) sm.kinv[row][c8 + j] = kx[j] * ei;
          else sm.kt[c8 + j][row] = kx[j] * ei;   // linear rule: no Gram needs kinv
        }
      }
    }
    __syncthreads();

    // ================= phase 1: Gram matrices =================
    // Lower 16x16 tiles (I >= J): KK^T feeds R (delta rule), QK^T feeds A.
    {
      constexpr int NTASK = DELTA ? 20 : 10;
      for (int task = w; task < NTASK; task += 4) {
        const bool isq = DELTA ? (task >= 10) : true;
        const int tt = DELTA ? task % 10 : task;
        int I = 0;
        while ((I + 1) * (I + 2) / 2 <= tt) ++I;
        const int J = tt - I * (I + 1) / 2;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const Op *arow = isq ? &sm.qq[0][0] : &sm.kk[0][0];
        const Op *bsrc;
        if constexpr (GATE == GDR_GATE_CHANNEL && DELTA) bsrc = &sm.kinv[0][0];
        else bsrc = &sm.kk[0][0];
        // channel gate, linear rule: B operand e^{-G} k is only held transposed
        if constexpr (GATE == GDR_GATE_CHANNEL && !DELTA) {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            Frag fa, fb;
            ldfrag(arow, SM::PK, 16 * I + r, 32 * s, g, fa);
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int kcol = 32 * s + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
              x[j] = sm.kt[kcol][16 * J + r];
            }
            split8(x, fb);
            acc = mm<true, true>(fa, fb, acc);
          }
        } else {
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            Frag fa, fb;
            ldfrag(arow, SM::PK, 16 * I + r, 32 * s, g, fa);
            ldfrag(bsrc, SM::PK, 16 * J + r, 32 * s, g, fb);
            acc = mm<OPF32, OPF32>(fa, fb, acc);
          }
        }
        const int jj = 16 * J + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ii = 16 * I + 4 * g + i;
          float gam = 1.f;
          if constexpr (GATE == GDR_GATE_SCALAR) gam = __expf(sm.G[ii] - sm.G[jj]);
          if (isq) {
            sm.aq[ii][jj] = (jj <= ii) ? p.scale * acc[i] * gam : 0.f;
          } else if constexpr (DELTA) {
            sm.rt[ii][jj] = (jj < ii) ? sm.beta[ii] * acc[i] * gam : 0.f;
          }
        }
      }
      // zero the strictly upper tiles (read by the 32-wide k steps below)
      for (int e = tid; e < 6 * 256; e += 256) {
        const int tu = e / 256, el = e % 256;
        // upper tiles (I, J), I < J: (0,1),(0,2),(0,3),(1,2),(1,3),(2,3)
        const int I = tu < 3 ? 0 : (tu < 5 ? 1 : 2);
        const int J = tu < 3 ? tu + 1 : (tu < 5 ? tu - 1 : 3);
        const int ii = 16 * I + el / 16, jj = 16 * J + el % 16;
        sm.aq[ii][jj] = 0.f;
        if constexpr (DELTA) sm.rt[ii][jj] = 0.f;
      }
    }
    __syncthreads();

    if constexpr (GATE == GDR_GATE_CHANNEL && DELTA) {
      // e^{-G} k: token-major (Gram operand) -> key-major (update operand)
      float tmp[C * D / 256];
#pragma unroll
      for (int e = 0; e < C * D / 256; ++e) {
        const int idx = tid + 256 * e;
        tmp[e] = sm.kinv[idx / D][idx % D];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < C * D / 256; ++e) {
        const int idx = tid + 256 * e;
        sm.kt[idx % D][idx / D] = tmp[e];
      }
    }

    // ================= phase 2: T = (I + R)^-1 =================
    if constexpr (DELTA) {
      if (tid < 64) {
        // forward substitution, one column of one 16x16 diagonal block per lane
        const int bb = tid >> 4, c = tid & 15, o = 16 * bb;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
          for (int j = 0; j < i; ++j) acc -= sm.rt[o + i][o + j] * x[j];
          x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.rt[o + i][o + c] = x[i];
      }
      __syncthreads();
      // merges T21 = -T22 R21 T11: 16 -> 32 (two blocks), then 32 -> 64
#pragma unroll
      for (int lvl = 0; lvl < 2; ++lvl) {
        const int nb = lvl == 0 ? 16 : 32;   // size of T11 / T22
        const int per = lvl == 0 ? 2 : 4;    // outputs per thread
        float pv[4];
        int pi[4], pj[4], po[4];
        // P = R21 T11
#pragma unroll
        for (int u = 0; u < per; ++u) {
          const int e = tid + 256 * u;
          int base, i, j;
          if (lvl == 0) { base = 32 * (e / 256); i = (e % 256) / 16; j = e % 16; }
          else { base = 0; i = e / 32; j = e % 32; }
          pi[u] = i; pj[u] = j; po[u] = base;
          float acc = 0.f;
          for (int kx = j; kx < nb; ++kx) acc += sm.rt[base + nb + i][base + kx] * sm.rt[base + kx][base + j];
          pv[u] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < per; ++u) sm.rt[po[u] + nb + pi[u]][po[u] + pj[u]] = pv[u];
        __syncthreads();
        // T21 = -T22 P
#pragma unroll
        for (int u = 0; u < per; ++u) {
          const int base = po[u], i = pi[u], j = pj[u];
          float acc = 0.f;
          for (int kx = 0; kx <= i; ++kx) acc += sm.rt[base + nb + i][base + nb + kx] * sm.rt[base + nb + kx][base + j];
          pv[u] = -acc;
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < per; ++u) sm.rt[po[u] + nb + pi[u]][po[u] + pj[u]] = pv[u];
        __syncthreads();
      }
    } else {
      __syncthreads();
    }

    // ================= phase 3: state-dependent products (per wave) =================
    // state B fragments over the key dim
    Frag sf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) chainfrag(st[2 * s], st[2 * s + 1], sf[s]);

    // value tiles of this wave: vt[I][i] = V[16I + 4g + i][col]
    f32x4 vt[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto x = sm.vv[16 * I + 4 * g + i][16 * w + r];
        if constexpr (IN_F32) vt[I][i] = x;
        else vt[I][i] = bf16_to_f32(x);
      }

    f32x4 vbar[4];   // corrected values (delta) or values (linear)
    if constexpr (DELTA) {
      // X = K_l S^T, then R_v = beta (V - X)
      f32x4 rv[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Frag fa;
          ldfrag(&sm.kk[0][0], SM::PK, 16 * I + r, 32 * s, g, fa);
          acc = mm<OPF32, true>(fa, sf[s], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ii = 16 * I + 4 * g + i;
          float x = acc[i];
          if constexpr (GATE == GDR_GATE_SCALAR) x *= sm.eG[ii];
          rv[I][i] = sm.beta[ii] * (vt[I][i] - x);
        }
      }
      // Vb = T R_v (T lower triangular: row tile I needs k steps s <= I/2)
      Frag rf[2];
      chainfrag(rv[0], rv[1], rf[0]);
      chainfrag(rv[2], rv[3], rf[1]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s <= I / 2; ++s) {
          Frag fa;
          ldfrag(&sm.rt[0][0], SM::PF, 16 * I + r, 32 * s, g, fa);
          acc = mm<true, true>(fa, rf[s], acc);
        }
        vbar[I] = acc;
      }
    } else {
#pragma unroll
      for (int I = 0; I < 4; ++I) vbar[I] = vt[I];
    }

    // O = s e^{G} (.) Q S^T + A Vb
    {
      Frag vf[2];
      chainfrag(vbar[0], vbar[1], vf[0]);
      chainfrag(vbar[2], vbar[3], vf[1]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Frag fa;
          ldfrag(&sm.qq[0][0], SM::PK, 16 * I + r, 32 * s, g, fa);
          acc = mm<OPF32, true>(fa, sf[s], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = p.scale;
          if constexpr (GATE == GDR_GATE_SCALAR) sc *= sm.eG[16 * I + 4 * g + i];
          acc[i] *= sc;
        }
#pragma unroll
        for (int s = 0; s <= I / 2; ++s) {
          Frag fa;
          ldfrag(&sm.aq[0][0], SM::PF, 16 * I + r, 32 * s, g, fa);
          acc = mm<true, (DELTA || IN_F32)>(fa, vf[s], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ii = 16 * I + 4 * g + i;
          if (ii < L) {
            const int64_t oe = (t0 + ii) * HVD + (int64_t)h * D + col;
            if (p.out_bf16) static_cast<uint16_t *>(p.o)[oe] = f32_to_bf16(acc[i]);
            else static_cast<float *>(p.o)[oe] = acc[i];
          }
        }
      }
    }

    // S^T <- decay (S^T) + K_end^T Vb
    {
      f32x4 vs[4];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = vbar[I][i];
          if constexpr (GATE == GDR_GATE_SCALAR) x *= sm.eGl[16 * I + 4 * g + i];
          vs[I][i] = x;
        }
      Frag uf[2];
      chainfrag(vs[0], vs[1], uf[0]);
      chainfrag(vs[2], vs[3], uf[1]);
      if constexpr (GATE == GDR_GATE_SCALAR) {
        const float a = sm.eGlast;
#pragma unroll
        for (int m = 0; m < NT; ++m) st[m] *= a;
      }
      constexpr bool USPLIT = DELTA || IN_F32 || GATE == GDR_GATE_SCALAR;
#pragma unroll
      for (int m = 0; m < NT; ++m) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag fa;
          ldfrag(&sm.kt[0][0], SM::PT, 16 * m + r, 32 * s, g, fa);
          st[m] = mm<OPF32, USPLIT>(fa, uf[s], st[m]);
        }
        if constexpr (GATE == GDR_GATE_CHANNEL) {
#pragma unroll
          for (int i = 0; i < 4; ++i) st[m][i] *= sm.eGlastc[16 * m + 4 * g + i];
        }
      }
    }
    __syncthreads();   // LDS is rewritten by the next chunk
  }

  // ---- final state back to the pool slot ----
#pragma unroll
  for (int m = 0; m < NT; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e = sbase + (int64_t)(16 * m + 4 * g + i) * D + col;
      if (p.st_bf16) static_cast<uint16_t *>(p.pool)[e] = f32_to_bf16(st[m][i]);
      else static_cast<float *>(p.pool)[e] = st[m][i];
    }
  }
}

template <bool IN_F32, int GATE, bool DELTA, int D>
hipError_t launch_t(const ChunkParams &p, int N, hipStream_t stream) {
  const int blocks = N * p.HV * (D / BV);
  hipLaunchKernelGGL((chunk_fwd_kernel<IN_F32, GATE, DELTA, D>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <bool IN_F32, int GATE, bool DELTA>
hipError_t by_dim(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.DK == 128) return launch_t<IN_F32, GATE, DELTA, 128>(p, a.N, s);
  return launch_t<IN_F32, GATE, DELTA, 64>(p, a.N, s);
}

template <bool IN_F32, int GATE>
hipError_t by_rule(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.rule == GDR_RULE_DELTA) return by_dim<IN_F32, GATE, true>(a, p, s);
  return by_dim<IN_F32, GATE, false>(a, p, s);
}

template <bool IN_F32>
hipError_t by_gate(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  switch (a.gate) {
    case GDR_GATE_SCALAR: return by_rule<IN_F32, GDR_GATE_SCALAR>(a, p, s);
    case GDR_GATE_CHANNEL: return by_rule<IN_F32, GDR_GATE_CHANNEL>(a, p, s);
    default: return by_rule<IN_F32, GDR_GATE_NONE>(a, p, s);
  }
}

}  // namespace

hipError_t launch_chunk_fwd(const gdr_args &a, hipStream_t stream) {
  ChunkParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  if (a.in_dtype == GDR_BF16) return by_gate<false>(a, p, stream);
  return by_gate<true>(a, p, stream);
}

}  // namespace gdr
