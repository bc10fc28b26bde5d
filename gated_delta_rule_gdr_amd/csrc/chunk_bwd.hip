// Chunkwise backward of the gated delta rule (scalar gate or none): the
// reverse-mode gradient of the chunk equations, regrouped the way "From
// Attention to Learned Memory" regroups the linear-attention backward
// (section "Backward: reverse the boundary scan, then differentiate each
// chunk"): one scan of the state's gradient over the chunk boundaries, from
// the last chunk back, then every chunk differentiated on its own.
//
// Forward chunk (C = 64 tokens, incoming state S_c as S^T [DK, DV], G the
// in-chunk cumulative log-decay, gamma_i = e^{G_i}, Gamma_ij = e^{G_i - G_j}
// for j <= i, s the query scale; the chunk equations of "You Could Have Come
// Up With Kimi Delta Attention", section 6, with a scalar gate):
//   K_l = gamma (.) K,  Q_l = gamma (.) Q,  K_e = e^{G_last - G} (.) K
//   R  = strict-lower( beta_i Gamma_ij k_i.k_j ),  T = (I + R)^{-1}
//   A  = lower( s Gamma_ij q_i.k_j )
//   X  = K_l S^T,  Rv = beta (.) (V - X),  E = T Rv
//   O  = s Q_l S^T + A E
//   S^T_{c+1} = e^{G_last} S^T_c + K_e^T E
// Backward, with dS^T_{c+1} the gradient of the state after the chunk and
// dO the outputs' gradient:
//   dE  = A^T dO + K_e dS^T_{c+1},  dRv = T^T dE,  dV = beta (.) dRv
//   dX  = -beta (.) dRv,  dA = dO E^T (lower),  dR = -dRv E^T (strict lower)
//   dQ_l = s dO S,  dK_l = dX S,  dK_e = E dS_{c+1}
//   dS^T_c = e^{G_last} dS^T_{c+1} + K_l^T dX + s Q_l^T dO = M dS^T_{c+1} + Y
// with W = T Diag(beta) K_l, M = e^{G_last} I - W^T K_e (the transpose of
// the linear part of the forward map S^T_c -> S^T_{c+1}, as the adjoint of a
// linear map must be) and Y = (s Q_l - A W)^T dO. Through the Gram matrices (KK = K K^T, QK = Q K^T):
//   P_R = dR (.) beta_i Gamma_ij,  P_A = dA (.) s Gamma_ij
//   dk = P_R K + P_R^T K + P_A^T Q + gamma (.) dK_l + e^{G_last - G} (.) dK_e
//   dq = P_A K + gamma (.) dQ_l
//   dbeta_i = sum_v (V - X)_iv dRv_iv + sum_j dR_ij Gamma_ij k_i.k_j
//   dG_i = rowsum_i(N) - colsum_i(N) + gamma_i (k_i.dK_l,i + q_i.dQ_l,i)
//          - e^{G_last - G_i} k_i.dK_e,i   (N = dR (.) R + dA (.) A)
//   dG_last += sum_j e^{G_last - G_j} k_j.dK_e,j + e^{G_last} <dS_{c+1}, S_c>
//   dg_t = sum_{i >= t} dG_i over the chunk (G is a prefix sum of g).
//
// Kernels, in order:
//   1. a prefill kernel in its checkpointing form: S^T_c at every chunk start
//      (bf16 inputs: the warp-specialised kernel, on a scratch copy of the
//      initial states and with scratch outputs; fp32 inputs: the general
//      kernel, which writes neither);
//   2. bwd_prep_kernel, one workgroup of eight waves per (chunk, value head):
//      the Grams, T, W and the reverse map's M and Y, written as fp32
//      [DK, DK] / [DK, DV];
//   3. bwd_walk_kernel, one workgroup per (sequence, value head, 16 value
//      columns): dS^T from zero at the sequence end back to the start,
//      dS^T_{c+1} stored per chunk; the last one is the initial state's
//      gradient;
//   4. bwd_grad_kernel, one workgroup of eight waves per (chunk, value head):
//      the formulas above, over 16-column blocks of the value dimension, dq
//      and dk per value head in fp32;
//   5. bwd_group_sum_kernel: dq and dk summed over each key head's group of
//      value heads, in the output dtype (with one value head per key head
//      the gradient kernel writes them directly instead).
// Everything is fp32: the matrix products on v_mfma_f32_16x16x4_f32 with
// operands from LDS (or, in the walk, from memory), fp32 accumulation.
#include <cstdint>

#include "chunk_common.h"

namespace gdr {
namespace {

using chunk::f32x4;
constexpr int CB = 64;        // tokens per chunk
constexpr int PC = CB + 4;    // pitch of the C x C matrices in LDS
constexpr int BW = 16;        // value columns per block of the gradient kernel
constexpr int PB = BW + 4;    // pitch of those blocks

__device__ __forceinline__ f32x4 mf(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc (one 16 x 16 tile) += A (16 x 4n) B (4n x 16), n a multiple of 4.
// A's element (i, k) is a[i * ai + k * ak], B's element (k, j) is
// b[k * bk + j * bj]. The k range is taken in blocks of 16, four MFMAs each:
// at step j of a block lane (r, g) supplies A(r, k) and B(k, r) for
// k = 16 blk + 4g + j (any assignment of the k's to steps gives the same
// sum as long as A and B agree), so that a lane's four A values (four B
// values) of a block are adjacent in memory when ak == 1 (bk == 1): one
// 16-byte read. The tile's element (4g + e, r) is acc[e].
template <bool AK1, bool BK1>
__device__ __forceinline__ f32x4 mm(const float *a, int ai, int ak, const float *b, int bk, int bj, int n,
                                    f32x4 acc, int r, int g) {
  const float *pa = a + r * ai + 4 * g * (AK1 ? 1 : ak);
  const float *pb = b + 4 * g * (BK1 ? 1 : bk) + r * bj;
  const int sa = 16 * (AK1 ? 1 : ak), sb = 16 * (BK1 ? 1 : bk);
#pragma unroll 2
  for (int s = 0; s < n; s += 4) {
    float av[4], bv[4];
    if constexpr (AK1) {
      const float4 x = *reinterpret_cast<const float4 *>(pa);
      av[0] = x.x; av[1] = x.y; av[2] = x.z; av[3] = x.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = pa[j * ak];
    }
    if constexpr (BK1) {
      const float4 x = *reinterpret_cast<const float4 *>(pb);
      bv[0] = x.x; bv[1] = x.y; bv[2] = x.z; bv[3] = x.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = pb[j * bk];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mf(av[j], bv[j], acc);
    pa += sa;
    pb += sb;
  }
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <bool BF16>
__device__ __forceinline__ float ld_in(const void *p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  else return static_cast<const float *>(p)[i];
}

struct BwdParams {
  const void *q, *k, *v, *dout;
  int64_t q_stride, k_stride, v_stride;   // elements between tokens (dout: HV * D)
  const float *g, *beta;
  const int32_t *cu_seqlens;
  int32_t N, HK, HV, ratio;
  float scale;
  int gated, out_bf16;
  int64_t flat;                           // flat chunk indices: [0, flat)
  const float *ckf;                       // S^T_c per (flat chunk, value head)
  float *ckb;                             // dS^T_{c+1} per (flat chunk, value head)
  float *M, *Y;                           // the reverse map per (flat chunk, value head)
  float *dqh, *dkh;                       // [T, HV, D] fp32
  void *dq, *dk;                          // [T, HK, D] out dtype (written here when HV == HK)
  void *dv;                               // [T, HV, D] out dtype
  float *dbeta, *dg;                      // [T, HV]
  float *dstate0;                         // [N, HV, D, D] or NULL
};

// The chunk of flat index F: sequence n (the last with base(n) <= F, base(n)
// = floor(cu[n] / 64) + n) and its first token t0; valid is false for an
// index between two sequences' ranges.
struct ChunkAt {
  int64_t t0;
  int n, L;
  bool valid;
};

__device__ __forceinline__ ChunkAt chunk_at(const int32_t *cu, int N, int64_t F) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)(cu[mid] >> 6) + mid <= F) lo = mid;
    else hi = mid - 1;
  }
  ChunkAt c;
  c.n = lo;
  const int64_t bos = cu[lo], eos = cu[lo + 1];
  c.t0 = bos + (int64_t)CB * (F - ((int64_t)(bos >> 6) + lo));
  c.valid = c.t0 < eos;
  c.L = c.valid ? (int)min<int64_t>(CB, eos - c.t0) : 0;
  return c;
}

// ---------------------------------------------------------------------------
// shared chunk set-up: inputs into LDS, the gate's prefix sums, the Gram
// matrices and T = (I + R)^{-1}
// ---------------------------------------------------------------------------

template <int D>
struct ChunkSm {
  static constexpr int PD = D + 4;
  // (16-byte aligned arrays: their rows are read 16 bytes at a time)
  alignas(16) float kk[CB][PD];   // keys (fp32), rows >= L zero
  alignas(16) float kg[CB][PC];   // Gamma (.) K K^T, strictly lower
  alignas(16) float ag[CB][PC];   // A = s Gamma (.) Q K^T, lower
  alignas(16) float tt[CB][PC];   // T
  float G[CB], eG[CB], eGl[CB], beta[CB];
  float gl;                       // e^{G_last}
};

template <bool BF16, int D, int NTH>
__device__ __forceinline__ void load_rows(float (*dst)[D + 4], const void *src, int64_t stride, int64_t off0,
                                          int L, int tid) {
  constexpr int Q4 = D / 4;
  for (int it = tid; it < CB * Q4; it += NTH) {
    const int row = it / Q4, c = 4 * (it - row * Q4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < L) {
      const int64_t e = off0 + row * stride + c;
      if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(src) + e);
        x = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                        __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
      } else {
        x = *reinterpret_cast<const float4 *>(static_cast<const float *>(src) + e);
      }
    }
    *reinterpret_cast<float4 *>(&dst[row][c]) = x;
  }
}

// Keys and queries (into qq), beta and the gate; then the Grams and T, with
// NW = 4 or 8 waves: wave w forms Gram row block w & 3, column blocks J of
// parity w >> 2 when NW = 8; the inverse runs on waves 0-3. Ends with a
// barrier.
template <bool BF16, int D, int NW>
__device__ void chunk_setup(ChunkSm<D> &sm, float (*qq)[D + 4], const BwdParams &p, const ChunkAt &ck, int h,
                            int tid) {
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6), w = w8 & 3, hf = w8 >> 2, lane = tid & 63,
            r = lane & 15, g = lane >> 4;
  constexpr int JS = NW / 4;   // column-block stride of one wave
  const int hk = h / p.ratio;
  load_rows<BF16, D, 64 * NW>(sm.kk, p.k, p.k_stride, ck.t0 * p.k_stride + (int64_t)hk * D, ck.L, tid);
  load_rows<BF16, D, 64 * NW>(qq, p.q, p.q_stride, ck.t0 * p.q_stride + (int64_t)hk * D, ck.L, tid);
  if (w8 == 0) {
    const bool ok = lane < ck.L;
    const float gv = (ok && p.gated) ? p.g[(ck.t0 + lane) * p.HV + h] : 0.f;
    const float G = chunk::wave_scan(gv);
    const float Gl = __shfl(G, 63, 64);
    sm.G[lane] = G;
    sm.eG[lane] = __expf(G);
    sm.eGl[lane] = __expf(Gl - G);
    sm.beta[lane] = ok ? p.beta[(ck.t0 + lane) * p.HV + h] : 0.f;
    if (lane == 0) sm.gl = __expf(Gl);
  }
  __syncthreads();
  // Grams: row block w against column blocks J <= w
  for (int J = hf; J <= w; J += JS) {
    f32x4 a = mm<true, true>(&sm.kk[16 * w][0], D + 4, 1, &sm.kk[16 * J][0], 1, D + 4, D / 4, zero4(), r, g);
    f32x4 b = mm<true, true>(&qq[16 * w][0], D + 4, 1, &sm.kk[16 * J][0], 1, D + 4, D / 4, zero4(), r, g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, j = 16 * J + r;
      const float gm = j <= i ? __expf(sm.G[i] - sm.G[j]) : 0.f;
      sm.kg[i][j] = j < i ? a[e] * gm : 0.f;
      sm.ag[i][j] = p.scale * b[e] * gm;
    }
  }
  for (int J = w + 1 + hf; J < 4; J += JS)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e, j = 16 * J + r;
      sm.kg[i][j] = 0.f;
      sm.ag[i][j] = 0.f;
    }
  __syncthreads();
  // diagonal blocks of T: lane b < 16 of wave w solves column b of
  // (I + R_ww) T_ww = I by forward substitution, R = beta_i kg
  if (hf == 0 && lane < 16) {
    float t[16];
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      const int i = 16 * w + a;
      float x = a == lane ? 1.f : 0.f;
      const float bi = sm.beta[i];
#pragma unroll
      for (int c = 0; c < a; ++c) x -= bi * sm.kg[i][16 * w + c] * t[c];
      t[a] = x;
    }
#pragma unroll
    for (int a = 0; a < 16; ++a) sm.tt[16 * w + a][16 * w + lane] = t[a];
  }
  // the blocks above the diagonal are zero
  for (int J = w + 1 + hf; J < 4; J += JS)
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.tt[16 * w + 4 * g + e][16 * J + r] = 0.f;
  __syncthreads();
  // blocks below: T_IJ = -T_II sum_{K=J}^{I-1} R_IK T_KJ, by distance I - J
  for (int d = 1; d < 4; ++d) {
    const int I = w, J = w - d;
    if (hf == 0 && J >= 0) {
      f32x4 y = mm<true, false>(&sm.kg[16 * I][16 * J], PC, 1, &sm.tt[16 * J][16 * J], PC, 1, 4 * d, zero4(), r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] *= sm.beta[16 * I + 4 * g + e];
      // Y through the block's own slot (this wave alone reads and writes it)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.tt[16 * I + 4 * g + e][16 * J + r] = y[e];
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the slot holds Y
      __builtin_amdgcn_wave_barrier();
      const f32x4 t = mm<true, false>(&sm.tt[16 * I][16 * I], PC, 1, &sm.tt[16 * I][16 * J], PC, 1, 4, zero4(), r, g);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.tt[16 * I + 4 * g + e][16 * J + r] = -t[e];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 2. the reverse map of each chunk: M = e^{G_last} I - W^T K_e,
//    Y = (s Q_l - A W)^T dO, W = T Diag(beta) K_l
// ---------------------------------------------------------------------------

template <int D>
struct PrepBwdSm {
  ChunkSm<D> c;
  alignas(16) float qq[CB][D + 4];   // queries, then Z = s Q_l - A W
  alignas(16) float ww[CB][D + 4];   // W, then dO
};

// Eight waves (w8 = 4 hf + w). Every product runs over 16-token blocks kb of
// its contraction with all of a wave's output tiles at once (one operand
// load feeds several independent accumulator chains): W and Z by row block
// w and key tiles of parity hf; M and Y (D x D) by 16-row tiles of the key
// dimension, D / 16 of them over the eight waves.
template <bool BF16, int D>
__global__ __launch_bounds__(512) void bwd_prep_kernel(BwdParams p) {
  __shared__ PrepBwdSm<D> sm;
  constexpr int NH = D / 32;               // key tiles per wave in W and Z
  constexpr int RTT = D / 16;              // row tiles of M and Y
  constexpr int CT = RTT * RTT / 8;        // M / Y tiles per wave
  constexpr int WPR = 8 / RTT;             // waves per row tile of M / Y
  const int64_t F = blockIdx.x / p.HV;
  const int h = blockIdx.x - (int)F * p.HV;
  const ChunkAt ck = chunk_at(p.cu_seqlens, p.N, F);
  if (!ck.valid) return;
  const int tid = threadIdx.x, w8 = __builtin_amdgcn_readfirstlane(tid >> 6), w = w8 & 3, hf = w8 >> 2,
            lane = tid & 63, r = lane & 15, g = lane >> 4;
  chunk_setup<BF16, D, 8>(sm.c, sm.qq, p, ck, h, tid);
  // T <- T Diag(beta gamma), so that T K = W
  for (int it = tid; it < CB * CB; it += 512) {
    const int i = it / CB, j = it - i * CB;
    sm.c.tt[i][j] *= sm.c.beta[j] * sm.c.eG[j];
  }
  __syncthreads();
  // W, row block w, key tiles 2 mm + hf (T lower: tokens < 16 (w + 1))
  {
    f32x4 acc[NH];
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_) acc[mm_] = zero4();
    for (int kb = 0; kb <= w; ++kb) {
      const float4 t4 = *reinterpret_cast<const float4 *>(&sm.c.tt[16 * w + r][16 * kb + 4 * g]);
      const float a[4] = {t4.x, t4.y, t4.z, t4.w};
      float b[NH][4];
#pragma unroll
      for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[mm_][j] = sm.c.kk[16 * kb + 4 * g + j][16 * (2 * mm_ + hf) + r];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mm_ = 0; mm_ < NH; ++mm_) acc[mm_] = mf(a[j], b[mm_][j], acc[mm_]);
    }
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.ww[16 * w + 4 * g + e][16 * (2 * mm_ + hf) + r] = acc[mm_][e];
  }
  __syncthreads();
  // keys decayed to the chunk's end, in place
  for (int it = tid; it < CB * D; it += 512) {
    const int i = it / D, j = it - i * D;
    sm.c.kk[i][j] *= sm.c.eGl[i];
  }
  __syncthreads();
  const int64_t mbase = (F * p.HV + h) * (int64_t)(D * D);
  // X^T Y' over the chunk's 64 tokens for one row tile (a0) and CT column
  // tiles c0 + WPR u: A(a, k) = xa[k][a0 + a], B(k, b) = xb[k][16 (c0 + WPR u) + b]
  const int a0 = 16 * (w8 / WPR), c0 = w8 % WPR;
  auto tprod = [&](const float (*xa)[D + 4], const float (*xb)[D + 4], f32x4 (&acc)[CT]) {
#pragma unroll
    for (int u = 0; u < CT; ++u) acc[u] = zero4();
    for (int kb = 0; kb < CB / 16; ++kb) {
      float a[4], b[CT][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = xa[16 * kb + 4 * g + j][a0 + r];
#pragma unroll
      for (int u = 0; u < CT; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[u][j] = xb[16 * kb + 4 * g + j][16 * (c0 + WPR * u) + r];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < CT; ++u) acc[u] = mf(a[j], b[u][j], acc[u]);
    }
  };
  // M = gl I - W^T K_e
  {
    f32x4 acc[CT];
    tprod(sm.ww, sm.c.kk, acc);
#pragma unroll
    for (int u = 0; u < CT; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = a0 + 4 * g + e, col = 16 * (c0 + WPR * u) + r;
        p.M[mbase + (int64_t)row * D + col] = (row == col ? sm.c.gl : 0.f) - acc[u][e];
      }
  }
  // Z = s Q_l - A W, row block w, key tiles 2 mm + hf, in place of the queries
  {
    f32x4 acc[NH];
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_) acc[mm_] = zero4();
    for (int kb = 0; kb <= w; ++kb) {
      const float4 t4 = *reinterpret_cast<const float4 *>(&sm.c.ag[16 * w + r][16 * kb + 4 * g]);
      const float a[4] = {t4.x, t4.y, t4.z, t4.w};
      float b[NH][4];
#pragma unroll
      for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[mm_][j] = sm.ww[16 * kb + 4 * g + j][16 * (2 * mm_ + hf) + r];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mm_ = 0; mm_ < NH; ++mm_) acc[mm_] = mf(a[j], b[mm_][j], acc[mm_]);
    }
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e, j = 16 * (2 * mm_ + hf) + r;
        sm.qq[i][j] = p.scale * sm.c.eG[i] * sm.qq[i][j] - acc[mm_][e];
      }
  }
  __syncthreads();
  // dO into W's place
  load_rows<BF16, D, 512>(sm.ww, p.dout, (int64_t)p.HV * D, ck.t0 * (int64_t)p.HV * D + (int64_t)h * D, ck.L,
                          tid);
  __syncthreads();
  // Y = Z^T dO
  {
    f32x4 acc[CT];
    tprod(sm.qq, sm.ww, acc);
#pragma unroll
    for (int u = 0; u < CT; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.Y[mbase + (int64_t)(a0 + 4 * g + e) * D + 16 * (c0 + WPR * u) + r] = acc[u][e];
  }
}

// ---------------------------------------------------------------------------
// 3. the reverse walk: dS^T_c = M_c dS^T_{c+1} + Y_c from dS^T = 0 at the
//    sequence's end; dS^T_{c+1} stored for chunk c; dS^T_0 to dstate0
// ---------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(256) void bwd_walk_kernel(BwdParams p) {
  // the state gradient's 16 columns, column-major (a lane's four k of a
  // 16-wide k block are one 16-byte read), by parity
  __shared__ alignas(16) float xs[2][16][D + 4];
  constexpr int GRP = D / 16;
  constexpr int RT = D / 64;       // 16-row tiles per wave
  constexpr int KB = D / 16;       // 16-wide k blocks
  // all workgroups of one (sequence, head) get ids equal modulo 8: one XCD,
  // whose L2 serves them each chunk's M
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7), vb = (b >> 3) % GRP;
  if (gi >= p.N * p.HV) return;
  const int n = gi / p.HV, h = gi - n * p.HV;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15,
            g = lane >> 4;
  const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  const int64_t nc = (eos - bos + CB - 1) / CB;
  const int64_t base = (int64_t)(p.cu_seqlens[n] >> 6) + n;
  const int col0 = 16 * vb;
  // A operands of M (rows (D/4) w + 16 t + r, k = 16 kb + 4g + j) and the
  // accumulators' Y, loaded one chunk ahead
  auto load_ops = [&](int64_t c, float4 (&am)[RT][KB], f32x4 (&ya)[RT]) {
    const int64_t mb = ((base + c) * p.HV + h) * (int64_t)(D * D);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int a0 = (D / 4) * w + 16 * t;
      const float *mr = p.M + mb + (int64_t)(a0 + r) * D + 4 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) am[t][kb] = *reinterpret_cast<const float4 *>(mr + 16 * kb);
#pragma unroll
      for (int e = 0; e < 4; ++e) ya[t][e] = p.Y[mb + (int64_t)(a0 + 4 * g + e) * D + col0 + r];
    }
  };
  f32x4 x[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) x[t] = zero4();
  // chunk c with operands in (am, ya), loading chunk c - 1's into (an, yn)
  // (chunk 0 loads its own again: every step issues the same loads); two
  // register sets used in turn, so that no copy waits for loads in flight
  auto step = [&](int64_t c, int par, const float4 (&am)[RT][KB], const f32x4 (&ya)[RT], float4 (&an)[RT][KB],
                  f32x4 (&yn)[RT]) {
    const int64_t mb = ((base + c) * p.HV + h) * (int64_t)(D * D);
    // dS^T_{c+1}: to the checkpoint and to LDS
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int row0 = (D / 4) * w + 16 * t + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) p.ckb[mb + (int64_t)(row0 + e) * D + col0 + r] = x[t][e];
      *reinterpret_cast<float4 *>(&xs[par][r][row0]) = make_float4(x[t][0], x[t][1], x[t][2], x[t][3]);
    }
    load_ops(c > 0 ? c - 1 : 0, an, yn);
    __syncthreads();
    float4 bx[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) bx[kb] = *reinterpret_cast<const float4 *>(&xs[par][r][16 * kb + 4 * g]);
    f32x4 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = ya[t];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const float bv[4] = {bx[kb].x, bx[kb].y, bx[kb].z, bx[kb].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const float a = j == 0 ? am[t][kb].x : j == 1 ? am[t][kb].y : j == 2 ? am[t][kb].z : am[t][kb].w;
          acc[t] = mf(a, bv[j], acc[t]);
        }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) x[t] = acc[t];
  };
  float4 a0[RT][KB], a1[RT][KB];
  f32x4 y0[RT], y1[RT];
  if (nc > 0) load_ops(nc - 1, a0, y0);
  int64_t c = nc - 1;
  for (; c >= 1; c -= 2) {
    step(c, 0, a0, y0, a1, y1);
    step(c - 1, 1, a1, y1, a0, y0);
  }
  if (c == 0) step(0, 0, a0, y0, a1, y1);
  if (p.dstate0) {
    float *d0 = p.dstate0 + ((int64_t)n * p.HV + h) * (int64_t)(D * D);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) d0[(int64_t)((D / 4) * w + 16 * t + 4 * g + e) * D + col0 + r] = x[t][e];
  }
}

// ---------------------------------------------------------------------------
// 4. per-chunk gradients
// ---------------------------------------------------------------------------

template <int D>
struct GradSm {
  ChunkSm<D> c;
  union alignas(16) {
    float qq[CB][D + 4];        // queries (set-up, and again for the last step)
    struct {
      float sb[D][PB];          // S^T_c, this block's columns
      float db[D][PB];          // dS^T_{c+1}, this block's columns
      float vb[CB][PB];         // V
      float ob[CB][PB];         // dO
      float rv[CB][PB];         // Rv
      float eb[CB][PB];         // E
      float de[CB][PB];         // dE
      float dr[CB][PB];         // dRv
      float dx[CB][PB];         // dX
    } b;
  } u;
  // per-wave partial sums of dG (by row and by column), dbeta and the last
  // row's scalar terms, each written by one wave and summed in wave order
  // (so the results do not depend on the order in which waves finish)
  float pr[8][CB], pc[8][CB], pb[8][CB], pl[8];
  float dG[CB];
};

// Eight waves: wave w8 = 4 hf + w. The products over a block's 16 value
// columns along the chain (one 16 x 16 tile per row block) are split
// between the two wave sets: X and E on hf = 0, K dS^T and dE on hf = 1,
// dRv on hf = 0; the Gram-side products (dA, dR: column blocks J of
// parity hf) and those over the key dimension (dQ_l, dK_l, dK_e, and dq, dk
// at the end: key tiles m of parity hf) are shared by all eight. Waves w and
// w + 4 share a SIMD.
template <bool BF16, int D>
__global__ __launch_bounds__(512) void bwd_grad_kernel(BwdParams p) {
  __shared__ GradSm<D> sm;
  constexpr int PD = D + 4;
  constexpr int NH = D / 32;   // key tiles per wave
  const int64_t F = blockIdx.x / p.HV;
  const int h = blockIdx.x - (int)F * p.HV;
  const ChunkAt ck = chunk_at(p.cu_seqlens, p.N, F);
  if (!ck.valid) return;
  const int tid = threadIdx.x, w8 = __builtin_amdgcn_readfirstlane(tid >> 6), w = w8 & 3, hf = w8 >> 2,
            lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int hk = h / p.ratio;
  chunk_setup<BF16, D, 8>(sm.c, sm.u.qq, p, ck, h, tid);
  for (int i = tid; i < 8 * CB; i += 512) {
    (&sm.pr[0][0])[i] = 0.f;
    (&sm.pc[0][0])[i] = 0.f;
    (&sm.pb[0][0])[i] = 0.f;
  }

  const int64_t mb = (F * p.HV + h) * (int64_t)(D * D);
  const int64_t HVD = (int64_t)p.HV * D;
  f32x4 dA[2], dR[2], dQl[NH], dKl[NH], dKe[NH];   // column blocks hf, hf + 2; key tiles 2 mm + hf
#pragma unroll
  for (int J = 0; J < 2; ++J) dA[J] = dR[J] = zero4();
#pragma unroll
  for (int m = 0; m < NH; ++m) dQl[m] = dKl[m] = dKe[m] = zero4();
  float dbl[4] = {0.f, 0.f, 0.f, 0.f};   // sum over columns of (V - X) dRv, rows 16w + 4g + e
  float sds = 0.f;
  float beta_r[4], eG_r[4], eGl_r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = 16 * w + 4 * g + e;
    beta_r[e] = sm.c.beta[i];
    eG_r[e] = sm.c.eG[i];
    eGl_r[e] = sm.c.eGl[i];
  }

  // a block's S^T, dS^T, V and dO columns, fetched into registers one block
  // ahead
  constexpr int NSB = D * BW / 512, NVB = CB * BW / 512;
  float ps[NSB], pd[NSB], pv[NVB], po[NVB];
  auto fetch = [&](int vb) {
    const int col0 = BW * vb;
#pragma unroll
    for (int u = 0; u < NSB; ++u) {
      const int it = tid + 512 * u, row = it / BW, c = it - row * BW;
      ps[u] = p.ckf[mb + (int64_t)row * D + col0 + c];
      pd[u] = p.ckb[mb + (int64_t)row * D + col0 + c];
    }
#pragma unroll
    for (int u = 0; u < NVB; ++u) {
      const int it = tid + 512 * u, row = it / BW, c = it - row * BW;
      const bool ok = row < ck.L;
      const int64_t tr = ck.t0 + (ok ? row : 0);
      const float v = ld_in<BF16>(p.v, tr * p.v_stride + (int64_t)h * D + col0 + c);
      const float o = ld_in<BF16>(p.dout, tr * HVD + (int64_t)h * D + col0 + c);
      pv[u] = ok ? v : 0.f;
      po[u] = ok ? o : 0.f;
    }
  };
  fetch(0);
  for (int vb = 0; vb < D / BW; ++vb) {
    const int col0 = BW * vb;
    __syncthreads();   // the previous block (or the queries) is no longer read
#pragma unroll
    for (int u = 0; u < NSB; ++u) {
      const int it = tid + 512 * u, row = it / BW, c = it - row * BW;
      sm.u.b.sb[row][c] = ps[u];
      sm.u.b.db[row][c] = pd[u];
      sds += ps[u] * pd[u];
    }
#pragma unroll
    for (int u = 0; u < NVB; ++u) {
      const int it = tid + 512 * u, row = it / BW, c = it - row * BW;
      sm.u.b.vb[row][c] = pv[u];
      sm.u.b.ob[row][c] = po[u];
    }
    fetch(vb + 1 < D / BW ? vb + 1 : vb);   // (the last block fetches itself again)
    __syncthreads();
    // X = K_l S^T, Rv = beta (V - X) on waves hf = 0; K dS^T (kept) on the others
    float vx[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 kds = zero4();
    if (hf == 0) {
      const f32x4 x = mm<true, false>(&sm.c.kk[16 * w][0], PD, 1, &sm.u.b.sb[0][0], PB, 1, D / 4, zero4(), r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e;
        vx[e] = sm.u.b.vb[i][r] - eG_r[e] * x[e];
        sm.u.b.rv[i][r] = beta_r[e] * vx[e];
      }
    } else {
      kds = mm<true, false>(&sm.c.kk[16 * w][0], PD, 1, &sm.u.b.db[0][0], PB, 1, D / 4, zero4(), r, g);
    }
    __syncthreads();
    // E = T Rv on waves hf = 0;  dE = A^T dO + K_e dS^T on the others
    if (hf == 0) {
      const f32x4 ev = mm<true, false>(&sm.c.tt[16 * w][0], PC, 1, &sm.u.b.rv[0][0], PB, 1, 4 * (w + 1), zero4(), r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.b.eb[16 * w + 4 * g + e][r] = ev[e];
    } else {
      const f32x4 a = mm<false, false>(&sm.c.ag[16 * w][16 * w], 1, PC, &sm.u.b.ob[16 * w][0], PB, 1, 4 * (4 - w), zero4(), r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.u.b.de[16 * w + 4 * g + e][r] = a[e] + eGl_r[e] * kds[e];
    }
    __syncthreads();
    // dRv = T^T dE; dV = beta dRv; dX = -beta dRv
    if (hf == 0) {
      const f32x4 d = mm<false, false>(&sm.c.tt[16 * w][16 * w], 1, PC, &sm.u.b.de[16 * w][0], PB, 1, 4 * (4 - w), zero4(), r, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e;
        dbl[e] += vx[e] * d[e];
        sm.u.b.dr[i][r] = d[e];
        sm.u.b.dx[i][r] = -beta_r[e] * d[e];
        if (i < ck.L) {
          const int64_t o = (ck.t0 + i) * HVD + (int64_t)h * D + col0 + r;
          const float dvv = beta_r[e] * d[e];
          if (p.out_bf16) static_cast<uint16_t *>(p.dv)[o] = f32_to_bf16(dvv);
          else static_cast<float *>(p.dv)[o] = dvv;
        }
      }
    }
    __syncthreads();
    // over the block's 16 columns k (lane (r, g) holds k = 4g .. 4g + 3):
    // dA += dO E^T, dR += dRv E^T (negated at the end) for blocks J <= w;
    // dQ_l += dO S, dK_l += dX S, dK_e += E dS for the wave's key tiles
    // (S's element (v, j) is sb[j][v]); every product of the step shares its
    // operand loads and runs as an independent accumulator chain
    {
      const float4 aob = *reinterpret_cast<const float4 *>(&sm.u.b.ob[16 * w + r][4 * g]);
      const float4 adr = *reinterpret_cast<const float4 *>(&sm.u.b.dr[16 * w + r][4 * g]);
      const float4 adx = *reinterpret_cast<const float4 *>(&sm.u.b.dx[16 * w + r][4 * g]);
      const float4 aeb = *reinterpret_cast<const float4 *>(&sm.u.b.eb[16 * w + r][4 * g]);
      float4 be[2], bs[NH], bd[NH];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int J = min(hf + 2 * jj, 3);
        be[jj] = *reinterpret_cast<const float4 *>(&sm.u.b.eb[16 * J + r][4 * g]);
      }
#pragma unroll
      for (int mm_ = 0; mm_ < NH; ++mm_) {
        const int m = 2 * mm_ + hf;
        bs[mm_] = *reinterpret_cast<const float4 *>(&sm.u.b.sb[16 * m + r][4 * g]);
        bd[mm_] = *reinterpret_cast<const float4 *>(&sm.u.b.db[16 * m + r][4 * g]);
      }
      const bool j0 = hf <= w, j1 = hf + 2 <= w;
      const float a_ob[4] = {aob.x, aob.y, aob.z, aob.w}, a_dr[4] = {adr.x, adr.y, adr.z, adr.w};
      const float a_dx[4] = {adx.x, adx.y, adx.z, adx.w}, a_eb[4] = {aeb.x, aeb.y, aeb.z, aeb.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const float b = jj == 0 ? (j == 0 ? be[0].x : j == 1 ? be[0].y : j == 2 ? be[0].z : be[0].w)
                                  : (j == 0 ? be[1].x : j == 1 ? be[1].y : j == 2 ? be[1].z : be[1].w);
          if (jj == 0 ? j0 : j1) {
            dA[jj] = mf(a_ob[j], b, dA[jj]);
            dR[jj] = mf(a_dr[j], b, dR[jj]);
          }
        }
#pragma unroll
        for (int mm_ = 0; mm_ < NH; ++mm_) {
          const float b1 = j == 0 ? bs[mm_].x : j == 1 ? bs[mm_].y : j == 2 ? bs[mm_].z : bs[mm_].w;
          const float b2 = j == 0 ? bd[mm_].x : j == 1 ? bd[mm_].y : j == 2 ? bd[mm_].z : bd[mm_].w;
          dQl[mm_] = mf(a_ob[j], b1, dQl[mm_]);
          dKl[mm_] = mf(a_dx[j], b1, dKl[mm_]);
          dKe[mm_] = mf(a_eb[j], b2, dKe[mm_]);
        }
      }
    }
  }
  __syncthreads();   // the blocks are dead: the queries return
  load_rows<BF16, D, 512>(sm.u.qq, p.q, p.q_stride, ck.t0 * p.q_stride + (int64_t)hk * D, ck.L, tid);
  // dbeta from Rv; the Gram terms of dG and dbeta; P_R, P_A in place of
  // kg and ag
  // (sums over the 16 lanes of a row group, or over the four row groups of
  // a column, by xor shuffles: a fixed order)
  auto sum16 = [](float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
  };
  auto sum_g = [](float x) {
    x += __shfl_xor(x, 16, 64);
    return x + __shfl_xor(x, 32, 64);
  };
  float rowp[4] = {0.f, 0.f, 0.f, 0.f}, rowb[4] = {0.f, 0.f, 0.f, 0.f};
  {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int J = hf + 2 * jj;
      if (J > w) continue;
      float colp = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e, j = 16 * J + r;
        const float kgv = sm.c.kg[i][j], agv = sm.c.ag[i][j];
        const float dr = -dR[jj][e], da = dA[jj][e];
        const float gm = j <= i ? __expf(sm.c.G[i] - sm.c.G[j]) : 0.f;
        const float nn = dr * beta_r[e] * kgv + da * agv;
        rowp[e] += nn;
        colp += nn;
        rowb[e] += dr * kgv;
        sm.c.kg[i][j] = j < i ? dr * beta_r[e] * gm : 0.f;
        sm.c.ag[i][j] = j <= i ? da * p.scale * gm : 0.f;
      }
      colp = sum_g(colp);
      if (g == 0) sm.pc[w8][16 * J + r] = -colp;
    }
  }
  __syncthreads();   // queries loaded, P_R and P_A written
  // row terms of dG; dk, dq start from the decayed-operand terms
  {
    float last = 0.f;
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * w + 4 * g + e, j = 16 * (2 * mm_ + hf) + r;
        const float kv = sm.c.kk[i][j], qv = sm.u.qq[i][j];
        const float ke = eGl_r[e] * kv * dKe[mm_][e];
        rowp[e] += eG_r[e] * (kv * dKl[mm_][e] + p.scale * qv * dQl[mm_][e]) - ke;
        last += ke;
        dKl[mm_][e] = eG_r[e] * dKl[mm_][e] + eGl_r[e] * dKe[mm_][e];   // dk
        dQl[mm_][e] = p.scale * eG_r[e] * dQl[mm_][e];                  // dq
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float rs = sum16(rowp[e]), bs = sum16(rowb[e] + dbl[e]);
      if (r == 0) {
        sm.pr[w8][16 * w + 4 * g + e] = rs;
        sm.pb[w8][16 * w + 4 * g + e] = bs;
      }
    }
    // the last row's scalar terms: sum_j e^{G_last - G_j} k_j . dK_e,j and
    // e^{G_last} <dS_{c+1}, S_c> (this thread's share of both)
    float lt = last + sm.c.gl * sds;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lt += __shfl_xor(lt, off, 64);
    if (lane == 0) sm.pl[w8] = lt;
  }
  // dk += P_R K + P_R^T K + P_A^T Q;  dq += P_A K, over 16-token blocks kb
  // of the contraction (lane (r, g) holds tokens 16 kb + 4g .. + 3), every
  // key tile of the wave at once: P_R and P_A rows for kb <= w, their
  // columns for kb >= w
  for (int kb = 0; kb <= w; ++kb) {
    const float4 pr = *reinterpret_cast<const float4 *>(&sm.c.kg[16 * w + r][16 * kb + 4 * g]);
    const float4 pa = *reinterpret_cast<const float4 *>(&sm.c.ag[16 * w + r][16 * kb + 4 * g]);
    const float a_pr[4] = {pr.x, pr.y, pr.z, pr.w}, a_pa[4] = {pa.x, pa.y, pa.z, pa.w};
    float bk[NH][4];
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
      for (int j = 0; j < 4; ++j) bk[mm_][j] = sm.c.kk[16 * kb + 4 * g + j][16 * (2 * mm_ + hf) + r];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mm_ = 0; mm_ < NH; ++mm_) {
        dKl[mm_] = mf(a_pr[j], bk[mm_][j], dKl[mm_]);
        dQl[mm_] = mf(a_pa[j], bk[mm_][j], dQl[mm_]);
      }
  }
  for (int kb = w; kb < 4; ++kb) {
    float a_pr[4], a_pa[4], bk[NH][4], bq[NH][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a_pr[j] = sm.c.kg[16 * kb + 4 * g + j][16 * w + r];
      a_pa[j] = sm.c.ag[16 * kb + 4 * g + j][16 * w + r];
    }
#pragma unroll
    for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bk[mm_][j] = sm.c.kk[16 * kb + 4 * g + j][16 * (2 * mm_ + hf) + r];
        bq[mm_][j] = sm.u.qq[16 * kb + 4 * g + j][16 * (2 * mm_ + hf) + r];
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mm_ = 0; mm_ < NH; ++mm_) {
        dKl[mm_] = mf(a_pr[j], bk[mm_][j], dKl[mm_]);
        dKl[mm_] = mf(a_pa[j], bq[mm_][j], dKl[mm_]);
      }
  }
#pragma unroll
  for (int mm_ = 0; mm_ < NH; ++mm_)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * w + 4 * g + e;
      if (i < ck.L) {
        const int64_t o = (ck.t0 + i) * HVD + (int64_t)h * D + 16 * (2 * mm_ + hf) + r;
        if (p.ratio > 1) {
          p.dkh[o] = dKl[mm_][e];
          p.dqh[o] = dQl[mm_][e];
        } else if (p.out_bf16) {   // one value head per key head: the final dq, dk
          static_cast<uint16_t *>(p.dk)[o] = f32_to_bf16(dKl[mm_][e]);
          static_cast<uint16_t *>(p.dq)[o] = f32_to_bf16(dQl[mm_][e]);
        } else {
          static_cast<float *>(p.dk)[o] = dKl[mm_][e];
          static_cast<float *>(p.dq)[o] = dQl[mm_][e];
        }
      }
    }
  __syncthreads();   // the partial sums are complete
  if (tid < CB) {
    float x = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) x += sm.pr[u][tid] + sm.pc[u][tid];
    if (tid == CB - 1)
#pragma unroll
      for (int u = 0; u < 8; ++u) x += sm.pl[u];
    sm.dG[tid] = x;
  }
  __syncthreads();
  if (tid < ck.L) {
    const int64_t o = (ck.t0 + tid) * p.HV + h;
    float b = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) b += sm.pb[u][tid];
    p.dbeta[o] = b;
    if (p.gated) {
      float s = 0.f;
      for (int i = tid; i < CB; ++i) s += sm.dG[i];
      p.dg[o] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// 5. dq, dk of a key head: the sum over its value heads
// ---------------------------------------------------------------------------

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float *dqh, const float *dkh, void *dq, void *dk,
                                                            int HK, int R, int D) {
  const int64_t t = blockIdx.x;
  const int HV = HK * R;
  for (int e = threadIdx.x; e < HK * D; e += 256) {
    const int hk = e / D, d = e - hk * D;
    float sq = 0.f, sk = 0.f;
    for (int j = 0; j < R; ++j) {
      const int64_t s = (t * HV + hk * R + j) * (int64_t)D + d;
      sq += dqh[s];
      sk += dkh[s];
    }
    const int64_t o = t * HK * (int64_t)D + e;
    if constexpr (OUT_BF16) {
      static_cast<uint16_t *>(dq)[o] = f32_to_bf16(sq);
      static_cast<uint16_t *>(dk)[o] = f32_to_bf16(sk);
    } else {
      static_cast<float *>(dq)[o] = sq;
      static_cast<float *>(dk)[o] = sk;
    }
  }
}

// dst[n][h] = pool[slot_idx[n]][h] in fp32 (D x D values), and slots[n] = n:
// the initial states as a scratch pool the warp-specialised walk may write.
// (COPY false: the slots alone, for a walk from zero states)
template <bool ST_BF16, bool COPY = true>
__global__ __launch_bounds__(256) void copy_states_kernel(const void *pool, const int32_t *slot_idx, float *dst,
                                                          int32_t *slots, int HV, int DD) {
  const int nh = blockIdx.x, n = nh / HV, h = nh - n * HV;
  const int64_t src = ((int64_t)slot_idx[n] * HV + h) * DD, o = (int64_t)nh * DD;
  for (int e = threadIdx.x; COPY && e < DD; e += 256) {
    if constexpr (ST_BF16) dst[o + e] = bf16_to_f32(static_cast<const uint16_t *>(pool)[src + e]);
    else dst[o + e] = static_cast<const float *>(pool)[src + e];
  }
  if (h == 0 && threadIdx.x == 0) slots[n] = n;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdWs {
  size_t ckf, ckb, M, Y, dqh, dkh, total;
};

BwdWs ws_layout(const gdr_args &a) {
  const size_t flat = (size_t)((a.T_total + CB - 1) / CB + a.N);
  const size_t mat = flat * a.HV * (size_t)a.DK * a.DK * 4;
  const size_t rows = (size_t)a.T_total * a.HV * a.DK * 4;
  BwdWs l;
  size_t o = 0;
  l.ckf = o; o += al256(mat);
  l.ckb = o; o += al256(mat);
  l.M = o; o += al256(mat);
  l.Y = o; o += al256(mat);
  l.dqh = o; o += al256(rows);
  l.dkh = o; o += al256(rows);
  l.total = o;
  return l;
}

template <bool BF16, int D>
hipError_t launch_bwd(const BwdParams &p, const gdr_args &a, void *dq, void *dk, hipStream_t stream) {
  const unsigned items = (unsigned)(p.flat * p.HV);
  hipLaunchKernelGGL((bwd_prep_kernel<BF16, D>), dim3(items), dim3(512), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_walk_kernel<D>), dim3((unsigned)(((p.N * p.HV + 7) / 8) * 8 * (D / 16))), dim3(256), 0,
                     stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<BF16, D>), dim3(items), dim3(512), 0, stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.T_total == 0 || p.ratio == 1) return hipSuccess;   // (HV == HK: dq, dk already final)
  if (p.out_bf16)
    hipLaunchKernelGGL((bwd_group_sum_kernel<true>), dim3((unsigned)a.T_total), dim3(256), 0, stream, p.dqh, p.dkh,
                       dq, dk, a.HK, p.ratio, D);
  else
    hipLaunchKernelGGL((bwd_group_sum_kernel<false>), dim3((unsigned)a.T_total), dim3(256), 0, stream, p.dqh,
                       p.dkh, dq, dk, a.HK, p.ratio, D);
  return hipGetLastError();
}

}  // namespace

size_t chunk_bwd_workspace(const gdr_args &a) { return ws_layout(a).total; }

hipError_t launch_chunk_bwd(const gdr_args &a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                            float *dg, float *dstate0, void *ws, hipStream_t stream) {
  const BwdWs l = ws_layout(a);
  char *w = static_cast<char *>(ws);
  hipError_t e;
  if (a.in_dtype == GDR_BF16 && !prefill_force_generic()) {
    // the warp-specialised kernel, on a scratch copy of the initial states
    // (in M's place) with its outputs in dq's fp32 scratch (both rewritten
    // later)
    gdr_args b = a;
    b.state_pool = w + l.M;
    b.state_dtype = GDR_F32;
    b.num_slots = a.N;
    b.slot_idx = reinterpret_cast<const int32_t *>(w + l.Y);
    b.o = w + l.dqh;
    b.out_dtype = GDR_F32;
    if (a.flags & GDR_FLAG_ZERO_INIT)
      hipLaunchKernelGGL((copy_states_kernel<false, false>), dim3((unsigned)(a.N * a.HV)), dim3(256), 0, stream,
                         a.state_pool, a.slot_idx, reinterpret_cast<float *>(w + l.M),
                         reinterpret_cast<int32_t *>(w + l.Y), a.HV, a.DK * a.DK);
    else if (a.state_dtype == GDR_BF16)
      hipLaunchKernelGGL(copy_states_kernel<true>, dim3((unsigned)(a.N * a.HV)), dim3(256), 0, stream, a.state_pool,
                         a.slot_idx, reinterpret_cast<float *>(w + l.M), reinterpret_cast<int32_t *>(w + l.Y), a.HV,
                         a.DK * a.DK);
    else
      hipLaunchKernelGGL(copy_states_kernel<false>, dim3((unsigned)(a.N * a.HV)), dim3(256), 0, stream,
                         a.state_pool, a.slot_idx, reinterpret_cast<float *>(w + l.M),
                         reinterpret_cast<int32_t *>(w + l.Y), a.HV, a.DK * a.DK);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = launch_chunk_states_ws(b, reinterpret_cast<float *>(w + l.ckf), stream);
  } else {
    e = launch_chunk_states(a, reinterpret_cast<float *>(w + l.ckf), stream);
  }
  if (e != hipSuccess) return e;
  BwdParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = dout;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta;
  p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HK = a.HK; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.gated = a.gate == GDR_GATE_SCALAR;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  p.flat = (a.T_total + CB - 1) / CB + a.N;
  p.ckf = reinterpret_cast<const float *>(w + l.ckf);
  p.ckb = reinterpret_cast<float *>(w + l.ckb);
  p.M = reinterpret_cast<float *>(w + l.M);
  p.Y = reinterpret_cast<float *>(w + l.Y);
  p.dqh = reinterpret_cast<float *>(w + l.dqh);
  p.dkh = reinterpret_cast<float *>(w + l.dkh);
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dbeta = dbeta;
  p.dg = dg;
  p.dstate0 = dstate0;
  const bool bf = a.in_dtype == GDR_BF16;
  if (a.DK == 128) return bf ? launch_bwd<true, 128>(p, a, dq, dk, stream) : launch_bwd<false, 128>(p, a, dq, dk, stream);
  return bf ? launch_bwd<true, 64>(p, a, dq, dk, stream) : launch_bwd<false, 64>(p, a, dq, dk, stream);
}

}  // namespace gdr
