// Chunkwise prefill with a per-key-channel gate, bf16 q/k/v: KDA (the delta
// rule) and GLA (the linear rule: no correction, records without region 1).
//
// Math (section 6 of "You Could Have Come Up With Kimi Delta Attention",
// section 4 of "From Attention to Learned Memory"): per chunk of C = 64
// tokens with incoming state S (value-by-key) and the inclusive in-chunk
// cumulative log-decay G_i in R^{d_k} (one value per key channel),
//
//   K_l = e^{G} (.) K,   Q^ = s e^{G} (.) Q,   K_end = e^{G_last - G} (.) K
//   R   = strict-lower( beta_i sum_c k_ic k_jc e^{G_ic - G_jc} )
//   A^  = lower( s sum_c q_ic k_jc e^{G_ic - G_jc} )
//   T   = (I + R)^{-1},  T' = T Diag(beta),  W = T' K_l,  U = T' V
//   Vb  = U - W S^T                         (the solved errors e_i)
//   O   = Q^ S^T + A^ Vb
//   S^T <- gamma (.) S^T + K_end^T Vb,      gamma = e^{G_last}   (per key row)
//
// Vb equals T (beta (V - K_l S^T)) of the chunk equations; forming W and U
// ahead of time leaves two products on the serial chain from one chunk's state
// to the next (W S^T and the update).
//
// Decay references. The Gram sums are taken over 16-token blocks (the KDA
// page's token sub-blocks of the chunked form) with the reference at a block
// boundary, so that no factor can overflow whatever the gate: for row block I
// and an earlier key block J the rows are q_i e^{G_i - B_I} and the keys
// k_j e^{B_I - G_j}, B_I being G just before block I, both factors <= 1; the
// diagonal block I uses the keys k_j e^{B_I - G_j} >= 1 when the block's
// strongest channel decay is at most 80 (factors <= e^{80}), and is summed
// pair by pair in fp32 otherwise (prep_exact_diagonal). K_l, Q^, K_end and
// gamma carry exponentials of non-positive numbers only.
//
// Two kernels per slice of chunks:
//   * kda_prep_kernel, persistent workgroups over the (chunk, value head)
//     items, fully parallel: gate prefix sums, the decayed operands, the Gram
//     matrices R and A^, the inverse T and the products W; it writes one
//     record per (chunk, head) to the workspace with every operand the state
//     kernel multiplies, already split into bf16 hi / lo planes and laid out
//     as MFMA fragments;
//   * kda_state_kernel, one workgroup per (sequence, value head, 16 value
//     columns): a chain wave (S^T[DK, 16] in MFMA accumulators: Vb and the
//     update) walks the slice's chunks in order, an output wave follows one
//     chunk behind, and six loader waves copy the next chunks' records (and
//     values) from the workspace into registers and into LDS region by region
//     as the computing waves release them (LDS counters, no workgroup
//     barrier).
// A sequence's state crosses slice boundaries through an fp32 carry area of
// the workspace. The workspace is sized by the caller: a larger one means
// fewer, longer slices.
//
// Precision as in the other prefill kernels: every computed operand is split
// hi = bf16(x), lo = bf16(x - hi) and multiplied in three passes (two when one
// side is an exact bf16 input), fp32 accumulation.
//
// Fragment convention (v_mfma_f32_16x16x32_bf16; chunk_common.h): lane
// (r, g) of a fragment holds row r and the eight k of slot set K(g); slot j
// is k = 4g + j for j < 4 and 16 + 4g + (j - 4) otherwise. A record fragment
// is 2 KB: the hi plane (64 lanes x 16 bytes, lane-major) then the lo plane.
#include <cstdint>

#include "chunk_common.h"

namespace gdr {
namespace {

using namespace chunk;

// Layout of one (chunk, value head) record, in bytes. Region 1 holds what the
// first products of a chunk read (W, T'), region 2 the output operands (Q^,
// A^), region 3 the update operands (K_end^T, gamma).
//   W(I, s):  lane (r, g) holds -W[16I + r][32s + k(j)]          (I < 4, s < DK/32)
//   T'(p):    T'[16I + r][32s + k(j)] for the six (I, s) with s <= I/2
//   Q^(I, s): as W;  A^(p): as T'
//   K(m, s):  K_end[32s + k(j)][16m + r]                          (m < DK/16, s < 2)
//   gamma:    DK fp32 values
template <int D>
struct KdaRec {
  static constexpr int NS = D / 32;
  static constexpr int NT = D / 16;
  static constexpr int FB = 2048;
  static constexpr int NF = 4 * NS + 6;   // fragments in region 1 and in region 2
  static constexpr int R1 = 0;
  static constexpr int R2 = NF * FB;
  static constexpr int R3 = 2 * NF * FB;
  static constexpr int GAM = R3 + 2 * NT * FB;
  static constexpr int BYTES = GAM + 4 * D;
  static constexpr int R1_BLOCKS = 2 * NF;   // 1 KB blocks per region
  static constexpr int R3_BLOCKS = 4 * NT;   // without gamma
  __host__ __device__ static constexpr int wq(int I, int s) { return (I * NS + s) * FB; }
  __host__ __device__ static constexpr int tp(int pr) { return (4 * NS + pr) * FB; }
  __host__ __device__ static constexpr int kf(int m, int s) { return R3 + (2 * m + s) * FB; }
};

// Index of the (I, s) fragment of a lower triangular C x C operand (s <= I/2).
__host__ __device__ constexpr int pair_index(int I, int s) { return I < 2 ? I : 2 * I - 2 + s; }

struct KdaParams {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  void *o;
  void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t N, HK, HV, ratio;
  float scale;
  int zero_init, st_bf16, out_bf16;
  int delta;         // the delta rule (else the linear rule: T' = I, W = 0)
  char *rec;         // records of this slice: [(F - F0) * HV + h]
  float *carry;      // [N, HV, D, D] fp32 S^T between slices
  int64_t F0, F1;    // flat chunk range of this slice
};

// Flat chunk index: chunk c of sequence n is base(n) + c with
// base(n) = floor(cu[n] / 64) + n, unique over the batch and below
// ceil(T_total / 64) + N.
__device__ __forceinline__ int64_t flat_base(const int32_t *cu, int n) {
  return (int64_t)(cu[n] >> 6) + n;
}

__device__ __forceinline__ void st_frag(char *base, int off, int lane, const Frag &f) {
  *reinterpret_cast<uint4 *>(base + off + 16 * lane) = __builtin_bit_cast(uint4, f.hi);
  *reinterpret_cast<uint4 *>(base + off + 1024 + 16 * lane) = __builtin_bit_cast(uint4, f.lo);
}

__device__ __forceinline__ void ld_frag(const char *base, int off, int lane, Frag &f) {
  f.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(base + off + 16 * lane));
  f.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(base + off + 1024 + 16 * lane));
}

// Pass P of a split product: lo x hi, hi x lo, hi x hi (the products of
// several independent accumulators are issued pass by pass, so that
// consecutive MFMAs never wait on each other's results).
template <int P, bool B_SPLIT = true>
__device__ __forceinline__ f32x4 mpass(const Frag &a, const Frag &b, f32x4 c) {
  if constexpr (P == 0) return mfma(a.lo, b.hi, c);
  else if constexpr (P == 1) return B_SPLIT ? mfma(a.hi, b.lo, c) : c;
  else return mfma(a.hi, b.hi, c);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Slot j of lane group g: offset of its k inside a 32-wide step.
__device__ __forceinline__ int slot_k(int g, int j) { return (j < 4 ? 4 * g + j : 12 + 4 * g + j); }

// ===========================================================================
// prep kernel
// ===========================================================================

template <int D>
struct PrepSmem {
  static constexpr int PK = D + 4;   // fp32 rows, key columns permuted (perm32)
  float kl[C][PK];                   // K_l = e^{G} (.) K, token-major
  union {
    float kd[C][PK];                 // keys decayed to the end of their own 16-token block
    struct {
      float tt[C][C + 4];            // T, row-major (once the Grams are done)
      float rd[4][16][20];           // R's diagonal blocks, negated
    } t;
  };
  float tot[4][D];                   // per 16-token block: gate sum of each channel (<= 0)
  float etot[4][D];                  // its exponential: the block's decay of each channel
  float fend[4][D];                  // decay of the blocks after block b (keys to the chunk's end)
  float dmid[3][D];                  // decay of the blocks strictly between J and w: (2,0), (3,1), (3,0)
  float beta[C];
};

// T_IJ = -T_II (sum_{K=J}^{I-1} R_IK T_KJ) for one block of T below the
// diagonal (16x16x16 products: R_IK and T_II in row layout as A operands,
// T_KJ read in column layout as the B operand). The last product is taken
// with swapped operands, (T_II Y)^T = Y^T T_II^T, which leaves the block in
// row layout for the row-major store.
template <int I, int J, int D>
__device__ __forceinline__ void t_block(PrepSmem<D> &sm, const f32x4 (&rv)[4], int r, int g) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int K = J; K < I; ++K) {
    Frag4 fr, fc;
    split4(rv[K], fr);
    f32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = sm.t.tt[16 * K + 4 * g + i][16 * J + r];
    split4(c, fc);
    acc = mm16(fr, fc, acc);
  }
  Frag4 ft, fy;
  const float4 d = *reinterpret_cast<const float4 *>(&sm.t.tt[16 * I + r][16 * I + 4 * g]);
  split4(f32x4{d.x, d.y, d.z, d.w}, ft);
  split4(acc, fy);
  const f32x4 t = -mm16(fy, ft, f32x4{0.f, 0.f, 0.f, 0.f});
  *reinterpret_cast<float4 *>(&sm.t.tt[16 * I + r][16 * J + 4 * g]) = make_float4(t[0], t[1], t[2], t[3]);
}

// One (chunk, value head) item of the prep kernel: where its record goes and
// which tokens it covers (valid is false for a flat index that names no chunk).
struct PrepItem {
  int64_t t0;
  int L, h;
  bool valid;
};

__device__ __forceinline__ PrepItem prep_item(const KdaParams &p, int64_t item) {
  PrepItem it;
  const int64_t jb = item / p.HV;
  it.h = (int)(item - jb * p.HV);
  const int64_t F = p.F0 + jb;
  // the sequence owning flat chunk F: the last n with base(n) <= F
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (flat_base(p.cu_seqlens, mid) <= F) lo = mid;
    else hi = mid - 1;
  }
  const int64_t bos = p.cu_seqlens[lo], eos = p.cu_seqlens[lo + 1];
  it.t0 = bos + 64 * (F - flat_base(p.cu_seqlens, lo));
  it.valid = it.t0 < eos;
  it.L = it.valid ? (int)min<int64_t>(C, eos - it.t0) : 1;
  if (!it.valid) it.t0 = 0;   // (loads of such an item read token 0 and are not used)
  return it;
}

// A lane's raw inputs of one item: token 16w + r, channels 32s + slot_k(g, j)
// (gate fp32, keys and queries bf16 pairs), and beta; held in registers from
// one item to the next so that their loads overlap the previous item's work.
template <int D>
struct PrepIn {
  static constexpr int NS = D / 32;
  typename U32Vec<8 * NS>::type g;
  typename U32Vec<4 * NS>::type k, q;
  float beta;
};

template <int D, bool DELTA>
__device__ __forceinline__ void prep_load(PrepIn<D> &in, const KdaParams &p, const PrepItem &it, int w,
                                          int r, int g) {
  constexpr int NS = D / 32;
  const int i = 16 * w + r;
  const int64_t t = it.t0 + min(i, it.L - 1);
  const int hk = it.h / p.ratio;
  const float *gp = p.g + (t * p.HV + it.h) * (int64_t)D;
  const uint16_t *kp = static_cast<const uint16_t *>(p.k) + t * p.k_stride + (int64_t)hk * D;
  const uint16_t *qp = static_cast<const uint16_t *>(p.q) + t * p.q_stride + (int64_t)hk * D;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int col = 32 * s + 16 * hf + 4 * g;
      const float4 g4 = *reinterpret_cast<const float4 *>(gp + col);
      const uint2 k2 = *reinterpret_cast<const uint2 *>(kp + col);
      const uint2 q2 = *reinterpret_cast<const uint2 *>(qp + col);
      const int u = 2 * s + hf;
      in.g[4 * u] = __float_as_uint(g4.x);
      in.g[4 * u + 1] = __float_as_uint(g4.y);
      in.g[4 * u + 2] = __float_as_uint(g4.z);
      in.g[4 * u + 3] = __float_as_uint(g4.w);
      in.k[2 * u] = k2.x;
      in.k[2 * u + 1] = k2.y;
      in.q[2 * u] = q2.x;
      in.q[2 * u + 1] = q2.y;
    }
  in.beta = DELTA ? p.beta[t * p.HV + it.h] : 0.f;
}

// The diagonal 16x16 block of the Gram matrices of row block w, summed pair
// by pair (the token-parallel form of the diagonal interaction blocks on the
// KDA page, section 6), for a block whose channel decay is too strong for
// the factored form: lane (r, g) reloads its token's inputs, sums over its
// own channels k_i k_j e^{G_i - G_j} and q_i k_j e^{G_i - G_j} for every row
// j of the block (row j's key and gate fetched from lane (j, g)), and the
// four channel groups are then summed. Every exponent is <= 0 for j <= i.
template <int D, bool DELTA>
__device__ __forceinline__ void prep_exact_diagonal(const KdaParams &p, const PrepItem &it, int w, int r, int g,
                                                    float bi, f32x4 (&rv)[4], f32x4 (&av)[4]) {
  constexpr int NS = D / 32;
  PrepIn<D> in;
  prep_load<D, DELTA>(in, p, it, w, r, g);
  const bool ok = 16 * w + r < it.L;
  float gv[NS][8], kv[NS][8], qv[NS][8];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int u = 2 * s + hf;
      const uint32_t kw[2] = {in.k[2 * u], in.k[2 * u + 1]}, qw[2] = {in.q[2 * u], in.q[2 * u + 1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gv[s][4 * hf + j] = ok ? __uint_as_float(in.g[4 * u + j]) : 0.f;
        kv[s][4 * hf + j] = ok ? ((j & 1) ? bf_hi(kw[j >> 1]) : bf_lo(kw[j >> 1])) : 0.f;
        qv[s][4 * hf + j] = ok ? ((j & 1) ? bf_hi(qw[j >> 1]) : bf_lo(qw[j >> 1])) : 0.f;
      }
    }
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = gv[s][j];
      x = dpp_add<0x111, 0xf>(x);
      x = dpp_add<0x112, 0xf>(x);
      x = dpp_add<0x114, 0xf>(x);
      x = dpp_add<0x118, 0xf>(x);
      gv[s][j] = x;
    }
  f32x4 rr = {0.f, 0.f, 0.f, 0.f}, ra = rr;
  for (int jj = 0; jj < 16; ++jj) {
    const int src = 16 * g + jj;
    float sr = 0.f, sa = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float kj = __shfl(kv[s][j], src, 64), gj = __shfl(gv[s][j], src, 64);
        const float t = kj * __expf(fminf(gv[s][j] - gj, 0.f));   // (pairs j > i are masked below)
        if constexpr (DELTA) sr += kv[s][j] * t;
        sa += qv[s][j] * t;
      }
    if constexpr (DELTA) sr = sum_lane_rows(sr);
    sa = sum_lane_rows(sa);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (jj == 4 * g + e) {
        rr[e] = sr;
        ra[e] = sa;
      }
  }
  f32x4 dr, da;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int jj = 4 * g + e;
    dr[e] = jj < r ? bi * rr[e] : 0.f;
    da[e] = jj <= r ? p.scale * ra[e] : 0.f;
  }
#pragma unroll
  for (int J = 0; J < 4; ++J)
    if (J == w) {
      rv[J] = dr;
      av[J] = da;
    }
}

// Persistent: each workgroup takes items blockIdx.x, blockIdx.x + gridDim.x, ...
// and loads the next item's inputs while it works on the current one.
// DELTA false (the linear rule, GLA's channel-gated linear attention): no
// correction (Vb = V), so no R, T or W: the record's region 1 is not
// written, and the state kernel's linear variant neither reads it.
template <int D, bool DELTA>
__global__ __launch_bounds__(256, 2) void kda_prep_kernel(KdaParams p) {
  using RC = KdaRec<D>;
  using SM = PrepSmem<D>;
  constexpr int NS = RC::NS, NT = RC::NT, PK = SM::PK;
  __shared__ SM sm;

  const int HV = p.HV;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int i = 16 * w + r;   // this lane's token
  const int64_t items = (p.F1 - p.F0) * HV;
  int64_t item = blockIdx.x;
  PrepItem nx = prep_item(p, item);
  PrepIn<D> in;
  prep_load<D, DELTA>(in, p, nx, w, r, g);
  for (; item < items; item += gridDim.x) {
    const PrepItem it = nx;
    const bool ok = i < it.L;
    float gv[NS][8], kv[NS][8], qv[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int u = 2 * s + hf;
        const uint32_t kw[2] = {in.k[2 * u], in.k[2 * u + 1]}, qw[2] = {in.q[2 * u], in.q[2 * u + 1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          gv[s][4 * hf + j] = ok ? __uint_as_float(in.g[4 * u + j]) : 0.f;
          kv[s][4 * hf + j] = ok ? ((j & 1) ? bf_hi(kw[j >> 1]) : bf_lo(kw[j >> 1])) : 0.f;
          qv[s][4 * hf + j] = ok ? ((j & 1) ? bf_hi(qw[j >> 1]) : bf_lo(qw[j >> 1])) : 0.f;
        }
      }
    if (g == 0) sm.beta[i] = ok ? in.beta : 0.f;
    // the next item's inputs are loaded once this item's operands are formed
    // (below), so that their registers are free meanwhile
    auto prefetch = [&]() {
      if (item + gridDim.x < items) {
        nx = prep_item(p, item + gridDim.x);
        prep_load<D, DELTA>(in, p, nx, w, r, g);
      }
    };
    if (!it.valid) prefetch();
    if (it.valid) {
      const int h = it.h;
      const int L = it.L;
      char *rec = p.rec + item * (int64_t)RC::BYTES;
      (void)L;

  // ---- gate prefix sums within the 16-token block (DPP row scan over r):
  //      gv becomes the log-decay from the start of the lane's block ----
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = gv[s][j];
      x = dpp_add<0x111, 0xf>(x);
      x = dpp_add<0x112, 0xf>(x);
      x = dpp_add<0x114, 0xf>(x);
      x = dpp_add<0x118, 0xf>(x);
      gv[s][j] = x;
    }
  if (r == 15) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 32 * s + 16 * hf + 4 * g;
        const float *x = &gv[s][4 * hf];
        *reinterpret_cast<float4 *>(&sm.tot[w][c0]) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4 *>(&sm.etot[w][c0]) =
            make_float4(__expf(x[0]), __expf(x[1]), __expf(x[2]), __expf(x[3]));
      }
  }
  __syncthreads();
  if (tid < D) {
    const float Gl = ((sm.tot[0][tid] + sm.tot[1][tid]) + sm.tot[2][tid]) + sm.tot[3][tid];
    reinterpret_cast<float *>(rec + RC::GAM)[tid] = __expf(Gl);
    const float e1 = sm.etot[1][tid], e2 = sm.etot[2][tid], e3 = sm.etot[3][tid];
    sm.fend[0][tid] = e1 * (e2 * e3);
    sm.fend[1][tid] = e2 * e3;
    sm.fend[2][tid] = e3;
    sm.fend[3][tid] = 1.f;
    sm.dmid[0][tid] = e1;
    sm.dmid[1][tid] = e2;
    sm.dmid[2][tid] = e1 * e2;
  }

  // ---- operands of this lane's token i (G_i = B_w + gv, B_w the log-decay
  //      before block w): every factor below but the diagonal-block one is
  //      an exponential of a non-positive number ----
  //   nk, nq  the Gram rows, decayed from the start of block w: k e^{gv},
  //           s q e^{gv}
  //   md      the diagonal block's key operand, k e^{-gv} (<= e^{span}),
  //           multiplied into the diagonal tile right away
  //   kd      the key decayed to the end of block w, k e^{tot_w - gv} (LDS)
  //   kl      K_l = nk e^{B_w} (LDS); Q^ = nq e^{B_w} (record)
  // The strongest decay of any channel over block w decides the diagonal
  // tile's form: up to 80 the factors e^{-gv} stay far inside the fp32
  // range and the tile is the product md^T (nk, nq) (transposed, as the
  // other tiles below); beyond, it is summed pair by pair.
  float span = 0.f;
  for (int c = lane; c < D; c += 64) span = fmaxf(span, -sm.tot[w][c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) span = fmaxf(span, __shfl_xor(span, off, 64));
  const bool fast = __builtin_amdgcn_readfirstlane(__float_as_int(span)) <= __float_as_int(80.f);
  Frag nk[NS], nq[NS];
  f32x4 rdiag = {0.f, 0.f, 0.f, 0.f}, adiag = rdiag;
  const float sc = p.scale;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    float a[8], b[8], c8[8], d[8], e[8], f[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int c0 = 32 * s + 16 * hf + 4 * g;
      const float4 tw = *reinterpret_cast<const float4 *>(&sm.tot[w][c0]);
      float4 eb = make_float4(1.f, 1.f, 1.f, 1.f);   // e^{B_w}: the decay of the earlier blocks
      for (int w2 = 0; w2 < w; ++w2) {
        const float4 x = *reinterpret_cast<const float4 *>(&sm.etot[w2][c0]);
        eb.x *= x.x; eb.y *= x.y; eb.z *= x.z; eb.w *= x.w;
      }
      const float twv[4] = {tw.x, tw.y, tw.z, tw.w}, ebv[4] = {eb.x, eb.y, eb.z, eb.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * hf + jj;
        const float G = gv[s][j];
        const float e1 = __expf(G);
        a[j] = kv[s][j] * e1;                        // nk
        c8[j] = (sc * qv[s][j]) * e1;                // nq
        b[j] = kv[s][j] * __expf(-G);                // md
        d[j] = kv[s][j] * __expf(twv[jj] - G);       // kd
        e[j] = a[j] * ebv[jj];                       // K_l
        f[j] = c8[j] * ebv[jj];                      // Q^
      }
    }
    // slot j of step s sits at physical column 32s + 8g + j (perm32)
    float *pl = &sm.kl[i][32 * s + 8 * g];
    float *pd = &sm.kd[i][32 * s + 8 * g];
    *reinterpret_cast<float4 *>(pl) = make_float4(e[0], e[1], e[2], e[3]);
    *reinterpret_cast<float4 *>(pl + 4) = make_float4(e[4], e[5], e[6], e[7]);
    *reinterpret_cast<float4 *>(pd) = make_float4(d[0], d[1], d[2], d[3]);
    *reinterpret_cast<float4 *>(pd + 4) = make_float4(d[4], d[5], d[6], d[7]);
    split8(a, nk[s]);
    split8(c8, nq[s]);
    if (fast) {
      Frag md;
      split8(b, md);
      if constexpr (DELTA) rdiag = mm<true, true>(md, nk[s], rdiag);
      adiag = mm<true, true>(md, nq[s], adiag);
    }
    Frag fq;
    split8(f, fq);
    st_frag(rec, RC::R2 + RC::wq(w, s), lane, fq);
  }
  prefetch();
  __syncthreads();

  // ---- Grams of row block w: tile (w, J) computed transposed (keys of
  //      block J as the M operand), so lane (r, g) holds row 16w + r,
  //      columns 16J + 4g .. +3. For J < w the keys are those of block J
  //      decayed to the start of block w (kd times the decay of the blocks
  //      between, <= 1 per channel); tile (w, w) is the diagonal above ----
  f32x4 rv[4], av[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    f32x4 ar = {0.f, 0.f, 0.f, 0.f}, aa = ar;
    if (J == w) {
      ar = rdiag;
      aa = adiag;
    } else if (J < w) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float *src = &sm.kd[16 * J + r][32 * s + 8 * g];
        const float4 x0 = *reinterpret_cast<const float4 *>(src);
        const float4 x1 = *reinterpret_cast<const float4 *>(src + 4);
        float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        if (J + 1 < w) {
          const float *dm = sm.dmid[w == 2 ? 0 : (J == 1 ? 1 : 2)];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const float4 y = *reinterpret_cast<const float4 *>(&dm[32 * s + 16 * hf + 4 * g]);
            x[4 * hf] *= y.x; x[4 * hf + 1] *= y.y; x[4 * hf + 2] *= y.z; x[4 * hf + 3] *= y.w;
          }
        }
        Frag fk;
        split8(x, fk);
        if constexpr (DELTA) ar = mm<true, true>(fk, nk[s], ar);
        aa = mm<true, true>(fk, nq[s], aa);
      }
    }
    const float bi = sm.beta[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = 4 * g + e;
      rv[J][e] = (J < w || (J == w && jj < r)) ? bi * ar[e] : 0.f;
      av[J][e] = (J < w || (J == w && jj <= r)) ? aa[e] : 0.f;
    }
  }
  if (!fast) prep_exact_diagonal<D, DELTA>(p, it, w, r, g, sm.beta[i], rv, av);

  // A^ fragments of row block w
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (2 * s <= w) {
      const float x[8] = {av[2 * s][0], av[2 * s][1], av[2 * s][2], av[2 * s][3],
                          av[2 * s + 1][0], av[2 * s + 1][1], av[2 * s + 1][2], av[2 * s + 1][3]};
      Frag f;
      split8(x, f);
      st_frag(rec, RC::R2 + RC::tp(pair_index(w, s)), lane, f);
    }
  }
  // K_end^T fragments (update operands): the keys decayed to the chunk's
  // end, kd times the decay of the blocks after the key's own; wave w takes
  // fragments w, w + 4, ...
#pragma unroll
  for (int u = 0; u < NT / 2; ++u) {
    const int fi = w + 4 * u;
    const int m = fi >> 1, s = fi & 1;
    const int ch = 16 * m + r, pc = perm32(ch);
    // tokens of slots 0-3 lie in block 2s, those of slots 4-7 in block 2s + 1
    const float fe0 = sm.fend[2 * s][ch], fe1 = sm.fend[2 * s + 1][ch];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sm.kd[32 * s + slot_k(g, j)][pc] * (j < 4 ? fe0 : fe1);
    Frag f;
    split8(x, f);
    st_frag(rec, RC::kf(m, s), lane, f);
  }
  __syncthreads();   // kd is dead: its storage holds T from here on

  // (the linear rule stops here: its records need no region 1)
  if constexpr (DELTA) {
  // ---- T = (I + R)^{-1}: diagonal blocks in registers, then the blocks
  //      below the diagonal by block forward substitution (three rounds) ----
  {
    f32x4 rdg = rv[0];
    if (w == 1) rdg = rv[1];
    if (w == 2) rdg = rv[2];
    if (w == 3) rdg = rv[3];
    *reinterpret_cast<float4 *>(&sm.t.rd[w][r][4 * g]) = make_float4(-rdg[0], -rdg[1], -rdg[2], -rdg[3]);
    float nn[16], tq[4];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const float4 v4 = *reinterpret_cast<const float4 *>(&sm.t.rd[w][r][4 * i4]);
      nn[4 * i4] = v4.x; nn[4 * i4 + 1] = v4.y; nn[4 * i4 + 2] = v4.z; nn[4 * i4 + 3] = v4.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tq[e] = (r == 4 * g + e) ? 1.f : 0.f;
    unit_lower_inverse16(tq, nn);
    *reinterpret_cast<float4 *>(&sm.t.tt[16 * w + r][16 * w + 4 * g]) = make_float4(tq[0], tq[1], tq[2], tq[3]);
  }
  __syncthreads();
  if (w == 1) t_block<1, 0, D>(sm, rv, r, g);
  if (w == 2) t_block<2, 1, D>(sm, rv, r, g);
  if (w == 3) t_block<3, 2, D>(sm, rv, r, g);
  __syncthreads();
  if (w == 2) t_block<2, 0, D>(sm, rv, r, g);
  if (w == 3) t_block<3, 1, D>(sm, rv, r, g);
  __syncthreads();
  if (w == 3) t_block<3, 0, D>(sm, rv, r, g);
  __syncthreads();

  // ---- T' = T Diag(beta) fragments (all six in every wave: B operands of W) ----
  Frag tf[6];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (2 * s > I) continue;
      float x[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c0 = 32 * s + 16 * hf + 4 * g;
        const bool live = 2 * s + hf <= I;   // blocks above the diagonal are zero
        const float4 tv = *reinterpret_cast<const float4 *>(&sm.t.tt[16 * I + r][c0]);
        const float4 bv = *reinterpret_cast<const float4 *>(&sm.beta[c0]);
        x[4 * hf] = live ? tv.x * bv.x : 0.f;
        x[4 * hf + 1] = live ? tv.y * bv.y : 0.f;
        x[4 * hf + 2] = live ? tv.z * bv.z : 0.f;
        x[4 * hf + 3] = live ? tv.w * bv.w : 0.f;
      }
      split8(x, tf[pair_index(I, s)]);
    }
#pragma unroll
  for (int pr = 0; pr < 6; ++pr)
    if (pr % 4 == w) st_frag(rec, RC::tp(pr), lane, tf[pr]);

  // ---- W^T = K_l^T T'^T: wave w < NS forms key tiles m = 2w, 2w + 1, which
  //      are exactly the W fragments (I, s = w); the record holds -W ----
  if (w < NS) {
    f32x4 acc[2][4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int m = 2 * w + h2;
      const int pc = perm32(16 * m + r);
      Frag fa[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = sm.kl[32 * s + slot_k(g, j)][pc];
        split8(x, fa[s]);
      }
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
          if (2 * s <= I) a = mm<true, true>(fa[s], tf[pair_index(I, s)], a);
        acc[h2][I] = a;
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const float x[8] = {-acc[0][I][0], -acc[0][I][1], -acc[0][I][2], -acc[0][I][3],
                          -acc[1][I][0], -acc[1][I][1], -acc[1][I][2], -acc[1][I][3]};
      Frag f;
      split8(x, f);
      st_frag(rec, RC::R1 + RC::wq(I, w), lane, f);
    }
  }
  }   // DELTA
    }
    __syncthreads();   // the next item reuses the LDS
  }
}

// ===========================================================================
// state kernel
// ===========================================================================

constexpr int NLW = 4;   // loader waves of regions 1 and 3 (and values, gamma)
constexpr int NLO = 2;   // loader waves of region 2

// A workgroup owns 16 NSW value columns: NSW chain waves (16 columns each:
// the state, U, Vb and the update), NSW output waves (the outputs of the same
// columns, one chunk behind), NLW loader waves for the chain's operands and
// NLO for the output waves'.
template <int D, int NSW>
struct StateSmem {
  static constexpr int VP = 16 * NSW + 16;  // pitch (bf16) of the value tile
  static constexpr int XB = (KdaRec<D>::NS + 2) * 2048;   // exchange: S^T fragments, then Vb's
  alignas(16) char rec[KdaRec<D>::BYTES];   // the current chunk's record
  alignas(16) uint16_t vv[C][VP];           // its values: 64 tokens x 16 NSW columns
  alignas(16) char xs[NSW][XB];             // chain wave -> output wave, per column block
  int ready[3];                             // loader waves: regions stored (NLW, NLO, NLW per chunk)
  int freed[3];                             // regions released (NSW per chunk; region 2 by the output waves)
  int xready[NSW];                          // chain wave: chunks published to xs
  int xfree[NSW];                           // output wave: chunks read from xs
};

// A loader lane's share of one chunk's record and values, in registers
// (vector types, not arrays, so that they stay there): region 1 with the
// values (LoadR1), region 3 with gamma (LoadR3), region 2 (LoadR2).
template <int D>
struct LoadN {
  static constexpr int N1 = KdaRec<D>::R1_BLOCKS / NLW;   // 1 KB blocks per loader wave
  static constexpr int N3 = KdaRec<D>::R3_BLOCKS / NLW;
};
template <int NSW>
constexpr int value_units() { return (128 * NSW + 64 * NLW - 1) / (64 * NLW); }   // 16-byte units per lane
template <int D, int NSW>
struct LoadR1 {
  typename U32Vec<4 * LoadN<D>::N1>::type r1;
  typename U32Vec<4 * value_units<NSW>()>::type v;
};
template <int D>
struct LoadR3 {
  typename U32Vec<4 * LoadN<D>::N3>::type r3;
  typename U32Vec<4>::type gam;
};
template <int D>
struct LoadR2 {
  typename U32Vec<4 * KdaRec<D>::R1_BLOCKS / NLO>::type r2;
};

// (the linear rule needs no region 1: its corrected values are the values)
template <int D, int NSW, bool DELTA>
__device__ __forceinline__ void issue_r1(LoadR1<D, NSW> &l1, const KdaParams &p, const char *rec,
                                         int64_t t0, int L, int h, int vb, int lw, int lane) {
  const char *base = rec + 16 * lane;
  if constexpr (DELTA) {
#pragma unroll
    for (int u = 0; u < LoadN<D>::N1; ++u)
      put4(l1.r1, u, *reinterpret_cast<const uint4 *>(base + KdaRec<D>::R1 + 1024 * (lw + NLW * u)));
  }
  // values: 64 rows of 2 NSW 16-byte units
  const uint16_t *vb_ = static_cast<const uint16_t *>(p.v) + (int64_t)h * D + 16 * NSW * vb;
#pragma unroll
  for (int u = 0; u < value_units<NSW>(); ++u) {
    const int q = 64 * lw + lane + 64 * NLW * u;
    const int row = min(q / (2 * NSW), C - 1);
    const int64_t tr = t0 + min(row, L - 1);
    const uint4 x = *reinterpret_cast<const uint4 *>(vb_ + tr * p.v_stride + 8 * (q % (2 * NSW)));
    put4(l1.v, u, row < L ? x : make_uint4(0, 0, 0, 0));
  }
}

template <int D>
__device__ __forceinline__ void issue_r3(LoadR3<D> &l3, const char *rec, int lw, int lane) {
  const char *base = rec + 16 * lane;
#pragma unroll
  for (int u = 0; u < LoadN<D>::N3; ++u)
    put4(l3.r3, u, *reinterpret_cast<const uint4 *>(base + KdaRec<D>::R3 + 1024 * (lw + NLW * u)));
  if (lw == 0 && lane < D / 4) put4(l3.gam, 0, *reinterpret_cast<const uint4 *>(base + KdaRec<D>::GAM));
}

template <int D>
__device__ __forceinline__ void issue_r2(LoadR2<D> &l2, const char *rec, int lw, int lane) {
  const char *base = rec + 16 * lane;
#pragma unroll
  for (int u = 0; u < KdaRec<D>::R1_BLOCKS / NLO; ++u)
    put4(l2.r2, u, *reinterpret_cast<const uint4 *>(base + KdaRec<D>::R2 + 1024 * (lw + NLO * u)));
}

template <int D, int NSW, bool DELTA>
__device__ __forceinline__ void store_r1(const LoadR1<D, NSW> &l1, StateSmem<D, NSW> &sm, int lw, int lane) {
  char *base = sm.rec + 16 * lane;
  if constexpr (DELTA) {
#pragma unroll
    for (int u = 0; u < LoadN<D>::N1; ++u)
      *reinterpret_cast<uint4 *>(base + KdaRec<D>::R1 + 1024 * (lw + NLW * u)) = get4(l1.r1, u);
  }
#pragma unroll
  for (int u = 0; u < value_units<NSW>(); ++u) {
    const int q = 64 * lw + lane + 64 * NLW * u;
    if (q < 128 * NSW) *reinterpret_cast<uint4 *>(&sm.vv[q / (2 * NSW)][8 * (q % (2 * NSW))]) = get4(l1.v, u);
  }
}

template <int D, int NSW>
__device__ __forceinline__ void store_r3(const LoadR3<D> &l3, StateSmem<D, NSW> &sm, int lw, int lane) {
  char *base = sm.rec + 16 * lane;
#pragma unroll
  for (int u = 0; u < LoadN<D>::N3; ++u)
    *reinterpret_cast<uint4 *>(base + KdaRec<D>::R3 + 1024 * (lw + NLW * u)) = get4(l3.r3, u);
  if (lw == 0 && lane < D / 4) *reinterpret_cast<uint4 *>(base + KdaRec<D>::GAM) = get4(l3.gam, 0);
}

template <int D, int NSW>
__device__ __forceinline__ void store_r2(const LoadR2<D> &l2, StateSmem<D, NSW> &sm, int lw, int lane) {
  char *base = sm.rec + 16 * lane;
#pragma unroll
  for (int u = 0; u < KdaRec<D>::R1_BLOCKS / NLO; ++u)
    *reinterpret_cast<uint4 *>(base + KdaRec<D>::R2 + 1024 * (lw + NLO * u)) = get4(l2.r2, u);
}

// DELTA false: the linear rule (GLA), Vb = V, region 1 neither loaded nor used.
template <int D, int NSW, bool DELTA>
__global__ __launch_bounds__(64 * (2 * NSW + NLW + NLO)) void kda_state_kernel(KdaParams p) {
  using RC = KdaRec<D>;
  using SM = StateSmem<D, NSW>;
  constexpr int NS = RC::NS, NT = RC::NT;
  constexpr int GRP = D / (16 * NSW);   // workgroups per (sequence, value head)
  __shared__ SM sm;

  // all workgroups of one (sequence, head) get ids equal modulo 8 (one XCD,
  // one L2 for the records they share)
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7);
  if (gi >= p.N * p.HV) return;
  const int vb = (b >> 3) % GRP;
  const int n = gi / p.HV;
  const int h = gi - n * p.HV;

  const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  const int64_t base = flat_base(p.cu_seqlens, n);
  const int64_t nc = (eos - bos + C - 1) / C;
  const int64_t cb = max<int64_t>(p.F0 - base, 0), ce = min<int64_t>(p.F1 - base, nc);

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int pw = w < NSW ? w : w - NSW;            // column block of a chain / output wave
  const int col = 16 * NSW * vb + 16 * pw + r;    // the value column this lane owns
  const int64_t slot = p.slot_idx[n];
  const int64_t pbase = (slot * p.HV + h) * (int64_t)(D * D) + col;

  if (nc == 0) {
    // a zero-length sequence writes its initial state back: zeros under
    // ZERO_INIT (once, in the slice holding its flat index), else nothing
    if (p.zero_init && w < NSW && base >= p.F0 && base < p.F1) {
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t idx = pbase + (int64_t)(16 * m + 4 * g + e) * D;
          if (p.st_bf16) static_cast<uint16_t *>(p.pool)[idx] = 0;
          else static_cast<float *>(p.pool)[idx] = 0.f;
        }
    }
    return;
  }
  if (cb >= ce) return;

  if (tid < 6 + 2 * NSW) {
    int *ctr = tid < 3 ? &sm.ready[tid] : tid < 6 ? &sm.freed[tid - 3]
             : tid < 6 + NSW ? &sm.xready[tid - 6] : &sm.xfree[tid - 6 - NSW];
    *ctr = 0;
  }
  __syncthreads();

  auto rec_of = [&](int64_t c) -> const char * {
    return p.rec + ((base + c - p.F0) * p.HV + h) * (int64_t)RC::BYTES;
  };

  if (w >= 2 * NSW + NLW) {
    // ================= region-2 loader waves: two chunks ahead =================
    const int lw = w - 2 * NSW - NLW;
    // (Every refill is issued, past the slice's last chunk as a reload of that
    // chunk, so each loop trip issues the same loads and the compiler's
    // memory-counter waits before a store cover only the loads it reads.)
    auto last = [&](int64_t c) { return c < ce ? c : ce - 1; };
    LoadR2<D> a0, a1;
    issue_r2<D>(a0, rec_of(cb), lw, lane);
    store_r2<D, NSW>(a0, sm, lw, lane);
    count_in(&sm.ready[1], lane);
    issue_r2<D>(a1, rec_of(last(cb + 1)), lw, lane);
    issue_r2<D>(a0, rec_of(last(cb + 2)), lw, lane);
    auto step = [&](LoadR2<D> &l2, int64_t c) {
      const int k = (int)(c - cb);
      spin_until(&sm.freed[1], NSW * (k + 1));
      store_r2<D, NSW>(l2, sm, lw, lane);
      count_in(&sm.ready[1], lane);
      issue_r2<D>(l2, rec_of(last(c + 3)), lw, lane);
    };
    for (int64_t c = cb; c + 1 < ce; c += 2) {
      step(a1, c);
      if (c + 2 < ce) step(a0, c + 1);
    }
    return;
  }
  if (w >= 2 * NSW) {
    // ================= region-1 / region-3 loader waves =================
    // Region 1 and the values (the first operands of a chunk) are loaded
    // two chunks ahead, alternating between two register sets; region 3 one
    // chunk ahead (it is used at the end of its chunk).
    const int lw = w - 2 * NSW;
    LoadR1<D, NSW> s0, s1;
    LoadR3<D> l3;
    auto i1 = [&](LoadR1<D, NSW> &l1, int64_t c) {
      const int64_t t0 = bos + C * c;
      issue_r1<D, NSW, DELTA>(l1, p, rec_of(c), t0, (int)min<int64_t>(C, eos - t0), h, vb, lw, lane);
    };
    i1(s0, cb);
    issue_r3<D>(l3, rec_of(cb), lw, lane);
    store_r1<D, NSW, DELTA>(s0, sm, lw, lane);
    store_r3<D, NSW>(l3, sm, lw, lane);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) {
      atomicAdd(&sm.ready[0], 1);
      atomicAdd(&sm.ready[2], 1);
    }
    auto last = [&](int64_t c) { return c < ce ? c : ce - 1; };
    i1(s1, last(cb + 1));
    issue_r3<D>(l3, rec_of(last(cb + 1)), lw, lane);
    i1(s0, last(cb + 2));
    // Store chunk c + 1's regions as chunk c releases them (region 1 early
    // in chunk c, region 3 at its end), each followed by the loads that
    // refill its registers.
    auto step = [&](LoadR1<D, NSW> &l1, int64_t c) {
      const int k = (int)(c - cb);
      spin_until(&sm.freed[0], NSW * (k + 1));
      store_r1<D, NSW, DELTA>(l1, sm, lw, lane);
      count_in(&sm.ready[0], lane);
      spin_until(&sm.freed[2], NSW * (k + 1));
      store_r3<D, NSW>(l3, sm, lw, lane);
      count_in(&sm.ready[2], lane);
      issue_r3<D>(l3, rec_of(last(c + 2)), lw, lane);
      i1(l1, last(c + 3));
    };
    for (int64_t c = cb; c + 1 < ce; c += 2) {
      step(s1, c);
      if (c + 2 < ce) step(s0, c + 1);
    }
    return;
  }

  char *xs = sm.xs[pw];
  const int64_t HVD = (int64_t)p.HV * D;

  if (w >= NSW) {
    // ================= output waves: O = Q^ S^T + A^ Vb, one chunk behind the chain =================
    for (int64_t c = cb; c < ce; ++c) {
      const int k = (int)(c - cb);
      const int64_t t0 = bos + C * c;
      const int L = (int)min<int64_t>(C, eos - t0);
      Frag sf[NS], vbf[2];
      spin_until(&sm.xready[pw], k + 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) ld_frag(xs, 2048 * s, lane, sf[s]);
#pragma unroll
      for (int s = 0; s < 2; ++s) ld_frag(xs, 2048 * (NS + s), lane, vbf[s]);
      count_in(&sm.xfree[pw], lane);

      spin_until(&sm.ready[1], NLO * (k + 1));
      f32x4 oa[4];
      {
        Frag qf[2][4], aa[6];
#pragma unroll
        for (int I = 0; I < 4; ++I) ld_frag(sm.rec, RC::R2 + RC::wq(I, 0), lane, qf[0][I]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int I = 0; I < 4; ++I) oa[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 1 < NS) {
#pragma unroll
            for (int I = 0; I < 4; ++I) ld_frag(sm.rec, RC::R2 + RC::wq(I, s + 1), lane, qf[(s + 1) & 1][I]);
          } else {
#pragma unroll
            for (int pr = 0; pr < 6; ++pr) ld_frag(sm.rec, RC::R2 + RC::tp(pr), lane, aa[pr]);
          }
#pragma unroll
          for (int I = 0; I < 4; ++I) oa[I] = mpass<0>(qf[s & 1][I], sf[s], oa[I]);
#pragma unroll
          for (int I = 0; I < 4; ++I) oa[I] = mpass<1>(qf[s & 1][I], sf[s], oa[I]);
#pragma unroll
          for (int I = 0; I < 4; ++I) oa[I] = mpass<2>(qf[s & 1][I], sf[s], oa[I]);
          if (s + 1 < NS) interleave<8, 0, 1>();
          else interleave<12, 0, 1>();
          __builtin_amdgcn_sched_barrier(0);
        }
        // + A^ Vb (lower triangular: k steps s <= I / 2)
        oa[0] = mpass<0>(aa[0], vbf[0], oa[0]);
        oa[1] = mpass<0>(aa[1], vbf[0], oa[1]);
        oa[2] = mpass<0>(aa[2], vbf[0], oa[2]);
        oa[3] = mpass<0>(aa[4], vbf[0], oa[3]);
        oa[0] = mpass<1>(aa[0], vbf[0], oa[0]);
        oa[1] = mpass<1>(aa[1], vbf[0], oa[1]);
        oa[2] = mpass<1>(aa[2], vbf[0], oa[2]);
        oa[3] = mpass<1>(aa[4], vbf[0], oa[3]);
        oa[0] = mpass<2>(aa[0], vbf[0], oa[0]);
        oa[1] = mpass<2>(aa[1], vbf[0], oa[1]);
        oa[2] = mpass<2>(aa[2], vbf[0], oa[2]);
        oa[3] = mpass<2>(aa[4], vbf[0], oa[3]);
        oa[2] = mpass<0>(aa[3], vbf[1], oa[2]);
        oa[3] = mpass<0>(aa[5], vbf[1], oa[3]);
        oa[2] = mpass<1>(aa[3], vbf[1], oa[2]);
        oa[3] = mpass<1>(aa[5], vbf[1], oa[3]);
        oa[2] = mpass<2>(aa[3], vbf[1], oa[2]);
        oa[3] = mpass<2>(aa[5], vbf[1], oa[3]);
      }
      count_in(&sm.freed[1], lane);

      // Buffer stores against a descriptor over this chunk's L output rows:
      // row 16I + e is a scalar offset and the lane part (row group 4g,
      // column) a fixed one; rows past a partial chunk's end fall outside the
      // descriptor and are dropped by the hardware.
      const uint32_t osz = p.out_bf16 ? 2u : 4u;
      const uint32_t orow = (uint32_t)HVD * osz;
      char *obase = static_cast<char *>(p.o) + (t0 * HVD + (int64_t)h * D) * osz;
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(obase, 0, (int)(L * orow), 0x00020000);
      const uint32_t olane = (uint32_t)(4 * g) * orow + (uint32_t)col * osz;
      if (!p.out_bf16) {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[I][e]), ors, olane,
                                                  (16 * I + e) * (int)orow, 0);
      } else {
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(oa[I][e]), ors, olane,
                                                  (16 * I + e) * (int)orow, 0);
      }
    }
    return;
  }

  // ================= chain waves =================
  f32x4 st[NT];   // st[m][e] = S^T[16m + 4g + e][col]
  if (cb == 0) {
#pragma unroll
    for (int m = 0; m < NT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!p.zero_init) {
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t idx = pbase + (int64_t)(16 * m + 4 * g + e) * D;
          st[m][e] = p.st_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p.pool)[idx])
                               : static_cast<const float *>(p.pool)[idx];
        }
    }
  } else {
    const float *cp = p.carry + ((int64_t)n * p.HV + h) * (int64_t)(D * D) + col;
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[m][e] = cp[(16 * m + 4 * g + e) * D];
  }

  for (int64_t c = cb; c < ce; ++c) {
    const int k = (int)(c - cb);

    // S^T as B fragments over key rows 32s .. 32s + 31, also handed to the
    // output wave once it has read the previous chunk's
    Frag sf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) chainfrag(st[2 * s], st[2 * s + 1], sf[s]);
    spin_until(&sm.xfree[pw], k);
#pragma unroll
    for (int s = 0; s < NS; ++s) st_frag(xs, 2048 * s, lane, sf[s]);

    // ---- region 1: Vb = U + (-W) S^T with U = T' V (the record holds -W) ----
    // Each block of products issues one LDS read of the next block's
    // fragments after each MFMA (interleave), so reads and products overlap.
    spin_until(&sm.ready[0], NLW * (k + 1));
    f32x4 acc[4];
    if constexpr (!DELTA) {
      // linear rule: Vb = V, read in the accumulator layout (row 16I + 4g + i)
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[I][i] = bf16_to_f32(sm.vv[16 * I + 4 * g + i][16 * pw + r]);
    } else {
      Frag vf[2], ta[6], wf[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s) ldfrag_tr(&sm.vv[0][0], SM::VP, 16 * pw + 4 * (r & 3), s, r, g, vf[s]);
#pragma unroll
      for (int pr = 0; pr < 6; ++pr) ld_frag(sm.rec, RC::tp(pr), lane, ta[pr]);
      __builtin_amdgcn_sched_barrier(0);
      // U = T' V: four accumulators (T' split, V exact)
#pragma unroll
      for (int I = 0; I < 4; ++I) ld_frag(sm.rec, RC::wq(I, 0), lane, wf[0][I]);
#pragma unroll
      for (int I = 0; I < 4; ++I) acc[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[0] = mpass<0, false>(ta[0], vf[0], acc[0]);
      acc[1] = mpass<0, false>(ta[1], vf[0], acc[1]);
      acc[2] = mpass<0, false>(ta[2], vf[0], acc[2]);
      acc[3] = mpass<0, false>(ta[4], vf[0], acc[3]);
      acc[0] = mpass<2, false>(ta[0], vf[0], acc[0]);
      acc[1] = mpass<2, false>(ta[1], vf[0], acc[1]);
      acc[2] = mpass<2, false>(ta[2], vf[0], acc[2]);
      acc[3] = mpass<2, false>(ta[4], vf[0], acc[3]);
      acc[2] = mpass<0, false>(ta[3], vf[1], acc[2]);
      acc[3] = mpass<0, false>(ta[5], vf[1], acc[3]);
      acc[2] = mpass<2, false>(ta[3], vf[1], acc[2]);
      acc[3] = mpass<2, false>(ta[5], vf[1], acc[3]);
      interleave<8, 0, 1>();
      __builtin_amdgcn_sched_barrier(0);
      // + (-W) S^T, k step by k step
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + 1 < NS) {
#pragma unroll
          for (int I = 0; I < 4; ++I) ld_frag(sm.rec, RC::wq(I, s + 1), lane, wf[(s + 1) & 1][I]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) acc[I] = mpass<0>(wf[s & 1][I], sf[s], acc[I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) acc[I] = mpass<1>(wf[s & 1][I], sf[s], acc[I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) acc[I] = mpass<2>(wf[s & 1][I], sf[s], acc[I]);
        if (s + 1 < NS) interleave<8, 0, 1>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    count_in(&sm.freed[0], lane);

    // Vb to the output wave
    Frag vbf[2];
    chainfrag(acc[0], acc[1], vbf[0]);
    chainfrag(acc[2], acc[3], vbf[1]);
#pragma unroll
    for (int s = 0; s < 2; ++s) st_frag(xs, 2048 * (NS + s), lane, vbf[s]);
    count_in(&sm.xready[pw], lane);

    // ---- region 3: S^T <- gamma (.) S^T + K_end^T Vb, in blocks of four key
    //      tiles and one k step (four independent accumulators), the next
    //      block's fragments in flight ----
    spin_until(&sm.ready[2], NLW * (k + 1));
    {
      const float *gam = reinterpret_cast<const float *>(sm.rec + RC::GAM);
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const float4 gm = *reinterpret_cast<const float4 *>(gam + 16 * m + 4 * g);
        st[m][0] *= gm.x;
        st[m][1] *= gm.y;
        st[m][2] *= gm.z;
        st[m][3] *= gm.w;
      }
      constexpr int NB = NT / 4 * 2;   // blocks (key tile group, k step)
      Frag kf[2][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ld_frag(sm.rec, RC::kf(j, 0), lane, kf[0][j]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bk = 0; bk < NB; ++bk) {
        const int mg = bk >> 1, s = bk & 1;
        if (bk + 1 < NB) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            ld_frag(sm.rec, RC::kf(4 * ((bk + 1) >> 1) + j, (bk + 1) & 1), lane, kf[(bk + 1) & 1][j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st[4 * mg + j] = mpass<0>(kf[bk & 1][j], vbf[s], st[4 * mg + j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) st[4 * mg + j] = mpass<1>(kf[bk & 1][j], vbf[s], st[4 * mg + j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) st[4 * mg + j] = mpass<2>(kf[bk & 1][j], vbf[s], st[4 * mg + j]);
        if (bk + 1 < NB) interleave<8, 0, 1>();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    count_in(&sm.freed[2], lane);
  }

  // ---- state out: the pool at the sequence's end, else the carry ----
  if (ce == nc) {
    if (p.st_bf16) {
      uint16_t *sp = static_cast<uint16_t *>(p.pool) + pbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(16 * m + 4 * g + e) * D] = f32_to_bf16(st[m][e]);
    } else {
      float *sp = static_cast<float *>(p.pool) + pbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(16 * m + 4 * g + e) * D] = st[m][e];
    }
  } else {
    float *cp = p.carry + ((int64_t)n * p.HV + h) * (int64_t)(D * D) + col;
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) cp[(16 * m + 4 * g + e) * D] = st[m][e];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

size_t record_bytes(int D) { return D == 128 ? KdaRec<128>::BYTES : KdaRec<64>::BYTES; }

size_t carry_bytes(const gdr_args &a) {
  const size_t b = (size_t)a.N * a.HV * a.DK * a.DK * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

int64_t flat_chunks(const gdr_args &a) { return (a.T_total + C - 1) / C + a.N; }

// Records per slice the preferred workspace holds: about 192 MB of them, so a
// slice's records are still in the 256 MB last-level cache when the state
// kernel reads them.
constexpr size_t kSliceRecordBytes = (size_t)192 << 20;

template <int D, int NSW>
hipError_t launch_slices(const KdaParams &p0, int64_t flat, int64_t per, hipStream_t stream) {
  const int cus = cu_count();
  const int grp = D / (16 * NSW);
  const int sblocks = ((p0.N * p0.HV + 7) / 8) * 8 * grp;
  for (int64_t F0 = 0; F0 < flat; F0 += per) {
    KdaParams p = p0;
    p.F0 = F0;
    p.F1 = F0 + per < flat ? F0 + per : flat;
    const int64_t items = (p.F1 - p.F0) * p.HV;
    const int64_t pblocks = items < 2 * (int64_t)cus ? items : 2 * (int64_t)cus;   // two per compute unit
    if (p.delta)
      hipLaunchKernelGGL((kda_prep_kernel<D, true>), dim3((unsigned)pblocks), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((kda_prep_kernel<D, false>), dim3((unsigned)pblocks), dim3(256), 0, stream, p);
    if (p.delta)
      hipLaunchKernelGGL((kda_state_kernel<D, NSW, true>), dim3(sblocks), dim3(64 * (2 * NSW + NLW + NLO)), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((kda_state_kernel<D, NSW, false>), dim3(sblocks), dim3(64 * (2 * NSW + NLW + NLO)), 0,
                         stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t kda_wait_flag(int *out, bool clear, hipStream_t stream) {
  return chunk::wait_flag_access(out, clear, stream);
}

bool chunk_fwd_kda_applies(const gdr_args &a) {
  return a.in_dtype == GDR_BF16 && a.gate == GDR_GATE_CHANNEL && products_of(a) == 1;
}

size_t chunk_fwd_kda_min_workspace(const gdr_args &a) {
  return carry_bytes(a) + record_bytes(a.DK) * (size_t)a.HV;
}

size_t chunk_fwd_kda_workspace(const gdr_args &a) {
  const size_t row = record_bytes(a.DK) * (size_t)a.HV;   // one flat chunk of every head
  int64_t per = (int64_t)(kSliceRecordBytes / row);
  if (per < 1) per = 1;
  const int64_t flat = flat_chunks(a);
  if (per > flat) per = flat;
  return carry_bytes(a) + row * (size_t)per;
}

hipError_t launch_chunk_fwd_kda(const gdr_args &a, void *ws, size_t ws_bytes, hipStream_t stream) {
  KdaParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HK = a.HK; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  p.delta = a.rule == GDR_RULE_DELTA;
  const size_t cb = carry_bytes(a);
  p.carry = static_cast<float *>(ws);
  p.rec = static_cast<char *>(ws) + cb;
  const size_t row = record_bytes(a.DK) * (size_t)a.HV;
  const int64_t flat = flat_chunks(a);
  int64_t per = (int64_t)((ws_bytes - cb) / row);
  if (per > flat) per = flat;
  p.F0 = p.F1 = 0;
  // 16 value columns per workgroup: each workgroup reads the whole record of
  // every chunk, so narrow ones spread that LDS traffic over many compute
  // units (a batch with more (sequence, head) pairs than fit at once runs in
  // more than one round of workgroups).
  if (a.DK == 128) return launch_slices<128, 1>(p, flat, per, stream);
  return launch_slices<64, 1>(p, flat, per, stream);
}

}  // namespace gdr
