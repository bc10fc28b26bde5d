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
//   * kda_state_kernel, one workgroup of four waves per (sequence, value
//     head, 16 value columns) walks the slice's chunks in order: wave q
//     holds the key rows q DK/4 .. (q+1) DK/4 - 1 of S^T[DK, 16] in MFMA
//     accumulators and forms the Vb and output rows 16q .. 16q+15; each wave
//     loads the record fragments it multiplies straight into registers (one
//     set, each group reloaded with the next chunk's right after its last
//     use), and LDS carries only the state and Vb fragments every wave reads
//     whole, with two LDS-only barriers per chunk.
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
#include <numeric>

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

// A record fragment stored at the record's uniform base plus the fragment's
// offset (scalar) and a 32-bit lane offset voff = 16 x lane shared by every
// store, so that no 64-bit address per fragment occupies vector registers.
// (Global stores, not buffer stores: the compiler guards the data registers
// of a 128-bit global store against being rewritten before the store has
// read them, but assumes no such hazard for a buffer store whose scalar
// offset is a register, and on gfx950 such stores have been seen to write
// the registers' next contents.)
__device__ __forceinline__ void st_frag(char *rec, uint32_t voff, int off, const Frag &f) {
  char *base = rec + off;
  *reinterpret_cast<u32x4 *>(base + voff) = __builtin_bit_cast(u32x4, f.hi);
  *reinterpret_cast<u32x4 *>(base + 1024 + voff) = __builtin_bit_cast(u32x4, f.lo);
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

// The prep kernel keeps the gate in base-2 units (g log2 e), so that every
// decay factor is one v_exp_f32 (2^x) of a prefix-sum difference.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16, round to nearest even, by integer arithmetic. (The state
// kernel's write-back to a bf16 pool uses this rather than the hardware
// conversion: with the conversion instruction in that epilogue the compiler
// schedules the chunk loop differently and the kernel runs 3-4 % slower.)
__device__ __forceinline__ uint16_t rne_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Slot j of lane group g: offset of its k inside a 32-wide step.
__device__ __forceinline__ int slot_k(int g, int j) { return (j < 4 ? 4 * g + j : 12 + 4 * g + j); }

// ===========================================================================
// prep kernel
// ===========================================================================

template <int D>
struct PrepSmem {
  static constexpr int PK = D + 4;   // fp32 rows, key columns permuted (perm32)
  // (the small fixed-address arrays first, within the 64 KiB that an LDS
  // instruction's immediate offset reaches, so they need no address register)
  float tot[4][D];                   // per 16-token block: gate sum of each channel (<= 0)
  float etot[4][D];                  // its exponential: the block's decay of each channel
  float fend[4][D];                  // decay of the blocks after block b (keys to the chunk's end)
  float dmid[3][D];                  // decay of the blocks strictly between J and w: (2,0), (3,1), (3,0)
  float beta[C];
  float kl[C][PK];                   // K_l = e^{G} (.) K, token-major
  union {
    float kd[C][PK];                 // keys decayed to the end of their own 16-token block
    struct {
      float tt[C][C + 4];            // T, row-major (once the Grams are done)
      float rd[4][16][20];           // R's diagonal blocks, negated
    } t;
  };
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

// Item jb * HV + h: flat chunk F0 + jb, value head h.
__device__ __forceinline__ PrepItem prep_item(const KdaParams &p, int64_t jb, int h) {
  PrepItem it;
  it.h = h;
  const int64_t F = p.F0 + jb;
  // the sequence owning flat chunk F: the last n with base(n) <= F (the
  // offsets through scalar loads: uniform, and not queued behind the vector
  // stores of the item in flight)
  const int32_t *cu = p.cu_seqlens;
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)(scalar_load(cu + mid) >> 6) + mid <= F) lo = mid;
    else hi = mid - 1;
  }
  const int64_t bos = scalar_load(cu + lo), eos = scalar_load(cu + lo + 1);
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
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  // buffer loads against descriptors over the item's L token rows (scalar
  // bases, one lane offset per tensor); a lane past the chunk's end falls
  // outside them (its row offset alone passes the range) and reads zeros
  const int row = 16 * w + r;
  const int hk = it.h / p.ratio;
  const int64_t HVD = (int64_t)p.HV * D;
  const __amdgpu_buffer_rsrc_t gr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(p.g + it.t0 * HVD + (int64_t)it.h * D), 0, (int)((it.L - 1) * HVD * 4 + 4 * D),
      0x00020000);
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(p.k) + it.t0 * p.k_stride + (int64_t)hk * D), 0,
      (int)((it.L - 1) * p.k_stride * 2 + 2 * D), 0x00020000);
  const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(static_cast<const uint16_t *>(p.q) + it.t0 * p.q_stride + (int64_t)hk * D), 0,
      (int)((it.L - 1) * p.q_stride * 2 + 2 * D), 0x00020000);
  const uint32_t gv = (uint32_t)(row * HVD * 4) + 16u * g;
  const uint32_t kv = (uint32_t)(row * p.k_stride * 2) + 8u * g;
  const uint32_t qv = (uint32_t)(row * p.q_stride * 2) + 8u * g;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int col = 32 * s + 16 * hf;
      const u32x4 g4 = __builtin_amdgcn_raw_buffer_load_b128(gr, gv, 4 * col, 0);
      const u32x2 k2 = __builtin_amdgcn_raw_buffer_load_b64(kr, kv, 2 * col, 0);
      const u32x2 q2 = __builtin_amdgcn_raw_buffer_load_b64(qr, qv, 2 * col, 0);
      const int u = 2 * s + hf;
      in.g[4 * u] = g4[0];
      in.g[4 * u + 1] = g4[1];
      in.g[4 * u + 2] = g4[2];
      in.g[4 * u + 3] = g4[3];
      in.k[2 * u] = k2[0];
      in.k[2 * u + 1] = k2[1];
      in.q[2 * u] = q2[0];
      in.q[2 * u + 1] = q2[1];
    }
  if constexpr (DELTA) {
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(p.beta + it.t0 * p.HV + it.h), 0, (int)((it.L - 1) * p.HV * 4 + 4), 0x00020000);
    in.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(br, (uint32_t)(row * p.HV * 4), 0, 0));
  } else {
    in.beta = 0.f;
  }
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
  float gv[NS][8], kv[NS][8], qv[NS][8];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int u = 2 * s + hf;
      const uint32_t kw[2] = {in.k[2 * u], in.k[2 * u + 1]}, qw[2] = {in.q[2 * u], in.q[2 * u + 1]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gv[s][4 * hf + j] = __uint_as_float(in.g[4 * u + j]) * LOG2E;
        kv[s][4 * hf + j] = (j & 1) ? bf_hi(kw[j >> 1]) : bf_lo(kw[j >> 1]);
        qv[s][4 * hf + j] = (j & 1) ? bf_hi(qw[j >> 1]) : bf_lo(qw[j >> 1]);
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
        const float t = kj * exp2_(fminf(gv[s][j] - gj, 0.f));   // (pairs j > i are masked below)
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
  // (the wave index through readfirstlane, so that conditions on it are
  // scalar branches)
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15,
            g = lane >> 4;
  const int i = 16 * w + r;   // this lane's token
  const int64_t items = (p.F1 - p.F0) * HV;
  int64_t item = blockIdx.x;
  // item = jb * HV + h, advanced by the grid stride (dj, dh) without a
  // division per item
  const int dj = (int)(gridDim.x / HV), dh = (int)(gridDim.x - dj * HV);
  int64_t jb = blockIdx.x / HV;
  int hh = (int)(blockIdx.x - jb * HV);
  PrepItem nx = prep_item(p, jb, hh);
  PrepIn<D> in;
  prep_load<D, DELTA>(in, p, nx, w, r, g);
  for (; item < items; item += gridDim.x) {
    const PrepItem it = nx;
    float gv[NS][8], kv[NS][8], qv[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int u = 2 * s + hf;
        const uint32_t kw[2] = {in.k[2 * u], in.k[2 * u + 1]}, qw[2] = {in.q[2 * u], in.q[2 * u + 1]};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // (rows past the chunk's end were read as zeros)
          gv[s][4 * hf + j] = __uint_as_float(in.g[4 * u + j]) * LOG2E;
          kv[s][4 * hf + j] = (j & 1) ? bf_hi(kw[j >> 1]) : bf_lo(kw[j >> 1]);
          qv[s][4 * hf + j] = (j & 1) ? bf_hi(qw[j >> 1]) : bf_lo(qw[j >> 1]);
        }
      }
    if (g == 0) sm.beta[i] = in.beta;
    // the next item's inputs are loaded once this item's operands are formed
    // (below), so that their registers are free meanwhile
    auto prefetch = [&]() {
      if (item + gridDim.x < items) {
        jb += dj;
        hh += dh;
        if (hh >= HV) {
          hh -= HV;
          ++jb;
        }
        nx = prep_item(p, jb, hh);
        prep_load<D, DELTA>(in, p, nx, w, r, g);
      }
    };
    if (!it.valid) prefetch();
    if (it.valid) {
      const int h = it.h;
      const int L = it.L;
      char *rec = p.rec + item * (int64_t)RC::BYTES;
      const uint32_t voff = 16u * (uint32_t)lane;
      (void)L;

  // ---- gate prefix sums within the 16-token block (DPP row scan over r):
  //      gv becomes the log-decay (base 2) from the start of the lane's
  //      block ----
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
            make_float4(exp2_(x[0]), exp2_(x[1]), exp2_(x[2]), exp2_(x[3]));
      }
  }
  lds_barrier();
  if (tid < D) {
    const float Gl = ((sm.tot[0][tid] + sm.tot[1][tid]) + sm.tot[2][tid]) + sm.tot[3][tid];
    *reinterpret_cast<float *>(rec + RC::GAM + 4u * (uint32_t)tid) = exp2_(Gl);
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
  // tile's form: up to 80 (in natural-log units; 80 log2 e in the kernel's
  // base-2 units) the factors e^{-gv} stay far inside the fp32 range and the tile is the product md^T (nk, nq) (transposed, as the
  // other tiles below); beyond, it is summed pair by pair.
  float span = 0.f;
  for (int c = lane; c < D; c += 64) span = fmaxf(span, -sm.tot[w][c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) span = fmaxf(span, __shfl_xor(span, off, 64));
  const bool fast = __builtin_amdgcn_readfirstlane(__float_as_int(span)) <= __float_as_int(80.f * LOG2E);
  // Gram tiles of row block w, by k step s: tile (w, J) is computed
  // transposed (keys of block J as the M operand), so lane (r, g) holds row
  // 16w + r, columns 16J + 4g .. +3. For J < w the keys are those of block J
  // decayed to the start of block w (kd times the decay of the blocks
  // between, <= 1 per channel); tile (w, w) takes md. One k step's operands
  // are live at a time; each step's kd columns are published by a barrier.
  f32x4 ar[4], aa[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) ar[J] = aa[J] = f32x4{0.f, 0.f, 0.f, 0.f};
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
        const float e1 = exp2_(G);
        a[j] = kv[s][j] * e1;                        // nk
        c8[j] = (sc * qv[s][j]) * e1;                // nq
        b[j] = kv[s][j] * exp2_(-G);                 // md
        d[j] = kv[s][j] * exp2_(twv[jj] - G);        // kd
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
    Frag nk, nq;
    split8(a, nk);
    split8(c8, nq);
    {
      Frag fq;
      split8(f, fq);
      st_frag(rec, voff, RC::R2 + RC::wq(w, s), fq);
    }
    if (fast) {
      Frag md;
      split8(b, md);
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J == w) {
          if constexpr (DELTA) ar[J] = mm<true, true>(md, nk, ar[J]);
          aa[J] = mm<true, true>(md, nq, aa[J]);
        }
    }
    if (s + 1 == NS) {
      // (fenced, so that the loads are not hoisted above the operand work and
      // their registers stay free until here)
      __builtin_amdgcn_sched_barrier(0);
      prefetch();
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
#pragma unroll
    for (int J = 0; J < 3; ++J) {
      if (J < w) {
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
        if constexpr (DELTA) ar[J] = mm<true, true>(fk, nk, ar[J]);
        aa[J] = mm<true, true>(fk, nq, aa[J]);
      }
    }
  }
  // write strength and causal masks
  f32x4 rv[4], av[4];
  const float bi = sm.beta[i];
#pragma unroll
  for (int J = 0; J < 4; ++J)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = 4 * g + e;
      rv[J][e] = (J < w || (J == w && jj < r)) ? bi * ar[J][e] : 0.f;
      av[J][e] = (J < w || (J == w && jj <= r)) ? aa[J][e] : 0.f;
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
      st_frag(rec, voff, RC::R2 + RC::tp(pair_index(w, s)), f);
    }
  }
  // K_end^T fragments (update operands): the keys decayed to the chunk's
  // end, kd times the decay of the blocks after the key's own; wave w takes
  // fragments w, w + 4, ... (the row index passes through an empty asm so
  // that these LDS addresses are formed here, not kept live, or spilled,
  // across the whole item loop)
  int ro = r;
  asm volatile("" : "+v"(ro));
#pragma unroll
  for (int u = 0; u < NT / 2; ++u) {
    const int fi = w + 4 * u;
    const int m = fi >> 1, s = fi & 1;
    const int ch = 16 * m + ro, pc = perm32(ch);
    // tokens of slots 0-3 lie in block 2s, those of slots 4-7 in block 2s + 1
    const float fe0 = sm.fend[2 * s][ch], fe1 = sm.fend[2 * s + 1][ch];
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sm.kd[32 * s + slot_k(g, j)][pc] * (j < 4 ? fe0 : fe1);
    Frag f;
    split8(x, f);
    st_frag(rec, voff, RC::kf(m, s), f);
  }
  lds_barrier();   // kd is dead: its storage holds T from here on

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
    // (the identity from an opaque copy of the lane index: formed here
    // rather than hoisted out of the item loop and spilled)
    int lq = lane;
    asm volatile("" : "+v"(lq));
#pragma unroll
    for (int e = 0; e < 4; ++e) tq[e] = ((lq & 15) == 4 * (lq >> 4) + e) ? 1.f : 0.f;
    unit_lower_inverse16(tq, nn);
    *reinterpret_cast<float4 *>(&sm.t.tt[16 * w + r][16 * w + 4 * g]) = make_float4(tq[0], tq[1], tq[2], tq[3]);
  }
  lds_barrier();
  if (w == 1) t_block<1, 0, D>(sm, rv, r, g);
  if (w == 2) t_block<2, 1, D>(sm, rv, r, g);
  if (w == 3) t_block<3, 2, D>(sm, rv, r, g);
  lds_barrier();
  if (w == 2) t_block<2, 0, D>(sm, rv, r, g);
  if (w == 3) t_block<3, 1, D>(sm, rv, r, g);
  lds_barrier();
  if (w == 3) t_block<3, 0, D>(sm, rv, r, g);
  lds_barrier();

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
    if (pr % 4 == w) st_frag(rec, voff, RC::tp(pr), tf[pr]);

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
      st_frag(rec, voff, RC::R1 + RC::wq(I, w), f);
    }
  }
  }   // DELTA
    }
    lds_barrier();   // the next item reuses the LDS
  }
}

// ===========================================================================
// state kernel
// ===========================================================================

// One workgroup of four waves per (sequence, value head, 16 value columns).
// Wave q owns the chunk's token rows 16q .. 16q+15 (U, Vb and the outputs of
// those rows) and the key rows q D/4 .. (q+1) D/4 - 1 of S^T (their state and
// its update). Each wave loads the record fragments it multiplies straight
// from the workspace into registers (one set, each group of fragments
// reloaded with chunk c + 1's right after chunk c's last use of it), so the
// record never passes through LDS; LDS carries only what the waves exchange:
// the state's tiles (every wave reads S^T whole), the Vb tiles (every wave
// reads Vb whole) and the values, double-buffered by chunk parity, with two
// barriers per chunk that wait for LDS only.
template <int D>
struct StateSmem {
  static constexpr int NS = D / 32;
  static constexpr int VP = 32;                   // pitch (bf16) of the value tile
  // S^T and Vb as split B fragments, [parity][k step][lane]: the wave that
  // holds a 16-row tile splits it once and writes its half of the fragment
  // (words 0-1 of hi and lo for the even tile of a k step, 2-3 for the odd)
  u32x4 sfh[2][NS][64], sfl[2][NS][64];
  u32x4 vbh[2][2][64], vbl[2][2][64];
  alignas(16) uint16_t vv[2][C][VP];              // values: [parity][token][column]
};

// Split an accumulator tile and write it as half h of split fragment slot
// (hi, lo) of this lane.
__device__ __forceinline__ void put_half(u32x4 *hi, u32x4 *lo, int lane, int h, const f32x4 &t) {
  uint32_t h0, l0, h1, l1;
  split_pair(t[0], t[1], h0, l0);
  split_pair(t[2], t[3], h1, l1);
  *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(&hi[lane]) + 2 * h) = make_uint2(h0, h1);
  *reinterpret_cast<uint2 *>(reinterpret_cast<uint32_t *>(&lo[lane]) + 2 * h) = make_uint2(l0, l1);
}

__device__ __forceinline__ void get_frag(const u32x4 *hi, const u32x4 *lo, int lane, Frag &f) {
  f.hi = __builtin_bit_cast(bf16x8, hi[lane]);
  f.lo = __builtin_bit_cast(bf16x8, lo[lane]);
}

// Fragment at byte offset `off` of a record, through a buffer descriptor
// over it: the lane part of the address (16 bytes per lane) is a fixed
// register, the fragment's offset a scalar.
__device__ __forceinline__ void buf_frag(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int off, Frag &f) {
  f.hi = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, off, 0));
  f.lo = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, off + 1024, 0));
}

// The record fragments wave q multiplies in one chunk.
template <int D>
struct WaveOps {
  static constexpr int NS = D / 32, KT = D / 64;
  Frag w[NS];       // -W, row block q
  Frag t[2];        // T', row block q, k steps s <= q / 2
  Frag qh[NS];      // Q^, row block q
  Frag a[2];        // A^, row block q, k steps s <= q / 2
  Frag ke[KT][2];   // K_end^T, this wave's key tiles, k steps 0 and 1
  float4 gam[KT];   // gamma of the lane's four key rows in each of those tiles
};

// voff2 is the lane offset for the second k step of the lower-triangular
// operands: voff for row blocks 2 and 3, beyond the record for blocks 0 and 1
// (whose fragment is zero), so that such a load returns zeros and reads
// nothing. Every wave then issues the same loads and the compiler's wait
// counts stay exact.
template <int D>
__device__ __forceinline__ void load_r1(WaveOps<D> &o, __amdgpu_buffer_rsrc_t rs, int q, uint32_t voff,
                                        uint32_t voff2) {
  using RC = KdaRec<D>;
#pragma unroll
  for (int s = 0; s < RC::NS; ++s) buf_frag(rs, voff, RC::R1 + RC::wq(q, s), o.w[s]);
  buf_frag(rs, voff, RC::tp(pair_index(q, 0)), o.t[0]);
  buf_frag(rs, voff2, RC::tp(pair_index(max(q, 2), 1)), o.t[1]);
}

template <int D>
__device__ __forceinline__ void load_r2(WaveOps<D> &o, __amdgpu_buffer_rsrc_t rs, int q, uint32_t voff,
                                        uint32_t voff2) {
  using RC = KdaRec<D>;
#pragma unroll
  for (int s = 0; s < RC::NS; ++s) buf_frag(rs, voff, RC::R2 + RC::wq(q, s), o.qh[s]);
  buf_frag(rs, voff, RC::R2 + RC::tp(pair_index(q, 0)), o.a[0]);
  buf_frag(rs, voff2, RC::R2 + RC::tp(pair_index(max(q, 2), 1)), o.a[1]);
}

template <int D>
__device__ __forceinline__ void load_r3(WaveOps<D> &o, __amdgpu_buffer_rsrc_t rs, int q, uint32_t voff, int g) {
  using RC = KdaRec<D>;
  constexpr int KT = WaveOps<D>::KT;
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const int m = KT * q + t;
    buf_frag(rs, voff, RC::kf(m, 0), o.ke[t][0]);
    buf_frag(rs, voff, RC::kf(m, 1), o.ke[t][1]);
    const u32x4 gm = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(16 * g), RC::GAM + 64 * m, 0);
    o.gam[t] = make_float4(__uint_as_float(gm[0]), __uint_as_float(gm[1]), __uint_as_float(gm[2]),
                           __uint_as_float(gm[3]));
  }
}

// Values of the chunk starting at token t0 (L rows): wave q's 16 rows of the
// workgroup's 16 columns, 8 bytes per lane, through a buffer descriptor over
// the chunk's L rows of this head's columns: rows past the chunk's end fall
// outside it and read as zeros. vlane = row x (row pitch in bytes) + 8 (lane
// mod 4), the same for every chunk.
__device__ __forceinline__ uint2 load_vals(const KdaParams &p, int64_t t0, int L, int h, int D, int vb,
                                           uint32_t vlane) {
  const char *base = static_cast<const char *>(p.v) + (t0 * p.v_stride + (int64_t)h * D + 16 * vb) * 2;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), 0, (int)(L * p.v_stride * 2), 0x00020000);
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs, vlane, 0, 0);
  return make_uint2(x[0], x[1]);
}

// DELTA false: the linear rule (GLA), Vb = V; region 1 is neither written by
// the prep kernel nor read here.
template <int D, bool DELTA>
__global__ __launch_bounds__(256, 2) void kda_state_kernel(KdaParams p) {
  using RC = KdaRec<D>;
  using SM = StateSmem<D>;
  constexpr int NS = RC::NS, KT = WaveOps<D>::KT;
  constexpr int GRP = D / 16;   // workgroups per (sequence, value head)
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

  // (the wave index through readfirstlane: the compiler then knows it is
  // uniform, so the conditions on it below are scalar branches, never
  // exec-masked regions around MFMAs)
  const int tid = threadIdx.x, q = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15,
            g = lane >> 4;
  const int col = 16 * vb + r;                    // the value column this lane owns
  const int64_t slot = p.slot_idx[n];
  const int64_t pbase = (slot * p.HV + h) * (int64_t)(D * D) + col;
  // key row of element e of this wave's key tile t: 16 (KT q + t) + 4g + e
  auto key_row = [&](int t, int e) { return 16 * (KT * q + t) + 4 * g + e; };

  if (nc == 0) {
    // a zero-length sequence writes its initial state back: zeros under
    // ZERO_INIT (once, in the slice holding its flat index), else nothing
    if (p.zero_init && base >= p.F0 && base < p.F1) {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t idx = pbase + (int64_t)key_row(t, e) * D;
          if (p.st_bf16) static_cast<uint16_t *>(p.pool)[idx] = 0;
          else static_cast<float *>(p.pool)[idx] = 0.f;
        }
    }
    return;
  }
  if (cb >= ce) return;

  auto rec_of = [&](int64_t c) -> __amdgpu_buffer_rsrc_t {
    const char *rec = p.rec + ((base + c - p.F0) * p.HV + h) * (int64_t)RC::BYTES;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(rec), 0, RC::BYTES, 0x00020000);
  };
  const uint32_t voff = 16u * (uint32_t)lane;
  uint32_t voff2 = q >= 2 ? voff : 0x80000000u;
  asm volatile("" : "+v"(voff2));
  auto len_of = [&](int64_t c) { return (int)min<int64_t>(C, eos - (bos + C * c)); };

  // ---- the state's tiles: the pool (or zeros) at the sequence's start, the
  //      carry between slices ----
  f32x4 st[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t kr = key_row(t, e);
      if (cb > 0) {
        st[t][e] = p.carry[((int64_t)n * p.HV + h) * (int64_t)(D * D) + kr * D + col];
      } else if (!p.zero_init) {
        const int64_t idx = pbase + kr * D;
        st[t][e] = p.st_bf16 ? bf16_to_f32(static_cast<const uint16_t *>(p.pool)[idx])
                             : static_cast<const float *>(p.pool)[idx];
      }
    }
  }

  // (Barriers wait for LDS only, lds_barrier: the next chunk's operand loads
  // stay in flight across them.)

  // The record operands in one register set: each group of fragments is
  // reloaded with chunk c + 1's right after chunk c's last use of it (W and
  // T' after Vb, Q^ and A^ after the outputs, K_end and gamma after the
  // update), so every load has about a chunk's time to land while the
  // registers stay within two workgroups per compute unit.
  WaveOps<D> ops;
  // this wave's state tiles as halves of the split S^T fragments
  auto publish_state = [&](int par) {
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int m = KT * q + t;
      put_half(sm.sfh[par][m >> 1], sm.sfl[par][m >> 1], lane, m & 1, st[t]);
    }
  };
  // values of the next chunk, loaded two chunks ahead of their use;
  // vlane = row x (row pitch in bytes) + 8 (lane mod 4)
  const uint32_t vlane = (uint32_t)((16 * q + (lane >> 2)) * p.v_stride * 2) + 8u * (uint32_t)(lane & 3);
  uint2 vq;
  {
    const __amdgpu_buffer_rsrc_t rec = rec_of(cb);
    if constexpr (DELTA) load_r1<D>(ops, rec, q, voff, voff2);
    load_r2<D>(ops, rec, q, voff, voff2);
    load_r3<D>(ops, rec, q, voff, g);
    const uint2 v0 = load_vals(p, bos + C * cb, len_of(cb), h, D, vb, vlane);
    const int64_t c1 = min(cb + 1, ce - 1);
    vq = load_vals(p, bos + C * c1, len_of(c1), h, D, vb, vlane);
    const int par = (int)(cb & 1);
    publish_state(par);
    *reinterpret_cast<uint2 *>(&sm.vv[par][16 * q + (lane >> 2)][4 * (lane & 3)]) = v0;
  }
  lds_barrier();

  const int64_t HVD = (int64_t)p.HV * D;
  // output rows of this lane: 16q + 4g + e, at e row pitches past the lane
  // offset, which is the same for every chunk; both widths are issued, the
  // other one at a lane offset beyond the chunk's descriptor, so that no
  // branch makes the compiler's wait counts assume fewer stores in flight
  const uint32_t osz = p.out_bf16 ? 2u : 4u;
  const uint32_t orow = (uint32_t)HVD * osz;
  const uint32_t olane = (uint32_t)(16 * q + 4 * g) * orow + (uint32_t)col * osz;
  uint32_t olane32 = p.out_bf16 ? 0x80000000u : olane, olane16 = p.out_bf16 ? olane : 0x80000000u;
  asm volatile("" : "+v"(olane32), "+v"(olane16));
  const int nts = q < 2 ? 1 : 2;   // k steps of row block q's lower-triangular operands
  auto chunk = [&](int64_t c) {
    const int par = (int)(c & 1);
    // The next chunk's loads are issued on every chunk, the last one
    // reloading its own record (unused): with loads under a branch the
    // compiler's wait counts must assume the branch that issued none, and a
    // wait for one group of operands then also waits for every load issued
    // after it.
    const bool more = c + 1 < ce;
    const __amdgpu_buffer_rsrc_t nrec = rec_of(more ? c + 1 : c);
    const int64_t c2 = min(c + 2, ce - 1);
    const uint2 vload = load_vals(p, bos + C * c2, len_of(c2), h, D, vb, vlane);

    // ---- S^T as B fragments over key rows 32s .. 32s + 31 ----
    Frag sf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) get_frag(sm.sfh[par][s], sm.sfl[par][s], lane, sf[s]);

    // ---- Vb rows of block q: U = T' V, then + (-W) S^T (the record holds
    //      -W); even and odd k steps in two accumulators ----
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DELTA) {
      Frag vf[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        if (s < nts) ldfrag_tr(&sm.vv[par][0][0], SM::VP, 4 * (r & 3), s, r, g, vf[s]);
      f32x4 a0 = acc, a1 = acc;
      a0 = mm<true, false>(ops.t[0], vf[0], a0);
      if (nts > 1) a1 = mm<true, false>(ops.t[1], vf[1], a1);
#pragma unroll
      for (int s = 0; s < NS; s += 2) {
#pragma unroll
        for (int ps = 0; ps < 3; ++ps) {
          if (ps == 0) { a0 = mm_pass<0, true, true>(ops.w[s], sf[s], a0); a1 = mm_pass<0, true, true>(ops.w[s + 1], sf[s + 1], a1); }
          if (ps == 1) { a0 = mm_pass<1, true, true>(ops.w[s], sf[s], a0); a1 = mm_pass<1, true, true>(ops.w[s + 1], sf[s + 1], a1); }
          if (ps == 2) { a0 = mm_pass<2, true, true>(ops.w[s], sf[s], a0); a1 = mm_pass<2, true, true>(ops.w[s + 1], sf[s + 1], a1); }
        }
      }
      acc = a0 + a1;
    } else {
      // linear rule: Vb = V, read in the accumulator layout (row 16q + 4g + i)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = bf16_to_f32(sm.vv[par][16 * q + 4 * g + i][r]);
    }
    put_half(sm.vbh[par][q >> 1], sm.vbl[par][q >> 1], lane, q & 1, acc);
    if constexpr (DELTA) load_r1<D>(ops, nrec, q, voff, voff2);
    lds_barrier();

    // ---- Vb as B fragments over tokens 32s .. 32s + 31 ----
    Frag vbf[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) get_frag(sm.vbh[par][s], sm.vbl[par][s], lane, vbf[s]);

    // ---- outputs of row block q: O = Q^ S^T + A^ Vb ----
    {
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
#pragma unroll
      for (int s = 0; s < NS; s += 2) {
        o0 = mm_pass<0, true, true>(ops.qh[s], sf[s], o0);
        o1 = mm_pass<0, true, true>(ops.qh[s + 1], sf[s + 1], o1);
        o0 = mm_pass<1, true, true>(ops.qh[s], sf[s], o0);
        o1 = mm_pass<1, true, true>(ops.qh[s + 1], sf[s + 1], o1);
        o0 = mm_pass<2, true, true>(ops.qh[s], sf[s], o0);
        o1 = mm_pass<2, true, true>(ops.qh[s + 1], sf[s + 1], o1);
      }
      o0 = mm<true, true>(ops.a[0], vbf[0], o0);
      if (nts > 1) o1 = mm<true, true>(ops.a[1], vbf[1], o1);
      const f32x4 oa = o0 + o1;
      // buffer stores against a descriptor over this chunk's L output rows:
      // rows past a partial chunk's end fall outside it and are dropped
      const int64_t t0 = bos + C * c;
      const int L = len_of(c);
      char *obase = static_cast<char *>(p.o) + (t0 * HVD + (int64_t)h * D) * osz;
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(obase, 0, (int)(L * orow), 0x00020000);
      const bf16x2 b01 = {static_cast<__bf16>(oa[0]), static_cast<__bf16>(oa[1])};
      const bf16x2 b23 = {static_cast<__bf16>(oa[2]), static_cast<__bf16>(oa[3])};
      const uint32_t w01 = __builtin_bit_cast(uint32_t, b01), w23 = __builtin_bit_cast(uint32_t, b23);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[e]), ors, olane32, e * (int)orow, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w01, ors, olane16, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w01 >> 16), ors, olane16, (int)orow, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w23, ors, olane16, 2 * (int)orow, 0);
      __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w23 >> 16), ors, olane16, 3 * (int)orow, 0);
    }

    load_r2<D>(ops, nrec, q, voff, voff2);

    // ---- this wave's key rows: S^T <- gamma (.) S^T + K_end^T Vb ----
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      // (gamma through an opaque copy here: hoisted into the Vb products
      // instead, its wait would stall them on loads issued at the end of
      // the previous chunk)
      float4 gm = ops.gam[t];
      asm volatile("" : "+v"(gm.x), "+v"(gm.y), "+v"(gm.z), "+v"(gm.w));
      st[t][0] *= gm.x;
      st[t][1] *= gm.y;
      st[t][2] *= gm.z;
      st[t][3] *= gm.w;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ps = 0; ps < 3; ++ps)
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          if (ps == 0) st[t] = mm_pass<0, true, true>(ops.ke[t][s], vbf[s], st[t]);
          if (ps == 1) st[t] = mm_pass<1, true, true>(ops.ke[t][s], vbf[s], st[t]);
          if (ps == 2) st[t] = mm_pass<2, true, true>(ops.ke[t][s], vbf[s], st[t]);
        }

    load_r3<D>(ops, nrec, q, voff, g);

    // ---- publish the next chunk's state fragments and values ----
    publish_state(par ^ 1);
    if (more) *reinterpret_cast<uint2 *>(&sm.vv[par ^ 1][16 * q + (lane >> 2)][4 * (lane & 3)]) = vq;
    vq = vload;
    lds_barrier();
  };
  // (the first chunk peeled: the loop's first wait then follows a chunk's
  // loads, as on every later iteration, not the prologue's different order)
  chunk(cb);
  for (int64_t c = cb + 1; c < ce; ++c) chunk(c);

  // ---- state out: the pool at the sequence's end, else the carry ----
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t kr = key_row(t, e);
      if (ce == nc) {
        const int64_t idx = pbase + kr * D;
        if (p.st_bf16) static_cast<uint16_t *>(p.pool)[idx] = rne_bf16(st[t][e]);
        else static_cast<float *>(p.pool)[idx] = st[t][e];
      } else {
        p.carry[((int64_t)n * p.HV + h) * (int64_t)(D * D) + kr * D + col] = st[t][e];
      }
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

// Records per slice, at most: about 128 MB for the delta rule, 192 MB for
// the linear rule (whose prep kernel is lighter). On the 131072-token,
// 32-head KDA call, slices of 16, 32, 48 and 64 chunk rows (60 to 240 MB)
// took 7.9, 7.3, 7.4 and 8.8 ms: larger slices find fewer of their records
// still in the 256 MB last-level cache when the state kernel reads them,
// smaller ones pay more per-slice launch and drain. GLA took 5.7 ms with 48
// rows and 5.9 ms with 32.
size_t slice_record_bytes(const gdr_args &a) {
  return (size_t)(a.rule == GDR_RULE_DELTA ? 128 : 192) << 20;
}

int64_t slice_rows(const gdr_args &a) {
  const size_t row = record_bytes(a.DK) * (size_t)a.HV;
  int64_t per = (int64_t)(slice_record_bytes(a) / row);
  if (per < 1) per = 1;
  const int64_t wg = 2 * (int64_t)cu_count();
  const int64_t q = wg / std::gcd(wg, (int64_t)a.HV);
  if (per >= q) per = per / q * q;
  return per;
}

template <int D>
void launch_prep(const KdaParams &p, int64_t blocks, hipStream_t stream) {
  if (p.delta)
    hipLaunchKernelGGL((kda_prep_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kda_prep_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
}

template <int D>
void launch_state(const KdaParams &p, hipStream_t stream) {
  const int blocks = ((p.N * p.HV + 7) / 8) * 8 * (D / 16);
  if (p.delta)
    hipLaunchKernelGGL((kda_state_kernel<D, true>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((kda_state_kernel<D, false>), dim3(blocks), dim3(256), 0, stream, p);
}

KdaParams slice_of(const KdaParams &p0, int64_t F0, int64_t per, int64_t flat, char *rec) {
  KdaParams p = p0;
  p.F0 = F0;
  p.F1 = F0 + per < flat ? F0 + per : flat;
  p.rec = rec;
  return p;
}

// Each slice: its prep launch (two workgroups per compute unit), then its
// state launch. (Running the next slice's prep beside this slice's state
// kernel, one workgroup of each per compute unit, was slower: each kernel
// then took about twice as long.)
template <int D>
hipError_t launch_slices(const KdaParams &p0, int64_t flat, int64_t per, hipStream_t stream) {
  const int64_t cap = 2 * (int64_t)cu_count();
  for (int64_t F0 = 0; F0 < flat; F0 += per) {
    const KdaParams p = slice_of(p0, F0, per, flat, p0.rec);
    const int64_t items = (p.F1 - p.F0) * p.HV;
    launch_prep<D>(p, items < cap ? items : cap, stream);
    launch_state<D>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t kda_wait_flag(int *out, bool clear, hipStream_t stream) {
  return chunk::wait_flag_access(out, clear, stream);
}

bool chunk_fwd_kda_applies(const gdr_args &a) {
  return a.in_dtype == GDR_BF16 && a.gate == GDR_GATE_CHANNEL && products_of(a) == 1 && a.chunk_size == 64;
}

size_t chunk_fwd_kda_min_workspace(const gdr_args &a) {
  return carry_bytes(a) + record_bytes(a.DK) * (size_t)a.HV;
}

size_t chunk_fwd_kda_workspace(const gdr_args &a) {
  const size_t row = record_bytes(a.DK) * (size_t)a.HV;   // one flat chunk of every head
  int64_t per = slice_rows(a);
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
  p.F0 = p.F1 = 0;
  // (16 value columns per state workgroup: the record's fragments are read
  // by every workgroup of a (sequence, head) from the L2 they share; narrow
  // workgroups spread that traffic over many compute units)
  int64_t per = (int64_t)((ws_bytes - cb) / row);
  const int64_t cap = slice_rows(a);   // (a larger workspace does not make larger slices)
  if (per > cap) per = cap;
  if (per > flat) per = flat;
  if (a.DK == 128) return launch_slices<128>(p, flat, per, stream);
  return launch_slices<64>(p, flat, per, stream);
}

}  // namespace gdr
